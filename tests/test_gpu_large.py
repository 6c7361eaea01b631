"""GPU parity past 32-bit offsets: the RWKV-4 forward and backward on 2^30-element bf16 inputs,
whose float32 outputs span 4 GiB, against the float64 C oracle on a sample of whole channels.

Every lane (batch row, channel) of the recurrence is independent ("RWKV（Receptance Weighted Key
Value）概念", section 3.2: the weighted sum runs per channel), so the oracle run on the sampled
channels' full sequences gives those channels' outputs exactly, and dw, du (sums over batch rows
and tokens of one channel) for them too.  Two shapes: B=8 T=32768 C=4096 takes the whole-tile
kernels, B=1 T=262144 C=4096 the time-split ones with chained carries.  Inputs follow the bf16
workload (1 % key spikes), drawn on the device.  Bounds as for the bf16 workload: y rtol 2e-3,
gradients rtol 1e-3 (atol as in the other parity tests)."""
import numpy as np
import pytest
import torch

from _helpers import bwd_atol, check_close
from oracle.ctwin import ctwin_backward, ctwin_forward
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def host(t):
    return t.float().cpu().numpy()


@pytest.mark.parametrize("B,T,C", [(8, 32768, 4096), (1, 262144, 4096)])
def test_outputs_beyond_4gib(B, T, C):
    from rwkv_wkv_mixing_amd import ops

    assert B * T * C == 1 << 30
    print(f"case large bf16 B={B} T={T} C={C}: inputs", flush=True)
    w, u, k, v, gy = W.large_bf16_torch(B, T, C, seed=B * 7 + 5, device=DEV)
    wd, ud = torch.from_numpy(w).to(DEV), torch.from_numpy(u).to(DEV)
    print("  forward", flush=True)
    y = ops.wkv_forward(wd, ud, k, v)
    torch.cuda.synchronize()
    # whole channels from the first, a middle and the last tile, and a seeded scatter
    rng = np.random.default_rng(11)
    cols = np.unique(np.concatenate([np.arange(0, 16), np.arange(2040, 2056), np.arange(C - 16, C),
                                     rng.choice(C, 16, replace=False)]))
    ci = torch.from_numpy(cols).to(DEV)
    ys = host(y.index_select(2, ci))
    del y
    print("  backward", flush=True)
    dk, dv, dw, du = ops.wkv_backward(wd, ud, k, v, gy)
    torch.cuda.synchronize()
    got = (host(dk.index_select(2, ci)), host(dv.index_select(2, ci)), host(dw[ci]), host(du[ci]))
    del dk, dv
    ks, vs, gs = (np.ascontiguousarray(host(t.index_select(2, ci))) for t in (k, v, gy))
    del k, v, gy
    torch.cuda.empty_cache()
    print(f"  oracle on {cols.size} channels", flush=True)
    ref_y = ctwin_forward(w[cols], u[cols], ks, vs)[0]
    check_close(f"large B={B} T={T} y (bf16 bound)", ys, ref_y, 2e-3, 2e-5 * rms(ref_y))
    rk, rv, rw, ru = ctwin_backward(w[cols], u[cols], ks, vs, gs)[:4]
    for n, g_, r_ in (("dk", got[0], rk), ("dv", got[1], rv), ("dw", got[2], rw), ("du", got[3], ru)):
        check_close(f"large B={B} T={T} {n}", g_, r_, 1e-3, bwd_atol(r_, gy=gs, v=vs))


# ---- the matrix-state calls (RWKV-5 and RWKV-6) past 4 GiB -----------------------------------
# Every (batch row, head) pair is independent ("RWKV模型深度研究报告", sections 1.3.2-1.3.3: one
# state per head), so the oracle on one head's full sequences gives that head's outputs, and its
# dw, du (sums over the batch rows) when every row of the head is taken.  Bounds and norm checks
# as in the matrix-state parity tests.

def _head(x, b, h):
    """Pair (b, h) of a [B, T, 64 H] device tensor as a float64 host array [1, T, 64]."""
    return x[b:b + 1, :, 64 * h:64 * h + 64].double().cpu().numpy()


@pytest.mark.parametrize("gen,B,T,H,rows", [(5, 8, 32768, 64, (7,)), (5, 1, 262144, 64, (0,)),
                                             (6, 8, 32768, 64, (7,))])
def test_matrix_state_beyond_4gib(gen, B, T, H, rows):
    """2^30-element bf16 inputs: RWKV-5 and RWKV-6 at B=8 T=32768 (512 pairs: one workgroup walks
    each sequence) and RWKV-5 at B=1 T=262144 (64 pairs: both calls split each sequence into
    segments chained through the state); forward (outputs, final state) and backward of the last
    head in the given batch rows against the oracle; RWKV-5's dw and du (sums over the batch rows)
    where every row is taken, RWKV-6's du at B = 1 (its dw is per token, checked with the rest)."""
    import test_gpu_wkv5 as F5
    import test_gpu_wkv5_bwd as B5
    import test_gpu_wkv6 as F6
    import test_gpu_wkv6_bwd as B6
    from oracle import wkv5_backward_ref
    from rwkv_wkv_mixing_amd import ops

    assert B * T * 64 * H == 1 << 30
    print(f"case large wkv{gen} B={B} T={T} H={H}: inputs", flush=True)
    w, u, r, k, v, go, _ = W.large_matrix_torch(gen, B, T, H, seed=gen * 10 + B, device=DEV)
    wd = torch.from_numpy(w).to(DEV) if gen == 5 else w
    ud = torch.from_numpy(u).to(DEV)
    fwd, bwd = (ops.wkv5_forward, ops.wkv5_backward) if gen == 5 else (ops.wkv6_forward, ops.wkv6_backward)
    print("  forward", flush=True)
    o, S = fwd(wd, ud, r, k, v, return_state=True)
    torch.cuda.synchronize()
    h = H - 1
    o_h = {b: _head(o, b, h) for b in rows}
    S_h = S[:, h:h + 1].cpu().numpy()
    del o, S
    print("  backward", flush=True)
    got = bwd(wd, ud, r, k, v, go, need_state_grad=True)
    torch.cuda.synchronize()
    per_tok = (0, 1, 2) if gen == 5 else (0, 1, 2, 3)  # dr, dk, dv (and RWKV-6's per-token dw)
    g_h = {i: {b: _head(got[i], b, h) for b in rows} for i in per_tok}
    all_rows = len(rows) == B
    g_sum = {i: got[i][h:h + 1].cpu().numpy() for i in ((3, 4) if gen == 5 else (4,))}  # [1, 64]
    g_ds = got[5][:, h:h + 1].cpu().numpy()
    del got
    sums = {}
    for b in rows:
        name = f"large wkv{gen} B={B} T={T} pair ({b}, {h})"
        print(f"  oracle {name}", flush=True)
        rb, kb, vb, gb = (_head(t, b, h) for t in (r, k, v, go))
        wb = w[h:h + 1] if gen == 5 else _head(w, b, h)
        p = W.Wkv5Problem(name, 1, T, 1, wb, u[h:h + 1], rb, kb, vb, None, None, None, None)
        (F5 if gen == 5 else F6).check(p, torch.from_numpy(o_h[b]), torch.from_numpy(S_h[b:b + 1]))
        mine = [g_h[i][b] if i in g_h else None for i in range(5)] + [g_ds[b:b + 1]]
        if gen == 5:
            ref = wkv5_backward_ref(p.w, p.u, p.r, p.k, p.v, gb, 1)
            bnd = B5.bounds(p.w.astype(np.float64), p.u, p.r, p.k, p.v, gb, 1, None, None)
            for i in (0, 1, 2, 5):
                B5.check_bound(f"{name} {B5.NAMES[i]}", mine[i], ref[i], bnd[i])
                B5.check_norm(f"{name} {B5.NAMES[i]}", mine[i], ref[i])
            for i in (3, 4):
                sums.setdefault(i, [0.0, 0.0])
                sums[i][0] = sums[i][0] + ref[i]
                sums[i][1] = sums[i][1] + bnd[i]
        else:
            mine[4] = g_sum[4] if B == 1 else None  # du sums over the rows: one row holds it all only at B = 1
            B6.check(p, gb, mine, name=name)
    for i in (sums if all_rows else ()):
        B5.check_bound(f"large wkv5 head {h} {B5.NAMES[i]} (all rows)", g_sum[i], sums[i][0], sums[i][1])
        B5.check_norm(f"large wkv5 head {h} {B5.NAMES[i]} (all rows)", g_sum[i], sums[i][0])
