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
