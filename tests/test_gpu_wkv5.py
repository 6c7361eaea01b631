"""GPU parity of the RWKV-5 matrix-state WKV (wkv5_forward) against the float64
oracle, through the C ABI.

Bound, from the arithmetic of the kernel (bf16 matrix-core operands, float32
accumulation and state; ub = 2^-8 is the unit roundoff of bf16, whose 8
significant bits round to nearest within 2^-8 relative): every term of an
output passes through at most three bf16 roundings (the decay-scaled
receptance, the decay-scaled key or the bf16 copy of the state, and the
attention entry), so
    |o_gpu - o| <= (3 ub (1 + 2^-7) + 2^-17) * o_abs,
with o_abs the oracle run on |r|, |k|, |v|, |u|, |S0| (every term made
non-negative: the sum of the terms' magnitudes); 2^-17 covers float32
accumulation over at most a few hundred terms per stage.  The final state's
terms pass through one rounding (the scaled key): (ub (1 + 2^-7) + 2^-17) S_abs.
A dropped term, a wrong decay exponent or a transposed operand exceeds these
bounds by orders of magnitude (the bounds are ~1.2 % of the magnitudes summed).
"""
import numpy as np
import pytest
import torch

from _helpers import to_dev
from oracle import wkv5_forward_ref
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UB = 2.0 ** -8
C_O = 3 * UB * (1 + 2.0 ** -7) + 2.0 ** -17
C_S = UB * (1 + 2.0 ** -7) + 2.0 ** -17


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def check_bound(name, got, ref, bound):
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    err = np.abs(g - o)
    ratio = err / (np.asarray(bound, dtype=np.float64) + 1e-30)
    worst = float(ratio.max(initial=0.0))
    print(f"  {name}: max_abs={float(err.max(initial=0.0)):.3e} worst_err/bound={worst:.3f}", flush=True)
    if worst > 1.0:
        idx = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError(f"{name}: {int((ratio > 1).sum())} of {ratio.size} out of bound; worst at {idx}: "
                             f"got {g[idx]!r} ref {o[idx]!r} bound {np.asarray(bound)[idx]!r}")


def dev_inputs(p):
    bt = lambda bits: to_dev(None, DEV, bits)
    d = dict(w=to_dev(p.w, DEV), u=to_dev(p.u, DEV), r=bt(p.r_bits), k=bt(p.k_bits), v=bt(p.v_bits))
    d["S0"] = None if p.S0 is None else to_dev(p.S0, DEV)
    return d



NORM_TOL = 2.0 ** -7


def check_norm(name, got, ref):
    """Normwise accuracy on random inputs: ||got - ref|| <= 2^-7 ||ref||.  Not a rounding bound:
    it checks that the errors do not add up coherently, which a magnitude-sum bound cannot see
    where a signed sum cancels."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    nr, ne = float(np.linalg.norm(r)), float(np.linalg.norm(g - r))
    print(f"  {name}: normwise relative error {ne / nr if nr else ne:.2e}", flush=True)
    assert (ne == 0.0) if nr == 0.0 else (ne <= NORM_TOL * nr), (name, ne, nr)


def check(p, o, S, S0=None, name=None):
    S0 = p.S0 if S0 is None else S0
    ref_o, ref_S = wkv5_forward_ref(p.w, p.u, p.r, p.k, p.v, p.H, S0)
    abs_o, abs_S = wkv5_forward_ref(p.w, np.abs(p.u), np.abs(p.r), np.abs(p.k), np.abs(p.v), p.H,
                                    None if S0 is None else np.abs(S0))
    name = name or p.name
    check_bound(f"{name} o", o.cpu().numpy(), ref_o, C_O * abs_o)
    check_norm(f"{name} o", o.cpu().numpy(), ref_o)
    if S is not None:
        check_bound(f"{name} state", S.cpu().numpy(), ref_S, C_S * abs_S)
        check_norm(f"{name} state", S.cpu().numpy(), ref_S)


SHAPES = [(2, 1, 1), (1, 63, 2), (2, 64, 1), (1, 65, 1), (2, 200, 3), (1, 1000, 2), (3, 129, 4)]


@pytest.mark.parametrize("B,T,H", SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_shapes(B, T, H, with_state):
    """Whole and ragged chunks of 64 tokens, one to several heads, from the zero
    state and from a given one."""
    p = W.make_wkv5(B, T, H, seed=B * 100 + T + H, with_state=with_state)
    print(f"case {p.name} state={with_state}", flush=True)
    d = dev_inputs(p)
    o, S = ops().wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    torch.cuda.synchronize()
    check(p, o, S)


@pytest.mark.parametrize("rates", [(20.0, 80.0), (1e-6, 1e-3), (8.0, 12.0)])
def test_extreme_decay_rates(rates):
    """Decay factors from e^{-80} (every older term vanishes) to nearly 1, and
    around the in-block cap of 10."""
    p = W.make_wkv5(2, 150, 2, seed=7, with_state=True)
    p.w[:] = np.exp(np.random.default_rng(8).uniform(np.log(rates[0]), np.log(rates[1]), p.w.shape)).astype(np.float32)
    print(f"case rates {rates}", flush=True)
    d = dev_inputs(p)
    o, S = ops().wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    torch.cuda.synchronize()
    check(p, o, S, name=f"rates {rates}")


def test_split_sequence_through_the_state():
    p = W.make_wkv5(2, 300, 2, seed=9)
    print(f"case split {p.name}", flush=True)
    d = dev_inputs(p)
    O = ops()
    for t1 in (1, 64, 100):
        sl = lambda x, a, b: x[:, a:b].contiguous()
        o1, S1 = O.wkv5_forward(d["w"], d["u"], sl(d["r"], 0, t1), sl(d["k"], 0, t1), sl(d["v"], 0, t1),
                                return_state=True)
        o2, S2 = O.wkv5_forward(d["w"], d["u"], sl(d["r"], t1, 300), sl(d["k"], t1, 300), sl(d["v"], t1, 300),
                                state_in=S1, state_out=S1, return_state=True)
        torch.cuda.synchronize()
        check(p, torch.cat([o1, o2], dim=1), S2, name=f"split at {t1}")


def test_zero_length_and_determinism():
    p = W.make_wkv5(2, 130, 3, seed=10, with_state=True)
    d = dev_inputs(p)
    O = ops()
    z = torch.zeros((2, 0, 192), dtype=torch.bfloat16, device=DEV)
    S = torch.full((2, 3, 64, 64), 9.0, device=DEV)
    O.wkv5_forward(d["w"], d["u"], z, z, z, state_in=d["S0"], state_out=S)
    torch.cuda.synchronize()
    assert torch.equal(S, d["S0"])
    O.wkv5_forward(d["w"], d["u"], z, z, z, state_out=S)
    torch.cuda.synchronize()
    assert torch.all(S == 0)
    a = O.wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    b = O.wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_bench_shape_every_head():
    """The 7B-shaped layer (B=8, T=1024, 64 heads of 64) in the launch the bench
    times: every output and the final state of every (batch row, head) against
    the oracle, one batch row (all 64 heads) at a time."""
    p = W.wkv5_config()
    print(f"case {p.name}", flush=True)
    d = dev_inputs(p)
    o, S = ops().wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], return_state=True)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    S = S.cpu().numpy()
    for b in range(p.B):
        q = W.Wkv5Problem(f"bench row {b}", 1, p.T, p.H, p.w, p.u, p.r[b:b + 1], p.k[b:b + 1], p.v[b:b + 1],
                          None, None, None, None)
        check(q, torch.from_numpy(o[b:b + 1]), torch.from_numpy(S[b:b + 1]))


def test_long_sequence_slow_decay():
    """4,096 tokens (64 chunks) with decay rates 1e-4 to 1e-2, so the state
    carries most of its history through every chunk: float32 rounding of the
    carried state accumulates most here."""
    p = W.make_wkv5(1, 4096, 1, seed=31, with_state=True)
    p.w[:] = np.exp(np.random.default_rng(32).uniform(np.log(1e-4), np.log(1e-2), p.w.shape)).astype(np.float32)
    print(f"case {p.name} slow decay", flush=True)
    d = dev_inputs(p)
    o, S = ops().wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    torch.cuda.synchronize()
    check(p, o, S, name="long slow decay")


def test_decode_steps_in_place():
    """Decoding: 40 single-token calls, each carrying the state in place (state_in = state_out),
    equal the oracle over the 40 tokens.  One token takes the float32 one-token kernel: each term
    of an output is exact up to float32 rounding of a 64-term sum and of the state carried over
    the steps, so |o - ref| <= (64 + 2 T) 2^-24 o_abs, and the same for the state."""
    p = W.make_wkv5(3, 40, 2, seed=71, with_state=True)
    d = dev_inputs(p)
    O = ops()
    S = d["S0"].clone()
    outs = []
    for t in range(p.T):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(O.wkv5_forward(d["w"], d["u"], sl(d["r"]), sl(d["k"]), sl(d["v"]), state_in=S, state_out=S))
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).cpu().numpy()
    ref_o, ref_S = wkv5_forward_ref(p.w, p.u, p.r, p.k, p.v, p.H, p.S0)
    abs_o, abs_S = wkv5_forward_ref(p.w, np.abs(p.u), np.abs(p.r), np.abs(p.k), np.abs(p.v), p.H, np.abs(p.S0))
    c = (64 + 2 * p.T) * 2.0 ** -24
    check_bound("decode o", o, ref_o, c * abs_o)
    check_bound("decode state", S.cpu().numpy(), ref_S, c * abs_S)


@pytest.mark.parametrize("T", [2, 5, 16, 17])
def test_few_tokens(T):
    """Up to 16 tokens take the token-by-token kernel (float32: within (64 + 2T) 2^-24 of the
    magnitudes); 17 takes the chunked one (its bound)."""
    p = W.make_wkv5(3, T, 2, seed=80 + T, with_state=True)
    d = dev_inputs(p)
    o, S = ops().wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], return_state=True)
    torch.cuda.synchronize()
    check(p, o, S, name=f"T={T}")
    if T <= 16:
        ref_o, ref_S = wkv5_forward_ref(p.w, p.u, p.r, p.k, p.v, p.H, p.S0)
        abs_o, abs_S = wkv5_forward_ref(p.w, np.abs(p.u), np.abs(p.r), np.abs(p.k), np.abs(p.v), p.H, np.abs(p.S0))
        c = (64 + 2 * T) * 2.0 ** -24
        check_bound(f"T={T} o (float32)", o.cpu().numpy(), ref_o, c * abs_o)
        check_bound(f"T={T} state (float32)", S.cpu().numpy(), ref_S, c * abs_S)


def test_time_split_long_sequence():
    """Few (batch row, head) pairs: the sequence splits into segments run in parallel (here 8 of
    2 chunks); outputs and final state within the bound, the state carried in place, and the
    saved chunk-start states within one bf16 rounding of the unsplit run's."""
    p = W.make_wkv5(1, 1000, 2, seed=101, with_state=True)
    assert ops().L.lib().wkv5_forward_workspace_bytes(1, 1000, 2, 64) > 0
    d = dev_inputs(p)
    O = ops()
    cks, outs = [], []
    for split in (True, False):
        S = d["S0"].clone()
        ck = O.new_wkv5_ckpt(1, 1000, 2, DEV)
        o = O.wkv5_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=S, state_out=S, ckpt=ck, split=split)
        torch.cuda.synchronize()
        check(p, o, S, name=f"split={split}")
        n = 2 * 16 * 64 * 64
        cks.append(ck[: 2 * n].view(torch.bfloat16).float())
        outs.append(o)
    assert torch.allclose(cks[0], cks[1], rtol=2.0 ** -7, atol=1e-30)
