"""GPU parity of the RWKV-6 backward (wkv6_backward) against the float64 oracle,
through the C ABI.

Bound, from the kernel's arithmetic (bf16 matrix-core operands, float32
accumulation, adjoint state and tables; ub = 2^-8 the unit roundoff of bf16).
As for RWKV-5, every term of dr, dk, dv and dw passes through at most three
bf16 roundings:
  dv: the decay-scaled key and the bf16 copy of the adjoint state G (itself a
      sum of terms with one rounding), or the scaled receptance and key and the
      bf16 attention entry;
  dk: the bf16 G (two), or the bf16 C = go v^T entry and the scaled receptance;
  dr: the bf16 chunk-start state (two), or the bf16 C entry and the scaled key;
  dw: the bf16 G or chunk-start state (two), or the bf16 C entry and a scaled
      receptance or key (two); its pairs inside one 16-token block are float32
      elementwise.
The decay factors come from float32 cumulative rates (sums of up to 64 capped
rates, largest in-chunk sum Emax): each factor's exponent is off by at most
2^-17 Emax.  A term carries at most two such factors inside a chunk, and the
adjoint state and chunk-start state carry their own from other chunks, which
are smaller the more chunks they span (x e^{-x} <= 1/e); 2^-15 Emax covers
them.  fp = 2^-12 covers float32 rounding (prefix sums and products of at most
a few hundred terms per chunk).  Rates above 10 act as 10: every term's decay
then lies between the true one and that of w' = min(w, 10), so the bound adds
x_abs(w') - x_abs(w) and takes the rounding part on the w' magnitudes:
    |x_gpu - x| <= (3 ub (1 + 2^-7) + fp + 2^-15 Emax) x_abs(w') + (x_abs(w') - x_abs(w))
with x_abs the oracle run on |r|, |k|, |v|, |go|, |u|, |S0|, |dS_T|.
dS0 = G before the first token: one rounding, (ub (1 + 2^-7) + fp + 2^-15 Emax).
du has no decay and is float32 throughout (exact bf16 products, float32 sums):
2^-14 x_abs.
"""
import numpy as np
import pytest
import torch

from _helpers import to_dev
from oracle import wkv5_backward_ref, wkv6_backward_ref
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UB = 2.0 ** -8
FP = 2.0 ** -12
C_DU = 2.0 ** -14
CAP = 10.0
NAMES = ("dr", "dk", "dv", "dw", "du", "dS0")


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


def emax(w):
    """Largest sum of capped rates over one channel of one 64-token chunk."""
    wc = np.minimum(np.asarray(w, np.float64), CAP)
    B, T, C = wc.shape
    pad = (-T) % 64
    wc = np.concatenate([wc, np.zeros((B, pad, C))], axis=1).reshape(B, -1, 64, C)
    return float(wc.sum(axis=2).max(initial=0.0))


def bounds(w, u, r, k, v, go, H, S0, dST):
    """Per-element bounds of (dr, dk, dv, dw, du, dS0) as described above."""
    a = lambda x: None if x is None else np.abs(x)
    absin = (np.abs(u), np.abs(r), np.abs(k), np.abs(v), np.abs(go), H, a(S0), a(dST))
    absx = [np.abs(x) for x in wkv6_backward_ref(w, *absin)]
    wc = np.minimum(w, CAP)
    capx = absx if np.array_equal(wc, w) else [np.abs(x) for x in wkv6_backward_ref(wc, *absin)]
    ce = 2.0 ** -15 * emax(w)
    c3 = 3 * UB * (1 + 2.0 ** -7) + FP + ce
    c1 = UB * (1 + 2.0 ** -7) + FP + ce
    out = [c3 * capx[i] + (capx[i] - absx[i]) for i in range(4)]
    out.append(C_DU * absx[4])
    out.append(c1 * capx[5] + (capx[5] - absx[5]))
    return out


def bf16_dev(bits):
    return to_dev(None, DEV, bits)


def dev_inputs(p, go_bits, dST=None):
    d = dict(w=to_dev(p.w, DEV), u=to_dev(p.u, DEV), r=bf16_dev(p.r_bits), k=bf16_dev(p.k_bits),
             v=bf16_dev(p.v_bits), go=bf16_dev(go_bits))
    d["S0"] = None if p.S0 is None else to_dev(p.S0, DEV)
    d["dST"] = None if dST is None else to_dev(dST, DEV)
    return d


def run(d, need_state_grad=True, ckpt=None, split=True):
    res = ops().wkv6_backward(d["w"], d["u"], d["r"], d["k"], d["v"], d["go"], state_in=d["S0"],
                              grad_state_out=d["dST"], need_state_grad=need_state_grad, ckpt=ckpt, split=split)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in res]



NORM_TOL = 2.0 ** -7


def check_norm(name, got, ref):
    """Normwise accuracy on random inputs: ||got - ref|| <= 2^-7 ||ref|| (exactly 0 where ref is).
    Not a rounding bound: it checks that the errors do not add up coherently, which the
    magnitude-sum bound cannot see where a signed sum cancels (a summed dw, a long sequence)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    nr, ne = float(np.linalg.norm(r)), float(np.linalg.norm(g - r))
    print(f"  {name}: normwise relative error {ne / nr if nr else ne:.2e}", flush=True)
    assert (ne == 0.0) if nr == 0.0 else (ne <= NORM_TOL * nr), (name, ne, nr)


def check(p, go, got, dST=None, name=None):
    """Every output within its bound of the oracle, and within 2^-7 in the norm of the oracle on
    the operator the kernel computes (rates capped at 10; at a capped token dw is that of the rate
    10, up to e^{w - 10} times the true one)."""
    name = name or p.name
    w = np.asarray(p.w, np.float64)
    ref = wkv6_backward_ref(w, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
    bnd = bounds(w, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
    wc = np.minimum(w, CAP)
    refc = ref if np.array_equal(wc, w) else wkv6_backward_ref(wc, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
    for i, n in enumerate(NAMES):
        if got[i] is not None:
            check_bound(f"{name} {n}", got[i], ref[i], bnd[i])
            check_norm(f"{name} {n}", got[i], refc[i])


SHAPES = [(2, 1, 1), (2, 5, 2), (1, 63, 2), (2, 64, 1), (1, 65, 1), (2, 200, 3), (1, 1000, 2), (3, 129, 4)]


@pytest.mark.parametrize("B,T,H", SHAPES)
@pytest.mark.parametrize("with_state", [False, True])
def test_shapes(B, T, H, with_state):
    """Whole and ragged 64-token chunks, one to several heads, from the zero
    state and from a given one (then also with a final-state gradient)."""
    p = W.make_wkv6(B, T, H, seed=B * 100 + T + H + 21, with_state=with_state)
    go_bits, go = W.wkv5_go(p, seed=B + T + H + 1)
    dST = np.random.default_rng(T + 1).standard_normal((B, H, 64, 64)).astype(np.float32) if with_state else None
    print(f"case {p.name} state={with_state}", flush=True)
    check(p, go, run(dev_inputs(p, go_bits, dST)), dST)


@pytest.mark.parametrize("split,B,T,H", [(False, 2, 300, 2), (True, 2, 300, 2), (True, 1, 1000, 2),
                                         (True, 4, 256, 64)])
def test_with_forward_ckpt_matches_recompute(split, B, T, H):
    """The chunk-start states a wkv6_forward call saved give the same gradients,
    bit for bit, as the backward's own recomputation of them: unsplit both, or
    each with its workspace (below 256 pairs both split the sequence the same
    way; at 256 the backward splits its adjoint pass but, as the forward, not
    the recompute of the states)."""
    p = W.make_wkv6(B, T, H, seed=23 + T + H, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=24)
    d = dev_inputs(p, go_bits)
    O = ops()
    print(f"case ckpt split={split} B={B} T={T} H={H}", flush=True)
    ck = O.new_wkv5_ckpt(B, T, H, DEV)
    O.wkv6_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], ckpt=ck, split=split)
    a = run(d, ckpt=ck, split=split)
    b = run(d, split=split)
    for n, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), n
    if B * H <= 8:
        check(p, go, a, name="with ckpt")


@pytest.mark.parametrize("rates", [(20.0, 80.0), (1e-6, 1e-3), (6.0, 14.0), (0.0, 0.0)])
def test_extreme_decay_rates(rates):
    """Per-token rates from 0 (no decay) and nearly 0 to e^{-80}, and across the cap of 10."""
    p = W.make_wkv6(2, 150, 2, seed=25, with_state=True)
    rng = np.random.default_rng(26)
    if rates[1] == 0.0:
        p.w[:] = 0.0
    else:
        p.w[:] = np.exp(rng.uniform(np.log(rates[0]), np.log(rates[1]), p.w.shape)).astype(np.float32)
    go_bits, go = W.wkv5_go(p, seed=27)
    dST = np.random.default_rng(28).standard_normal((2, 2, 64, 64)).astype(np.float32)
    print(f"case rates {rates}", flush=True)
    check(p, go, run(dev_inputs(p, go_bits, dST)), dST, name=f"rates {rates}")


def test_mixed_resets():
    """Ordinary rates with scattered tokens whose rate is 30 (a near reset)."""
    p = W.make_wkv6(2, 300, 2, seed=29, with_state=True)
    mask = np.random.default_rng(30).random(p.w.shape) < 0.02
    p.w[mask] = 30.0
    go_bits, go = W.wkv5_go(p, seed=31)
    check(p, go, run(dev_inputs(p, go_bits)), name="mixed resets")


def test_fast_channel_dw_has_no_cancellation():
    """Channels with rates near 5 next to slow ones: dw of a fast channel is
    small next to the terms that make it up, and stays within its bound
    (a difference of large partial sums would not)."""
    p = W.make_wkv6(1, 256, 1, seed=33, base_range=(-6.0, 1.7), spread=0.2, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=34)
    check(p, go, run(dev_inputs(p, go_bits)), name="fast channels")


def test_constant_rates_match_rwkv5_backward():
    """With the same rate at every token the operator is RWKV-5's: both oracles
    agree, and the RWKV-6 kernel's dw summed over tokens and batch rows lies
    within its bound of the RWKV-5 oracle's dw."""
    p = W.make_wkv5(2, 130, 2, seed=35, with_state=True)
    p.w[:] = np.minimum(p.w, 9.0)  # below the cap of either kernel's terms
    go_bits, go = W.wkv5_go(p, seed=36)
    w6 = np.broadcast_to(p.w.reshape(1, 1, -1), (2, 130, 128)).astype(np.float32).copy()
    p6 = W.Wkv5Problem("wkv6 as wkv5", p.B, p.T, p.H, w6, p.u, p.r, p.k, p.v, p.r_bits, p.k_bits, p.v_bits, p.S0)
    got = run(dev_inputs(p6, go_bits))
    check(p6, go, got, name="constant rates")
    ref5 = wkv5_backward_ref(p.w.astype(np.float64), p.u, p.r, p.k, p.v, go, p.H, p.S0)
    bnd = bounds(w6.astype(np.float64), p.u, p.r, p.k, p.v, go, p.H, p.S0, None)
    check_bound("summed dw vs RWKV-5", got[3].sum(axis=(0, 1)).reshape(p.H, 64), ref5[3],
                bnd[3].sum(axis=(0, 1)).reshape(p.H, 64))


def test_zero_length_and_determinism():
    p = W.make_wkv6(2, 130, 3, seed=37, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=38)
    dST = np.random.default_rng(39).standard_normal((2, 3, 64, 64)).astype(np.float32)
    d = dev_inputs(p, go_bits, dST)
    O = ops()
    z = torch.empty((2, 0, 192), dtype=torch.bfloat16, device=DEV)
    zw = torch.empty((2, 0, 192), dtype=torch.float32, device=DEV)
    dr, dk, dv, dw, du, ds = O.wkv6_backward(zw, d["u"], z, z, z, z, state_in=d["S0"], grad_state_out=d["dST"],
                                             need_state_grad=True)
    torch.cuda.synchronize()
    assert dw.shape == (2, 0, 192) and torch.equal(du, torch.zeros_like(du)) and torch.equal(ds, d["dST"])
    a = run(d)
    b = run(d)
    for n, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), n


def test_autograd_function():
    """Wkv6Function: the gradients torch.autograd routes through wkv6_backward
    for o = wkv6(w, u, r, k, v, S0) and L = sum(go * o)."""
    p = W.make_wkv6(1, 100, 2, seed=41, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=42)
    d = dev_inputs(p, go_bits)
    O = ops()
    w = d["w"].clone().requires_grad_()
    u = d["u"].clone().requires_grad_()
    r, k, v = (d[n].clone().requires_grad_() for n in ("r", "k", "v"))
    S0 = d["S0"].clone().requires_grad_()
    o = O.Wkv6Function.apply(w, u, r, k, v, S0)
    (o * d["go"].float()).sum().backward()
    torch.cuda.synchronize()
    got = [r.grad.float(), k.grad.float(), v.grad.float(), w.grad, u.grad, S0.grad]
    ref = wkv6_backward_ref(p.w.astype(np.float64), p.u, p.r, p.k, p.v, go, p.H, p.S0)
    bnd = bounds(p.w.astype(np.float64), p.u, p.r, p.k, p.v, go, p.H, p.S0, None)
    for i, n in enumerate(NAMES):
        b = bnd[i] * (1 + UB) + np.abs(ref[i]) * UB if i < 3 else bnd[i]  # dr, dk, dv handed back in bf16
        check_bound(f"autograd {n}", got[i].cpu().numpy(), ref[i], b)


def test_full_size_every_head():
    """B=8, T=1024, 64 heads of 64 (the benchmarked shape and call sequence: the
    forward saves its chunk-start states, the backward reads them): every
    gradient of every (batch row, head) against the oracle, one batch row (all
    64 heads) at a time; du, summed over the batch rows, against the oracle's
    sum over the rows (and the bound summed likewise)."""
    p = W.wkv6_config(seed=5)
    go_bits, go = W.wkv5_go(p, seed=6)
    print(f"case {p.name}", flush=True)
    d = dev_inputs(p, go_bits)
    O = ops()
    ck = O.new_wkv5_ckpt(p.B, p.T, p.H, DEV)
    O.wkv6_forward(d["w"], d["u"], d["r"], d["k"], d["v"], ckpt=ck)
    got = run(d, need_state_grad=True, ckpt=ck)
    du_ref = du_refc = du_bnd = 0.0
    for b in range(p.B):
        name = f"{p.name} row {b}"
        w = np.asarray(p.w[b:b + 1], np.float64)
        args = (p.u, p.r[b:b + 1], p.k[b:b + 1], p.v[b:b + 1], go[b:b + 1], p.H, None, None)
        ref = wkv6_backward_ref(w, *args)
        bnd = bounds(w, *args)
        wc = np.minimum(w, CAP)
        refc = ref if np.array_equal(wc, w) else wkv6_backward_ref(wc, *args)
        for i in (0, 1, 2, 3, 5):
            check_bound(f"{name} {NAMES[i]}", got[i][b:b + 1], ref[i], bnd[i])
            check_norm(f"{name} {NAMES[i]}", got[i][b:b + 1], refc[i])
        du_ref = du_ref + ref[4]
        du_refc = du_refc + refc[4]
        du_bnd = du_bnd + bnd[4]
    check_bound(f"{p.name} du (all rows)", got[4], du_ref, du_bnd)
    check_norm(f"{p.name} du (all rows)", got[4], du_refc)


@pytest.mark.parametrize("rates", [None, (6.0, 14.0)])
def test_capped_rates_are_the_operator(rates):
    """Rates above 10 act as 10: against the oracle run on min(w, 10) the
    outputs stay within the rounding bound alone (no allowance for the cap),
    on the default rate mix (a few rates above 10) and on rates around 10."""
    p = W.make_wkv6(3, 129, 4, seed=43, with_state=True)
    if rates is not None:
        rng = np.random.default_rng(44)
        p.w[:] = np.exp(rng.uniform(np.log(rates[0]), np.log(rates[1]), p.w.shape)).astype(np.float32)
    assert (p.w > CAP).any()
    go_bits, go = W.wkv5_go(p, seed=45)
    dST = np.random.default_rng(46).standard_normal((3, 4, 64, 64)).astype(np.float32)
    got = run(dev_inputs(p, go_bits, dST))
    wc = np.minimum(p.w.astype(np.float64), CAP)
    pc = W.Wkv5Problem("capped", p.B, p.T, p.H, wc, p.u, p.r, p.k, p.v, None, None, None, p.S0)
    check(pc, go, got, dST, name=f"capped {rates}")


def test_long_sequence_slow_decay():
    """4,096 tokens (64 chunks) with per-token rates 1e-4 to 1e-2 and a
    final-state gradient: the adjoint state carries most of its history through
    every chunk."""
    p = W.make_wkv6(1, 4096, 1, seed=39, with_state=True)
    p.w[:] = np.exp(np.random.default_rng(40).uniform(np.log(1e-4), np.log(1e-2), p.w.shape)).astype(np.float32)
    go_bits, go = W.wkv5_go(p, seed=41)
    dST = np.random.default_rng(42).standard_normal((1, 1, 64, 64)).astype(np.float32)
    print(f"case {p.name} slow decay", flush=True)
    # the terms' summed magnitudes dwarf the signed results here, so the normwise check in check()
    # is what holds the gradients to bf16 accuracy
    check(p, go, run(dev_inputs(p, go_bits, dST)), dST, name="long slow decay")


SPLIT_TOL = 2.0 ** -9


@pytest.mark.parametrize("B,T,H", [(1, 1000, 2), (2, 200, 3), (1, 4100, 1), (4, 256, 64)])
def test_backward_time_split_matches_unsplit(B, T, H):
    """Few (batch row, head) pairs: the backward runs the sequence's segments in parallel, each
    from the adjoint after it (chained with the segments' summed capped rates).  Both the split
    and the unsplit backward are within the oracle's bounds, and they agree in the norm to 2^-9."""
    p = W.make_wkv6(B, T, H, seed=45 + T, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=46)
    dST = np.random.default_rng(47).standard_normal((B, H, 64, 64)).astype(np.float32)
    d = dev_inputs(p, go_bits, dST)
    lib = ops().L.lib()
    assert lib.wkv6_backward_workspace_bytes(B, T, H, 64, 0) > lib.wkv6_backward_workspace_bytes(B, T, H, 64, 2)
    print(f"case split backward {p.name}", flush=True)
    a = run(d, split=True)
    b = run(d, split=False)
    check(p, go, a, dST, name="split")
    for n, x, y in zip(NAMES, a, b):
        g_, r_ = np.asarray(x, np.float64), np.asarray(y, np.float64)
        ne, nr = float(np.linalg.norm(g_ - r_)), float(np.linalg.norm(r_))
        print(f"  split vs unsplit {n}: {ne / nr if nr else ne:.2e}", flush=True)
        assert ne <= SPLIT_TOL * nr, (n, ne, nr)


def test_backward_from_time_split_forward():
    """One long sequence with two heads: the forward runs split into segments, and the backward
    from the chunk-start states it saved stays within the bounds of the oracle."""
    p = W.make_wkv6(1, 1000, 2, seed=103, with_state=True)
    go_bits, go = W.wkv5_go(p, seed=104)
    d = dev_inputs(p, go_bits)
    O = ops()
    assert O.L.lib().wkv6_forward_workspace_bytes(1, 1000, 2, 64) > 0
    ck = O.new_wkv5_ckpt(1, 1000, 2, DEV)
    O.wkv6_forward(d["w"], d["u"], d["r"], d["k"], d["v"], state_in=d["S0"], ckpt=ck)
    check(p, go, run(d, ckpt=ck), name="from the split forward")
