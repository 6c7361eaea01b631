"""GPU parity of the whole-tile forward: with bf16 inputs, at least two 64-channel
tiles per CU, C a multiple of 8 and 16-byte aligned k, v, the forward runs one
workgroup per tile over the whole sequence with each next block staged in LDS.
These shapes take that path: B = 2 rows of ncu + 1 tiles, the last tile ragged
(C = 64 ncu + 24, its lanes past C read as zeros); T ragged against the
128-token blocks.

Bounds as the forward tests: y rtol 2e-3 against the oracle on the bf16-rounded
inputs, atol 2e-3 * 1e-2 * RMS; states through a/b and ln b + p at 1e-4; the
gated output as y.
"""
import numpy as np
import pytest
import torch

from _helpers import check_close, problem_to_dev, to_dev
from oracle import wkv_forward_ref, wkv_gated_forward_ref, wkv_state_from_sums
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2))) if np.size(a) else 0.0


def tile_C():
    return 64 * torch.cuda.get_device_properties(0).multi_processor_count + 24


def check_y(name, got, ref):
    return check_close(f"{name} y (bf16 bound)", got, ref, 2e-3, 2e-5 * rms(ref))


@pytest.mark.parametrize("T", [1, 77, 128, 200, 1000])
def test_tile_forward_parity(T):
    p = W.make_problem(2, T, tile_C(), dtype="bf16", seed=900 + T, spike_frac=0.01, name=f"tile fwd T={T}")
    print(f"case {p.name} C={p.C}", flush=True)
    d = problem_to_dev(p, DEV)
    O = ops()
    ck = O.new_ckpt(p.B, p.T, p.C, DEV)
    y = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], ckpt=ck)
    torch.cuda.synchronize()
    check_y(p.name, y.cpu().numpy(), wkv_forward_ref(p.w, p.u, p.k, p.v))
    # the saved states serve the backward exactly as the ones it recomputes (the same kernel)
    g1 = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], ckpt=ck)
    g2 = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"])
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T1,T2", [(300, 457), (128, 1), (1, 255)])
def test_tile_forward_split_through_state(T1, T2):
    """Forward over T1 tokens returning its state, then T2 more from that state
    (also updated in place): outputs and final state equal the whole-sequence oracle."""
    p = W.make_problem(2, T1 + T2, tile_C(), dtype="bf16", seed=T1 + 7 * T2, spike_frac=0.01,
                       name=f"tile split T={T1}+{T2}")
    print(f"case {p.name} C={p.C}", flush=True)
    O = ops()
    d = problem_to_dev(p, DEV)
    k1, v1 = d["k"][:, :T1].contiguous(), d["v"][:, :T1].contiguous()
    k2, v2 = d["k"][:, T1:].contiguous(), d["v"][:, T1:].contiguous()
    y1, st = O.wkv_forward(d["w"], d["u"], k1, v1, return_state=True)
    y2 = O.wkv_forward(d["w"], d["u"], k2, v2, state_in=st, state_out=st)
    torch.cuda.synchronize()
    ref, A, Bs = wkv_forward_ref(p.w, p.u, p.k, p.v, return_sums=True)
    check_y(p.name, np.concatenate([y1.cpu().numpy(), y2.cpu().numpy()], axis=1), ref)
    a, b, pp = (t.cpu().numpy().astype(np.float64) for t in st)
    ra, rb, rp = wkv_state_from_sums(A, Bs)
    check_close(f"{p.name} state a/b", a / b, ra / rb, 1e-4, 1e-4)
    check_close(f"{p.name} state ln b + p", np.log(b) + pp, np.log(rb) + rp, 1e-4, 1e-4)


@pytest.mark.parametrize("T", [77, 300])
def test_tile_forward_gated(T):
    p = W.make_problem(2, T, tile_C(), dtype="bf16", seed=950 + T, spike_frac=0.01, name=f"tile gated T={T}")
    r, rb = W.receptance(p)
    print(f"case {p.name} C={p.C}", flush=True)
    d = problem_to_dev(p, DEV)
    out = ops().wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], to_dev(r, DEV, rb))
    torch.cuda.synchronize()
    ref = wkv_gated_forward_ref(p.w, p.u, p.k, p.v, r)
    check_close(f"{p.name} out (bf16 bound)", out.cpu().numpy(), ref, 2e-3, 2e-5 * rms(ref))


def test_tile_forward_extreme_inputs():
    """Key spikes of +-100, |u| up to 30 and w up to 80 (the general path inside
    the tile kernel), against the stress bound."""
    p = W.make_problem(2, 300, tile_C(), dtype="bf16", seed=977, spike_frac=0.03, spike_range=(60.0, 100.0),
                       name="tile extreme")
    rng = np.random.default_rng(5)
    p.u[:] = rng.uniform(-30.0, 30.0, p.C).astype(np.float32)
    p.w[: p.C // 4] = rng.uniform(0.0, 80.0, p.C // 4).astype(np.float32)
    print(f"case {p.name} C={p.C}", flush=True)
    d = problem_to_dev(p, DEV)
    y = ops().wkv_forward(d["w"], d["u"], d["k"], d["v"])
    torch.cuda.synchronize()
    check_close(f"{p.name} y (stress bound)", y.cpu().numpy(), wkv_forward_ref(p.w, p.u, p.k, p.v), 1e-4, 1e-5)
