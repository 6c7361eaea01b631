"""GPU parity of the fused receptance gate (wkv_forward_gated,
wkv_backward_gated) against the float64 oracle.

Bounds: out as the forward (fp32 rtol 1e-5 atol 1e-6; bf16 rtol 2e-3, atol
2e-3 * 1e-2 * RMS); every gradient, dr included, as the backward (rtol 1e-3,
atol 1e-3 * 1e-2 * RMS, at least 1e-12 of the gradient scale).
"""
import numpy as np
import pytest
import torch

from _helpers import bwd_atol, check_close, problem_to_dev, to_dev
from oracle import wkv_gated_backward_ref, wkv_gated_forward_ref
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2))) if np.size(a) else 0.0


def run_and_check(p, r, r_bits, with_ckpt=False):
    O = ops()
    d = problem_to_dev(p, DEV)
    rd = to_dev(r, DEV, r_bits)
    ck = O.new_ckpt(p.B, p.T, p.C, DEV) if with_ckpt else None
    out = O.wkv_forward_gated(d["w"], d["u"], d["k"], d["v"], rd, ckpt=ck)
    grads = O.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], rd, d["gy"], ckpt=ck)
    torch.cuda.synchronize()
    ref = wkv_gated_forward_ref(p.w, p.u, p.k, p.v, r)
    if p.dtype == "bf16":
        check_close(f"{p.name} out (bf16 bound)", out.cpu().numpy(), ref, 2e-3, 2e-5 * rms(ref))
    else:
        check_close(f"{p.name} out", out.cpu().numpy(), ref, 1e-5, 1e-6)
    rgrads = wkv_gated_backward_ref(p.w, p.u, p.k, p.v, r, p.gy)
    for n, g, rr in zip(("dk", "dv", "dr", "dw", "du"), grads, rgrads):
        check_close(f"{p.name} {n}", g.cpu().numpy(), rr, 1e-3, bwd_atol(rr, gy=p.gy, v=p.v))


@pytest.mark.parametrize("dtype,B,T,C", [("f32", 1, 64, 8), ("f32", 2, 300, 70), ("bf16", 3, 77, 13),
                                         ("bf16", 2, 1000, 129)])
def test_gated_parity(dtype, B, T, C):
    spikes = 0.01 if dtype == "bf16" else 0.0
    p = W.make_problem(B, T, C, dtype=dtype, seed=B + T + C, spike_frac=spikes, name=f"gated {dtype} B={B} T={T} C={C}")
    r, rb = W.receptance(p)
    print(f"case {p.name}", flush=True)
    run_and_check(p, r, rb, with_ckpt=(T == 300))


def test_gated_whole_tile_backward():
    """Enough tiles for the whole-tile backward, ragged T and tile, saved states reused."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    p = W.make_problem(2, 77, 64 * ncu + 17, dtype="bf16", seed=61, spike_frac=0.01, name="gated tile bf16")
    r, rb = W.receptance(p)
    print(f"case {p.name}", flush=True)
    run_and_check(p, r, rb, with_ckpt=True)


def test_gated_whole_tile_staged_ragged():
    """The whole-tile backward with its inputs (r included, bf16) staged in LDS: C a whole number
    of 16-byte rows, a ragged last time block, saved states reused."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    p = W.make_problem(2, 77, 64 * ncu, dtype="bf16", seed=63, spike_frac=0.01, name="gated tile staged bf16")
    r, rb = W.receptance(p)
    print(f"case {p.name}", flush=True)
    run_and_check(p, r, rb, with_ckpt=True)


def test_gated_config3_shape():
    p = W.config3()
    r, rb = W.receptance(p)
    print(f"case gated {p.name}", flush=True)
    run_and_check(p, r, rb, with_ckpt=True)


def test_gate_saturation():
    """r far in both tails: sigmoid and 1 - sigmoid are formed without overflow or cancellation."""
    p = W.make_problem(2, 120, 40, dtype="f32", seed=62, name="gate tails")
    r, _ = W.receptance(p, std=40.0)
    r[:, ::7] = 95.0
    r[:, 3::7] = -95.0
    print(f"case {p.name}", flush=True)
    run_and_check(p, r.astype(np.float32), None)
