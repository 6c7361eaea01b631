"""GPU parity of wkv_forward_state: the forward started from a given state and
returning the state after its last token, against the float64 oracle.

Bounds: outputs as the forward (fp32 rtol 1e-5 atol 1e-6; bf16 rtol 2e-3,
atol 2e-3 * 1e-2 * RMS); states compared only through the representation-free
a/b and ln b + p, rtol 1e-4 atol 1e-4 (the decode-step reading).
"""
import numpy as np
import pytest
import torch

from _helpers import check_close, problem_to_dev, to_dev
from oracle import wkv_forward_ref, wkv_state_from_sums, wkv_sums_from_state
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2))) if np.size(a) else 0.0


def check_y(name, got, ref, dtype):
    if dtype == "bf16":
        return check_close(f"{name} y (bf16 bound)", got, ref, 2e-3, 2e-5 * rms(ref))
    return check_close(f"{name} y", got, ref, 1e-5, 1e-6)


def check_state(name, st, A, Bs):
    a, b, p = (t.cpu().numpy().astype(np.float64) for t in st)
    ra, rb, rp = wkv_state_from_sums(A, Bs)
    check_close(f"{name} state a/b", a / b, ra / rb, 1e-4, 1e-4)
    check_close(f"{name} state ln b + p", np.log(b) + p, np.log(rb) + rp, 1e-4, 1e-4)


def sub(p, t0, t1):
    """Device tensors of tokens [t0, t1) of a problem."""
    d = problem_to_dev(p, DEV)
    return {n: (d[n][:, t0:t1].contiguous() if d[n].dim() == 3 else d[n]) for n in d}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T1,T2,C", [(2, 300, 457, 70), (1, 1, 5, 3), (3, 256, 256, 129), (1, 1000, 3097, 64)])
def test_split_sequence_equals_whole(dtype, B, T1, T2, C):
    """Forward over T1 tokens returning its state, then over T2 more from that
    state: outputs and final state equal the whole-sequence oracle."""
    spikes = 0.01 if dtype == "bf16" else 0.0
    p = W.make_problem(B, T1 + T2, C, dtype=dtype, seed=T1 + 7 * T2 + C, spike_frac=spikes,
                       name=f"split {dtype} B={B} T={T1}+{T2} C={C}")
    print(f"case {p.name}", flush=True)
    O = ops()
    d1, d2 = sub(p, 0, T1), sub(p, T1, T1 + T2)
    y1, st = O.wkv_forward(d1["w"], d1["u"], d1["k"], d1["v"], return_state=True)
    y2, st2 = O.wkv_forward(d2["w"], d2["u"], d2["k"], d2["v"], state_in=st, return_state=True)
    torch.cuda.synchronize()
    yref, A, Bs = wkv_forward_ref(p.w, p.u, p.k, p.v, return_sums=True)
    check_y(p.name, np.concatenate([y1.cpu().numpy(), y2.cpu().numpy()], axis=1), yref, dtype)
    check_state(p.name, st2, A, Bs)


def test_prefill_hands_off_to_decode_steps():
    """Forward prefill of 200 tokens, then 60 wkv_step calls from its state."""
    p = W.make_problem(2, 260, 96, dtype="bf16", seed=51, spike_frac=0.01, name="prefill+steps")
    print(f"case {p.name}", flush=True)
    O = ops()
    d = problem_to_dev(p, DEV)
    _, (a, b, pp) = O.wkv_forward(d["w"], d["u"], d["k"][:, :200].contiguous(), d["v"][:, :200].contiguous(),
                                  return_state=True)
    a, b, pp = a[None], b[None], pp[None]  # [L=1, B, C] for wkv_step
    w, u = d["w"][None].contiguous(), d["u"][None].contiguous()
    ys = []
    for t in range(200, 260):
        ys.append(O.wkv_step(w, u, d["k"][:, t][None].contiguous(), d["v"][:, t][None].contiguous(), a, b, pp)[0])
    torch.cuda.synchronize()
    yref = wkv_forward_ref(p.w, p.u, p.k, p.v)[:, 200:]
    check_y(p.name, torch.stack(ys, dim=1).cpu().numpy(), yref, "bf16")


@pytest.mark.parametrize("scale", [0.0, 37.0, -25.0])
def test_forward_from_given_state(scale):
    """State of an oracle prefix with key spikes, passed in several (a, b, p)
    representations (scaled by e^scale); the continuation matches the oracle
    started from the same sums."""
    B, T0, T, C = 2, 150, 333, 67
    p = W.make_problem(B, T0 + T, C, dtype="f32", seed=52, spike_frac=0.0, name=f"given state {scale}")
    print(f"case {p.name}", flush=True)
    _, A0, B0 = wkv_forward_ref(p.w, p.u, p.k[:, :T0], p.v[:, :T0], return_sums=True)
    ra, rb, rp = wkv_state_from_sums(A0, B0)
    ra, rb, rp = ra * np.exp(scale), rb * np.exp(scale), rp - scale
    sa, sb, spp = (np.asarray(x, np.float32) for x in (ra, rb, rp))
    A0f, B0f = wkv_sums_from_state(sa, sb, spp)  # the oracle starts from the float32 state it was given
    O = ops()
    d = sub(p, T0, T0 + T)
    st_in = tuple(to_dev(x, DEV) for x in (sa, sb, spp))
    y, st = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_in=st_in, return_state=True)
    torch.cuda.synchronize()
    yref, A, Bs = wkv_forward_ref(p.w, p.u, p.k[:, T0:], p.v[:, T0:], return_sums=True, A0=A0f, B0=B0f)
    check_y(p.name, y.cpu().numpy(), yref, "f32")
    check_state(p.name, st, A, Bs)


def test_state_update_in_place_and_empty_sequence():
    p = W.make_problem(2, 90, 40, dtype="f32", seed=53, name="in place")
    print(f"case {p.name}", flush=True)
    O = ops()
    d = problem_to_dev(p, DEV)
    st = tuple(torch.empty((2, 40), device=DEV) for _ in range(3))
    O.wkv_forward(d["w"], d["u"], d["k"][:, :30].contiguous(), d["v"][:, :30].contiguous(), state_out=st)
    # T = 0: the state passes through unchanged; with no input state it is the empty one
    z = torch.zeros((2, 0, 40), device=DEV)
    st0 = tuple(torch.full((2, 40), 5.0, device=DEV) for _ in range(3))
    O.wkv_forward(d["w"], d["u"], z, z, state_in=st, state_out=st0)
    torch.cuda.synchronize()
    for t0, t1 in zip(st0, st):
        assert torch.equal(t0, t1)
    O.wkv_forward(d["w"], d["u"], z, z, state_out=st0)
    torch.cuda.synchronize()
    assert torch.all(st0[0] == 0) and torch.all(st0[1] == 0) and torch.all(st0[2] <= -1e30)
    # continue in place: state_out is the state_in tensors
    y, _ = O.wkv_forward(d["w"], d["u"], d["k"][:, 30:].contiguous(), d["v"][:, 30:].contiguous(),
                         state_in=st, state_out=st, return_state=True)
    torch.cuda.synchronize()
    yref, A, Bs = wkv_forward_ref(p.w, p.u, p.k, p.v, return_sums=True)
    check_y(p.name, y.cpu().numpy(), yref[:, 30:], "f32")
    check_state(p.name, st, A, Bs)
