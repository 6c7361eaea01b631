"""GPU tests of the workspace protocol of wkv_forward / wkv_backward.

Where the calls chain workgroups in time (few 64-channel tiles), carries are
tagged with the call's generation instead of cleared per call, and the last
workgroup of each channel tile folds the dw / du partials.  These tests reuse
one zero-filled workspace over many calls (every call equals the first, bit for
bit, and the oracle), force every carry wait to give up from the host
(wkv_debug_spin_limit(0): every kernel still runs to its end) and check that
wkv_workspace_status reports it, and check that a workspace that was not
zero-filled before its first call is reported too.

Bounds as the parity tests: forward rtol 2e-3 (bf16) or 1e-5 (fp32) against the
oracle; backward rtol 1e-3 with the absolute floor of the parity tests.
"""
import numpy as np
import pytest
import torch

from _helpers import bwd_atol, check_close, problem_to_dev
from oracle import wkv_backward_ref, wkv_forward_ref
from rwkv_wkv_mixing_amd import _lib as L
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2))) if np.size(a) else 0.0


def check_y(p, y):
    ref = wkv_forward_ref(p.w, p.u, p.k, p.v)
    if p.dtype == "bf16":
        check_close(f"{p.name} y", y, ref, 2e-3, 2e-5 * rms(ref))
    else:
        check_close(f"{p.name} y", y, ref, 1e-5, 1e-6)


def check_grads(p, g):
    ref = wkv_backward_ref(p.w, p.u, p.k, p.v, p.gy)
    for n, a, r in zip(("dk", "dv", "dw", "du"), g, ref):
        check_close(f"{p.name} {n}", a.cpu().numpy(), r, 1e-3, bwd_atol(r, gy=p.gy, v=p.v))


@pytest.mark.parametrize("dtype,B,T,C", [("bf16", 1, 2000, 64), ("f32", 2, 700, 130), ("bf16", 8, 1024, 768)])
def test_workspace_reused_over_calls(dtype, B, T, C):
    """Time-split kernels (few tiles): forward and backward four times on one
    workspace each; every call equals the first bit for bit, the first equals
    the oracle, and the error word stays clear."""
    p = W.make_problem(B, T, C, dtype=dtype, seed=B * 7 + T + C, spike_frac=0.01 if dtype == "bf16" else 0.0,
                       name=f"reuse {dtype} B={B} T={T} C={C}")
    print(f"case {p.name}", flush=True)
    O = ops()
    d = problem_to_dev(p, DEV)
    dt = d["k"].dtype
    wsf = O.new_workspace(0, B, T, C, dt, DEV)
    wsb = O.new_workspace(1, B, T, C, dt, DEV)
    assert wsf.numel() > 1 and wsb.numel() > 1  # these shapes chain workgroups in time
    outs = []
    for _ in range(4):
        ck = O.new_ckpt(B, T, C, DEV)
        y = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], ckpt=ck, workspace=wsf)
        g = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], ckpt=ck, workspace=wsb)
        g2 = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], workspace=wsb)  # recomputes the states
        outs.append((y, g, g2))
    torch.cuda.synchronize()
    assert O.workspace_status(wsf) == L.WKV_OK
    assert O.workspace_status(wsb) == L.WKV_OK
    y0, g0, g20 = outs[0]
    check_y(p, y0.cpu().numpy())
    check_grads(p, g0)
    for y, g, g2 in outs[1:]:
        assert torch.equal(y, y0)
        for a, b in zip(g + g2, g0 + g20):
            assert torch.equal(a, b)


def test_timeout_is_reported():
    """With a spin limit of 0 every wait between workgroups gives up at once:
    the kernels still end, the error word is set and wkv_workspace_status
    reports WKV_ETIMEOUT; once cleared, the same workspace serves correct calls."""
    p = W.make_problem(1, 2000, 64, dtype="bf16", seed=77, spike_frac=0.01, name="timeout")
    print(f"case {p.name}", flush=True)
    O = ops()
    lib = L.lib()
    d = problem_to_dev(p, DEV)
    wsf = O.new_workspace(0, p.B, p.T, p.C, d["k"].dtype, DEV)
    wsb = O.new_workspace(1, p.B, p.T, p.C, d["k"].dtype, DEV)
    old = lib.wkv_debug_spin_limit(0)
    try:
        O.wkv_forward(d["w"], d["u"], d["k"], d["v"], workspace=wsf)
        O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], workspace=wsb)
        torch.cuda.synchronize()
    finally:
        lib.wkv_debug_spin_limit(old)
    assert O.workspace_status(wsf, clear=True) == L.WKV_ETIMEOUT
    assert O.workspace_status(wsb, clear=True) == L.WKV_ETIMEOUT
    assert O.workspace_status(wsf) == L.WKV_OK and O.workspace_status(wsb) == L.WKV_OK
    y = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], workspace=wsf)
    g = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], workspace=wsb)
    torch.cuda.synchronize()
    assert O.workspace_status(wsf) == L.WKV_OK and O.workspace_status(wsb) == L.WKV_OK
    check_y(p, y.cpu().numpy())
    check_grads(p, g)


def test_workspace_not_zero_filled_is_reported():
    """A workspace whose header was not zero-filled before its first call hands
    out tickets out of range: the affected workgroups do nothing, the waits on
    them give up (spin limit shortened here), and the error word says so."""
    p = W.make_problem(1, 1500, 64, dtype="bf16", seed=78, name="dirty workspace")
    print(f"case {p.name}", flush=True)
    O = ops()
    lib = L.lib()
    d = problem_to_dev(p, DEV)
    wsf = torch.full((O.workspace_bytes(0, p.B, p.T, p.C, d["k"].dtype),), 0x5A, dtype=torch.uint8, device=DEV)
    wsf[4:8] = 0  # a clear error word, with everything else dirty
    old = lib.wkv_debug_spin_limit(1000)
    try:
        O.wkv_forward(d["w"], d["u"], d["k"], d["v"], workspace=wsf)
        torch.cuda.synchronize()
    finally:
        lib.wkv_debug_spin_limit(old)
    assert O.workspace_status(wsf) == L.WKV_ETIMEOUT


def test_one_workspace_across_shapes():
    """One zero-filled buffer serves forward and backward calls of several shapes and
    dtypes in turn (the counters sit at fixed offsets for every shape, the carries
    start at one fixed offset, and every carry is tagged with the call's
    generation): each call equals the same call on a fresh workspace, bit for bit."""
    O = ops()
    shapes = [("bf16", 1, 2000, 64), ("f32", 2, 700, 130), ("bf16", 1, 1100, 192), ("f32", 1, 3000, 64),
              ("bf16", 1, 2000, 64)]
    probs = []
    for i, (dt, B, T, C) in enumerate(shapes):
        p = W.make_problem(B, T, C, dtype=dt, seed=300 + i, spike_frac=0.01 if dt == "bf16" else 0.0,
                           name=f"shapes {dt} B={B} T={T} C={C}")
        probs.append((p, problem_to_dev(p, DEV)))
    nbytes = max(O.workspace_bytes(op, p.B, p.T, p.C, d["k"].dtype) for p, d in probs for op in (0, 1))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    for p, d in probs:
        print(f"case {p.name}", flush=True)
        B, T, C = p.B, p.T, p.C
        dt = d["k"].dtype
        ck = O.new_ckpt(B, T, C, DEV)
        y = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], ckpt=ck, workspace=ws)
        g = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], ckpt=ck, workspace=ws)
        g2 = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], workspace=ws)
        ck_f = O.new_ckpt(B, T, C, DEV)
        y_f = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], ckpt=ck_f, workspace=O.new_workspace(0, B, T, C, dt, DEV))
        g_f = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], ckpt=ck_f,
                             workspace=O.new_workspace(1, B, T, C, dt, DEV))
        torch.cuda.synchronize()
        assert O.workspace_status(ws) == L.WKV_OK
        assert torch.equal(y, y_f)
        for a, b in zip(g + g2, g_f + g_f):
            assert torch.equal(a, b)
        check_y(p, y.cpu().numpy())
        check_grads(p, g)
