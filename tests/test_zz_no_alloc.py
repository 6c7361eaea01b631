"""GPU test of wkv_forward_state_noalloc, the forward for callers that cannot
allocate: its workspace is a static array inside the library, shared by every
call on the GPU.

Several calls in a row on that one array (no synchronisation between them,
sizes going down and up again, chained and whole-tile shapes, with and without
a given state) each give the same y, ckpt and final state, bit for bit, as
wkv_forward_state on a zero-filled workspace of its own: the same kernels on the
same inputs, so equality is exact.  Both entry points are called through the
C ABI.
"""
import ctypes

import numpy as np
import pytest
import torch

from _helpers import problem_to_dev
from rwkv_wkv_mixing_amd import _lib as L
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (dtype, B, T, C, with a given state); the first two are the large call and the
# smaller one after it on the same static array
CASES = [("bf16", 1, 6000, 128, True), ("bf16", 1, 1500, 64, False), ("f32", 2, 3000, 64, True),
         ("f32", 1, 900, 64, False), ("bf16", 8, 300, 4096, True), ("bf16", 1, 6000, 128, False)]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nan(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def inputs(i, dtype, B, T, C, with_state):
    p = W.make_problem(B, T, C, dtype=dtype, seed=900 + i, spike_frac=0.01 if dtype == "bf16" else 0.0,
                       with_gy=False, name=f"noalloc {dtype} B={B} T={T} C={C}")
    d = problem_to_dev(p, DEV)
    d["dt"] = L.WKV_BF16 if dtype == "bf16" else L.WKV_F32
    if with_state:  # a given state: any a, b > 0 and p
        rng = np.random.default_rng(950 + i)
        a = torch.tensor(rng.standard_normal((B, C)), dtype=torch.float32, device=DEV)
        b = torch.tensor(rng.uniform(0.5, 4.0, (B, C)), dtype=torch.float32, device=DEV)
        pp = torch.tensor(rng.uniform(-3.0, 3.0, (B, C)), dtype=torch.float32, device=DEV)
        d["state"] = (a, b, pp)
    else:
        d["state"] = (None, None, None)
    return p, d


def outputs(lib, B, T, C):
    return dict(y=_nan(B, T, C), ck=_nan(lib.wkv_ckpt_bytes(B, T, C) // 4), st=tuple(_nan(B, C) for _ in range(3)))


def call(lib, p, d, o, workspace=None, noalloc=True):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [p.B, p.T, p.C, d["dt"], _p(d["w"]), _p(d["u"]), _p(d["k"]), _p(d["v"]), _p(o["y"]),
            *[_p(t) for t in d["state"]], *[_p(t) for t in o["st"]], _p(o["ck"])]
    if noalloc:
        return lib.wkv_forward_state_noalloc(*args, stream)
    nbytes = workspace.numel()
    return lib.wkv_forward_state(*args, _p(workspace) if nbytes > 1 else None, nbytes, stream)


def test_noalloc_matches_forward_state_over_calls_in_a_row():
    lib = L.lib()
    probs = [inputs(i, *c) for i, c in enumerate(CASES)]
    torch.cuda.synchronize()
    got = []
    for (p, d), c in zip(probs, CASES):  # back to back on the static array
        print(f"case {p.name} state={c[4]} noalloc", flush=True)
        o = outputs(lib, p.B, p.T, p.C)
        assert call(lib, p, d, o) == L.WKV_OK
        got.append(o)
    torch.cuda.synchronize()
    for (p, d), c, o in zip(probs, CASES, got):
        print(f"case {p.name} state={c[4]} compare", flush=True)
        nbytes = lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, p.B, p.T, p.C, d["dt"])
        assert nbytes <= L.WKV_STATIC_SCRATCH_BYTES
        ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=DEV)
        ref = outputs(lib, p.B, p.T, p.C)
        assert call(lib, p, d, ref, workspace=ws, noalloc=False) == L.WKV_OK
        torch.cuda.synchronize()
        assert torch.isfinite(o["y"]).all()
        assert torch.equal(o["y"], ref["y"]), "y"
        assert torch.equal(o["ck"], ref["ck"]), "ckpt"
        for n, x, r in zip("abp", o["st"], ref["st"]):
            assert torch.equal(x, r), f"state {n}"



def test_binding_matches_wkv_forward():
    """The thin Python binding of the same entry point, with a state in and out."""
    from rwkv_wkv_mixing_amd import ops as O

    p, d = inputs(7, "bf16", 1, 2500, 64, True)
    print(f"case {p.name} binding", flush=True)
    y = torch.empty((p.B, p.T, p.C), dtype=torch.float32, device=DEV)
    st = tuple(torch.empty((p.B, p.C), dtype=torch.float32, device=DEV) for _ in range(3))
    O.wkv_forward_state_noalloc(d["w"], d["u"], d["k"], d["v"], y, state_in=d["state"], state_out=st)
    ref, ref_st = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_in=d["state"], return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    for x, r in zip(st, ref_st):
        assert torch.equal(x, r)
