"""GPU: a call bound once (ops' bind=True) and launched repeatedly gives, bit for bit, what the
same call gives unbound, also after the inputs' contents change between launches."""
import pytest
import torch

from _helpers import problem_to_dev
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


@pytest.mark.parametrize("dtype,B,T,C", [("bf16", 8, 300, 4096), ("f32", 2, 700, 130)])
def test_bound_forward_backward_equal_unbound(dtype, B, T, C):
    print(f"case bind {dtype} B={B} T={T} C={C}", flush=True)
    O = ops()
    p = W.make_problem(B, T, C, dtype=dtype, seed=B + T + C, name="bind")
    d = problem_to_dev(p, DEV)
    dt = d["k"].dtype
    y = torch.empty((B, T, C), device=DEV)
    ck = O.new_ckpt(B, T, C, DEV)
    out = (torch.empty((B, T, C), device=DEV), torch.empty((B, T, C), device=DEV), torch.empty(C, device=DEV),
           torch.empty(C, device=DEV))
    ws = torch.zeros(max(O.workspace_bytes(op, B, T, C, dt) for op in (0, 1)), dtype=torch.uint8, device=DEV)
    f = O.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, ckpt=ck, workspace=ws, bind=True)
    b = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"], ckpt=ck, out=out, workspace=ws, bind=True)
    for rep in range(3):
        if rep == 2:  # new contents in the bound buffers
            d["v"].copy_(d["v"].flip(1))
        assert f() is y
        got = b()
        ref_y = O.wkv_forward(d["w"], d["u"], d["k"], d["v"])
        ref = O.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["gy"])
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y)
        for a, r in zip(got, ref):
            assert torch.equal(a, r)


def test_bound_matrix_state_forward_equal_unbound():
    print("case bind wkv5/wkv6 forward", flush=True)
    O = ops()
    B, T, H = 2, 200, 4
    C = 64 * H
    g = torch.Generator(device="cpu").manual_seed(5)
    r, k, v = (torch.randn((B, T, C), generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    w5 = torch.rand((H, 64), generator=g).to(DEV)
    w6 = torch.rand((B, T, C), generator=g).to(DEV)
    u = torch.randn((H, 64), generator=g).to(DEV)
    for fn, w in ((O.wkv5_forward, w5), (O.wkv6_forward, w6)):
        o = torch.empty((B, T, C), device=DEV)
        st = torch.empty((B, H, 64, 64), device=DEV)
        call = fn(w, u, r, k, v, out=o, state_out=st, bind=True)
        for _ in range(2):
            call()
            ref, ref_st = fn(w, u, r, k, v, return_state=True)
            torch.cuda.synchronize()
            assert torch.equal(o, ref) and torch.equal(st, ref_st)
