"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects invalid calls on the host
before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from rwkv_wkv_mixing_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from rwkv_wkv_mixing_amd.build import build

        build()
    return L.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(wkv[0-9]*_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(L.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"


def test_version_and_status_strings(lib):
    assert lib.wkv_version().decode() == "0.1.0"
    for s in range(9):
        assert len(lib.wkv_status_str(s)) >= 2
    assert lib.wkv_status_str(99) == b"unknown status"
    assert lib.wkv_last_hip_error() == b""


def test_header_constants_match_binding():
    src = open(HEADER).read()
    assert "#define WKV_CKPT_LEN 16" in src and L.WKV_CKPT_LEN == 16
    for name, val in (("WKV_OK", 0), ("WKV_EINVAL", 1), ("WKV_EDTYPE", 2), ("WKV_ESIZE", 3),
                      ("WKV_EALIGN", 4), ("WKV_EWORKSPACE", 5), ("WKV_EHIP", 6), ("WKV_ETIMEOUT", 7),
                      ("WKV_ESCRATCH", 8)):
        assert re.search(rf"{name} = {val}\b", src), name
        assert getattr(L, name) == val


def test_workspace_and_ckpt_sizes(lib):
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, -1, 4, 4, L.WKV_F32) == 0
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, 1, 4, 4, 7) == 0
    assert lib.wkv_workspace_bytes(5, 1, 4, 4, L.WKV_F32) == 0
    assert lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 0, 4, 4, L.WKV_F32) == 0
    for dt in (L.WKV_F32, L.WKV_BF16):
        assert lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 8, 1024, 4096, dt) > 0
    # overflow of B*T*C
    assert lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 1 << 30, 1 << 30, 1 << 10, L.WKV_F32) == 0
    assert lib.wkv_ckpt_bytes(8, 1024, 4096) == 8 * 64 * 4096 * 12
    assert lib.wkv_ckpt_bytes(1, 17, 3) == 2 * 3 * 12
    assert lib.wkv_ckpt_bytes(1, 0, 3) == 0
    assert lib.wkv_ckpt_bytes(-1, 5, 3) == 0


P = ctypes.c_void_p


def fwd(lib, B, T, C, dt, w, u, k, v, y, ck=None, ws=None, nws=0):
    return lib.wkv_forward(B, T, C, dt, P(w), P(u), P(k), P(v), P(y), P(ck), P(ws), nws, None)


def bwd(lib, B, T, C, dt, w, u, k, v, gy, dk, dv, dw, du, ck=None, ws=None, nws=0):
    return lib.wkv_backward(B, T, C, dt, P(w), P(u), P(k), P(v), P(gy), P(dk), P(dv), P(dw), P(du),
                            P(ck), P(ws), nws, None)


def step(lib, Ln, B, C, dt, w, u, k, v, y, a, b, p):
    return lib.wkv_step(Ln, B, C, dt, P(w), P(u), P(k), P(v), P(y), P(a), P(b), P(p), None)


A16 = 0x10000  # fake, never dereferenced: every call below fails validation on the host


def test_forward_validation(lib):
    x = A16
    assert fwd(lib, -1, 4, 4, L.WKV_F32, x, x, x, x, x) == L.WKV_EINVAL
    assert fwd(lib, 1, 4, 4, 3, x, x, x, x, x) == L.WKV_EDTYPE
    assert fwd(lib, 1 << 30, 1 << 30, 1 << 10, L.WKV_F32, x, x, x, x, x) == L.WKV_ESIZE
    assert fwd(lib, 1, 4, 4, L.WKV_F32, None, x, x, x, x) == L.WKV_EINVAL
    assert fwd(lib, 1, 4, 4, L.WKV_F32, x, x, x, x, None) == L.WKV_EINVAL
    assert fwd(lib, 1, 4, 4, L.WKV_F32, x, x, x + 2, x, x) == L.WKV_EALIGN
    assert fwd(lib, 1, 4, 4, L.WKV_BF16, x, x, x + 1, x, x) == L.WKV_EALIGN
    assert fwd(lib, 1, 4, 4, L.WKV_F32, x, x, x, x, x + 1) == L.WKV_EALIGN
    # empty problems are no-ops and touch nothing
    assert fwd(lib, 0, 4, 4, L.WKV_F32, None, None, None, None, None) == L.WKV_OK
    assert fwd(lib, 3, 0, 4, L.WKV_F32, None, None, None, None, None) == L.WKV_OK


def fwd_state(lib, B, T, C, dt, w, u, k, v, y, ain=None, bin_=None, pin=None, aout=None, bout=None, pout=None):
    return lib.wkv_forward_state(B, T, C, dt, P(w), P(u), P(k), P(v), P(y), P(ain), P(bin_), P(pin), P(aout),
                                 P(bout), P(pout), None, None, 0, None)


def test_forward_state_validation(lib):
    x = A16
    base = (1, 4, 4, L.WKV_F32, x, x, x, x, x)
    # the three state pointers of each side are all NULL or all set
    assert fwd_state(lib, *base, ain=x) == L.WKV_EINVAL
    assert fwd_state(lib, *base, ain=x, bin_=x) == L.WKV_EINVAL
    assert fwd_state(lib, *base, bout=x) == L.WKV_EINVAL
    assert fwd_state(lib, *base, ain=x, bin_=x, pin=x, aout=x, bout=x) == L.WKV_EINVAL
    assert fwd_state(lib, *base, ain=x, bin_=x, pin=x + 2) == L.WKV_EALIGN
    assert fwd_state(lib, *base, aout=x + 1, bout=x, pout=x) == L.WKV_EALIGN
    assert fwd_state(lib, 1, 4, 4, 5, x, x, x, x, x, ain=x, bin_=x, pin=x) == L.WKV_EDTYPE
    # no lanes: nothing to do, states included
    assert fwd_state(lib, 0, 4, 4, L.WKV_F32, None, None, None, None, None, x, x, x, x, x, x) == L.WKV_OK


def test_backward_validation(lib):
    x = A16
    ws_need = lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 1, 4, 4, L.WKV_F32)
    args = [x] * 9
    assert bwd(lib, 1, -4, 4, L.WKV_F32, *args) == L.WKV_EINVAL
    assert bwd(lib, 1, 4, 4, 9, *args) == L.WKV_EDTYPE
    assert bwd(lib, 1, 4, 4, L.WKV_F32, x, x, x, x, x, x, x, None, x) == L.WKV_EINVAL
    assert bwd(lib, 1, 4, 4, L.WKV_F32, x, x, x, x, None, x, x, x, x) == L.WKV_EINVAL
    assert bwd(lib, 1, 4, 4, L.WKV_F32, x, x, x, x, x, x + 2, x, x, x) == L.WKV_EALIGN
    assert bwd(lib, 1, 4, 4, L.WKV_BF16, x, x, x, x, x + 1, x, x, x, x) == L.WKV_EALIGN
    if ws_need > 0:
        assert bwd(lib, 1, 4, 4, L.WKV_F32, *args) == L.WKV_EWORKSPACE
        assert bwd(lib, 1, 4, 4, L.WKV_F32, *args, ws=x, nws=ws_need - 1) == L.WKV_EWORKSPACE
    assert bwd(lib, 1, 4, 0, L.WKV_F32, *[None] * 9) == L.WKV_OK


def bwd_state(lib, B, T, C, dt, x, sin=(None,) * 3, sout=(None,) * 3, gin=(None,) * 3, dw=None):
    dw = x if dw is None else dw
    return lib.wkv_backward_state(B, T, C, dt, P(x), P(x), P(x), P(x), P(x), *[P(t) for t in sin],
                                  *[P(t) for t in sout], P(x), P(x), P(dw), P(x), *[P(t) for t in gin],
                                  None, None, 0, None)


def test_backward_state_validation(lib):
    """Each state triple all NULL or all set, the given state's gradients only
    with a given state, 4-byte alignment; checked before any HIP call."""
    x = A16
    three = (x, x, x)
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sin=(x, x, None)) == L.WKV_EINVAL
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sout=(None, x, x)) == L.WKV_EINVAL
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sin=three, gin=(x, None, x)) == L.WKV_EINVAL
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, gin=three) == L.WKV_EINVAL  # no given state
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sin=(x, x + 2, x)) == L.WKV_EALIGN
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sout=(x, x, x + 1)) == L.WKV_EALIGN
    assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sin=three, gin=(x + 2, x, x)) == L.WKV_EALIGN
    assert bwd_state(lib, 1, 4, 4, 9, x, sin=three) == L.WKV_EDTYPE
    assert bwd_state(lib, 1, 4, 0, L.WKV_F32, x, sin=three, sout=three, gin=three) == L.WKV_OK  # C = 0
    ws_need = lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 1, 4, 4, L.WKV_F32)
    if ws_need > 0:
        assert bwd_state(lib, 1, 4, 4, L.WKV_F32, x, sin=three, sout=three, gin=three) == L.WKV_EWORKSPACE


def test_step_validation(lib):
    x = A16
    args = [x] * 8
    assert step(lib, -1, 2, 4, L.WKV_F32, *args) == L.WKV_EINVAL
    assert step(lib, 1, 2, 4, 4, *args) == L.WKV_EDTYPE
    assert step(lib, 1 << 30, 1 << 30, 1 << 10, L.WKV_F32, *args) == L.WKV_ESIZE
    assert step(lib, 1, 2, 4, L.WKV_F32, x, x, x, x, x, x, x, None) == L.WKV_EINVAL
    assert step(lib, 1, 2, 4, L.WKV_F32, x, x, x, x, x, x + 3, x, x) == L.WKV_EALIGN
    assert step(lib, 0, 2, 4, L.WKV_F32, *[None] * 8) == L.WKV_OK


def test_binding_rejects_host_tensors():
    """There is no CPU path: host tensors are refused before the library is called."""
    import torch

    from rwkv_wkv_mixing_amd import ops

    w = torch.ones(4)
    with pytest.raises(ValueError):
        ops.wkv_forward(w, w, torch.zeros(1, 2, 4), torch.zeros(1, 2, 4))
    with pytest.raises(ValueError):
        ops.wkv_step(torch.ones(1, 4), torch.ones(1, 4), torch.zeros(1, 2, 4), torch.zeros(1, 2, 4),
                     torch.zeros(1, 2, 4), torch.zeros(1, 2, 4), torch.zeros(1, 2, 4))


def shift(lib, B, T, C, M, dt, mu, x, xp, out):
    return lib.wkv_token_shift(B, T, C, M, dt, P(mu), P(x), P(xp), P(out), None)


def shift_bwd(lib, B, T, C, M, dt, mu, x, xp, g, dx, dmu, dxp, ws=None, nws=0):
    return lib.wkv_token_shift_backward(B, T, C, M, dt, P(mu), P(x), P(xp), P(g), P(dx), P(dmu), P(dxp),
                                        P(ws), nws, None)


def test_token_shift_workspace_size(lib):
    # partial sums of dmu: one row per (batch row, block of 128 tokens), M * C floats each
    assert lib.wkv_token_shift_workspace_bytes(8, 1024, 4096, 3) == 8 * 8 * 3 * 4096 * 4
    assert lib.wkv_token_shift_workspace_bytes(2, 128, 7, 1) == 2 * 1 * 7 * 4
    assert lib.wkv_token_shift_workspace_bytes(2, 129, 7, 1) == 2 * 2 * 7 * 4
    assert lib.wkv_token_shift_workspace_bytes(2, 257, 7, 1) == 2 * 3 * 7 * 4
    assert lib.wkv_token_shift_workspace_bytes(2, 0, 7, 1) == 0
    assert lib.wkv_token_shift_workspace_bytes(2, 5, 7, 0) == 0   # M out of range
    assert lib.wkv_token_shift_workspace_bytes(2, 5, 7, 5) == 0
    assert lib.wkv_token_shift_workspace_bytes(-2, 5, 7, 1) == 0
    assert lib.wkv_token_shift_workspace_bytes(1 << 30, 1 << 30, 1 << 10, 1) == 0


def test_token_shift_validation(lib):
    x = A16
    assert shift(lib, 1, 4, 4, 0, L.WKV_F32, x, x, None, x) == L.WKV_EINVAL
    assert shift(lib, 1, 4, 4, 5, L.WKV_F32, x, x, None, x) == L.WKV_EINVAL
    assert shift(lib, -1, 4, 4, 3, L.WKV_F32, x, x, None, x) == L.WKV_EINVAL
    assert shift(lib, 1, 4, 4, 3, 2, x, x, None, x) == L.WKV_EDTYPE
    assert shift(lib, 1 << 30, 1 << 30, 1 << 10, 3, L.WKV_F32, x, x, None, x) == L.WKV_ESIZE
    assert shift(lib, 1, 4, 4, 3, L.WKV_F32, None, x, None, x) == L.WKV_EINVAL
    assert shift(lib, 1, 4, 4, 3, L.WKV_F32, x, x, None, None) == L.WKV_EINVAL
    assert shift(lib, 1, 4, 4, 3, L.WKV_F32, x, x + 2, None, x) == L.WKV_EALIGN
    assert shift(lib, 1, 4, 4, 3, L.WKV_BF16, x, x, x + 1, x) == L.WKV_EALIGN
    assert shift(lib, 1, 4, 4, 3, L.WKV_BF16, x + 2, x, None, x) == L.WKV_EALIGN
    assert shift(lib, 0, 4, 4, 3, L.WKV_F32, None, None, None, None) == L.WKV_OK
    assert shift(lib, 2, 0, 4, 3, L.WKV_F32, None, None, None, None) == L.WKV_OK
    need = lib.wkv_token_shift_workspace_bytes(1, 4, 4, 3)
    args = [x] * 7
    assert shift_bwd(lib, 1, 4, 4, 9, L.WKV_F32, *args, ws=x, nws=need) == L.WKV_EINVAL
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, x, x, None, x, x, None, None, ws=x, nws=need) == L.WKV_EINVAL
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, x, x, None, None, x, x, None, ws=x, nws=need) == L.WKV_EINVAL
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, x, x, None, x, x + 2, x, None, ws=x, nws=need) == L.WKV_EALIGN
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, x, x, None, x, x, x, x + 1, ws=x, nws=need) == L.WKV_EALIGN
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, *args) == L.WKV_EWORKSPACE
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, *args, ws=x, nws=need - 1) == L.WKV_EWORKSPACE
    assert shift_bwd(lib, 1, 4, 4, 3, L.WKV_F32, *args, ws=x + 16, nws=need) == L.WKV_EWORKSPACE
    assert shift_bwd(lib, 1, 4, 0, 3, L.WKV_F32, *[None] * 7) == L.WKV_OK


def wkv5(lib, B, T, H, N, dt, w, u, r, k, v, o, si=None, so=None, ck=None):
    return lib.wkv5_forward(B, T, H, N, dt, P(w), P(u), P(r), P(k), P(v), P(o), P(si), P(so), P(ck), None, 0, None)


def test_wkv5_validation(lib):
    x = A16
    args = [x] * 6
    assert wkv5(lib, 1, 4, 2, 32, L.WKV_BF16, *args) == L.WKV_EINVAL      # head size must be 64
    assert wkv5(lib, -1, 4, 2, 64, L.WKV_BF16, *args) == L.WKV_EINVAL
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_F32, *args) == L.WKV_EDTYPE       # bf16 operands only
    assert wkv5(lib, 1, 4, 2, 64, 7, *args) == L.WKV_EDTYPE
    assert wkv5(lib, 1 << 30, 1 << 30, 1 << 10, 64, L.WKV_BF16, *args) == L.WKV_ESIZE
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, None, x, x, x) == L.WKV_EINVAL
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x + 2, x, x, x) == L.WKV_EALIGN   # r, k, v 16-byte aligned
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x, x, x, x + 2) == L.WKV_EALIGN
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_BF16, *args, si=x + 1) == L.WKV_EALIGN
    assert wkv5(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ck=x + 8) == L.WKV_EALIGN   # ckpt 16-byte aligned
    assert wkv5(lib, 0, 4, 2, 64, L.WKV_BF16, *[None] * 6) == L.WKV_OK
    assert wkv5(lib, 2, 4, 0, 64, L.WKV_BF16, *[None] * 6) == L.WKV_OK


def test_wkv5_workspace_sizes(lib):
    # chunk-start states: bf16 64 x 64 per (batch row, head, 64-token chunk); partial sums: 2 x 64 float32
    assert lib.wkv5_ckpt_bytes(2, 100, 3, 64) == 2 * 3 * 2 * 64 * 64 * 2
    assert lib.wkv5_ckpt_bytes(1, 1, 1, 64) == 64 * 64 * 2
    assert lib.wkv5_ckpt_bytes(1, 1, 1, 32) == 0
    assert lib.wkv5_backward_workspace_bytes(2, 100, 3, 64, 1) == 2 * 3 * 2 * 64 * 4
    assert lib.wkv5_backward_workspace_bytes(2, 100, 3, 64, 0) == 2 * 3 * 2 * 64 * 4 + 2 * 3 * 2 * 64 * 64 * 2
    assert lib.wkv5_backward_workspace_bytes(2, 0, 3, 64, 0) == 0
    assert lib.wkv5_backward_workspace_bytes(2, 10, 3, 48, 0) == 0


def wkv5_bwd(lib, B, T, H, N, dt, w, u, r, k, v, go, dr, dk, dv, dw, du, si=None, dso=None, dsi=None, ck=None,
             ws=None, nws=0):
    return lib.wkv5_backward(B, T, H, N, dt, P(w), P(u), P(r), P(k), P(v), P(go), P(si), P(dso), P(dr), P(dk), P(dv),
                             P(dw), P(du), P(dsi), P(ck), P(ws), nws, None)


def test_wkv5_backward_validation(lib):
    x = A16
    args = [x] * 11
    need = lib.wkv5_backward_workspace_bytes(1, 4, 2, 64, 0)
    ok = dict(ws=x, nws=need)
    assert wkv5_bwd(lib, 1, 4, 2, 32, L.WKV_BF16, *args, **ok) == L.WKV_EINVAL       # head size must be 64
    assert wkv5_bwd(lib, 1, -4, 2, 64, L.WKV_BF16, *args, **ok) == L.WKV_EINVAL
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_F32, *args, **ok) == L.WKV_EDTYPE        # bf16 operands only
    assert wkv5_bwd(lib, 1 << 30, 1 << 30, 1 << 10, 64, L.WKV_BF16, *args, **ok) == L.WKV_ESIZE
    assert wkv5_bwd(lib, 1, 4, 0, 64, L.WKV_BF16, *[None] * 11) == L.WKV_OK          # no heads: nothing to do
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args[:9], None, x, **ok) == L.WKV_EINVAL   # dw NULL
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args[:9], x + 2, x, **ok) == L.WKV_EALIGN
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, dso=x + 1, **ok) == L.WKV_EALIGN
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, dsi=x + 1, **ok) == L.WKV_EALIGN
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, None, *args[3:], **ok) == L.WKV_EINVAL  # r NULL
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x, x, x, None, *args[6:], **ok) == L.WKV_EINVAL  # go NULL
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x, x, x, x + 2, *args[6:], **ok) == L.WKV_EALIGN  # go
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ck=x + 8, **ok) == L.WKV_EALIGN
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args) == L.WKV_EWORKSPACE
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x, nws=need - 1) == L.WKV_EWORKSPACE
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x + 16, nws=need) == L.WKV_EWORKSPACE
    # with a ckpt only the partial sums are needed
    small = lib.wkv5_backward_workspace_bytes(1, 4, 2, 64, 1)
    assert wkv5_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x, nws=small - 1, ck=x) == L.WKV_EWORKSPACE


def wkv6(lib, B, T, H, N, dt, w, u, r, k, v, o, si=None, so=None, ck=None):
    return lib.wkv6_forward(B, T, H, N, dt, P(w), P(u), P(r), P(k), P(v), P(o), P(si), P(so), P(ck), None, 0, None)


def test_wkv6_validation(lib):
    x = A16
    args = [x] * 6
    assert wkv6(lib, 1, 4, 2, 32, L.WKV_BF16, *args) == L.WKV_EINVAL      # head size must be 64
    assert wkv6(lib, 1, -4, 2, 64, L.WKV_BF16, *args) == L.WKV_EINVAL
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_F32, *args) == L.WKV_EDTYPE       # bf16 operands only
    assert wkv6(lib, 1 << 30, 1 << 30, 1 << 10, 64, L.WKV_BF16, *args) == L.WKV_ESIZE
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_BF16, None, x, x, x, x, x) == L.WKV_EINVAL   # w NULL
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_BF16, x + 4, x, x, x, x, x) == L.WKV_EALIGN  # w 16-byte aligned
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x + 2, x, x, x) == L.WKV_EALIGN
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_BF16, *args, so=x + 1) == L.WKV_EALIGN
    assert wkv6(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ck=x + 8) == L.WKV_EALIGN
    assert wkv6(lib, 0, 4, 2, 64, L.WKV_BF16, *[None] * 6) == L.WKV_OK


def test_wkv6_backward_sizes(lib):
    # the RWKV-6 calls share the RWKV-5 layouts of the chunk-start states and partial sums
    for args in ((2, 100, 3, 64), (1, 1, 1, 64), (1, 1, 1, 32), (2, 0, 3, 64)):
        assert lib.wkv6_ckpt_bytes(*args) == lib.wkv5_ckpt_bytes(*args)
        for have in (0, 1):
            assert lib.wkv6_backward_workspace_bytes(*args, have) == lib.wkv5_backward_workspace_bytes(*args, have)


def wkv6_bwd(lib, B, T, H, N, dt, w, u, r, k, v, go, dr, dk, dv, dw, du, si=None, dso=None, dsi=None, ck=None,
             ws=None, nws=0):
    return lib.wkv6_backward(B, T, H, N, dt, P(w), P(u), P(r), P(k), P(v), P(go), P(si), P(dso), P(dr), P(dk), P(dv),
                             P(dw), P(du), P(dsi), P(ck), P(ws), nws, None)


def test_wkv6_backward_validation(lib):
    x = A16
    args = [x] * 11
    need = lib.wkv6_backward_workspace_bytes(1, 4, 2, 64, 0)
    ok = dict(ws=x, nws=need)
    assert wkv6_bwd(lib, 1, 4, 2, 32, L.WKV_BF16, *args, **ok) == L.WKV_EINVAL       # head size must be 64
    assert wkv6_bwd(lib, 1, -4, 2, 64, L.WKV_BF16, *args, **ok) == L.WKV_EINVAL
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_F32, *args, **ok) == L.WKV_EDTYPE        # bf16 operands only
    assert wkv6_bwd(lib, 1 << 30, 1 << 30, 1 << 10, 64, L.WKV_BF16, *args, **ok) == L.WKV_ESIZE
    assert wkv6_bwd(lib, 1, 4, 0, 64, L.WKV_BF16, *[None] * 11) == L.WKV_OK          # no heads: nothing to do
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args[:10], None, **ok) == L.WKV_EINVAL    # du NULL
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args[:9], None, x, **ok) == L.WKV_EINVAL  # dw NULL
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args[:9], x + 2, x, **ok) == L.WKV_EALIGN
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x + 4, *args[1:], **ok) == L.WKV_EALIGN   # w 16-byte aligned
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, dso=x + 1, **ok) == L.WKV_EALIGN
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, dsi=x + 1, **ok) == L.WKV_EALIGN
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, None, *args[3:], **ok) == L.WKV_EINVAL  # r NULL
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x, x, x, None, *args[6:], **ok) == L.WKV_EINVAL  # go NULL
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, x, x, x, x, x, x + 2, *args[6:], **ok) == L.WKV_EALIGN  # go
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ck=x + 8, **ok) == L.WKV_EALIGN
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args) == L.WKV_EWORKSPACE
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x, nws=need - 1) == L.WKV_EWORKSPACE
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x + 16, nws=need) == L.WKV_EWORKSPACE
    small = lib.wkv6_backward_workspace_bytes(1, 4, 2, 64, 1)
    assert wkv6_bwd(lib, 1, 4, 2, 64, L.WKV_BF16, *args, ws=x, nws=small - 1, ck=x) == L.WKV_EWORKSPACE


def test_matrix_backward_split_workspace(lib):
    # 1 x 1000 x 2 heads: 8 segments of 2 chunks.  Split size = the dw/du partials (2 x 64 float32
    # per pair) for every segment + the forward split's region; WKV_WS_NO_SPLIT (2) = one set of
    # partials; without WKV_WS_HAVE_CKPT (1) both add the recomputed chunk-start states
    B, T, H = 1, 1000, 2
    full = lib.wkv5_backward_workspace_bytes(B, T, H, 64, 1)
    flat = lib.wkv5_backward_workspace_bytes(B, T, H, 64, 3)
    assert flat == B * H * 2 * 64 * 4
    assert full == 8 * flat + lib.wkv5_forward_workspace_bytes(B, T, H, 64)
    assert lib.wkv5_backward_workspace_bytes(B, T, H, 64, 0) == full + lib.wkv5_ckpt_bytes(B, T, H, 64)
    assert lib.wkv5_backward_workspace_bytes(B, T, H, 64, 2) == flat + lib.wkv5_ckpt_bytes(B, T, H, 64)
    assert full % 256 == 0 and flat % 256 == 0
    assert lib.wkv6_backward_workspace_bytes(B, T, H, 64, 1) == full
    # 256 pairs: the backward splits (2 segments), the forward does not
    assert lib.wkv5_forward_workspace_bytes(4, 1024, 64, 64) == 0
    assert lib.wkv5_backward_workspace_bytes(4, 1024, 64, 64, 1) > lib.wkv5_backward_workspace_bytes(4, 1024, 64, 64, 3)
    # 512 pairs (or 3 chunks): no split, one size whatever the flags
    for shape in ((8, 1024, 64), (1, 192, 2)):
        assert lib.wkv5_backward_workspace_bytes(*shape, 64, 1) == lib.wkv5_backward_workspace_bytes(*shape, 64, 3)


def test_matrix_forward_split_workspace(lib):
    # a split only below 256 (batch row, head) pairs and from 4 chunks: local and start states
    # (2 x 64 x 64 float32) and summed rates (64 float32) per pair and segment
    assert lib.wkv5_forward_workspace_bytes(8, 1024, 64, 64) == 0       # 512 pairs: no split
    assert lib.wkv5_forward_workspace_bytes(1, 192, 2, 64) == 0         # 3 chunks: no split
    assert lib.wkv5_forward_workspace_bytes(1, 1000, 2, 64) == 2 * 8 * (2 * 64 * 64 + 64) * 4  # 8 segments of 2 chunks
    assert lib.wkv5_forward_workspace_bytes(1, 1000, 2, 32) == 0
    assert lib.wkv6_forward_workspace_bytes(1, 1000, 2, 64) == lib.wkv5_forward_workspace_bytes(1, 1000, 2, 64)
    x = A16
    need = lib.wkv5_forward_workspace_bytes(1, 1000, 2, 64)
    for fn in (lib.wkv5_forward, lib.wkv6_forward):
        args = [P(x)] * 6
        assert fn(1, 1000, 2, 64, L.WKV_BF16, *args, None, None, None, P(x), need - 1, None) == L.WKV_EWORKSPACE
        assert fn(1, 1000, 2, 64, L.WKV_BF16, *args, None, None, None, P(x + 16), need, None) == L.WKV_EWORKSPACE


def test_workspace_status_validation(lib):
    """Rejected on the host, before any HIP call: NULL, too small, misaligned."""
    buf = ctypes.create_string_buffer(1024)
    base = ctypes.addressof(buf)
    aligned = (base + 255) // 256 * 256
    assert lib.wkv_workspace_status(None, 256, 0, None) == L.WKV_EINVAL
    assert lib.wkv_workspace_status(ctypes.c_void_p(aligned), 4, 0, None) == L.WKV_EWORKSPACE
    assert lib.wkv_workspace_status(ctypes.c_void_p(aligned + 16), 256, 0, None) == L.WKV_EWORKSPACE


def test_noalloc_forward_validation(lib):
    """The forward on the library's static scratch rejects on the host, before
    any HIP call: a problem whose workspace exceeds the static array
    (WKV_ESCRATCH), and the checks of wkv_forward_state."""
    f = lib.wkv_forward_state_noalloc
    nul = [None] * 12
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, 4, 32768, 4096, L.WKV_BF16) > L.WKV_STATIC_SCRATCH_BYTES
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, 2, 32768, 4096, L.WKV_BF16) <= L.WKV_STATIC_SCRATCH_BYTES
    assert f(4, 32768, 4096, L.WKV_BF16, *nul, None) == L.WKV_ESCRATCH
    assert f(2, 32768, 4096, L.WKV_BF16, *nul, None) == L.WKV_EINVAL
    assert f(1, 8, 4, 7, *nul, None) == L.WKV_EDTYPE
    assert f(-1, 8, 4, L.WKV_F32, *nul, None) == L.WKV_EINVAL
    assert f(1, 0, 4, L.WKV_F32, *nul, None) == L.WKV_OK  # nothing to do, no state: no launch
    assert "#define WKV_STATIC_SCRATCH_BYTES (32u << 20)" in open(HEADER).read()


def test_debug_spin_limit_exchanges():
    lib = L.lib()
    old = lib.wkv_debug_spin_limit(5)
    assert old == 1 << 22
    assert lib.wkv_debug_spin_limit(old) == 5
    assert lib.wkv_debug_spin_limit(old) == old


def test_carry_regions_beyond_32_bit_addressing_are_rejected(lib):
    """Carries between workgroups are addressed through 32-bit buffer resources:
    a shape whose carry region would pass 4 GiB gets no workspace size and the
    calls return WKV_ESIZE before touching any pointer."""
    T = 1 << 30  # one 64-channel tile, 2^22 blocks of 256 tokens: 4 GiB of 16-byte slots
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, 1, T, 64, L.WKV_BF16) == 0
    assert lib.wkv_workspace_bytes(L.WKV_OP_BACKWARD, 1, T, 64, L.WKV_BF16) == 0
    p = ctypes.c_void_p(256)
    assert lib.wkv_forward(1, T, 64, L.WKV_BF16, p, p, p, p, p, None, p, 1 << 20, None) == L.WKV_ESIZE
    assert lib.wkv_backward(1, T, 64, L.WKV_BF16, p, p, p, p, p, p, p, p, p, None, p, 1 << 20, None) == L.WKV_ESIZE
    assert lib.wkv_workspace_bytes(L.WKV_OP_FORWARD, 1, T // 8, 64, L.WKV_BF16) > 0
