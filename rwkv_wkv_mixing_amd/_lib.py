"""ctypes declarations of the C ABI in include/wkv.h (librwkv_wkv.so).

Loading never falls back to anything: if the library is missing, ``lib()``
raises, and every op in this package fails with it.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librwkv_wkv.so")

WKV_OK, WKV_EINVAL, WKV_EDTYPE, WKV_ESIZE, WKV_EALIGN, WKV_EWORKSPACE, WKV_EHIP, WKV_ETIMEOUT, WKV_ESCRATCH = range(9)
WKV_STATIC_SCRATCH_BYTES = 32 << 20
WKV_F32, WKV_BF16 = 0, 1
WKV_OP_FORWARD, WKV_OP_BACKWARD = 0, 1
WKV_CKPT_LEN = 16

# every symbol include/wkv.h declares
EXPORTS = (
    "wkv_workspace_bytes",
    "wkv_ckpt_bytes",
    "wkv_forward",
    "wkv_forward_state",
    "wkv_forward_state_noalloc",
    "wkv_backward",
    "wkv_backward_state",
    "wkv_forward_gated",
    "wkv_backward_gated",
    "wkv_step",
    "wkv5_forward",
    "wkv6_forward",
    "wkv5_forward_workspace_bytes",
    "wkv6_forward_workspace_bytes",
    "wkv5_ckpt_bytes",
    "wkv5_backward_workspace_bytes",
    "wkv5_backward",
    "wkv6_ckpt_bytes",
    "wkv6_backward_workspace_bytes",
    "wkv6_backward",
    "wkv_token_shift_workspace_bytes",
    "wkv_token_shift",
    "wkv_token_shift_backward",
    "wkv_workspace_status",
    "wkv_debug_spin_limit",
    "wkv_status_str",
    "wkv_last_hip_error",
    "wkv_version",
)

_lib = None


class WkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().wkv_status_str(status).decode()
        if status == WKV_EHIP:
            msg += ": " + lib().wkv_last_hip_error().decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load librwkv_wkv.so (built by rwkv_wkv_mixing_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing; run `python -m rwkv_wkv_mixing_amd.build`"
        )
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(L):
    """Attach the argument and return types of include/wkv.h to a loaded library."""
    i64, i32, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    L.wkv_workspace_bytes.restype = sz
    L.wkv_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
    L.wkv_ckpt_bytes.restype = sz
    L.wkv_ckpt_bytes.argtypes = [i64, i64, i64]
    L.wkv_forward.restype = i32
    L.wkv_forward.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, fp, vp, vp, sz, vp]
    L.wkv_forward_state.restype = i32
    L.wkv_forward_state.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, fp, fp, fp, fp, fp, fp, fp, vp, vp, sz, vp]
    L.wkv_forward_state_noalloc.restype = i32
    L.wkv_forward_state_noalloc.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, fp, fp, fp, fp, fp, fp, fp, vp, vp]
    L.wkv_backward.restype = i32
    L.wkv_backward.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, vp, fp, fp, fp, fp, vp, vp, sz, vp]
    L.wkv_backward_state.restype = i32
    L.wkv_backward_state.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                     fp, fp, fp, vp, vp, sz, vp]
    L.wkv_forward_gated.restype = i32
    L.wkv_forward_gated.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, vp, fp, vp, vp, sz, vp]
    L.wkv_backward_gated.restype = i32
    L.wkv_backward_gated.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, vp, vp, fp, fp, fp, fp, fp, vp, vp, sz, vp]
    L.wkv_step.restype = i32
    L.wkv_step.argtypes = [i64, i64, i64, i32, fp, fp, vp, vp, fp, fp, fp, fp, vp]
    L.wkv5_forward.restype = i32
    L.wkv5_forward.argtypes = [i64, i64, i64, i64, i32, fp, fp, vp, vp, vp, fp, fp, fp, vp, vp, sz, vp]
    L.wkv6_forward.restype = i32
    L.wkv6_forward.argtypes = [i64, i64, i64, i64, i32, fp, fp, vp, vp, vp, fp, fp, fp, vp, vp, sz, vp]
    L.wkv5_forward_workspace_bytes.restype = sz
    L.wkv5_forward_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.wkv6_forward_workspace_bytes.restype = sz
    L.wkv6_forward_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.wkv5_ckpt_bytes.restype = sz
    L.wkv5_ckpt_bytes.argtypes = [i64, i64, i64, i64]
    L.wkv5_backward_workspace_bytes.restype = sz
    L.wkv5_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.wkv5_backward.restype = i32
    L.wkv5_backward.argtypes = [i64, i64, i64, i64, i32, fp, fp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, vp, vp,
                                sz, vp]
    L.wkv6_ckpt_bytes.restype = sz
    L.wkv6_ckpt_bytes.argtypes = [i64, i64, i64, i64]
    L.wkv6_backward_workspace_bytes.restype = sz
    L.wkv6_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    L.wkv6_backward.restype = i32
    L.wkv6_backward.argtypes = [i64, i64, i64, i64, i32, fp, fp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, vp, vp,
                                sz, vp]
    L.wkv_token_shift_workspace_bytes.restype = sz
    L.wkv_token_shift_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.wkv_token_shift.restype = i32
    L.wkv_token_shift.argtypes = [i64, i64, i64, i64, i32, fp, vp, vp, vp, vp]
    L.wkv_token_shift_backward.restype = i32
    L.wkv_token_shift_backward.argtypes = [i64, i64, i64, i64, i32, fp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
    L.wkv_workspace_status.restype = i32
    L.wkv_workspace_status.argtypes = [vp, sz, i32, vp]
    L.wkv_debug_spin_limit.restype = ctypes.c_uint32
    L.wkv_debug_spin_limit.argtypes = [ctypes.c_uint32]
    L.wkv_status_str.restype = ctypes.c_char_p
    L.wkv_status_str.argtypes = [i32]
    L.wkv_last_hip_error.restype = ctypes.c_char_p
    L.wkv_last_hip_error.argtypes = []
    L.wkv_version.restype = ctypes.c_char_p
    L.wkv_version.argtypes = []
    return L


def check(fn: str, status: int) -> None:
    if status != WKV_OK:
        raise WkvError(fn, status)
