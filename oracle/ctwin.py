"""ctypes loader for the float64 C twin of the oracle (oracle/wkv_ref.c).

TEST INFRASTRUCTURE ONLY (see oracle/wkv_ref.py).  ``build_ctwin()`` compiles
the library with gcc; ``load_ctwin()`` loads what is built and raises if
nothing is.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "wkv_ref.c")
LIB = os.path.join(_HERE, "libwkv_ref.so")

_lib = None


def build_ctwin(verbose: bool = False) -> str:
    """Compile oracle/wkv_ref.c into oracle/libwkv_ref.so (gcc, OpenMP, -O2).

    No -ffast-math: the twin must keep IEEE double semantics.
    """
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def load_ctwin():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise RuntimeError(f"oracle C twin not built: {LIB} missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.wkv_ref_max_threads.restype = i32
    lib.wkv_ref_max_threads.argtypes = []
    lib.wkv_ref_forward.restype = i32
    lib.wkv_ref_forward.argtypes = [i64, i64, i64, fp, fp, fp, fp, dp, dp, dp, i32]
    lib.wkv_ref_backward.restype = i32
    lib.wkv_ref_backward.argtypes = [i64, i64, i64, fp, fp, fp, fp, fp, dp, dp, dp, dp, i32]
    vp = ctypes.c_void_p
    lib.wkv_ref_step.restype = i32
    lib.wkv_ref_step.argtypes = [i64, i64, i64, fp, fp, vp, vp, i32, dp, dp, dp, i32]
    _lib = lib
    return lib


def _fptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _dptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f32c(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def ctwin_forward(w, u, k, v, want_y=True, want_sums=False, nthreads=0):
    """Float64 forward of the C twin.  Inputs must be exactly representable in
    float32 (they are: fp32 or bf16-rounded workloads).  Returns
    (y or None, A or None, B or None, threads_used)."""
    lib = load_ctwin()
    w, u, k, v = _f32c(w), _f32c(u), _f32c(k), _f32c(v)
    Bsz, T, C = k.shape
    y = np.empty((Bsz, T, C)) if want_y else None
    A = np.empty((Bsz, C)) if want_sums else None
    Bs = np.empty((Bsz, C)) if want_sums else None
    used = lib.wkv_ref_forward(Bsz, T, C, _fptr(w), _fptr(u), _fptr(k), _fptr(v),
                               _dptr(y), _dptr(A), _dptr(Bs), int(nthreads))
    return y, A, Bs, used


def ctwin_backward(w, u, k, v, gy, nthreads=0):
    """Float64 backward of the C twin: (dk, dv, dw, du, threads_used)."""
    lib = load_ctwin()
    w, u, k, v, gy = _f32c(w), _f32c(u), _f32c(k), _f32c(v), _f32c(gy)
    Bsz, T, C = k.shape
    dk = np.empty((Bsz, T, C))
    dv = np.empty((Bsz, T, C))
    dw = np.empty(C)
    du = np.empty(C)
    used = lib.wkv_ref_backward(Bsz, T, C, _fptr(w), _fptr(u), _fptr(k), _fptr(v), _fptr(gy),
                                _dptr(dk), _dptr(dv), _dptr(dw), _dptr(du), int(nthreads))
    if used < 0:
        raise MemoryError("oracle C twin: scratch allocation failed")
    return dk, dv, dw, du, used


def ctwin_step(w, u, k, v, A, Bs, want_y=True, nthreads=0):
    """One float64 decode step of the C twin for [L, B, C] lanes, in place on the
    plain sums A, Bs (float64 [L, B, C], C-contiguous).  w, u: [L, C]; k, v:
    float32 values or uint16 bf16 bits, [L, B, C].  Returns (y or None,
    threads_used)."""
    lib = load_ctwin()
    w, u = _f32c(w), _f32c(u)
    bf16 = k.dtype == np.uint16
    if not bf16:
        k, v = _f32c(k), _f32c(v)
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)
    assert A.dtype == np.float64 and Bs.dtype == np.float64 and A.flags.c_contiguous and Bs.flags.c_contiguous
    Ln, Bsz, C = k.shape
    assert A.shape == k.shape == v.shape == Bs.shape and w.shape == u.shape == (Ln, C)
    y = np.empty((Ln, Bsz, C)) if want_y else None
    used = lib.wkv_ref_step(Ln, Bsz, C, _fptr(w), _fptr(u), k.ctypes.data_as(ctypes.c_void_p),
                            v.ctypes.data_as(ctypes.c_void_p), 1 if bf16 else 0, _dptr(A), _dptr(Bs), _dptr(y),
                            int(nthreads))
    if used < 0:
        raise MemoryError("oracle C twin: scratch allocation failed")
    return y, used
