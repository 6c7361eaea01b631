"""Build the HIP library librwkv_wkv.so in-tree for gfx950 with hipcc.

    python -m rwkv_wkv_mixing_amd.build        # or __graft_entry__.build()

Each csrc/*.hip file is compiled to an object in parallel, then linked into a
shared library next to this file.  Packed-FP32 instruction selection is
switched off (-packed-fp32-ops); hipcc's host pass warns that it does not know
that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librwkv_wkv.so")
STREAM_SRC = os.path.join(PKG, "stream", "stream.hip")
STREAM_LIB = os.path.join(PKG, "librwkv_stream.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link librwkv_wkv.so.  Always rebuilds."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


def build_stream(verbose: bool = False) -> str:
    """Compile the streaming-ceiling kernels (stream/stream.hip) into
    librwkv_stream.so: measurement only, not part of the operator library."""
    os.makedirs(OBJDIR, exist_ok=True)
    obj = _compile(STREAM_SRC, verbose)
    tmp = STREAM_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, STREAM_LIB)
    return STREAM_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_stream(verbose="-v" in sys.argv))
