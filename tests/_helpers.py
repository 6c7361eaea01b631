"""Shared test helpers: tolerance checks and host <-> device marshalling."""
from __future__ import annotations

import numpy as np


def check_close(name, got, ref, rtol, atol, report=None):
    """Element passes iff |g - o| <= max(atol, rtol |o|).  Asserts all pass."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (name, g.shape, o.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite values in GPU output"
    err = np.abs(g - o)
    tol = np.maximum(atol, rtol * np.abs(o))
    ok = err <= tol
    rel = err / np.maximum(np.abs(o), 1e-30)
    info = dict(name=name, max_abs=float(err.max(initial=0.0)), max_rel=float(rel.max(initial=0.0)),
                pass_frac=float(ok.mean()) if ok.size else 1.0, worst_ratio=float((err / tol).max(initial=0.0)))
    if report is not None:
        report.append(info)
    print(f"  {name}: max_abs={info['max_abs']:.3e} max_rel={info['max_rel']:.3e} "
          f"pass={info['pass_frac']:.6f} worst_err/tol={info['worst_ratio']:.3f}", flush=True)
    if not ok.all():
        idx = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{name}: {int((~ok).sum())} of {ok.size} elements out of tolerance; "
                             f"worst at {idx}: got {g[idx]!r} ref {o[idx]!r} (rtol={rtol}, atol={atol})")
    return info


def _rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def bwd_atol(ref, rtol=1e-3, gy=None, v=None):
    """Absolute floor where none is stated: rtol * 1e-2 * RMS of the reference
    tensor.  Where a gradient is exactly zero (dk, du, dw at T = 1) the
    reference holds only float64 rounding noise, so the floor is never below
    1e-12 of the gradient's natural scale RMS(gy) (1 + RMS(v)), when given."""
    floor = rtol * 1e-2 * _rms(ref)
    if gy is not None:
        floor = max(floor, 1e-12 * _rms(gy) * (1.0 + (_rms(v) if v is not None else 0.0)))
    return floor


def to_dev(x, device, bf16_bits=None):
    """numpy -> torch device tensor.  If ``bf16_bits`` (uint16) is given, upload it as bfloat16."""
    import torch

    if bf16_bits is not None:
        t = torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).view(torch.bfloat16)
        return t.to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def problem_to_dev(p, device):
    """Upload a workloads.WkvProblem: returns dict of device tensors."""
    out = dict(w=to_dev(p.w, device), u=to_dev(p.u, device))
    for n in ("k", "v", "gy"):
        arr = getattr(p, n)
        if arr is None:
            continue
        bits = getattr(p, n + "_bits") if p.dtype == "bf16" else None
        out[n] = to_dev(arr, device, bits)
    return out
