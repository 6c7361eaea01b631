"""Thin torch binding of the C ABI: argument marshalling only.

Every function takes device tensors, allocates outputs / workspace with torch
(plumbing), and calls the same-named entry point of librwkv_wkv.so on the
current HIP stream.  There is no CPU path: host tensors are rejected.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_DT = {torch.float32: L.WKV_F32, torch.bfloat16: L.WKV_BF16}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")



class BoundCall:
    """One library call with its arguments checked and marshalled once (device addresses, sizes,
    the stream): calling it launches the same call again, with no checks and no allocation, for a
    loop that repeats one call on the same buffers (the buffers' contents may change between
    calls, not their shapes or places).  It keeps the tensors it was bound to alive.  Returns what
    the unbound call returns."""

    __slots__ = ("name", "fn", "args", "result", "_keep")

    def __init__(self, name, fn, args, result, keep):
        self.name, self.fn, self.args, self.result, self._keep = name, fn, args, result, keep

    def __call__(self):
        L.check(self.name, self.fn(*self.args))
        return self.result


def _tensors(x, acc):
    if isinstance(x, torch.Tensor):
        acc.append(x)
    elif isinstance(x, (tuple, list)):
        for y in x:
            _tensors(y, acc)
    return acc


def _launch(bind, name, fn, args, result, scope):
    """Run a library call and check its status, or (bind) return it as a BoundCall holding every
    tensor of the calling function's scope."""
    if bind:
        return BoundCall(name, fn, args, result, tuple(_tensors(list(scope.values()), [])))
    L.check(name, fn(*args))
    return result


def workspace_bytes(op: int, B: int, T: int, C: int, in_dtype: torch.dtype) -> int:
    return int(L.lib().wkv_workspace_bytes(op, B, T, C, _DT[in_dtype]))


def ckpt_bytes(B: int, T: int, C: int) -> int:
    return int(L.lib().wkv_ckpt_bytes(B, T, C))


def new_ckpt(B: int, T: int, C: int, device) -> torch.Tensor:
    """Buffer for the forward's block-start states (opaque float32)."""
    return torch.empty(ckpt_bytes(B, T, C) // 4, dtype=torch.float32, device=device)


def new_workspace(op: int, B: int, T: int, C: int, in_dtype: torch.dtype, device) -> torch.Tensor:
    """A zero-filled workspace for wkv_forward (op 0) or wkv_backward (op 1) at
    this shape.  It may be reused by later calls on the same stream, of either
    op and any shape it is large enough for (each call leaves it ready for the
    next); it must not be written in between."""
    return torch.zeros(max(workspace_bytes(op, B, T, C, in_dtype), 1), dtype=torch.uint8, device=device)


def workspace_status(workspace: torch.Tensor, clear: bool = False) -> int:
    """Synchronise the current stream and read the workspace's error word:
    WKV_OK, or WKV_ETIMEOUT if a wait between workgroups gave up (or the
    workspace was not zero-filled before its first call) since it was last
    cleared; then the outputs written since are invalid."""
    st = int(L.lib().wkv_workspace_status(_p(workspace), workspace.numel() * workspace.element_size(),
                                          1 if clear else 0, _stream(workspace.device)))
    if st not in (L.WKV_OK, L.WKV_ETIMEOUT):
        L.check("wkv_workspace_status", st)
    return st


def _workspace(op, B, T, C, dt, device, workspace):
    nbytes = workspace_bytes(op, B, T, C, dt)
    if nbytes == 0:
        return None, 0
    if workspace is None:  # zero-filled: a workspace must hold zeros before its first call
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace, workspace.numel() * workspace.element_size()


def wkv_forward(w, u, k, v, *, y=None, ckpt=None, workspace=None, state_in=None, state_out=None,
                return_state=False, bind=False):
    """y [B,T,C] float32 from w, u [C] float32 and k, v [B,T,C] (float32 or bfloat16).

    state_in:  None (empty history) or (a, b, p), each [B, C] float32, in the
               representation of wkv_step: the state before the first token.
    state_out: None or (a, b, p) tensors to receive the state after the last
               token (they may be the state_in tensors).  With
               return_state=True and no state_out, they are allocated and the
               call returns (y, (a, b, p)).
    """
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    _need(v, "v", k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if y is None:
        y = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, (B, T, C), dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    if state_out is None and return_state:
        state_out = tuple(torch.empty((B, C), dtype=torch.float32, device=dev) for _ in range(3))
    for name, st3 in (("state_in", state_in), ("state_out", state_out)):
        if st3 is not None:
            for t, n in zip(st3, "abp"):
                _need(t, f"{name}.{n}", torch.float32, (B, C), dev)
    sin = state_in if state_in is not None else (None, None, None)
    sout = state_out if state_out is not None else (None, None, None)
    ws, ws_n = _workspace(L.WKV_OP_FORWARD, B, T, C, k.dtype, dev, workspace)
    args = (B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(y), *[_p(t) for t in sin],
            *[_p(t) for t in sout], _p(ckpt), _p(ws), ws_n, _stream(dev))
    return _launch(bind, "wkv_forward_state", L.lib().wkv_forward_state, args, (y, state_out) if return_state else y, locals())


def wkv_forward_state_noalloc(w, u, k, v, y, *, ckpt=None, state_in=None, state_out=None):
    """wkv_forward for callers that cannot allocate: every buffer is the
    caller's (y [B,T,C] float32 included), and the workspace is the library's
    static scratch, shared by all calls on the GPU (calls on one GPU must not
    overlap in time).  Arguments as wkv_forward; returns y."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    _need(v, "v", k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    _need(y, "y", torch.float32, (B, T, C), dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    for name, st3 in (("state_in", state_in), ("state_out", state_out)):
        if st3 is not None:
            for t, n in zip(st3, "abp"):
                _need(t, f"{name}.{n}", torch.float32, (B, C), dev)
    sin = state_in if state_in is not None else (None, None, None)
    sout = state_out if state_out is not None else (None, None, None)
    st = L.lib().wkv_forward_state_noalloc(B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(y),
                                           *[_p(t) for t in sin], *[_p(t) for t in sout], _p(ckpt), _stream(dev))
    L.check("wkv_forward_state_noalloc", st)
    return y


def wkv_forward_gated(w, u, k, v, r, *, out=None, ckpt=None, workspace=None, bind=False):
    """out = sigmoid(r) * wkv(w, u, k, v), [B,T,C] float32; r has the dtype of k."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    for t, n in ((v, "v"), (r, "r")):
        _need(t, n, k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, C), dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    ws, ws_n = _workspace(L.WKV_OP_FORWARD, B, T, C, k.dtype, dev, workspace)
    args = (B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(r), _p(out), _p(ckpt), _p(ws), ws_n,
            _stream(dev))
    return _launch(bind, "wkv_forward_gated", L.lib().wkv_forward_gated, args, out, locals())


def wkv_backward_gated(w, u, k, v, r, gout, *, ckpt=None, out=None, workspace=None, bind=False):
    """(dk, dv, dr, dw, du) for L = sum(gout * sigmoid(r) * wkv).  r, gout have the dtype of k."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    for t, n in ((v, "v"), (r, "r"), (gout, "gout")):
        _need(t, n, k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if out is None:
        out = tuple(torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(3)) + \
            tuple(torch.empty((C,), dtype=torch.float32, device=dev) for _ in range(2))
    dk, dv, dr, dw, du = out
    for t, n, s_ in ((dk, "dk", (B, T, C)), (dv, "dv", (B, T, C)), (dr, "dr", (B, T, C)), (dw, "dw", (C,)),
                     (du, "du", (C,))):
        _need(t, n, torch.float32, s_, dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    ws, ws_n = _workspace(L.WKV_OP_BACKWARD, B, T, C, k.dtype, dev, workspace)
    args = (B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(r), _p(gout), _p(dk), _p(dv), _p(dr), _p(dw),
            _p(du), _p(ckpt), _p(ws), ws_n, _stream(dev))
    return _launch(bind, "wkv_backward_gated", L.lib().wkv_backward_gated, args, (dk, dv, dr, dw, du), locals())


def wkv_backward(w, u, k, v, gy, *, ckpt=None, out=None, workspace=None, bind=False):
    """(dk, dv, dw, du) for L = sum(gy * y).  gy has the dtype of k."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    _need(v, "v", k.dtype, (B, T, C), dev)
    _need(gy, "gy", k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    if out is None:
        dk = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        dv = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        dw = torch.empty((C,), dtype=torch.float32, device=dev)
        du = torch.empty((C,), dtype=torch.float32, device=dev)
    else:
        dk, dv, dw, du = out
    for t, n, s in ((dk, "dk", (B, T, C)), (dv, "dv", (B, T, C)), (dw, "dw", (C,)), (du, "du", (C,))):
        _need(t, n, torch.float32, s, dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    ws, ws_n = _workspace(L.WKV_OP_BACKWARD, B, T, C, k.dtype, dev, workspace)
    args = (B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(gy), _p(dk), _p(dv), _p(dw), _p(du), _p(ckpt),
            _p(ws), ws_n, _stream(dev))
    return _launch(bind, "wkv_backward", L.lib().wkv_backward, args, (dk, dv, dw, du), locals())


def wkv_backward_state(w, u, k, v, gy, *, state_in=None, grad_state_out=None, need_state_grad=True, ckpt=None,
                       out=None, workspace=None):
    """Gradients through a segment run by wkv_forward from state_in = (a, b, p)
    (or the empty history) for L = sum(gy * y) + the loss carried by the state it
    handed on.  grad_state_out: None or (ga, gb, p_out), the gradient of L with
    respect to that state's (a_out, b_out) and the p_out the forward wrote.
    Returns (dk, dv, dw, du, (ga_in, gb_in, gp_in)), the last None unless
    state_in is given and need_state_grad; dw includes the history's decay."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    B, T, C = k.shape
    _need(v, "v", k.dtype, (B, T, C), dev)
    _need(gy, "gy", k.dtype, (B, T, C), dev)
    _need(w, "w", torch.float32, (C,), dev)
    _need(u, "u", torch.float32, (C,), dev)
    for name, st3 in (("state_in", state_in), ("grad_state_out", grad_state_out)):
        if st3 is not None:
            for t, n in zip(st3, "abp"):
                _need(t, f"{name}.{n}", torch.float32, (B, C), dev)
    if out is None:
        dk = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        dv = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        dw = torch.empty((C,), dtype=torch.float32, device=dev)
        du = torch.empty((C,), dtype=torch.float32, device=dev)
    else:
        dk, dv, dw, du = out
    for t, n, s in ((dk, "dk", (B, T, C)), (dv, "dv", (B, T, C)), (dw, "dw", (C,)), (du, "du", (C,))):
        _need(t, n, torch.float32, s, dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.float32, (ckpt_bytes(B, T, C) // 4,), dev)
    gin = None
    if state_in is not None and need_state_grad:
        gin = tuple(torch.empty((B, C), dtype=torch.float32, device=dev) for _ in range(3))
    sin = state_in if state_in is not None else (None, None, None)
    sout = grad_state_out if grad_state_out is not None else (None, None, None)
    gi = gin if gin is not None else (None, None, None)
    ws, ws_n = _workspace(L.WKV_OP_BACKWARD, B, T, C, k.dtype, dev, workspace)
    st = L.lib().wkv_backward_state(B, T, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(gy),
                                    *[_p(t) for t in sin], *[_p(t) for t in sout], _p(dk), _p(dv), _p(dw),
                                    _p(du), *[_p(t) for t in gi], _p(ckpt), _p(ws), ws_n, _stream(dev))
    L.check("wkv_backward_state", st)
    return dk, dv, dw, du, gin


def wkv_step(w, u, k, v, a, b, p, *, y=None, bind=False):
    """One decode token for [L,B,C] states (a, b, p updated in place); returns y."""
    _need(k, "k", (torch.float32, torch.bfloat16))
    dev = k.device
    Ln, B, C = k.shape
    _need(v, "v", k.dtype, (Ln, B, C), dev)
    _need(w, "w", torch.float32, (Ln, C), dev)
    _need(u, "u", torch.float32, (Ln, C), dev)
    for t, n in ((a, "a"), (b, "b"), (p, "p")):
        _need(t, n, torch.float32, (Ln, B, C), dev)
    if y is None:
        y = torch.empty((Ln, B, C), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, (Ln, B, C), dev)
    args = (Ln, B, C, _DT[k.dtype], _p(w), _p(u), _p(k), _p(v), _p(y), _p(a), _p(b), _p(p), _stream(dev))
    return _launch(bind, "wkv_step", L.lib().wkv_step, args, y, locals())


def empty_state(Ln: int, B: int, C: int, device):
    """The empty decode state: a = b = 0, p = -1e38."""
    a = torch.zeros((Ln, B, C), dtype=torch.float32, device=device)
    b = torch.zeros((Ln, B, C), dtype=torch.float32, device=device)
    p = torch.full((Ln, B, C), -1e38, dtype=torch.float32, device=device)
    return a, b, p


class WKVFunction(torch.autograd.Function):
    """Autograd wrapper: saves w, u, k, v and the forward's block-start states;
    the backward recomputes everything else on chip."""

    @staticmethod
    def forward(ctx, w, u, k, v):
        B, T, C = k.shape
        ckpt = new_ckpt(B, T, C, k.device)
        y = wkv_forward(w, u, k, v, ckpt=ckpt)
        ctx.save_for_backward(w, u, k, v, ckpt)
        return y

    @staticmethod
    def backward(ctx, gy):
        w, u, k, v, ckpt = ctx.saved_tensors
        gy = gy.to(k.dtype).contiguous()
        dk, dv, dw, du = wkv_backward(w, u, k, v, gy, ckpt=ckpt)
        return dw, du, dk.to(k.dtype), dv.to(v.dtype)


def wkv(w, u, k, v):
    """Differentiable WKV forward (see WKVFunction)."""
    return WKVFunction.apply(w, u, k, v)


class WKVStateFunction(torch.autograd.Function):
    """Autograd wrapper of a segment with carried state: (y, a_out, b_out,
    p_out) from (w, u, k, v, a, b, p), for training over a long input split into
    segments.  The gradient flows through the handed-on state's (a_out, b_out);
    p_out is marked non-differentiable (its gradient is a_out ga + b_out gb for
    any loss that depends on the state only through the sums it stands for)."""

    @staticmethod
    def forward(ctx, w, u, k, v, a, b, p):
        B, T, C = k.shape
        ckpt = new_ckpt(B, T, C, k.device)
        y, (a2, b2, p2) = wkv_forward(w, u, k, v, ckpt=ckpt, state_in=(a, b, p), return_state=True)
        ctx.save_for_backward(w, u, k, v, a, b, p, p2, ckpt)
        ctx.mark_non_differentiable(p2)
        return y, a2, b2, p2

    @staticmethod
    def backward(ctx, gy, ga, gb, _gp):
        w, u, k, v, a, b, p, p2, ckpt = ctx.saved_tensors
        gy = (torch.zeros_like(k) if gy is None else gy.to(k.dtype)).contiguous()
        ga = torch.zeros_like(a) if ga is None else ga.contiguous()
        gb = torch.zeros_like(b) if gb is None else gb.contiguous()
        dk, dv, dw, du, (ga_in, gb_in, gp_in) = wkv_backward_state(
            w, u, k, v, gy, state_in=(a, b, p), grad_state_out=(ga, gb, p2), ckpt=ckpt)
        return dw, du, dk.to(k.dtype), dv.to(v.dtype), ga_in, gb_in, gp_in


def wkv_with_state(w, u, k, v, a, b, p):
    """Differentiable WKV forward from a given state (a, b, p) [B, C]; returns
    (y, a_out, b_out, p_out) (see WKVStateFunction)."""
    return WKVStateFunction.apply(w, u, k, v, a, b, p)


def token_shift(mu, x, *, x_prev=None, out=None, bind=False):
    """The M token-shift mixes of x: out[j] = mu[j] * x_t + (1 - mu[j]) * x_{t-1}.

    mu [M, C] float32 (1 <= M <= 4); x [B, T, C] float32 or bfloat16; x_prev
    [B, C] of x's dtype (the previous segment's last input) or None (zeros).
    Returns out [M, B, T, C] in x's dtype.
    """
    _need(x, "x", (torch.float32, torch.bfloat16))
    dev = x.device
    B, T, C = x.shape
    _need(mu, "mu", torch.float32, None, dev)
    if mu.dim() != 2 or mu.shape[1] != C:
        raise ValueError(f"mu has shape {tuple(mu.shape)}, expected (M, {C})")
    M = mu.shape[0]
    if x_prev is not None:
        _need(x_prev, "x_prev", x.dtype, (B, C), dev)
    if out is None:
        out = torch.empty((M, B, T, C), dtype=x.dtype, device=dev)
    _need(out, "out", x.dtype, (M, B, T, C), dev)
    args = (B, T, C, M, _DT[x.dtype], _p(mu), _p(x), _p(x_prev), _p(out), _stream(dev))
    return _launch(bind, "wkv_token_shift", L.lib().wkv_token_shift, args, out, locals())


def token_shift_backward(mu, x, gout, *, x_prev=None, want_dx_prev=False, out=None, workspace=None, bind=False):
    """(dx [B,T,C], dmu [M,C], dx_prev [B,C] or None), float32, for L = sum(gout * token_shift(mu, x, x_prev)).

    gout [M, B, T, C] has x's dtype.  dx_prev is computed when want_dx_prev
    (or when ``out`` holds a third tensor).
    """
    _need(x, "x", (torch.float32, torch.bfloat16))
    dev = x.device
    B, T, C = x.shape
    _need(mu, "mu", torch.float32, None, dev)
    if mu.dim() != 2 or mu.shape[1] != C:
        raise ValueError(f"mu has shape {tuple(mu.shape)}, expected (M, {C})")
    M = mu.shape[0]
    _need(gout, "gout", x.dtype, (M, B, T, C), dev)
    if x_prev is not None:
        _need(x_prev, "x_prev", x.dtype, (B, C), dev)
    if out is None:
        out = (torch.empty((B, T, C), dtype=torch.float32, device=dev),
               torch.empty((M, C), dtype=torch.float32, device=dev),
               torch.empty((B, C), dtype=torch.float32, device=dev) if want_dx_prev else None)
    dx, dmu, dxp = out
    _need(dx, "dx", torch.float32, (B, T, C), dev)
    _need(dmu, "dmu", torch.float32, (M, C), dev)
    if dxp is not None:
        _need(dxp, "dx_prev", torch.float32, (B, C), dev)
    nbytes = int(L.lib().wkv_token_shift_workspace_bytes(B, T, C, M))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    args = (B, T, C, M, _DT[x.dtype], _p(mu), _p(x), _p(x_prev), _p(gout), _p(dx), _p(dmu), _p(dxp),
            _p(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    return _launch(bind, "wkv_token_shift_backward", L.lib().wkv_token_shift_backward, args, (dx, dmu, dxp), locals())


class TokenShiftFunction(torch.autograd.Function):
    """Autograd wrapper of token_shift: saves mu, x (and x_prev)."""

    @staticmethod
    def forward(ctx, mu, x, x_prev):
        out = token_shift(mu, x, x_prev=x_prev)
        ctx.save_for_backward(mu, x, x_prev)
        return out

    @staticmethod
    def backward(ctx, gout):
        mu, x, x_prev = ctx.saved_tensors
        gout = gout.to(x.dtype).contiguous()
        dx, dmu, dxp = token_shift_backward(mu, x, gout, x_prev=x_prev, want_dx_prev=x_prev is not None)
        return dmu, dx.to(x.dtype), None if dxp is None else dxp.to(x.dtype)


def token_shift_mix(mu, x, x_prev=None):
    """Differentiable token_shift (see TokenShiftFunction)."""
    return TokenShiftFunction.apply(mu, x, x_prev)


def wkv5_ckpt_bytes(B: int, T: int, H: int) -> int:
    return int(L.lib().wkv5_ckpt_bytes(B, T, H, 64))


def new_wkv5_ckpt(B: int, T: int, H: int, device) -> torch.Tensor:
    """Buffer for wkv5_forward's chunk-start states (opaque bytes)."""
    return torch.empty(max(wkv5_ckpt_bytes(B, T, H), 1), dtype=torch.uint8, device=device)


def wkv5_forward(w, u, r, k, v, *, state_in=None, state_out=None, return_state=False, out=None, ckpt=None, workspace=None, split=True, bind=False):
    """RWKV-5 matrix-state WKV: o [B, T, C] float32 from w, u [H, 64] float32 and
    r, k, v [B, T, C] bfloat16 (C = 64 H).  state_in: [B, H, 64, 64] float32 or
    None (zero).  state_out: tensor to receive the final state (may be
    state_in); with return_state and no state_out one is allocated and the
    call returns (o, state).  ckpt: None or a new_wkv5_ckpt() buffer that
    receives the chunk-start states for wkv5_backward.  With few (batch row, head) pairs
    the call splits each sequence into segments run in parallel, in a workspace it allocates
    (or is given); split=False keeps the whole sequence in one workgroup per pair."""
    _need(r, "r", torch.bfloat16)
    dev = r.device
    B, T, C = r.shape
    H = w.shape[0] if w.dim() == 2 else C // 64
    if C != 64 * H:
        raise ValueError(f"C = {C} is not 64 * H with H = {H}")
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, (B, T, C), dev)
    _need(w, "w", torch.float32, (H, 64), dev)
    _need(u, "u", torch.float32, (H, 64), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, C), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, 64, 64), dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, 64, 64), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (B, H, 64, 64), dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.uint8, None, dev)
        if ckpt.numel() < wkv5_ckpt_bytes(B, T, H):
            raise ValueError(f"ckpt has {ckpt.numel()} bytes, needs {wkv5_ckpt_bytes(B, T, H)}")
    nws = int(L.lib().wkv5_forward_workspace_bytes(B, T, H, 64)) if split else 0
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    args = (B, T, H, 64, L.WKV_BF16, _p(w), _p(u), _p(r), _p(k), _p(v), _p(out), _p(state_in), _p(state_out),
            _p(ckpt), _p(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(dev))
    return _launch(bind, "wkv5_forward", L.lib().wkv5_forward, args, (out, state_out) if return_state else out, locals())


def wkv5_backward(w, u, r, k, v, go, *, state_in=None, grad_state_out=None, need_state_grad=False, ckpt=None,
                  workspace=None, split=True, bind=False):
    """Gradients of sum <go, o> + <grad_state_out, S_T> for
    (o, S_T) = wkv5_forward(w, u, r, k, v, state_in=state_in, return_state=True):
    returns (dr, dk, dv [B, T, C] float32, dw, du [H, 64] float32 summed over
    the batch, ds_in [B, H, 64, 64] float32 or None).  go: [B, T, C] bfloat16.
    split: with few (batch row, head) pairs, run the sequence's segments in
    parallel (the adjoint state chained between them); False keeps one
    workgroup per pair walking the whole sequence."""
    _need(r, "r", torch.bfloat16)
    dev = r.device
    B, T, C = r.shape
    H = w.shape[0] if w.dim() == 2 else C // 64
    if C != 64 * H:
        raise ValueError(f"C = {C} is not 64 * H with H = {H}")
    for t, n in ((k, "k"), (v, "v"), (go, "go")):
        _need(t, n, torch.bfloat16, (B, T, C), dev)
    _need(w, "w", torch.float32, (H, 64), dev)
    _need(u, "u", torch.float32, (H, 64), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, 64, 64), dev)
    if grad_state_out is not None:
        _need(grad_state_out, "grad_state_out", torch.float32, (B, H, 64, 64), dev)
    dr, dk, dv = (torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(3))
    dw = torch.empty((H, 64), dtype=torch.float32, device=dev)
    du = torch.empty((H, 64), dtype=torch.float32, device=dev)
    ds = torch.empty((B, H, 64, 64), dtype=torch.float32, device=dev) if need_state_grad else None
    lib = L.lib()
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.uint8, None, dev)
        if ckpt.numel() < wkv5_ckpt_bytes(B, T, H):
            raise ValueError(f"ckpt has {ckpt.numel()} bytes, needs {wkv5_ckpt_bytes(B, T, H)}")
    flags = (1 if ckpt is not None else 0) | (0 if split else 2)  # WKV_WS_HAVE_CKPT, WKV_WS_NO_SPLIT
    nbytes = int(lib.wkv5_backward_workspace_bytes(B, T, H, 64, flags))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    # without split the call is told only the unsplit size, so it never splits
    wsz = workspace.numel() * workspace.element_size() if split else nbytes
    args = (B, T, H, 64, L.WKV_BF16, _p(w), _p(u), _p(r), _p(k), _p(v), _p(go), _p(state_in),
            _p(grad_state_out), _p(dr), _p(dk), _p(dv), _p(dw), _p(du), _p(ds), _p(ckpt), _p(workspace), wsz,
            _stream(dev))
    return _launch(bind, "wkv5_backward", lib.wkv5_backward, args, (dr, dk, dv, dw, du, ds), locals())


class Wkv5Function(torch.autograd.Function):
    """Autograd wrapper: o = wkv5_forward(...); backward through wkv5_backward
    (go rounded to bfloat16 for the matrix-core products)."""

    @staticmethod
    def forward(ctx, w, u, r, k, v, state_in=None):
        B, T, C = r.shape
        ckpt = new_wkv5_ckpt(B, T, C // 64, r.device)
        o = wkv5_forward(w, u, r, k, v, state_in=state_in, ckpt=ckpt)
        ctx.save_for_backward(w, u, r, k, v, state_in, ckpt)
        return o

    @staticmethod
    def backward(ctx, go):
        w, u, r, k, v, state_in, ckpt = ctx.saved_tensors
        dr, dk, dv, dw, du, ds = wkv5_backward(w, u, r, k, v, go.to(torch.bfloat16).contiguous(), state_in=state_in,
                                               need_state_grad=state_in is not None and ctx.needs_input_grad[5],
                                               ckpt=ckpt)
        return dw, du, dr.to(r.dtype), dk.to(k.dtype), dv.to(v.dtype), ds


def wkv6_forward(w, u, r, k, v, *, state_in=None, state_out=None, return_state=False, out=None, ckpt=None, workspace=None, split=True, bind=False):
    """RWKV-6 matrix-state WKV with per-token decay: o [B, T, C] float32 from
    w [B, T, C] float32 rates (>= 0), u [H, 64] float32 and r, k, v [B, T, C]
    bfloat16 (C = 64 H); state handling, ckpt, workspace and split as wkv5_forward."""
    _need(r, "r", torch.bfloat16)
    dev = r.device
    B, T, C = r.shape
    H = u.shape[0]
    if C != 64 * H:
        raise ValueError(f"C = {C} is not 64 * H with H = {H}")
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, (B, T, C), dev)
    _need(w, "w", torch.float32, (B, T, C), dev)
    _need(u, "u", torch.float32, (H, 64), dev)
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, C), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, 64, 64), dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, 64, 64), dtype=torch.float32, device=dev)
    if state_out is not None:
        _need(state_out, "state_out", torch.float32, (B, H, 64, 64), dev)
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.uint8, None, dev)
        if ckpt.numel() < wkv5_ckpt_bytes(B, T, H):
            raise ValueError(f"ckpt has {ckpt.numel()} bytes, needs {wkv5_ckpt_bytes(B, T, H)}")
    nws = int(L.lib().wkv6_forward_workspace_bytes(B, T, H, 64)) if split else 0
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    args = (B, T, H, 64, L.WKV_BF16, _p(w), _p(u), _p(r), _p(k), _p(v), _p(out), _p(state_in), _p(state_out),
            _p(ckpt), _p(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(dev))
    return _launch(bind, "wkv6_forward", L.lib().wkv6_forward, args, (out, state_out) if return_state else out, locals())


def wkv6_backward(w, u, r, k, v, go, *, state_in=None, grad_state_out=None, need_state_grad=False, ckpt=None,
                  workspace=None, split=True, bind=False):
    """Gradients of sum <go, o> + <grad_state_out, S_T> for
    (o, S_T) = wkv6_forward(w, u, r, k, v, state_in=state_in, return_state=True):
    returns (dr, dk, dv, dw [B, T, C] float32 (dw per token), du [H, 64]
    float32 summed over the batch, ds_in [B, H, 64, 64] float32 or None).
    go: [B, T, C] bfloat16; ckpt: None or what wkv6_forward wrote."""
    _need(r, "r", torch.bfloat16)
    dev = r.device
    B, T, C = r.shape
    H = u.shape[0]
    if C != 64 * H:
        raise ValueError(f"C = {C} is not 64 * H with H = {H}")
    for t, n in ((k, "k"), (v, "v"), (go, "go")):
        _need(t, n, torch.bfloat16, (B, T, C), dev)
    _need(w, "w", torch.float32, (B, T, C), dev)
    _need(u, "u", torch.float32, (H, 64), dev)
    if state_in is not None:
        _need(state_in, "state_in", torch.float32, (B, H, 64, 64), dev)
    if grad_state_out is not None:
        _need(grad_state_out, "grad_state_out", torch.float32, (B, H, 64, 64), dev)
    dr, dk, dv, dw = (torch.empty((B, T, C), dtype=torch.float32, device=dev) for _ in range(4))
    du = torch.empty((H, 64), dtype=torch.float32, device=dev)
    ds = torch.empty((B, H, 64, 64), dtype=torch.float32, device=dev) if need_state_grad else None
    lib = L.lib()
    if ckpt is not None:
        _need(ckpt, "ckpt", torch.uint8, None, dev)
        if ckpt.numel() < wkv5_ckpt_bytes(B, T, H):
            raise ValueError(f"ckpt has {ckpt.numel()} bytes, needs {wkv5_ckpt_bytes(B, T, H)}")
    flags = (1 if ckpt is not None else 0) | (0 if split else 2)  # WKV_WS_HAVE_CKPT, WKV_WS_NO_SPLIT
    nbytes = int(lib.wkv6_backward_workspace_bytes(B, T, H, 64, flags))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    # without split the call is told only the unsplit size, so it never splits
    wsz = workspace.numel() * workspace.element_size() if split else nbytes
    args = (B, T, H, 64, L.WKV_BF16, _p(w), _p(u), _p(r), _p(k), _p(v), _p(go), _p(state_in),
            _p(grad_state_out), _p(dr), _p(dk), _p(dv), _p(dw), _p(du), _p(ds), _p(ckpt), _p(workspace), wsz,
            _stream(dev))
    return _launch(bind, "wkv6_backward", lib.wkv6_backward, args, (dr, dk, dv, dw, du, ds), locals())


class Wkv6Function(torch.autograd.Function):
    """Autograd wrapper: o = wkv6_forward(...); backward through wkv6_backward
    (go rounded to bfloat16 for the matrix-core products)."""

    @staticmethod
    def forward(ctx, w, u, r, k, v, state_in=None):
        B, T, C = r.shape
        ckpt = new_wkv5_ckpt(B, T, C // 64, r.device)
        o = wkv6_forward(w, u, r, k, v, state_in=state_in, ckpt=ckpt)
        ctx.save_for_backward(w, u, r, k, v, state_in, ckpt)
        return o

    @staticmethod
    def backward(ctx, go):
        w, u, r, k, v, state_in, ckpt = ctx.saved_tensors
        dr, dk, dv, dw, du, ds = wkv6_backward(w, u, r, k, v, go.to(torch.bfloat16).contiguous(), state_in=state_in,
                                               need_state_grad=state_in is not None and ctx.needs_input_grad[5],
                                               ckpt=ckpt)
        return dw, du, dr.to(r.dtype), dk.to(k.dtype), dv.to(v.dtype), ds
