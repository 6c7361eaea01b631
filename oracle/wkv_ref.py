"""Float64 CPU oracle for the RWKV-4 WKV time-mixing operator.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``rwkv_wkv_mixing_amd`` and its HIP library) imports, links or calls this
module.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code, tables or constants with
the HIP path.

Every function is plain float64 numpy: loops over time, vectorised only over
the independent (batch, channel) lanes, with no blocking, fusion or reordering
beyond what the formula states.

Sources (page title, then section):

* [P4] "RWKV（Receptance Weighted Key Value）概念" (compassingai.com concept
  page), section 3.2 "时间混合（Time-mixing）与 WKV 算子": the weighted-sum
  definition of wkv_t over the history i < t with decay e^{-(t-1-i)w} and the
  current-token bonus e^{u+k_t}; section 3.4: time-parallel training versus
  constant-state recurrent inference.
* [P5] "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型" (paper notes on
  arXiv 2305.13048), section "一句话总结" and "关键设计 2：WKV 算子": the
  numerator/denominator recurrences a_t, b_t and the output formula that reads
  the state *before* token t; "关键设计 4：双执行模式": the decode step (output
  first from the undecayed state, then decay-and-add) and the remark that real
  implementations carry a stability exponent p.
* [P3] "RWKV模型深度研究报告", section 4.4.2: a long input is encoded segment by
  segment, the state carrying the history from one segment into the next.

Readings where the pages are silent:

* initial state is empty: the history sum over i = 1..t-1 is empty at t = 1;
* the stability-exponent update rule (not given on the pages) is the running
  max p' = max(p - w, k); it only changes the representation (a, b, p) of the
  same (A, B) = (a e^p, b e^p);
* the backward formulas are derived here by differentiating the [P4] sum; the
  pages give none.  Pinned by finite differences and by autograd of the
  direct definition, see tests/test_oracle_pins.py.
* a segment's backward through carried state (wkv_backward_state_ref) is the
  derivative of its outputs and of the state it hands on: the loss is
  sum(gy y) + sum(gA A_T) + sum(gB B_T), with (gA, gB) the gradient a later
  segment returns for the plain sums it started from.  Gradients of the
  stable representation (a, b, p) follow by the chain rule through
  A = a e^p, B = b e^p (wkv_state_grads_from_sums, wkv_sums_grads_from_state).

Parity status: every function here is pinned (no "parity unpinned" entries).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit, softmax

__all__ = [
    "wkv_forward_ref",
    "wkv_direct_ref",
    "wkv_backward_ref",
    "wkv_backward_state_ref",
    "wkv_state_grads_from_sums",
    "wkv_sums_grads_from_state",
    "wkv_step_ref",
    "wkv_state_from_sums",
]


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def wkv_forward_ref(w, u, k, v, return_sums: bool = False, A0=None, B0=None):
    """Recurrent WKV forward in float64.

    [P5] "一句话总结" / "关键设计 2": with d = e^{-w},
        y_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}),
        A_t = d A_{t-1} + e^{k_t} v_t,   B_t = d B_{t-1} + e^{k_t},
    and A_0 = B_0 = 0 (the empty history of the [P4] 3.2 sum), or the plain
    sums A0, B0 [B, C] of an earlier segment when given ([P3] 4.4.2: a long
    input is encoded segment by segment, the state carrying the history from
    one segment into the next).

    w, u: [C]; k, v: [B, T, C].  Returns y [B, T, C] (and the final plain sums
    A_T, B_T, each [B, C], when ``return_sums``).  The sums are kept unscaled:
    float64 holds e^{|k|+|u|} for every workload used here, and the function
    asserts that everything stayed finite.
    """
    w, u, k, v = _f64(w, u, k, v)
    Bsz, T, C = k.shape
    d = np.exp(-w)
    eu = np.exp(u)
    A = np.zeros((Bsz, C)) if A0 is None else np.array(A0, dtype=np.float64).reshape(Bsz, C)
    Bs = np.zeros((Bsz, C)) if B0 is None else np.array(B0, dtype=np.float64).reshape(Bsz, C)
    y = np.empty((Bsz, T, C))
    for t in range(T):
        ek = np.exp(k[:, t, :])
        cur = eu * ek
        y[:, t, :] = (A + cur * v[:, t, :]) / (Bs + cur)
        A = d * A + ek * v[:, t, :]
        Bs = d * Bs + ek
    assert np.isfinite(y).all(), "oracle forward left float64 range"
    if return_sums:
        return y, A, Bs
    return y


def wkv_gated_forward_ref(w, u, k, v, r):
    """Time-mixing output with the receptance gate, [P4] section 3.2:
    out_t = sigmoid(r_t) * wkv_t, elementwise per (b, t, c); r [B, T, C].
    sigmoid is scipy's ``expit``."""
    return expit(np.asarray(r, np.float64)) * wkv_forward_ref(w, u, k, v)


def wkv_gated_backward_ref(w, u, k, v, r, gout):
    """Gradients of L = sum(gout * out) through the gate: the WKV gradients of
    wkv_backward_ref for gy = gout sigmoid(r), and dr = gout y sigmoid(r)
    sigmoid(-r).  Returns (dk, dv, dr, dw, du)."""
    r, gout = _f64(r, gout)
    y = wkv_forward_ref(w, u, k, v)
    dk, dv, dw, du = wkv_backward_ref(w, u, k, v, gout * expit(r))
    dr = gout * y * expit(r) * expit(-r)
    return dk, dv, dr, dw, du


def wkv_direct_ref(w, u, k, v):
    """O(T^2) evaluation of the [P4] section 3.2 weighted sum, read literally.

    For each output t (1-based) the weights over i = 1..t are a softmax of the
    logits  k_i - (t-1-i) w  (i < t)  and  u + k_t  (i = t), applied to v.  The
    softmax is scipy's, so this shares no recurrence with wkv_forward_ref.
    """
    w, u, k, v = _f64(w, u, k, v)
    Bsz, T, C = k.shape
    y = np.empty((Bsz, T, C))
    for t in range(T):  # 0-based t here; token index t+1 on the page
        i = np.arange(t + 1)
        age = (t - 1 - i).astype(np.float64)  # (t+1)-1-(i+1) in 1-based terms
        logits = k[:, : t + 1, :] - age[None, :, None] * w[None, None, :]
        logits[:, t, :] = u[None, :] + k[:, t, :]
        p = softmax(logits, axis=1)
        y[:, t, :] = np.sum(p * v[:, : t + 1, :], axis=1)
    return y


def wkv_backward_ref(w, u, k, v, gy):
    """Gradients of L = sum(gy * y) with respect to k, v, w, u, in float64.

    Derived by differentiating the [P4] 3.2 sum (the pages print no backward).
    With D_t = B_{t-1} + e^{u+k_t}, pi_t = e^{u+k_t}/D_t and d = e^{-w}:

        G_t  = sum_{s>t} gy_s d^{s-1-t} / D_s         G_{t-1}  = d G_t + gy_t / D_t
        H_t  = sum_{s>t} gy_s y_s d^{s-1-t} / D_s     H_{t-1}  = d H_t + gy_t y_t / D_t
        G'_t = sum_{s>t} (s-1-t) gy_s d^{s-1-t}/D_s   G'_{t-1} = d (G'_t + G_t)
        H'_t likewise with y_s                         H'_{t-1} = d (H'_t + H_t)

        dv_t = gy_t pi_t + e^{k_t} G_t
        dk_t = gy_t pi_t (v_t - y_t) + e^{k_t} (v_t G_t - H_t)
        du   = sum_{b,t} gy_t pi_t (v_t - y_t)
        dw   = -sum_{b,t} e^{k_t} (v_t G'_t - H'_t)

    w is the decay *rate* (decay factor e^{-w}); dw is dL/dw for that argument.
    Returns dk, dv [B, T, C] and dw, du [C].
    """
    w, u, k, v, gy = _f64(w, u, k, v, gy)
    Bsz, T, C = k.shape
    d = np.exp(-w)
    eu = np.exp(u)
    # forward sweep, keeping y_t and D_t
    A = np.zeros((Bsz, C))
    Bs = np.zeros((Bsz, C))
    y = np.empty((Bsz, T, C))
    D = np.empty((Bsz, T, C))
    for t in range(T):
        ek = np.exp(k[:, t, :])
        cur = eu * ek
        D[:, t, :] = Bs + cur
        y[:, t, :] = (A + cur * v[:, t, :]) / D[:, t, :]
        A = d * A + ek * v[:, t, :]
        Bs = d * Bs + ek
    # reverse sweep
    G = np.zeros((Bsz, C))
    H = np.zeros((Bsz, C))
    Gp = np.zeros((Bsz, C))
    Hp = np.zeros((Bsz, C))
    dk = np.empty((Bsz, T, C))
    dv = np.empty((Bsz, T, C))
    du = np.zeros(C)
    dw = np.zeros(C)
    for t in range(T - 1, -1, -1):
        ek = np.exp(k[:, t, :])
        pi = eu * ek / D[:, t, :]
        gt, vt, yt = gy[:, t, :], v[:, t, :], y[:, t, :]
        cur_k = gt * pi * (vt - yt)
        dv[:, t, :] = gt * pi + ek * G
        dk[:, t, :] = cur_k + ek * (vt * G - H)
        du += cur_k.sum(axis=0)
        dw -= (ek * (vt * Gp - Hp)).sum(axis=0)
        # step the accumulators from "after t" to "after t-1"
        Gp = d * (Gp + G)
        Hp = d * (Hp + H)
        G = d * G + gt / D[:, t, :]
        H = d * H + gt * yt / D[:, t, :]
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    return dk, dv, dw, du


def wkv_backward_state_ref(w, u, k, v, gy, A0=None, B0=None, gA=None, gB=None):
    """Gradients through a segment that starts from a given history and hands
    its state on ([P3] 4.4.2), in float64:

        L = sum(gy * y) + sum(gA * A_T) + sum(gB * B_T),

    with y and the final plain sums (A_T, B_T) those of wkv_forward_ref from the
    initial sums (A0, B0) (zeros when None), and (gA, gB) the gradient of the
    loss with respect to (A_T, B_T) (zeros when None).

    Reverse mode written out on the [P5] recurrence, one token at a time, with
    d = e^{-w}, D_t = B_{t-1} + e^{u+k_t} and the adjoints (ga, gb) of the state
    after each token, starting from (gA, gB) after the last:
      the state update A_t = d A_{t-1} + e^{k_t} v_t, B_t = d B_{t-1} + e^{k_t}
        gives v_t the part ga e^{k_t}, k_t the part e^{k_t} (ga v_t + gb),
        w the part -d (ga A_{t-1} + gb B_{t-1}), and passes (d ga, d gb) back;
      the output y_t = (A_{t-1} + e^{u+k_t} v_t) / D_t
        gives v_t the part gy_t e^{u+k_t} / D_t, k_t and u the part
        gy_t e^{u+k_t} (v_t - y_t) / D_t, and adds gy_t / D_t and
        -gy_t y_t / D_t to the adjoints of A_{t-1} and B_{t-1}.
    Returns dk, dv [B, T, C], dw, du [C] and dA0, dB0 [B, C] (the adjoints of
    the initial sums).
    """
    w, u, k, v, gy = _f64(w, u, k, v, gy)
    Bsz, T, C = k.shape
    d = np.exp(-w)
    eu = np.exp(u)
    A = np.zeros((Bsz, C)) if A0 is None else np.array(A0, dtype=np.float64).reshape(Bsz, C)
    Bs = np.zeros((Bsz, C)) if B0 is None else np.array(B0, dtype=np.float64).reshape(Bsz, C)
    A_before = np.empty((Bsz, T, C))  # the sums before each token
    B_before = np.empty((Bsz, T, C))
    y = np.empty((Bsz, T, C))
    D = np.empty((Bsz, T, C))
    for t in range(T):
        A_before[:, t, :] = A
        B_before[:, t, :] = Bs
        ek = np.exp(k[:, t, :])
        cur = eu * ek
        D[:, t, :] = Bs + cur
        y[:, t, :] = (A + cur * v[:, t, :]) / D[:, t, :]
        A = d * A + ek * v[:, t, :]
        Bs = d * Bs + ek
    ga = np.zeros((Bsz, C)) if gA is None else np.array(gA, dtype=np.float64).reshape(Bsz, C)
    gb = np.zeros((Bsz, C)) if gB is None else np.array(gB, dtype=np.float64).reshape(Bsz, C)
    dk = np.zeros((Bsz, T, C))
    dv = np.zeros((Bsz, T, C))
    dw = np.zeros(C)
    du = np.zeros(C)
    for t in range(T - 1, -1, -1):
        ek = np.exp(k[:, t, :])
        cur = eu * ek
        vt, yt, gt, Dt = v[:, t, :], y[:, t, :], gy[:, t, :], D[:, t, :]
        # the state update of token t
        dv[:, t, :] += ga * ek
        dk[:, t, :] += ek * (ga * vt + gb)
        dw -= (d * (ga * A_before[:, t, :] + gb * B_before[:, t, :])).sum(axis=0)
        ga_prev = d * ga
        gb_prev = d * gb
        # the output of token t
        dv[:, t, :] += gt * cur / Dt
        dky = gt * cur * (vt - yt) / Dt
        dk[:, t, :] += dky
        du += dky.sum(axis=0)
        ga = ga_prev + gt / Dt
        gb = gb_prev - gt * yt / Dt
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    return dk, dv, dw, du, ga, gb


def wkv_state_grads_from_sums(a, b, p, dA, dB):
    """Gradient of the loss with respect to a stable state (a, b, p), from its
    gradient (dA, dB) with respect to the plain sums it stands for,
    A = a e^p, B = b e^p: ga = e^p dA, gb = e^p dB, gp = a ga + b gb.  An empty
    state (b <= 0, the empty history whatever a and p hold) is a constant: all
    three are zero."""
    a, b, p, dA, dB = _f64(a, b, p, dA, dB)
    live = b > 0
    f = np.where(live, np.exp(np.where(live, p, 0.0)), 0.0)
    ga = f * dA
    gb = f * dB
    return ga, gb, a * ga + b * gb


def wkv_sums_grads_from_state(ga, gb, p):
    """Gradient (gA, gB) with respect to the plain sums (A, B) = (a e^p, b e^p)
    from the gradient (ga, gb) with respect to (a, b) at that p:
    gA = ga e^{-p}, gB = gb e^{-p}.  (The gradient with respect to p is then
    a ga + b gb for any loss that depends on the state only through the sums,
    so it carries nothing more.)"""
    ga, gb, p = _f64(ga, gb, p)
    f = np.exp(-p)
    return ga * f, gb * f


def wkv_step_ref(w, u, k, v, a, b, p):
    """One recurrent-mode token (decode) on a stable state, in float64.

    [P5] "关键设计 4": the output is read from the *previous* state plus the
    current token with bonus u, then the state is decayed by e^{-w} and the
    current token is added.  The state is carried as (a, b, p) with
    A = a e^p, B = b e^p ([P5] lists the stability exponent p in the state
    tuple); the exponent follows the running max, so no exponential overflows:

        q  = max(p, u + k)
        y  = (e^{p-q} a + e^{u+k-q} v) / (e^{p-q} b + e^{u+k-q})
        p' = max(p - w, k)
        a' = e^{p-w-p'} a + e^{k-p'} v,   b' = e^{p-w-p'} b + e^{k-p'}

    All arguments broadcast elementwise (w, u per lane).  The empty state is
    a = b = 0 with p = -inf (or any very negative p).  Returns (y, a', b', p').
    """
    w, u, k, v, a, b, p = _f64(w, u, k, v, a, b, p)
    uk = u + k
    q = np.maximum(p, uk)
    e1 = np.exp(p - q)
    e2 = np.exp(uk - q)
    y = (e1 * a + e2 * v) / (e1 * b + e2)
    pw = p - w
    p2 = np.maximum(pw, k)
    f1 = np.exp(pw - p2)
    f2 = np.exp(k - p2)
    return y, f1 * a + f2 * v, f1 * b + f2, p2


def wkv_sums_from_state(a, b, p):
    """Plain sums of a stable state (a, b, p): A = a e^p, B = b e^p (the empty
    state, b = 0 with a very negative p, gives A = B = 0)."""
    a, b, p = _f64(a, b, p)
    f = np.exp(np.maximum(p, -745.0))
    return np.where(b > 0, a * f, 0.0), np.where(b > 0, b * f, 0.0)


def wkv_state_from_sums(A, B):
    """Stable state (a, b, p) for plain sums (A, B), B > 0: a = A/B, b = 1, p = ln B.

    One valid representation among (a e^s, b e^s, p - s) for any s.
    """
    A, B = _f64(A, B)
    return A / B, np.ones_like(B), np.log(B)
