"""Float64 CPU oracle for the multi-head, matrix-state WKV of RWKV-5.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or calls
this module; only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may.  It shares no code, tables or constants with the HIP
path.

Sources (page title, then section):

* [P2] the intelliparadigm.com post (its printed title is garbled), section
  "2.1 WKV的数学表达与实现": version 5 splits the feature channels into groups,
  each group with its own decay rate.
* [P3] "RWKV模型深度研究报告（截至2026年初）", section 1.3.2: RWKV-5/6 carry a
  matrix-valued state instead of RWKV-4's per-channel scalars, so that the
  channels keep independent time decays; section 1.3.3 writes the matrix
  state's update as the previous state times a diagonal decay plus an outer
  product of value and key (RWKV-7 adds a rank-one term, not used here);
  section 1.4.1: chunkwise-parallel training (matrix products inside a chunk,
  the state passed between chunks).
* [P4] "RWKV（Receptance Weighted Key Value）概念", section 3.2 and [P5]
  "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section "关键设计 2":
  the RWKV-4 operator this generalises, with its per-channel decay rate w
  (decay factor e^{-w}), the current token's bonus u, and the receptance that
  decides how much of the history a token receives.

Readings where the pages are silent:

* heads: C = H * N channels, head h owning channels h*N .. h*N + N - 1; the
  state of a head is an N x N matrix S (key index i, value index j);
* update: S_t = diag(e^{-w}) S_{t-1} + k_t^T v_t, w [H, N] the positive decay
  rate of each key channel (as in RWKV-4), constant over time (version 5);
* readout: o_t = r_t (S_{t-1} + diag(u) k_t^T v_t), i.e.
  o_t[j] = sum_i r_t[i] (S_{t-1}[i, j] + u[i] k_t[i] v_t[j]): the receptance
  reads the state before the token, and the current token enters with the
  bonus u, as in RWKV-4.  The matrix state holds the numerator only: the
  update on the pages has no normalising denominator;
* the initial state is zero unless given.

* the backward (derived here by differentiating the recurrence; the pages give
  none) is for L = sum_t <go_t, o_t> + <dS_T, S_T> (dS_T, the gradient of the
  final state, zero unless given): with the adjoint state
  G_{t-1} = diag(e^{-w}) G_t + r_t^T go_t (G_{T-1} = dS_T),
      dr_t = S_{t-1} go_t^T + u . k_t (v_t . go_t)
      dk_t = G_t v_t^T + u . r_t (v_t . go_t)
      dv_t = k_t G_t + (sum_i r_t,i u_i k_t,i) go_t
      du_i = sum_t r_t,i k_t,i (v_t . go_t)
      dw_i = -e^{-w_i} sum_t sum_j G_t[i, j] S_{t-1}[i, j]
      dS0  = G_{-1}
  (dw, du summed over the batch).

Parity status: every function here is pinned (tests/test_oracle_wkv5_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["wkv5_forward_ref", "wkv5_direct_ref", "wkv5_backward_ref"]


def _heads(x, H):
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    return x.reshape(B, T, H, C // H)


def wkv5_forward_ref(w, u, r, k, v, H, S0=None):
    """Token-by-token recurrence in float64.

    w, u: [H, N] (or [C]); r, k, v: [B, T, C] with C = H * N; S0: [B, H, N, N]
    or None (zero).  Returns (o [B, T, C], S_T [B, H, N, N]).
    """
    r, k, v = (_heads(x, H) for x in (r, k, v))
    B, T, _, N = r.shape
    w = np.asarray(w, dtype=np.float64).reshape(H, N)
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    d = np.exp(-w)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, dtype=np.float64).reshape(B, H, N, N)
    o = np.empty((B, T, H, N))
    for t in range(T):
        kv = k[:, t, :, :, None] * v[:, t, :, None, :]                 # k_t^T v_t, [B, H, N, N]
        o[:, t] = np.einsum("bhi,bhij->bhj", r[:, t], S + u[None, :, :, None] * kv)
        S = d[None, :, :, None] * S + kv
    assert np.isfinite(o).all() and np.isfinite(S).all()
    return o.reshape(B, T, H * N), S


def wkv5_direct_ref(w, u, r, k, v, H, S0=None):
    """The same outputs written as one sum over the history (no recurrence):

        o_t[j] = sum_i r_t[i] e^{-w_i t} S0[i, j]
               + sum_{s<t} (sum_i r_t[i] k_s[i] e^{-w_i (t-1-s)}) v_s[j]
               + (sum_i r_t[i] u_i k_t[i]) v_t[j]

    with an explicit [T, T, N] decay tensor and library matrix products.
    For small T only."""
    r, k, v = (_heads(x, H) for x in (r, k, v))
    B, T, _, N = r.shape
    w = np.asarray(w, dtype=np.float64).reshape(H, N)
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    t = np.arange(T)
    age = (t[:, None] - 1 - t[None, :]).astype(np.float64)              # t - 1 - s
    causal = age >= 0
    o = np.zeros((B, T, H, N))
    for h in range(H):
        dec = np.where(causal[:, :, None], np.exp(-w[h][None, None, :] * np.maximum(age, 0)[:, :, None]), 0.0)
        A = np.einsum("bti,tsi,bsi->bts", r[:, :, h], dec, k[:, :, h])   # [B, T, T]
        A = A + np.einsum("bti,i,bti->bt", r[:, :, h], u[h], k[:, :, h])[:, :, None] * np.eye(T)[None]
        o[:, :, h] = A @ v[:, :, h]
        if S0 is not None:
            S0h = np.asarray(S0, dtype=np.float64).reshape(B, H, N, N)[:, h]
            rd = r[:, :, h] * np.exp(-w[h][None, None, :] * t[None, :, None])
            o[:, :, h] += rd @ S0h
    return o.reshape(B, T, H * N)


def wkv5_backward_ref(w, u, r, k, v, go, H, S0=None, dST=None):
    """Gradients of L = sum_t <go_t, o_t> + <dST, S_T> for
    (o, S_T) = wkv5_forward_ref(w, u, r, k, v, H, S0), in float64: a forward
    pass keeping every S_{t-1}, then the adjoint state G (starting from dST,
    [B, H, N, N] or None for zero) walked backwards in time.

    Returns (dr, dk, dv [B, T, C], dw, du [H, N] summed over the batch, dS0
    [B, H, N, N]).
    """
    r, k, v, go = (_heads(x, H) for x in (r, k, v, go))
    B, T, _, N = r.shape
    w = np.asarray(w, dtype=np.float64).reshape(H, N)
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    d = np.exp(-w)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, dtype=np.float64).reshape(B, H, N, N)
    prev = np.empty((T, B, H, N, N))                                      # S_{t-1}
    for t in range(T):
        prev[t] = S
        S = d[None, :, :, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
    G = np.zeros((B, H, N, N)) if dST is None else np.array(dST, dtype=np.float64).reshape(B, H, N, N)
    dr, dk, dv = (np.empty((B, T, H, N)) for _ in range(3))
    dw = np.zeros((H, N))
    du = np.zeros((H, N))
    for t in range(T - 1, -1, -1):
        vg = np.einsum("bhj,bhj->bh", v[:, t], go[:, t])                 # v_t . go_t
        bonus = np.einsum("bhi,hi,bhi->bh", r[:, t], u, k[:, t])
        dr[:, t] = np.einsum("bhij,bhj->bhi", prev[t], go[:, t]) + u[None] * k[:, t] * vg[..., None]
        dk[:, t] = np.einsum("bhij,bhj->bhi", G, v[:, t]) + u[None] * r[:, t] * vg[..., None]
        dv[:, t] = np.einsum("bhi,bhij->bhj", k[:, t], G) + bonus[..., None] * go[:, t]
        du += np.einsum("bhi,bhi,bh->hi", r[:, t], k[:, t], vg)
        dw -= d * np.einsum("bhij,bhij->hi", G, prev[t])
        G = d[None, :, :, None] * G + r[:, t, :, :, None] * go[:, t, :, None, :]
    return (dr.reshape(B, T, H * N), dk.reshape(B, T, H * N), dv.reshape(B, T, H * N), dw, du, G)
