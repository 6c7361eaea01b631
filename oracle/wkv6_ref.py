"""Float64 CPU oracle for the matrix-state WKV with data-dependent decay (RWKV-6).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or calls
this module; only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may.  It shares no code, tables or constants with the HIP
path.

Sources (page title, then section):

* "RWKV模型深度研究报告（截至2026年初）", section 1.3.2: RWKV-5 and RWKV-6
  (Eagle, Finch) share the matrix-valued state with per-channel decay; section
  1.1.3: RWKV-6 makes the token-shift mix input dependent through a low-rank
  projection.
* "RWKV（Receptance Weighted Key Value）概念", section 13 (recent events): the
  sixth generation brings data-dependent time mixing.
* "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", the lineage figure and
  the resource table: Eagle/Finch add dynamic mix and dynamic decay.
* the intelliparadigm.com post, section 3.1 (the table of versions): v6's change
  is a dynamic decay adjustment.

Readings where the pages are silent:

* the decay rate becomes a per-token input: w [B, T, C] >= 0, decay factor
  e^{-w_t} applied to the key rows of the state at token t; whatever produces it
  (the low-rank projection of the pages) runs before this operator;
* otherwise as RWKV-5 (wkv5_ref.py): heads of N channels, state S (key x value),
      S_t = diag(e^{-w_t}) S_{t-1} + k_t^T v_t
      o_t = r_t (S_{t-1} + diag(u) k_t^T v_t)
  with the bonus u [H, N] constant, and the zero initial state unless given;
* the backward (derived here by differentiating the recurrence; the pages give
  none) is for L = sum_t <go_t, o_t> + <dS_T, S_T>, with the adjoint state
  G_{t-1} = diag(e^{-w_t}) G_t + r_t^T go_t (G_{T-1} = dS_T): dr, dk, dv, du
  and dS0 as for RWKV-5 (wkv5_ref.py), and the rate's gradient per token,
      dw_t = -e^{-w_t} . rowsum(G_t . S_{t-1})
  (dw [B, T, C], not summed: each token has its own rate).

Parity status: every function here is pinned (tests/test_oracle_wkv6_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["wkv6_forward_ref", "wkv6_direct_ref", "wkv6_backward_ref"]


def _heads(x, H):
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    return x.reshape(B, T, H, C // H)


def wkv6_forward_ref(w, u, r, k, v, H, S0=None):
    """Token-by-token recurrence in float64.

    w, r, k, v: [B, T, C] with C = H * N (w the per-token decay rates); u: [H, N];
    S0: [B, H, N, N] or None (zero).  Returns (o [B, T, C], S_T [B, H, N, N]).
    """
    w, r, k, v = (_heads(x, H) for x in (w, r, k, v))
    B, T, _, N = r.shape
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, dtype=np.float64).reshape(B, H, N, N)
    o = np.empty((B, T, H, N))
    with np.errstate(over="ignore"):
        d = np.exp(-w)                                                     # [B, T, H, N]
    for t in range(T):
        kv = k[:, t, :, :, None] * v[:, t, :, None, :]                     # k_t^T v_t, [B, H, N, N]
        o[:, t] = np.einsum("bhi,bhij->bhj", r[:, t], S + u[None, :, :, None] * kv)
        S = d[:, t, :, :, None] * S + kv
    assert np.isfinite(o).all() and np.isfinite(S).all()
    return o.reshape(B, T, H * N), S


def wkv6_direct_ref(w, u, r, k, v, H, S0=None):
    """The same outputs as one sum over the history, with the decay between two
    tokens written as the exponential of a difference of cumulative rates
    L_t = sum_{t' <= t} w_t' (no recurrence):

        o_t[j] = sum_i r_t[i] e^{-L_{t-1}[i]} S0[i, j]
               + sum_{s<t} (sum_i r_t[i] k_s[i] e^{-(L_{t-1}[i] - L_s[i])}) v_s[j]
               + (sum_i r_t[i] u_i k_t[i]) v_t[j]

    with an explicit [T, T, N] decay tensor per (batch row, head).  Small T and
    finite w only."""
    w, r, k, v = (_heads(x, H) for x in (w, r, k, v))
    B, T, _, N = r.shape
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    L = np.concatenate([np.zeros((B, 1, H, N)), np.cumsum(w, axis=1)], axis=1)   # L[t + 1] = L_t, L[0] = 0
    o = np.zeros((B, T, H, N))
    t = np.arange(T)
    causal = (t[:, None] - 1 - t[None, :]) >= 0                                    # s < t
    for b in range(B):
        for h in range(H):
            Lb = L[b, :, h]                                                        # [T + 1, N]
            gap = Lb[t][:, None, :] - Lb[t + 1][None, :, :]                        # L_{t-1} - L_s, [T, T, N]
            dec = np.where(causal[:, :, None], np.exp(-np.where(causal[:, :, None], gap, 0.0)), 0.0)
            A = np.einsum("ti,tsi,si->ts", r[b, :, h], dec, k[b, :, h])
            A += np.diag(np.einsum("ti,i,ti->t", r[b, :, h], u[h], k[b, :, h]))
            o[b, :, h] = A @ v[b, :, h]
            if S0 is not None:
                S0h = np.asarray(S0, dtype=np.float64).reshape(B, H, N, N)[b, h]
                o[b, :, h] += (r[b, :, h] * np.exp(-Lb[t])) @ S0h
    return o.reshape(B, T, H * N)


def wkv6_backward_ref(w, u, r, k, v, go, H, S0=None, dST=None):
    """Gradients of L = sum_t <go_t, o_t> + <dST, S_T> for
    (o, S_T) = wkv6_forward_ref(w, u, r, k, v, H, S0), in float64: a forward
    pass keeping every S_{t-1}, then the adjoint state G (starting from dST,
    [B, H, N, N] or None for zero) walked backwards in time.

    Returns (dr, dk, dv, dw [B, T, C], du [H, N] summed over the batch, dS0
    [B, H, N, N]).
    """
    w, r, k, v, go = (_heads(x, H) for x in (w, r, k, v, go))
    B, T, _, N = r.shape
    u = np.asarray(u, dtype=np.float64).reshape(H, N)
    with np.errstate(over="ignore"):
        d = np.exp(-w)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, dtype=np.float64).reshape(B, H, N, N)
    prev = np.empty((T, B, H, N, N))                                      # S_{t-1}
    for t in range(T):
        prev[t] = S
        S = d[:, t, :, :, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
    G = np.zeros((B, H, N, N)) if dST is None else np.array(dST, dtype=np.float64).reshape(B, H, N, N)
    dr, dk, dv, dw = (np.empty((B, T, H, N)) for _ in range(4))
    du = np.zeros((H, N))
    for t in range(T - 1, -1, -1):
        vg = np.einsum("bhj,bhj->bh", v[:, t], go[:, t])                 # v_t . go_t
        bonus = np.einsum("bhi,hi,bhi->bh", r[:, t], u, k[:, t])
        dr[:, t] = np.einsum("bhij,bhj->bhi", prev[t], go[:, t]) + u[None] * k[:, t] * vg[..., None]
        dk[:, t] = np.einsum("bhij,bhj->bhi", G, v[:, t]) + u[None] * r[:, t] * vg[..., None]
        dv[:, t] = np.einsum("bhi,bhij->bhj", k[:, t], G) + bonus[..., None] * go[:, t]
        du += np.einsum("bhi,bhi,bh->hi", r[:, t], k[:, t], vg)
        dw[:, t] = -d[:, t] * np.einsum("bhij,bhij->bhi", G, prev[t])
        G = d[:, t, :, :, None] * G + r[:, t, :, :, None] * go[:, t, :, None, :]
    return (dr.reshape(B, T, H * N), dk.reshape(B, T, H * N), dv.reshape(B, T, H * N), dw.reshape(B, T, H * N), du,
            G)
