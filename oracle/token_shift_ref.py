"""Float64 CPU oracle for the token-shift mix that produces the inputs of the
time-mixing projections.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or calls
this module; only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may.  It shares no code, tables or constants with the HIP
path.

Sources (page title, then section):

* [P5] "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section
  "关键设计 1：Token Shift - 给并行投影注入前一时刻": each of r, k, v is a
  linear projection of its own per-channel mix of the current token's input
  and the previous token's input, with mixing vectors mu_r, mu_k, mu_v
  (weight mu on x_t, 1 - mu on x_{t-1}); section "整体架构": the inference
  state tuple carries x, the previous token's input.
* [P4] "RWKV（Receptance Weighted Key Value）概念", section 3.3: channel mixing
  applies the same mix mu x_t + (1 - mu) x_{t-1} before its projections.
* [P3] "RWKV模型深度研究报告（截至2026年初）", section 1.1.3: token shift mixes
  each token's embedding with the previous token's by a learnt ratio.

Only the elementwise mix is computed here; the projections W_r, W_k, W_v are
ordinary matrix products outside this operator.

Readings where the pages are silent:

* before the first token the previous input is zero, unless the caller passes
  the last input of an earlier segment (the state tuple's x);
* one call computes M mixes (M mixing vectors) of the same x: 3 for the
  time-mixing r, k, v, 2 for channel mixing;
* the backward (derived here by differentiating the mix) gives dx, the
  gradient of every mixing vector summed over batch and time, and the
  gradient of the carried-in previous input.

Parity status: every function here is pinned (tests/test_oracle_shift_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["token_shift_ref", "token_shift_backward_ref", "shifted_inputs_ref"]


def shifted_inputs_ref(x, x_prev=None):
    """x_{t-1} for every token: [B, T, C] float64 whose token t holds x[:, t-1]
    and whose token 0 holds ``x_prev`` [B, C] (zeros when None)."""
    x = np.asarray(x, dtype=np.float64)
    xs = np.zeros_like(x)
    xs[:, 1:] = x[:, :-1]
    if x_prev is not None and x.shape[1] > 0:
        xs[:, 0] = np.asarray(x_prev, dtype=np.float64).reshape(x.shape[0], x.shape[2])
    return xs


def token_shift_ref(mu, x, x_prev=None):
    """The M mixes of [P5] "关键设计 1" in float64.

    mu: [M, C]; x: [B, T, C]; x_prev: [B, C] or None.
    Returns out [M, B, T, C] with
        out[j, b, t] = mu[j] x[b, t] + (1 - mu[j]) x[b, t-1].
    """
    mu = np.asarray(mu, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    xs = shifted_inputs_ref(x, x_prev)
    m = mu[:, None, None, :]
    return m * x[None] + (1.0 - m) * xs[None]


def token_shift_backward_ref(mu, x, gout, x_prev=None):
    """Gradients of L = sum(gout * out) for out = token_shift_ref(mu, x, x_prev).

    Differentiating out[j, t] = mu_j x_t + (1 - mu_j) x_{t-1}:
        dx_t     = sum_j mu_j gout[j, t] + (1 - mu_j) gout[j, t+1]   (no t+1 term at t = T-1)
        dmu_j    = sum_{b,t} gout[j, t] (x_t - x_{t-1})               [C]
        dx_prev  = sum_j (1 - mu_j) gout[j, 0]                        [B, C]
    (x_{-1} is x_prev, or zero).  Returns (dx [B, T, C], dmu [M, C],
    dx_prev [B, C]) in float64.
    """
    mu = np.asarray(mu, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gout, dtype=np.float64)
    Bsz, T, C = x.shape
    m = mu[:, None, None, :]
    dx = np.sum(m * g, axis=0)
    if T > 1:
        dx[:, :-1] += np.sum((1.0 - m) * g[:, :, 1:], axis=0)
    xs = shifted_inputs_ref(x, x_prev)
    dmu = np.sum(g * (x - xs)[None], axis=(1, 2))
    dx_prev = np.sum((1.0 - mu)[:, None, :] * g[:, :, 0], axis=0) if T > 0 else np.zeros((Bsz, C))
    return dx, dmu, dx_prev
