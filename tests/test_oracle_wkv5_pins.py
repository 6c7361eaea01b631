"""Pins for the RWKV-5 matrix-state oracle (oracle/wkv5_ref.py), by routes other
than its recurrence: the history-sum form with library matrix products, the
no-decay case as causal linear attention, the infinite-decay limit, the
one-channel case through scipy's linear filter, an exact worked example,
splitting a sequence through the state, and invariances."""
import math

import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import wkv5_backward_ref, wkv5_direct_ref, wkv5_forward_ref


def rand(B, T, H, N, seed, w_lo=-3.0, w_hi=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_lo, w_hi, (H, N)))
    u = rng.normal(0, 1, (H, N))
    r, k, v = (rng.normal(0, 1, (B, T, H * N)) for _ in range(3))
    S0 = rng.normal(0, 1, (B, H, N, N))
    return w, u, r, k, v, S0


@pytest.mark.parametrize("B,T,H,N", [(2, 13, 2, 4), (1, 1, 3, 2), (3, 30, 1, 8)])
def test_recurrence_equals_history_sum(B, T, H, N):
    w, u, r, k, v, S0 = rand(B, T, H, N, B + T + H + N)
    o, _ = wkv5_forward_ref(w, u, r, k, v, H)
    np.testing.assert_allclose(o, wkv5_direct_ref(w, u, r, k, v, H), rtol=1e-12, atol=1e-12)
    o, _ = wkv5_forward_ref(w, u, r, k, v, H, S0)
    np.testing.assert_allclose(o, wkv5_direct_ref(w, u, r, k, v, H, S0), rtol=1e-12, atol=1e-12)


def test_no_decay_is_causal_linear_attention():
    """w = 0, u = 1: o_t = sum_{s <= t} (r_t . k_s) v_s, per head, i.e. tril(R K^T) V."""
    B, T, H, N = 2, 17, 3, 5
    _, _, r, k, v, _ = rand(B, T, H, N, 1)
    o, S = wkv5_forward_ref(np.zeros((H, N)), np.ones((H, N)), r, k, v, H)
    for h in range(H):
        sl = slice(h * N, (h + 1) * N)
        for b in range(B):
            att = np.tril(r[b, :, sl] @ k[b, :, sl].T)
            np.testing.assert_allclose(o[b, :, sl], att @ v[b, :, sl], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S[b, h], k[b, :, sl].T @ v[b, :, sl], rtol=1e-12, atol=1e-12)


def test_infinite_decay_keeps_only_the_previous_token():
    """e^{-w} = 0: the state before token t is k_{t-1}^T v_{t-1} alone."""
    B, T, H, N = 1, 9, 2, 3
    _, u, r, k, v, _ = rand(B, T, H, N, 2)
    o, _ = wkv5_forward_ref(np.full((H, N), 1e4), u, r, k, v, H)
    for h in range(H):
        sl = slice(h * N, (h + 1) * N)
        for t in range(T):
            exp = (r[0, t, sl] * u[h] * k[0, t, sl]).sum() * v[0, t, sl]
            if t > 0:
                exp = exp + (r[0, t, sl] * k[0, t - 1, sl]).sum() * v[0, t - 1, sl]
            np.testing.assert_allclose(o[0, t, sl], exp, rtol=1e-12, atol=1e-12)


def test_one_channel_heads_are_a_linear_filter():
    """N = 1: s_t = e^{-w} s_{t-1} + k_t v_t (scipy's lfilter), o_t = r_t (s_{t-1} + u k_t v_t)."""
    B, T, H, N = 2, 40, 3, 1
    w, u, r, k, v, _ = rand(B, T, H, N, 3)
    o, S = wkv5_forward_ref(w, u, r, k, v, H)
    for b in range(B):
        for h in range(H):
            x = k[b, :, h] * v[b, :, h]
            s = lfilter([1.0], [1.0, -math.exp(-w[h, 0])], x)
            prev = np.concatenate([[0.0], s[:-1]])
            np.testing.assert_allclose(o[b, :, h], r[b, :, h] * (prev + u[h, 0] * x), rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(S[b, h, 0, 0], s[-1], rtol=1e-12)


def test_worked_example():
    # one head, N = 1, decay factor 1/2, u = 3; r = 1, k = (1, 2, 4), v = (1, 1, -1)
    # o_0 = u k0 v0 = 3;  o_1 = k0 v0 + u k1 v1 = 1 + 6 = 7
    # o_2 = (1/2) k0 v0 + k1 v1 + u k2 v2 = 0.5 + 2 - 12 = -9.5;  S_2 = 0.25 + 1 - 4 = -2.75
    w = np.array([[math.log(2.0)]])
    u = np.array([[3.0]])
    r = np.ones((1, 3, 1))
    k = np.array([1.0, 2.0, 4.0]).reshape(1, 3, 1)
    v = np.array([1.0, 1.0, -1.0]).reshape(1, 3, 1)
    o, S = wkv5_forward_ref(w, u, r, k, v, 1)
    np.testing.assert_allclose(o[0, :, 0], [3.0, 7.0, -9.5], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(S[0, 0, 0, 0], -2.75, rtol=1e-15)


def test_split_sequence_through_the_state():
    B, T, H, N = 2, 25, 2, 4
    w, u, r, k, v, S0 = rand(B, T, H, N, 4)
    whole, Sw = wkv5_forward_ref(w, u, r, k, v, H, S0)
    for t1 in (1, 11, 24):
        a, Sa = wkv5_forward_ref(w, u, r[:, :t1], k[:, :t1], v[:, :t1], H, S0)
        b, Sb = wkv5_forward_ref(w, u, r[:, t1:], k[:, t1:], v[:, t1:], H, Sa)
        np.testing.assert_allclose(np.concatenate([a, b], axis=1), whole, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Sb, Sw, rtol=1e-12, atol=1e-12)


def test_invariances():
    B, T, H, N = 1, 12, 2, 3
    w, u, r, k, v, _ = rand(B, T, H, N, 5)
    o, _ = wkv5_forward_ref(w, u, r, k, v, H)
    # linear in r and in v; bilinear scaling of k against v
    np.testing.assert_allclose(wkv5_forward_ref(w, u, 2.5 * r, k, v, H)[0], 2.5 * o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(wkv5_forward_ref(w, u, r, 4.0 * k, 0.25 * v, H)[0], o, rtol=1e-12, atol=1e-12)
    # heads are independent: head 1's inputs do not reach head 0's outputs
    r2 = r.copy()
    r2[:, :, N:] += 1.0
    k2 = k.copy()
    k2[:, :, N:] *= -3.0
    o2, _ = wkv5_forward_ref(w, u, r2, k2, v, H)
    np.testing.assert_array_equal(o2[:, :, :N], o[:, :, :N])


def _torch_direct(w, u, r, k, v, H, S0):
    """wkv5_direct_ref's history sum written in torch (float64, CPU), for autograd."""
    import torch

    B, T, C = r.shape
    N = C // H
    rh, kh, vh = (x.reshape(B, T, H, N) for x in (r, k, v))
    t = torch.arange(T, dtype=torch.float64)
    age = t[:, None] - 1 - t[None, :]
    mask = (age >= 0).to(torch.float64)
    outs = []
    for h in range(H):
        dec = torch.exp(-w[h][None, None, :] * torch.clamp(age, min=0)[:, :, None]) * mask[:, :, None]
        A = torch.einsum("bti,tsi,bsi->bts", rh[:, :, h], dec, kh[:, :, h])
        A = A + torch.einsum("bti,i,bti->bt", rh[:, :, h], u[h], kh[:, :, h])[:, :, None] * torch.eye(T, dtype=torch.float64)
        o = A @ vh[:, :, h]
        o = o + (rh[:, :, h] * torch.exp(-w[h][None, None, :] * t[None, :, None])) @ S0[:, h]
        outs.append(o)
    return torch.stack(outs, dim=2).reshape(B, T, C)


@pytest.mark.parametrize("B,T,H,N", [(2, 11, 2, 4), (1, 1, 2, 3), (1, 20, 1, 6)])
def test_backward_matches_torch_autograd_of_the_history_sum(B, T, H, N):
    import torch

    w, u, r, k, v, S0 = rand(B, T, H, N, 11 + T)
    go = np.random.default_rng(12 + T).normal(0, 1, r.shape)
    tw, tu, tr, tk, tv, tS = (torch.tensor(x, requires_grad=True) for x in (w, u, r, k, v, S0))
    (torch.tensor(go) * _torch_direct(tw, tu, tr, tk, tv, H, tS)).sum().backward()
    dr, dk, dv, dw, du, dS = wkv5_backward_ref(w, u, r, k, v, go, H, S0)
    for name, got, ref in (("dr", dr, tr), ("dk", dk, tk), ("dv", dv, tv), ("dw", dw, tw), ("du", du, tu),
                           ("dS0", dS, tS)):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-10, atol=1e-10, err_msg=name)


def test_backward_central_differences():
    B, T, H, N = 1, 7, 2, 3
    w, u, r, k, v, S0 = rand(B, T, H, N, 13)
    go = np.random.default_rng(14).normal(0, 1, r.shape)
    dr, dk, dv, dw, du, dS = wkv5_backward_ref(w, u, r, k, v, go, H, S0)
    loss = lambda *a: float(np.sum(go * wkv5_forward_ref(*a[:5], H, a[5])[0]))
    args = [w, u, r, k, v, S0]
    h = 1e-5
    for ai, grad, idx in ((0, dw, (1, 2)), (1, du, (0, 1)), (2, dr, (0, 3, 4)), (3, dk, (0, 5, 1)), (4, dv, (0, 0, 5)),
                          (5, dS, (0, 1, 2, 0))):
        a_p = [x.copy() for x in args]
        a_m = [x.copy() for x in args]
        a_p[ai][idx] += h
        a_m[ai][idx] -= h
        fd = (loss(*a_p) - loss(*a_m)) / (2 * h)
        assert abs(fd - grad[idx]) < 1e-6 * (1 + abs(fd)), (ai, fd, grad[idx])


def _torch_final_state(w, k, v, H, S0):
    """S_T = diag(e^{-w T}) S0 + sum_s diag(e^{-w (T-1-s)}) k_s^T v_s, written as one sum."""
    import torch

    B, T, C = k.shape
    N = C // H
    kh, vh = (x.reshape(B, T, H, N) for x in (k, v))
    t = torch.arange(T, dtype=torch.float64)
    dec = torch.exp(-w[None, :, :] * (T - 1 - t)[:, None, None])  # [T, H, N]
    S = torch.exp(-w * T)[None, :, :, None] * S0
    return S + torch.einsum("bthi,thi,bthj->bhij", kh, dec, vh)


@pytest.mark.parametrize("B,T,H,N", [(2, 9, 2, 4), (1, 1, 1, 3)])
def test_backward_with_final_state_gradient_matches_autograd(B, T, H, N):
    """L = <go, o> + <dS_T, S_T>: the final state's gradient enters as the
    adjoint after the last token."""
    import torch

    w, u, r, k, v, S0 = rand(B, T, H, N, 21 + T)
    rng = np.random.default_rng(22 + T)
    go = rng.normal(0, 1, r.shape)
    dST = rng.normal(0, 1, S0.shape)
    tw, tu, tr, tk, tv, tS = (torch.tensor(x, requires_grad=True) for x in (w, u, r, k, v, S0))
    loss = (torch.tensor(go) * _torch_direct(tw, tu, tr, tk, tv, H, tS)).sum()
    loss = loss + (torch.tensor(dST) * _torch_final_state(tw, tk, tv, H, tS)).sum()
    loss.backward()
    dr, dk, dv, dw, du, dS = wkv5_backward_ref(w, u, r, k, v, go, H, S0, dST)
    for name, got, ref in (("dr", dr, tr), ("dk", dk, tk), ("dv", dv, tv), ("dw", dw, tw), ("du", du, tu),
                           ("dS0", dS, tS)):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-10, atol=1e-10, err_msg=name)


def test_backward_of_a_split_sequence_chains_through_the_state():
    """Backward of a sequence cut in two: the second part's dS0 is the first
    part's dS_T, and the pieces equal the whole sequence's gradients."""
    B, T, H, N, t1 = 2, 12, 2, 3, 5
    w, u, r, k, v, S0 = rand(B, T, H, N, 31)
    go = np.random.default_rng(32).normal(0, 1, r.shape)
    whole = wkv5_backward_ref(w, u, r, k, v, go, H, S0)
    _, S1 = wkv5_forward_ref(w, u, r[:, :t1], k[:, :t1], v[:, :t1], H, S0)
    second = wkv5_backward_ref(w, u, r[:, t1:], k[:, t1:], v[:, t1:], go[:, t1:], H, S1)
    first = wkv5_backward_ref(w, u, r[:, :t1], k[:, :t1], v[:, :t1], go[:, :t1], H, S0, second[5])
    for i, name in enumerate(("dr", "dk", "dv")):
        np.testing.assert_allclose(np.concatenate([first[i], second[i]], axis=1), whole[i], rtol=1e-11, atol=1e-11,
                                   err_msg=name)
    np.testing.assert_allclose(first[3] + second[3], whole[3], rtol=1e-11, atol=1e-11, err_msg="dw")
    np.testing.assert_allclose(first[4] + second[4], whole[4], rtol=1e-11, atol=1e-11, err_msg="du")
    np.testing.assert_allclose(first[5], whole[5], rtol=1e-11, atol=1e-11, err_msg="dS0")
