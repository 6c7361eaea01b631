"""Pins of the float64 RWKV-6 oracle (oracle/wkv6_ref.py) to facts that do not
depend on it: its closed history-sum form, the RWKV-5 special case (constant
decay), an exact reset, and the state hand-over of a split sequence."""
import numpy as np
import pytest

from oracle import wkv5_forward_ref, wkv6_backward_ref, wkv6_direct_ref, wkv6_forward_ref


def rand(B, T, H, N, seed, w_lo=-3.0, w_hi=1.0):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_lo, w_hi, (B, T, H * N)))
    u = rng.normal(0, 1, (H, N))
    r, k, v = (rng.normal(0, 1, (B, T, H * N)) for _ in range(3))
    S0 = rng.normal(0, 1, (B, H, N, N))
    return w, u, r, k, v, S0


@pytest.mark.parametrize("B,T,H,N", [(2, 13, 2, 4), (1, 1, 3, 2), (3, 30, 1, 8)])
def test_recurrence_equals_history_sum(B, T, H, N):
    w, u, r, k, v, S0 = rand(B, T, H, N, B + T + H + N)
    o, _ = wkv6_forward_ref(w, u, r, k, v, H)
    np.testing.assert_allclose(o, wkv6_direct_ref(w, u, r, k, v, H), rtol=1e-11, atol=1e-11)
    o, _ = wkv6_forward_ref(w, u, r, k, v, H, S0)
    np.testing.assert_allclose(o, wkv6_direct_ref(w, u, r, k, v, H, S0), rtol=1e-11, atol=1e-11)


def test_constant_decay_is_rwkv5():
    """w_t the same for every token: the RWKV-5 operator, outputs and final state."""
    B, T, H, N = 2, 21, 3, 5
    _, u, r, k, v, S0 = rand(B, T, H, N, 3)
    w5 = np.exp(np.random.default_rng(4).uniform(-3, 1, (H, N)))
    w6 = np.broadcast_to(w5.reshape(1, 1, H * N), (B, T, H * N))
    o6, S6 = wkv6_forward_ref(w6, u, r, k, v, H, S0)
    o5, S5 = wkv5_forward_ref(w5, u, r, k, v, H, S0)
    np.testing.assert_allclose(o6, o5, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S6, S5, rtol=1e-12, atol=1e-12)


def test_infinite_decay_resets_the_state():
    """e^{-w_t0} = 0 in every channel: the state after token t0 holds only
    k_t0^T v_t0, so the outputs after t0 and the final state do not depend on
    anything before t0 (o_t0 itself still reads the state before t0)."""
    B, T, H, N, t0 = 2, 16, 2, 4, 7
    w, u, r, k, v, S0 = rand(B, T, H, N, 5)
    w[:, t0, :] = np.inf
    o, S = wkv6_forward_ref(w, u, r, k, v, H, S0)
    rng = np.random.default_rng(6)
    r2, k2, v2 = (x.copy() for x in (r, k, v))
    for x in (r2, k2, v2):
        x[:, :t0] = rng.normal(0, 1, x[:, :t0].shape)
    o2, S2 = wkv6_forward_ref(w, u, r2, k2, v2, H, rng.normal(0, 1, S0.shape))
    np.testing.assert_allclose(o2[:, t0 + 1:], o[:, t0 + 1:], rtol=1e-12, atol=1e-12)
    assert np.abs(o2[:, t0] - o[:, t0]).max() > 1e-3  # the reset token's own output does change
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_split_sequence_through_the_state():
    B, T, H, N = 2, 25, 2, 3
    w, u, r, k, v, S0 = rand(B, T, H, N, 7)
    o, S = wkv6_forward_ref(w, u, r, k, v, H, S0)
    for t1 in (1, 9, 24):
        o1, S1 = wkv6_forward_ref(w[:, :t1], u, r[:, :t1], k[:, :t1], v[:, :t1], H, S0)
        o2, S2 = wkv6_forward_ref(w[:, t1:], u, r[:, t1:], k[:, t1:], v[:, t1:], H, S1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_single_channel_worked_example():
    """N = 1 and three tokens, written out by hand: s_t = e^{-w_t} s_{t-1} + k_t v_t,
    o_t = r_t (s_{t-1} + u k_t v_t) with s_0 = 0."""
    w = np.array([[[np.log(2.0)], [np.log(4.0)], [0.0]]])          # decay factors 1/2, 1/4, 1
    r = np.array([[[1.0], [2.0], [-1.0]]])
    k = np.array([[[3.0], [1.0], [2.0]]])
    v = np.array([[[1.0], [-2.0], [0.5]]])
    u = np.array([[0.5]])
    o, S = wkv6_forward_ref(w, u, r, k, v, 1)
    # s after t=1: 3; after t=2: 3/4 - 2 = -5/4; after t=3: -5/4 + 1 = -1/4
    # o_1 = 1 (0 + 0.5 * 3) = 1.5; o_2 = 2 (3 + 0.5 * -2) = 4; o_3 = -1 (-5/4 + 0.5 * 1) = 0.75
    np.testing.assert_allclose(o[0, :, 0], [1.5, 4.0, 0.75], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], [[-0.25]], rtol=0, atol=1e-15)


def _torch_direct6(w, u, r, k, v, H, S0):
    """wkv6_direct_ref's history sum written again in torch (float64, CPU), so
    that autograd differentiates the closed form."""
    import torch

    B, T, C = r.shape
    N = C // H
    wh, rh, kh, vh = (x.reshape(B, T, H, N) for x in (w, r, k, v))
    L = torch.cat([torch.zeros(B, 1, H, N, dtype=torch.float64), torch.cumsum(wh, dim=1)], dim=1)  # L[t + 1] = L_t
    t = torch.arange(T)
    causal = ((t[:, None] - 1 - t[None, :]) >= 0).to(torch.float64)
    outs = []
    for h in range(H):
        Lh = L[:, :, h]                                                  # [B, T + 1, N]
        gap = Lh[:, :T][:, :, None, :] - Lh[:, 1:][:, None, :, :]        # L_{t-1} - L_s, [B, T, T, N]
        dec = torch.exp(-torch.clamp(gap, min=0)) * causal[None, :, :, None]
        A = torch.einsum("bti,btsi,bsi->bts", rh[:, :, h], dec, kh[:, :, h])
        A = A + torch.diag_embed(torch.einsum("bti,i,bti->bt", rh[:, :, h], u[h], kh[:, :, h]))
        o = A @ vh[:, :, h]
        o = o + (rh[:, :, h] * torch.exp(-Lh[:, :T])) @ S0[:, h]
        outs.append(o)
    return torch.stack(outs, dim=2).reshape(B, T, C)


def _torch_final_state6(w, k, v, H, S0):
    """S_T = diag(e^{-L_{T-1}}) S0 + sum_s diag(e^{-(L_{T-1} - L_s)}) k_s^T v_s."""
    import torch

    B, T, C = k.shape
    N = C // H
    wh, kh, vh = (x.reshape(B, T, H, N) for x in (w, k, v))
    L = torch.cumsum(wh, dim=1)                                          # L_s, [B, T, H, N]
    S = torch.exp(-L[:, -1])[:, :, :, None] * S0
    return S + torch.einsum("bthi,bthi,bthj->bhij", kh, torch.exp(-(L[:, -1:] - L)), vh)


@pytest.mark.parametrize("B,T,H,N", [(2, 9, 2, 4), (1, 1, 1, 3), (1, 14, 1, 5)])
def test_backward_matches_torch_autograd_of_the_history_sum(B, T, H, N):
    """All gradients, dw per token included, with a final-state gradient."""
    import torch

    w, u, r, k, v, S0 = rand(B, T, H, N, 41 + T)
    rng = np.random.default_rng(42 + T)
    go = rng.normal(0, 1, r.shape)
    dST = rng.normal(0, 1, S0.shape)
    tw, tu, tr, tk, tv, tS = (torch.tensor(x, requires_grad=True) for x in (w, u, r, k, v, S0))
    loss = (torch.tensor(go) * _torch_direct6(tw, tu, tr, tk, tv, H, tS)).sum()
    loss = loss + (torch.tensor(dST) * _torch_final_state6(tw, tk, tv, H, tS)).sum()
    loss.backward()
    dr, dk, dv, dw, du, dS = wkv6_backward_ref(w, u, r, k, v, go, H, S0, dST)
    for name, got, ref in (("dr", dr, tr), ("dk", dk, tk), ("dv", dv, tv), ("dw", dw, tw), ("du", du, tu),
                           ("dS0", dS, tS)):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-10, atol=1e-10, err_msg=name)


def test_backward_central_differences():
    B, T, H, N = 1, 6, 2, 3
    w, u, r, k, v, S0 = rand(B, T, H, N, 43)
    go = np.random.default_rng(44).normal(0, 1, r.shape)
    dr, dk, dv, dw, du, dS = wkv6_backward_ref(w, u, r, k, v, go, H, S0)
    loss = lambda *a: float(np.sum(go * wkv6_forward_ref(*a[:5], H, a[5])[0]))
    args = [w, u, r, k, v, S0]
    h = 1e-5
    for ai, grad, idx in ((0, dw, (0, 2, 4)), (0, dw, (0, 4, 1)), (1, du, (1, 2)), (2, dr, (0, 3, 4)),
                          (3, dk, (0, 1, 5)), (4, dv, (0, 0, 2)), (5, dS, (0, 1, 2, 0))):
        a_p = [x.copy() for x in args]
        a_m = [x.copy() for x in args]
        a_p[ai][idx] += h
        a_m[ai][idx] -= h
        fd = (loss(*a_p) - loss(*a_m)) / (2 * h)
        assert abs(fd - grad[idx]) < 1e-6 * (1 + abs(fd)), (ai, idx, fd, grad[idx])


def test_backward_constant_decay_is_rwkv5():
    """Constant rates: dr, dk, dv, du, dS0 equal RWKV-5's, and the per-token dw
    summed over tokens and the batch is RWKV-5's dw."""
    from oracle import wkv5_backward_ref

    B, T, H, N = 2, 11, 2, 4
    _, u, r, k, v, S0 = rand(B, T, H, N, 45)
    go = np.random.default_rng(46).normal(0, 1, r.shape)
    w5 = np.exp(np.random.default_rng(47).uniform(-3, 1, (H, N)))
    w6 = np.broadcast_to(w5.reshape(1, 1, H * N), (B, T, H * N)).copy()
    g6 = wkv6_backward_ref(w6, u, r, k, v, go, H, S0)
    g5 = wkv5_backward_ref(w5, u, r, k, v, go, H, S0)
    for i, name in ((0, "dr"), (1, "dk"), (2, "dv")):
        np.testing.assert_allclose(g6[i], g5[i], rtol=1e-12, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(g6[3].sum(axis=(0, 1)).reshape(H, N), g5[3], rtol=1e-11, atol=1e-11, err_msg="dw")
    np.testing.assert_allclose(g6[4], g5[4], rtol=1e-12, atol=1e-12, err_msg="du")
    np.testing.assert_allclose(g6[5], g5[5], rtol=1e-12, atol=1e-12, err_msg="dS0")
