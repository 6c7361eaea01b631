"""Pins for the token-shift oracle (oracle/token_shift_ref.py): what the pages
and the mathematics fix, checked by routes other than the oracle's formula.

The mix of "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section
"关键设计 1：Token Shift", puts weight mu on the current token and 1 - mu on
the previous one.  Pinned by: its limits mu = 1 (the input itself) and mu = 0
(the input delayed by one token, through numpy's pad), a worked example in
exact rationals, splitting a sequence through the carried previous input,
linearity, and for the backward torch autograd, finite differences and the
adjoint identities of a linear map.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import shifted_inputs_ref, token_shift_backward_ref, token_shift_ref


def rand(B, T, C, M, seed):
    rng = np.random.default_rng(seed)
    mu = rng.uniform(-0.5, 1.5, (M, C))
    x = rng.normal(0, 1, (B, T, C))
    xp = rng.normal(0, 1, (B, C))
    g = rng.normal(0, 1, (M, B, T, C))
    return mu, x, xp, g


def test_mu_one_is_identity():
    _, x, xp, _ = rand(2, 9, 5, 1, 0)
    mu = np.ones((1, 5))
    assert np.array_equal(token_shift_ref(mu, x, xp)[0], x)


def test_mu_zero_is_delay_by_one_token():
    _, x, xp, _ = rand(3, 7, 4, 1, 1)
    mu = np.zeros((1, 4))
    delayed = np.pad(x, ((0, 0), (1, 0), (0, 0)))[:, :-1]
    assert np.array_equal(token_shift_ref(mu, x)[0], delayed)
    delayed[:, 0] = xp
    assert np.array_equal(token_shift_ref(mu, x, xp)[0], delayed)


def test_worked_example_exact():
    # x = 1, 2, 4 on one channel, mu = 1/4, nothing before the first token:
    # 1/4 * 1 + 3/4 * 0 = 1/4;  1/4 * 2 + 3/4 * 1 = 5/4;  1/4 * 4 + 3/4 * 2 = 5/2
    x = np.array([[[1.0], [2.0], [4.0]]])
    out = token_shift_ref(np.array([[0.25]]), x)[0, 0, :, 0]
    assert [Fraction(v) for v in out] == [Fraction(1, 4), Fraction(5, 4), Fraction(5, 2)]
    # with a previous input of -8: 1/4 * 1 + 3/4 * (-8) = -23/4
    out = token_shift_ref(np.array([[0.25]]), x, np.array([[-8.0]]))[0, 0, :, 0]
    assert Fraction(out[0]) == Fraction(-23, 4)


def test_split_sequence_through_previous_input():
    mu, x, xp, _ = rand(2, 40, 6, 3, 2)
    whole = token_shift_ref(mu, x, xp)
    for t1 in (1, 17, 39):
        a = token_shift_ref(mu, x[:, :t1], xp)
        b = token_shift_ref(mu, x[:, t1:], x[:, t1 - 1])
        np.testing.assert_array_equal(np.concatenate([a, b], axis=2), whole)


def test_linear_in_x_and_affine_in_mu():
    mu, x, xp, _ = rand(2, 11, 3, 2, 3)
    _, z, zp, _ = rand(2, 11, 3, 2, 4)
    lhs = token_shift_ref(mu, 2.0 * x - 3.0 * z, 2.0 * xp - 3.0 * zp)
    rhs = 2.0 * token_shift_ref(mu, x, xp) - 3.0 * token_shift_ref(mu, z, zp)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)
    # mu = 1/2 is the mean of the two tokens
    half = token_shift_ref(np.full((1, 3), 0.5), x, xp)[0]
    np.testing.assert_allclose(half, (x + shifted_inputs_ref(x, xp)) / 2, rtol=0, atol=1e-15)


def _torch_mix(mu, x, xp):
    """The mix written with torch's pad for the delay, for autograd."""
    xs = torch.cat([xp[:, None, :], x[:, :-1]], dim=1)
    return mu[:, None, None, :] * x[None] + (1 - mu[:, None, None, :]) * xs[None]


@pytest.mark.parametrize("B,T,C,M", [(2, 13, 5, 3), (1, 1, 3, 2), (3, 2, 1, 4), (2, 30, 7, 1)])
def test_backward_matches_torch_autograd(B, T, C, M):
    mu, x, xp, g = rand(B, T, C, M, B * 100 + T + C + M)
    tm = torch.tensor(mu, requires_grad=True)
    tx = torch.tensor(x, requires_grad=True)
    tp = torch.tensor(xp, requires_grad=True)
    (torch.tensor(g) * _torch_mix(tm, tx, tp)).sum().backward()
    dx, dmu, dxp = token_shift_backward_ref(mu, x, g, xp)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dmu, tm.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dxp, tp.grad.numpy(), rtol=1e-13, atol=1e-13)


def test_backward_central_differences():
    B, T, C, M = 2, 6, 3, 3
    mu, x, xp, g = rand(B, T, C, M, 9)
    dx, dmu, dxp = token_shift_backward_ref(mu, x, g, xp)
    loss = lambda m, xx, pp: float(np.sum(g * token_shift_ref(m, xx, pp)))
    h = 1e-3  # the loss is bilinear in (mu, x): central differences are exact up to rounding
    for idx in [(0, 0, 0), (1, 3, 2), (0, T - 1, 1)]:
        e = np.zeros_like(x)
        e[idx] = h
        assert abs((loss(mu, x + e, xp) - loss(mu, x - e, xp)) / (2 * h) - dx[idx]) < 1e-9
    for idx in [(0, 0), (2, 2)]:
        e = np.zeros_like(mu)
        e[idx] = h
        assert abs((loss(mu + e, x, xp) - loss(mu - e, x, xp)) / (2 * h) - dmu[idx]) < 1e-9
    e = np.zeros_like(xp)
    e[1, 1] = h
    assert abs((loss(mu, x, xp + e) - loss(mu, x, xp - e)) / (2 * h) - dxp[1, 1]) < 1e-9


def test_backward_adjoint_identities():
    """For a map linear in (x, x_prev): <g, out> = <dx, x> + <dx_prev, x_prev>;
    and out = x_{t-1} + mu (x_t - x_{t-1}) gives <g, out> = <g, x_{t-1}> + <mu, dmu>."""
    mu, x, xp, g = rand(3, 25, 8, 3, 10)
    out = token_shift_ref(mu, x, xp)
    dx, dmu, dxp = token_shift_backward_ref(mu, x, g, xp)
    lhs = np.sum(g * out)
    assert abs(lhs - (np.sum(dx * x) + np.sum(dxp * xp))) < 1e-10 * np.sum(np.abs(g * out))
    xs = shifted_inputs_ref(x, xp)
    assert abs(lhs - (np.sum(g * xs[None]) + np.sum(mu * dmu))) < 1e-10 * np.sum(np.abs(g * out))


def test_empty_and_single_token():
    mu = np.array([[0.3, 0.7]])
    x = np.zeros((2, 0, 2))
    g = np.zeros((1, 2, 0, 2))
    dx, dmu, dxp = token_shift_backward_ref(mu, x, g)
    assert dx.shape == (2, 0, 2) and np.all(dmu == 0) and np.all(dxp == 0)
    x1 = np.array([[[2.0, -1.0]]])
    g1 = np.array([[[[1.0, 3.0]]]])
    dx, dmu, dxp = token_shift_backward_ref(mu, x1, g1, np.array([[5.0, 7.0]]))
    np.testing.assert_allclose(dx[0, 0], [0.3, 2.1], rtol=0, atol=1e-15)          # mu g
    np.testing.assert_allclose(dmu[0], [1.0 * (2 - 5), 3.0 * (-1 - 7)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dxp[0], [0.7, 0.9], rtol=0, atol=1e-15)             # (1 - mu) g
