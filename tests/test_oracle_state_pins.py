"""Pins for the oracle's backward through carried state (wkv_backward_state_ref)
and its conversions between plain-sum and stable-state gradients.

Each test checks the oracle against something other than itself: the closed-form
backward of oracle/wkv_ref.py (itself pinned by finite differences and autograd
of the direct definition), central finite differences of the whole loss, an
explicit closed form where only the handed-on state carries gradient, and the
chain rule across a split sequence ("RWKV模型深度研究报告" section 4.4.2: a long
input encoded segment by segment).
"""
import numpy as np
import pytest

from oracle import (
    wkv_backward_ref,
    wkv_backward_state_ref,
    wkv_forward_ref,
    wkv_state_grads_from_sums,
    wkv_sums_from_state,
    wkv_sums_grads_from_state,
)


def rand_case(B, T, C, seed, w_lo=-3.0, w_hi=1.5):
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_lo, w_hi, C))
    u = rng.normal(0, 1, C)
    k = rng.normal(0, 1, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    gy = rng.normal(0, 1, (B, T, C))
    B0 = rng.uniform(0.5, 3.0, (B, C))
    A0 = B0 * rng.normal(0, 1, (B, C))  # |A0| ~ B0: a mean of values
    gA = rng.normal(0, 1, (B, C))
    gB = rng.normal(0, 1, (B, C))
    return w, u, k, v, gy, A0, B0, gA, gB


def loss(w, u, k, v, gy, A0, B0, gA, gB):
    y, AT, BT = wkv_forward_ref(w, u, k, v, return_sums=True, A0=A0, B0=B0)
    return float(np.sum(gy * y) + np.sum(gA * AT) + np.sum(gB * BT))


@pytest.mark.parametrize("B,T,C", [(1, 1, 1), (2, 9, 3), (3, 40, 5)])
def test_no_state_is_the_closed_form_backward(B, T, C):
    """Empty history and no gradient on the handed-on state: the gradients of
    the closed-form accumulators (G, H, G', H')."""
    w, u, k, v, gy, *_ = rand_case(B, T, C, seed=T)
    got = wkv_backward_state_ref(w, u, k, v, gy)
    ref = wkv_backward_ref(w, u, k, v, gy)
    for g, r in zip(got[:4], ref):
        np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-13)
    # nothing flows into an empty history that is then never read
    assert got[4].shape == (B, C) and got[5].shape == (B, C)


def test_central_differences_of_the_whole_loss():
    """Every gradient, the initial sums' included, against central differences
    of L = sum(gy y) + sum(gA A_T) + sum(gB B_T) through wkv_forward_ref."""
    B, T, C = 2, 6, 3
    w, u, k, v, gy, A0, B0, gA, gB = rand_case(B, T, C, seed=11)
    dk, dv, dw, du, dA0, dB0 = wkv_backward_state_ref(w, u, k, v, gy, A0, B0, gA, gB)
    args = dict(w=w, u=u, k=k, v=v, A0=A0, B0=B0)
    grads = dict(w=dw, u=du, k=dk, v=dv, A0=dA0, B0=dB0)
    h = 1e-6
    for name, x in args.items():
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = dict(args, **{name: xp})
            am = dict(args, **{name: xm})
            fd[idx] = (loss(ap["w"], ap["u"], ap["k"], ap["v"], gy, ap["A0"], ap["B0"], gA, gB) -
                       loss(am["w"], am["u"], am["k"], am["v"], gy, am["A0"], am["B0"], gA, gB)) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_handed_on_state_only_has_a_closed_form():
    """With gy = 0 the loss is gA A_T + gB B_T, and A_T = d^T A0 + sum_t
    d^{T-t} e^{k_t} v_t (1-based t), B_T likewise: every gradient is explicit."""
    B, T, C = 2, 12, 4
    w, u, k, v, _, A0, B0, gA, gB = rand_case(B, T, C, seed=5)
    gy = np.zeros_like(k)
    dk, dv, dw, du, dA0, dB0 = wkv_backward_state_ref(w, u, k, v, gy, A0, B0, gA, gB)
    age = (T - 1 - np.arange(T)).astype(np.float64)  # T - t for the 1-based t = index + 1
    f = np.exp(-age[None, :, None] * w[None, None, :]) * np.exp(k)  # d^{T-t} e^{k_t}
    q = gA[:, None, :] * v + gB[:, None, :]
    dT = np.exp(-T * w)
    np.testing.assert_allclose(dv, gA[:, None, :] * f, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk, f * q, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(du, np.zeros(C))
    dw_ref = -(age[None, :, None] * f * q).sum(axis=(0, 1)) - T * (dT * (gA * A0 + gB * B0)).sum(axis=0)
    np.testing.assert_allclose(dw, dw_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dA0, dT * gA, rtol=1e-13)
    np.testing.assert_allclose(dB0, dT * gB, rtol=1e-13)


@pytest.mark.parametrize("cut", [1, 7, 19])
def test_two_segments_chain_to_the_whole_sequence(cut):
    """A sequence split at `cut`: the second segment's backward from the state
    the first hands on gives (dA, dB) for that state; the first segment's
    backward with that as its handed-on gradient gives the rest.  Together they
    equal the backward of the whole sequence (dk, dv joined, dw, du summed)."""
    B, T, C = 2, 20, 3
    w, u, k, v, gy, A0, B0, gA, gB = rand_case(B, T, C, seed=cut)
    whole = wkv_backward_state_ref(w, u, k, v, gy, A0, B0, gA, gB)
    _, Am, Bm = wkv_forward_ref(w, u, k[:, :cut], v[:, :cut], return_sums=True, A0=A0, B0=B0)
    s2 = wkv_backward_state_ref(w, u, k[:, cut:], v[:, cut:], gy[:, cut:], Am, Bm, gA, gB)
    s1 = wkv_backward_state_ref(w, u, k[:, :cut], v[:, :cut], gy[:, :cut], A0, B0, s2[4], s2[5])
    np.testing.assert_allclose(np.concatenate([s1[0], s2[0]], axis=1), whole[0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([s1[1], s2[1]], axis=1), whole[1], rtol=1e-11, atol=1e-13)
    for i in (2, 3):
        np.testing.assert_allclose(s1[i] + s2[i], whole[i], rtol=1e-11, atol=1e-13)
    for i in (4, 5):
        np.testing.assert_allclose(s1[i], whole[i], rtol=1e-11, atol=1e-13)


def test_stable_state_gradients_by_finite_differences():
    """The representation gradients (ga, gb, gp) of a segment started from a
    stable state (a, b, p), and the plain-sum gradient recovered from a
    gradient given at the representation of the handed-on state: both against
    central differences of the loss written in (a, b, p)."""
    B, T, C = 1, 5, 3
    w, u, k, v, gy, *_ = rand_case(B, T, C, seed=3)
    rng = np.random.default_rng(4)
    a = rng.normal(0, 1, (B, C))
    b = rng.uniform(0.5, 2.0, (B, C))
    p = rng.uniform(-2.0, 2.0, (B, C))
    # the next segment's gradient, given with respect to (a_T, b_T) at p_T
    ga_T = rng.normal(0, 1, (B, C))
    gb_T = rng.normal(0, 1, (B, C))
    p_T = rng.uniform(-1.0, 3.0, (B, C))
    gA, gB = wkv_sums_grads_from_state(ga_T, gb_T, p_T)

    def L(a_, b_, p_):
        A0, B0 = wkv_sums_from_state(a_, b_, p_)
        y, AT, BT = wkv_forward_ref(w, u, k, v, return_sums=True, A0=A0, B0=B0)
        # the loss in the handed-on state's representation at p_T
        return float(np.sum(gy * y) + np.sum(ga_T * AT * np.exp(-p_T)) + np.sum(gb_T * BT * np.exp(-p_T)))

    A0, B0 = wkv_sums_from_state(a, b, p)
    *_, dA0, dB0 = wkv_backward_state_ref(w, u, k, v, gy, A0, B0, gA, gB)
    ga, gb, gp = wkv_state_grads_from_sums(a, b, p, dA0, dB0)
    h = 1e-6
    for name, x, g in (("a", a, ga), ("b", b, gb), ("p", p, gp)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"a": a, "b": b, "p": p, name: xp}
            args_m = {"a": a, "b": b, "p": p, name: xm}
            fd[idx] = (L(args_p["a"], args_p["b"], args_p["p"]) - L(args_m["a"], args_m["b"], args_m["p"])) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_empty_state_has_no_gradient():
    """b <= 0 is the empty history whatever a and p hold: a constant, so its
    representation gradients are zero."""
    a = np.array([[0.0, 3.0, -1.0]])
    b = np.array([[0.0, 0.0, -2.0]])
    p = np.array([[-1e38, 5.0, 0.0]])
    ga, gb, gp = wkv_state_grads_from_sums(a, b, p, np.ones((1, 3)), np.ones((1, 3)))
    for g in (ga, gb, gp):
        np.testing.assert_array_equal(g, np.zeros((1, 3)))
