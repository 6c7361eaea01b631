"""The RWKV-5/6 forward and backward parity tests would catch plausible kernel
mistakes (CPU).  Each mistake is planted in a copy of the backward recurrence written
here (never in the product path); the copy's outputs are held to exactly the
criteria the GPU tests apply to the kernel: the per-element rounding bound and
the normwise check.  Every planted mistake must fail at least one of them,
and the unaltered copy must pass both."""
import numpy as np
import pytest
import torch  # CPU tensors only: the GPU tests' forward check() reads its inputs back with .cpu()

import test_gpu_wkv5 as F5
import test_gpu_wkv5_bwd as G5
import test_gpu_wkv6 as F6
import test_gpu_wkv6_bwd as G6
from oracle import wkv5_backward_ref, wkv6_backward_ref
from rwkv_wkv_mixing_amd import workloads as W

KINDS = ["dk_no_bonus", "dv_no_bonus", "dr_reads_S_after", "dk_G_transposed", "du_without_k", "dw_sign",
         "dw_no_decay_factor", "dw_reads_S_after", "dw_reads_G_before", "G_decayed_twice", "G_previous_rate"]


def backward_copy(wt, u, r, k, v, go, H, S0, dST, kind):
    """The adjoint recurrence with per-token rates wt [B, T, C] and, unless kind
    is None, one planted mistake.  Returns (dr, dk, dv, dw per token, du, dS0)."""
    hd = lambda x: np.asarray(x, np.float64).reshape(x.shape[0], x.shape[1], H, -1)
    wt, r, k, v, go = (hd(x) for x in (wt, r, k, v, go))
    B, T, _, N = r.shape
    u = np.asarray(u, np.float64).reshape(H, N)
    d = np.exp(-wt)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, np.float64).reshape(B, H, N, N)
    prev, after = np.empty((T, B, H, N, N)), np.empty((T, B, H, N, N))
    for t in range(T):
        prev[t] = S
        S = d[:, t, :, :, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
        after[t] = S
    Gs = np.zeros((B, H, N, N)) if dST is None else np.array(dST, np.float64).reshape(B, H, N, N)
    dr, dk, dv, dw = (np.empty((B, T, H, N)) for _ in range(4))
    du = np.zeros((H, N))
    for t in range(T - 1, -1, -1):
        vg = np.einsum("bhj,bhj->bh", v[:, t], go[:, t])
        bonus = np.einsum("bhi,hi,bhi->bh", r[:, t], u, k[:, t])
        Sr = after[t] if kind == "dr_reads_S_after" else prev[t]
        dr[:, t] = np.einsum("bhij,bhj->bhi", Sr, go[:, t]) + u[None] * k[:, t] * vg[..., None]
        Gk = np.swapaxes(Gs, -1, -2) if kind == "dk_G_transposed" else Gs
        dk[:, t] = np.einsum("bhij,bhj->bhi", Gk, v[:, t])
        if kind != "dk_no_bonus":
            dk[:, t] += u[None] * r[:, t] * vg[..., None]
        dv[:, t] = np.einsum("bhi,bhij->bhj", k[:, t], Gs)
        if kind != "dv_no_bonus":
            dv[:, t] += bonus[..., None] * go[:, t]
        du += np.einsum("bhi,bhi,bh->hi", r[:, t], np.ones_like(k[:, t]) if kind == "du_without_k" else k[:, t], vg)
        Gn = d[:, t, :, :, None] * Gs + r[:, t, :, :, None] * go[:, t, :, None, :]
        Sw = after[t] if kind == "dw_reads_S_after" else prev[t]
        Gw = Gn if kind == "dw_reads_G_before" else Gs
        fac = 1.0 if kind == "dw_no_decay_factor" else d[:, t]
        dw[:, t] = (1.0 if kind == "dw_sign" else -1.0) * fac * np.einsum("bhij,bhij->bhi", Gw, Sw)
        if kind == "G_decayed_twice":
            Gn = d[:, t, :, :, None] * (d[:, t, :, :, None] * Gs) + r[:, t, :, :, None] * go[:, t, :, None, :]
        if kind == "G_previous_rate" and t > 0:
            Gn = d[:, t - 1, :, :, None] * Gs + r[:, t, :, :, None] * go[:, t, :, None, :]
        Gs = Gn
    C = H * N
    return dr.reshape(B, T, C), dk.reshape(B, T, C), dv.reshape(B, T, C), dw.reshape(B, T, C), du, Gs


def caught(got, ref, bnd):
    """Whether the GPU tests' criteria reject these outputs: the worst
    element-to-bound ratio and the worst normwise relative error."""
    ratio = max(float((np.abs(np.asarray(g) - r) / (b + 1e-30)).max()) for g, r, b in zip(got, ref, bnd))
    norm = max(float(np.linalg.norm(np.asarray(g) - r) / max(np.linalg.norm(r), 1e-300)) for g, r in zip(got, ref))
    return ratio, norm


def case(gen):
    if gen == 5:
        p = W.make_wkv5(2, 130, 1, seed=51, with_state=True)
        wt = np.broadcast_to(p.w.reshape(1, 1, -1), (p.B, p.T, p.H * 64)).astype(np.float64)
    else:
        p = W.make_wkv6(2, 130, 1, seed=52, with_state=True)
        p.w[:] = np.minimum(p.w, 10.0)  # the operator the kernel computes
        wt = p.w.astype(np.float64)
    go = W.wkv5_go(p, seed=53)[1]
    dST = np.random.default_rng(54).standard_normal((p.B, p.H, 64, 64))
    return p, wt, go, dST


def reference_and_bounds(gen, p, wt, go, dST):
    if gen == 5:
        ref = wkv5_backward_ref(p.w, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
        bnd = G5.bounds(p.w.astype(np.float64), p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
    else:
        ref = wkv6_backward_ref(wt, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
        bnd = G6.bounds(wt, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST)
    return ref, bnd


def as_gen(gen, out):
    """RWKV-5's dw is summed over batch rows and tokens, [H, 64]."""
    dr, dk, dv, dw, du, ds = out
    if gen == 5:
        dw = dw.sum(axis=(0, 1)).reshape(du.shape)
    return dr, dk, dv, dw, du, ds


@pytest.mark.parametrize("gen", [5, 6])
def test_unaltered_copy_passes(gen):
    p, wt, go, dST = case(gen)
    ref, bnd = reference_and_bounds(gen, p, wt, go, dST)
    ratio, norm = caught(as_gen(gen, backward_copy(wt, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST, None)), ref, bnd)
    assert ratio < 1e-6 and norm < 1e-9, (ratio, norm)


# a per-token rate taken from the previous token is no mistake at RWKV-5's constant rates
CASES = [(g, k) for g in (5, 6) for k in KINDS if not (g == 5 and k == "G_previous_rate")]


@pytest.mark.parametrize("gen,kind", CASES)
def test_planted_mistake_is_caught(gen, kind):
    p, wt, go, dST = case(gen)
    ref, bnd = reference_and_bounds(gen, p, wt, go, dST)
    ratio, norm = caught(as_gen(gen, backward_copy(wt, p.u, p.r, p.k, p.v, go, p.H, p.S0, dST, kind)), ref, bnd)
    print(f"RWKV-{gen} {kind}: worst error / bound {ratio:.3g}, normwise {norm:.3g}", flush=True)
    assert ratio > 1.0 or norm > G6.NORM_TOL, (kind, ratio, norm)


# ---- the forwards ---------------------------------------------------------------------------

FWD_KINDS = ["no_bonus", "decay_before_read", "state_transposed", "bonus_without_u", "previous_rate"]


def forward_copy(wt, u, r, k, v, H, S0, kind):
    """The forward recurrence with per-token rates wt [B, T, C] and, unless kind
    is None, one planted mistake.  Returns (o [B, T, C], S_T)."""
    hd = lambda x: np.asarray(x, np.float64).reshape(x.shape[0], x.shape[1], H, -1)
    wt, r, k, v = (hd(x) for x in (wt, r, k, v))
    B, T, _, N = r.shape
    u = np.asarray(u, np.float64).reshape(H, N)
    d = np.exp(-wt)
    S = np.zeros((B, H, N, N)) if S0 is None else np.array(S0, np.float64).reshape(B, H, N, N)
    o = np.empty((B, T, H, N))
    for t in range(T):
        kv = k[:, t, :, :, None] * v[:, t, :, None, :]
        dt = d[:, t - 1] if (kind == "previous_rate" and t > 0) else d[:, t]
        if kind == "decay_before_read":
            S = dt[..., None] * S
        read = np.swapaxes(S, -1, -2) if kind == "state_transposed" else S
        uu = np.ones_like(u) if kind == "bonus_without_u" else u
        cur = 0.0 if kind == "no_bonus" else uu[None, :, :, None] * kv
        o[:, t] = np.einsum("bhi,bhij->bhj", r[:, t], read + cur)
        S = (S if kind == "decay_before_read" else dt[..., None] * S) + kv
    return o.reshape(B, T, H * N), S


def fwd_case(gen):
    if gen == 5:
        p = W.make_wkv5(2, 130, 1, seed=61, with_state=True)
        wt = np.broadcast_to(p.w.reshape(1, 1, -1), (p.B, p.T, p.H * 64)).astype(np.float64)
    else:
        p = W.make_wkv6(2, 130, 1, seed=62, with_state=True)
        p.w[:] = np.minimum(p.w, 10.0)
        wt = p.w.astype(np.float64)
    return p, wt


def fwd_check(gen, p, o, S):
    (F5 if gen == 5 else F6).check(p, torch.from_numpy(o), torch.from_numpy(S), name=f"RWKV-{gen} planted")


@pytest.mark.parametrize("gen", [5, 6])
def test_unaltered_forward_copy_passes(gen):
    p, wt = fwd_case(gen)
    fwd_check(gen, p, *forward_copy(wt, p.u, p.r, p.k, p.v, p.H, p.S0, None))


FWD_CASES = [(g, k) for g in (5, 6) for k in FWD_KINDS if not (g == 5 and k == "previous_rate")]


@pytest.mark.parametrize("gen,kind", FWD_CASES)
def test_planted_forward_mistake_is_caught(gen, kind):
    p, wt = fwd_case(gen)
    o, S = forward_copy(wt, p.u, p.r, p.k, p.v, p.H, p.S0, kind)
    with pytest.raises(AssertionError):
        fwd_check(gen, p, o, S)
