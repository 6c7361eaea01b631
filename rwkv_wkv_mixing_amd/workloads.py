"""Seeded synthetic inputs shaped like the RWKV-4 models on the pages.

This module holds only input generation (random draws, bf16 rounding, shapes):
none of the operator's arithmetic.  Tests feed the same arrays to the float64
oracle and to the HIP path, and the oracle never imports this module.

Shapes follow the model table of "RWKV - 把 RNN 重新带回 Transformer 时代的线性
大模型", section "实验关键数据" (169M: 12 layers x 768; 7B: 32 layers x 4096).
No public dataset underlies these workloads; all values are synthetic.

Draw conventions (one ``numpy.random.default_rng(seed)`` stream per workload,
seed 0 unless a test says otherwise):

* ``N(m, s)`` means mean m and *standard deviation* s;
* draw order: w, u, k, v, spikes, gy (then decode-prefix inputs);
* w_c = exp(U(lo, hi)) is drawn in float64 and rounded to float32;
* spikes: an independent Bernoulli(0.01) mask per k entry, sign +-1 with equal
  probability, magnitude U(20, 40), applied before bf16 rounding;
* float64 -> float32 and float32 -> bf16 both round to nearest even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32 = "f32"
BF16 = "bf16"


def bf16_round(x) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bfloat16 (nearest even).

    Returns (bits as uint16, the same values widened back to float32)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    hi = ((u + bias) >> np.uint64(16)).astype(np.uint16)
    vals = (hi.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return hi, vals


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class WkvProblem:
    """One forward(+backward) workload.

    ``k, v, gy`` are float32 arrays holding the exact values both sides
    consume; when ``dtype == "bf16"`` the ``*_bits`` arrays hold the bf16
    encodings handed to the GPU.  ``gy`` is None for forward-only workloads.
    """

    name: str
    B: int
    T: int
    C: int
    dtype: str
    w: np.ndarray
    u: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gy: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    gy_bits: np.ndarray | None = None
    note: str = ""
    seed: int = 0

    @property
    def n(self) -> int:
        return self.B * self.T * self.C

    def device_inputs(self, name: str) -> np.ndarray:
        """Array to upload for input ``name`` in the GPU input dtype."""
        if self.dtype == BF16:
            return getattr(self, name + "_bits")
        return getattr(self, name)


def _finish(p: WkvProblem) -> WkvProblem:
    if p.dtype == BF16:
        p.k_bits, p.k = bf16_round(p.k)
        p.v_bits, p.v = bf16_round(p.v)
        if p.gy is not None:
            p.gy_bits, p.gy = bf16_round(p.gy)
    else:
        p.k = np.ascontiguousarray(p.k, dtype=np.float32)
        p.v = np.ascontiguousarray(p.v, dtype=np.float32)
        if p.gy is not None:
            p.gy = np.ascontiguousarray(p.gy, dtype=np.float32)
    p.w = np.ascontiguousarray(p.w, dtype=np.float32)
    p.u = np.ascontiguousarray(p.u, dtype=np.float32)
    return p


def _normal(rng, std, shape):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def make_problem(B, T, C, *, dtype=F32, seed=0, w_range=(-6.0, 1.5), u_std=1.0,
                 k_std=1.0, v_std=1.0, spike_frac=0.0, spike_range=(20.0, 40.0),
                 with_gy=True, name="custom", note="") -> WkvProblem:
    """General generator in the fixed draw order w, u, k, v, spikes, gy."""
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_range[0], w_range[1], C)).astype(np.float32)
    u = _normal(rng, u_std, C)
    k = _normal(rng, k_std, (B, T, C))
    v = _normal(rng, v_std, (B, T, C))
    if spike_frac > 0.0:
        mask = rng.random((B, T, C)) < spike_frac
        n = int(mask.sum())
        sign = rng.integers(0, 2, n).astype(np.float32) * 2.0 - 1.0
        mag = rng.uniform(spike_range[0], spike_range[1], n).astype(np.float32)
        k[mask] = sign * mag
    gy = _normal(rng, 1.0, (B, T, C)) if with_gy else None
    return _finish(WkvProblem(name, B, T, C, dtype, w, u, k, v, gy, note=note, seed=seed))


# --- the five workloads -----------------------------------------------------

def config1(seed=0) -> WkvProblem:
    """B=1, T=64, C=8, fp32; w = exp(U(-3,2)), u ~ N(0,0.5), k, v, gy ~ N(0,1)."""
    return make_problem(1, 64, 8, dtype=F32, seed=seed, w_range=(-3.0, 2.0), u_std=0.5,
                        name="wkv4 fp32 B=1 T=64 C=8")


def config2(seed=0) -> WkvProblem:
    """169M-model shape: B=8, T=1024, C=768, fp32; w = exp(U(-6,1.5)), u, k, v, gy ~ N(0,1)."""
    return make_problem(8, 1024, 768, dtype=F32, seed=seed, w_range=(-6.0, 1.5),
                        name="wkv4 fp32 B=8 T=1024 C=768")


def receptance(p: WkvProblem, std: float = 2.0):
    """Receptance r [B, T, C] for the gated operator: N(0, std) from its own
    stream (seed, 2), so the other inputs of ``p`` are unchanged; rounded like
    the problem's inputs.  Returns (r as float32 values, bf16 bits or None)."""
    rng = np.random.default_rng([p.seed, 2])
    r = _normal(rng, std, (p.B, p.T, p.C))
    if p.dtype == BF16:
        bits, r = bf16_round(r)
        return r, bits
    return r, None


def config3(seed=0) -> WkvProblem:
    """7B-model shape: B=8, T=1024, C=4096; bf16 k, v, gy; 1% of k set to +-U(20,40)."""
    return make_problem(8, 1024, 4096, dtype=BF16, seed=seed, w_range=(-6.0, 1.5),
                        spike_frac=0.01, name="wkv4 bf16 B=8 T=1024 C=4096")


def config4(seed=0) -> WkvProblem:
    """Long context: B=1, T=32768, C=4096, fp32; w = exp(U(-8,1)), k ~ N(0,2), forward only."""
    return make_problem(1, 32768, 4096, dtype=F32, seed=seed, w_range=(-8.0, 1.0), k_std=2.0,
                        with_gy=False, name="wkv4 fp32 B=1 T=32768 C=4096")


def large_bf16_torch(B, T, C, *, seed=0, w_range=(-6.0, 1.5), spike_frac=0.01, spike_range=(20.0, 40.0),
                     device="cuda:0"):
    """The bf16 workload's distributions (config 3: w = exp(U(lo, hi)), u, k, v, gy ~ N(0, 1), a
    fraction of k set to +-U(20, 40)) at sizes too large to draw on the host: w, u [C] float32 from
    numpy's generator (as make_problem), k, v, gy [B, T, C] bf16 drawn on ``device`` with torch's
    seeded Philox generator, spikes applied before the bf16 rounding.  Deterministic per seed."""
    import torch

    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(w_range[0], w_range[1], C)).astype(np.float32)
    u = _normal(rng, 1.0, C)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 17)
    out = []
    for name in ("k", "v", "gy"):
        x = torch.randn((B, T, C), generator=g, device=device, dtype=torch.float32)
        if name == "k" and spike_frac > 0.0:
            mask = torch.rand((B, T, C), generator=g, device=device) < spike_frac
            mag = torch.empty((B, T, C), device=device).uniform_(spike_range[0], spike_range[1], generator=g)
            sign = torch.where(torch.rand((B, T, C), generator=g, device=device) < 0.5, -1.0, 1.0)
            x = torch.where(mask, sign * mag, x)
            del mask, mag, sign
        out.append(x.to(torch.bfloat16))
        del x
    return w, u, out[0], out[1], out[2]


@dataclass
class DecodeProblem:
    """Recurrent-mode workload: L layers x B streams x C channels.

    Per-layer w, u are [L, C].  The state-seeding prefix k, v are [B, Tp, C]
    per stream and shared by all layers (each layer still gets its own state
    because w, u differ per layer).  Per-step inputs are drawn on demand by
    ``step_inputs``.
    """

    L: int
    B: int
    C: int
    Tp: int
    w: np.ndarray
    u: np.ndarray
    pk: np.ndarray
    pv: np.ndarray
    seed: int = 0
    extra: dict = field(default_factory=dict)


def make_decode(L, B, C, Tp, seed=0) -> DecodeProblem:
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-6.0, 1.5, (L, C))).astype(np.float32)
    u = _normal(rng, 1.0, (L, C))
    pk = np.empty((B, Tp, C), np.float32)
    pv = np.empty((B, Tp, C), np.float32)
    for b in range(B):  # per stream, to bound temporaries
        pk[b] = rng.standard_normal((Tp, C), dtype=np.float32)
    for b in range(B):
        pv[b] = rng.standard_normal((Tp, C), dtype=np.float32)
    _, pk = bf16_round(pk)
    _, pv = bf16_round(pv)
    return DecodeProblem(L, B, C, Tp, w, u, pk, pv, seed)


def config5(seed=0) -> DecodeProblem:
    """256 streams x 32 layers, C=4096; prefix T=512 of bf16 k, v ~ N(0,1)."""
    return make_decode(32, 256, 4096, 512, seed)


def step_inputs_numpy(dp: DecodeProblem, step: int):
    """Per-step bf16 k, v [L, B, C] drawn with numpy (small decode problems)."""
    rng = np.random.default_rng([dp.seed, 1, step])
    k = rng.standard_normal((dp.L, dp.B, dp.C), dtype=np.float32)
    v = rng.standard_normal((dp.L, dp.B, dp.C), dtype=np.float32)
    kb, kf = bf16_round(k)
    vb, vf = bf16_round(v)
    return kb, vb, kf, vf


def step_inputs_torch(dp: DecodeProblem, step: int, device):
    """Per-step bf16 k, v [L, B, C] drawn on ``device`` with torch's seeded
    Philox generator (the full decode workload is too large to draw on the
    host: 1000 steps x 2 x 33.5M values).  Deterministic per (seed, step)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(dp.seed) * 1_000_003 + 7919 * int(step) + 1)
    k = torch.randn((dp.L, dp.B, dp.C), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((dp.L, dp.B, dp.C), generator=g, device=device, dtype=torch.float32)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


@dataclass
class ShiftProblem:
    """Inputs of the token-shift mix: mu [M, C] float32, x [B, T, C], x_prev
    [B, C] (or None), gout [M, B, T, C].  As for WkvProblem, the float32
    arrays hold the exact values both sides consume and ``*_bits`` the bf16
    encodings handed to the GPU."""

    name: str
    B: int
    T: int
    C: int
    M: int
    dtype: str
    mu: np.ndarray
    x: np.ndarray
    x_prev: np.ndarray | None
    gout: np.ndarray
    x_bits: np.ndarray | None = None
    x_prev_bits: np.ndarray | None = None
    gout_bits: np.ndarray | None = None

    def device_inputs(self, name: str) -> np.ndarray:
        if self.dtype == BF16:
            return getattr(self, name + "_bits")
        return getattr(self, name)


def make_shift(B, T, C, M, *, dtype=BF16, seed=0, with_prev=True, name="") -> ShiftProblem:
    """Draw order: mu ~ U(0, 1) (the mixing ratios of the pages lie between
    the two tokens), x ~ N(0, 1), x_prev ~ N(0, 1) (always drawn, dropped when
    not wanted), gout ~ N(0, 1); then bf16 rounding of x, x_prev, gout."""
    rng = np.random.default_rng(seed)
    mu = rng.uniform(0.0, 1.0, (M, C)).astype(np.float32)
    x = _normal(rng, 1.0, (B, T, C))
    xp = _normal(rng, 1.0, (B, C))
    g = _normal(rng, 1.0, (M, B, T, C))
    p = ShiftProblem(name or f"shift {dtype} B={B} T={T} C={C} M={M}", B, T, C, M, dtype, mu, x,
                     xp if with_prev else None, g)
    if dtype == BF16:
        p.x_bits, p.x = bf16_round(x)
        p.gout_bits, p.gout = bf16_round(g)
        if with_prev:
            p.x_prev_bits, p.x_prev = bf16_round(xp)
    return p


def shift_config(seed=0) -> ShiftProblem:
    """The three time-mixing mixes (r, k, v) of a 7B-shaped layer at the bf16
    training workload's size: B=8, T=1024, C=4096."""
    return make_shift(8, 1024, 4096, 3, dtype=BF16, seed=seed, with_prev=False,
                      name="token shift bf16 B=8 T=1024 C=4096 M=3")


@dataclass
class Wkv5Problem:
    """Inputs of the RWKV-5 matrix-state WKV: w, u [H, 64] float32, r, k, v
    [B, T, 64 H] (float32 values exactly representable in bf16, with their
    bf16 encodings in ``*_bits``), optional state S0 [B, H, 64, 64]."""

    name: str
    B: int
    T: int
    H: int
    w: np.ndarray
    u: np.ndarray
    r: np.ndarray
    k: np.ndarray
    v: np.ndarray
    r_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    S0: np.ndarray | None = None


def make_wkv5(B, T, H, *, seed=0, w_range=(-4.0, 1.5), kv_std=1.0, with_state=False, name="") -> Wkv5Problem:
    """Draw order: w = exp(U(lo, hi)) per (head, key channel), u ~ N(0, 1),
    r, k, v ~ N(0, kv_std) rounded to bf16, then (if wanted) S0 ~ N(0, 1).
    The rate range gives decay factors from e^{-e^{1.5}} = 0.011 to
    e^{-e^{-4}} = 0.98 per token."""
    rng = np.random.default_rng(seed)
    N = 64
    w = np.exp(rng.uniform(w_range[0], w_range[1], (H, N))).astype(np.float32)
    u = _normal(rng, 1.0, (H, N))
    r_bits, r = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    k_bits, k = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    v_bits, v = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    S0 = _normal(rng, 1.0, (B, H, N, N)) if with_state else None
    return Wkv5Problem(name or f"wkv5 B={B} T={T} H={H}", B, T, H, w, u, r, k, v, r_bits, k_bits, v_bits, S0)


def make_wkv6(B, T, H, *, seed=0, base_range=(-4.0, 1.5), spread=0.5, kv_std=1.0, with_state=False,
              name="") -> Wkv5Problem:
    """Inputs of the RWKV-6 operator (a Wkv5Problem whose w is [B, T, 64 H]).
    Draw order: a base log-rate per (head, key channel) ~ U(lo, hi), then
    per-token rates w = exp(base + spread * N(0, 1)) (data-dependent decay
    around each channel's base), u ~ N(0, 1), r, k, v ~ N(0, kv_std) rounded to
    bf16, then (if wanted) S0 ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    N = 64
    base = rng.uniform(base_range[0], base_range[1], (H * N,))
    w = np.exp(base[None, None, :] + spread * rng.standard_normal((B, T, H * N))).astype(np.float32)
    u = _normal(rng, 1.0, (H, N))
    r_bits, r = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    k_bits, k = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    v_bits, v = bf16_round(_normal(rng, kv_std, (B, T, H * N)))
    S0 = _normal(rng, 1.0, (B, H, N, N)) if with_state else None
    return Wkv5Problem(name or f"wkv6 B={B} T={T} H={H}", B, T, H, w, u, r, k, v, r_bits, k_bits, v_bits, S0)


def wkv6_config(seed=0) -> Wkv5Problem:
    """A 7B-shaped layer in RWKV-6 form: B=8, T=1024, C=4096 as 64 heads of 64."""
    return make_wkv6(8, 1024, 64, seed=seed, name="wkv6 bf16 B=8 T=1024 H=64 N=64")


def wkv5_go(p: Wkv5Problem, *, seed=1, std=1.0) -> tuple[np.ndarray, np.ndarray]:
    """A gradient of the output for a Wkv5Problem: go ~ N(0, std) of shape
    [B, T, 64 H], rounded to bf16.  Returns (bits as uint16, values as float32)."""
    rng = np.random.default_rng(seed)
    return bf16_round(_normal(rng, std, (p.B, p.T, p.H * 64)))


def large_matrix_torch(gen, B, T, H, *, seed=0, rate_range=(-4.0, 1.5), spread=0.5, device="cuda:0"):
    """make_wkv5 (gen 5) or make_wkv6 (gen 6) inputs, with go ~ N(0, 1), at sizes too large to draw
    on the host.  Host (numpy, as those generators): the log-rates per (head, key channel) ~ U(lo,
    hi) (gen 5: w = their exp, [H, 64]; gen 6: the per-channel base) and u ~ N(0, 1) [H, 64].
    Device (torch's seeded Philox generator): r, k, v, go ~ N(0, 1) [B, T, 64 H] rounded to bf16,
    and for gen 6 the per-token rates w = exp(base + spread N(0, 1)) [B, T, 64 H] float32.
    Returns (w, u, r, k, v, go, base) with w a numpy array (gen 5) or a device tensor (gen 6) and
    base the gen-6 log-rates (None for gen 5)."""
    import torch

    rng = np.random.default_rng(seed)
    N = 64
    lw = rng.uniform(rate_range[0], rate_range[1], (H, N))
    u = _normal(rng, 1.0, (H, N))
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + 29)
    shape = (B, T, H * N)
    r, k, v, go = (torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    if gen == 5:
        return np.exp(lw).astype(np.float32), u, r, k, v, go, None
    base = torch.from_numpy(lw.reshape(-1)).to(device=device, dtype=torch.float32)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(spread).add_(base).exp_()
    return w, u, r, k, v, go, lw.reshape(-1)


def wkv5_config(seed=0) -> Wkv5Problem:
    """A 7B-shaped layer in RWKV-5 form: B=8, T=1024, C=4096 as 64 heads of 64."""
    return make_wkv5(8, 1024, 64, seed=seed, name="wkv5 bf16 B=8 T=1024 H=64 N=64")
