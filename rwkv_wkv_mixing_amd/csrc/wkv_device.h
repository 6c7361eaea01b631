// Device-side building blocks of the WKV kernels (gfx950).
//
// Lane recurrence ("RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型",
// sections "一句话总结" and "关键设计 2：WKV 算子"):
//     y_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t})
//     A_t = d A_{t-1} + e^{k_t} v_t,   B_t = d B_{t-1} + e^{k_t},  d = e^{-w}
//
// Representation used on chip.  The state of a lane is (a, b, s) with
// A = a * 2^s and B = b * 2^s: an INTEGER log2-scale s plus two float32
// mantissas ("the stability exponent" of section "关键设计 4", kept in base 2).
// Unlike a per-token running max, s only moves on a RESCALE, when a new key
// would exceed the scale by 2^32 or b leaves [2^-32, 2^32]; in between, the
// decay is applied to (a, b) as a product with d split into float32 hi + lo
// parts.  A per-token exponent update p <- p - w would round the same way at
// every token and act as a systematic error in w that grows with the memory
// length 1/w; the split product keeps the decay exact to ~2^-48 instead.
//
// Each key enters as e^k = em * 2^n with the integer n = rint(k log2 e) and
// em = 2^{k log2 e - n} in [2^-1/2, 2^1/2], a function of k alone.  Because s
// is an integer, moving a weight or a state to another scale is an exact
// ldexp: a token's weight carries the same float32 rounding in every pass and
// kernel that meets it, and joining states of different scales adds no
// rounding.  (A fractional scale would put the rounding of k log2 e - s, up
// to 2^-19 relative near |x| = 32, into every weight, differently in every
// pass; sums that cancel, such as the gradient at a dominant token, amplify
// such inconsistencies.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr float kL2E = 1.4426950408889634f;   // log2(e), rounded to float32
// log2(e) - kL2E: the float32 constant is 1.3e-8 relative short, which would
// put 5e-7 relative error into the weight of a key of 40; k log2 e is formed
// as fma(k, kL2E, k kL2E_lo) (exact to ~2^-24 of the product) wherever a key
// becomes a weight.
constexpr float kL2E_lo = 1.925963033500011e-08f;
constexpr float kLN2 = 0.6931471805599453f;   // ln(2)
constexpr float kHi = 0x1p32f;               // rescale bounds for b and new terms
constexpr float kLo = 0x1p-32f;
constexpr float kBig = 32.0f;                // log2(kHi)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float ldx(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

// ---- inputs: float32 or bfloat16 (raw bits), widened exactly to float32 ----
template <typename TIn>
struct Ld;

template <>
struct Ld<float> {
    static __device__ __forceinline__ float at(const float* p, int64_t i) { return p[i]; }
};

template <>
struct Ld<uint16_t> {
    static __device__ __forceinline__ float at(const uint16_t* p, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
    }
};

// ---- raw buffer access ----------------------------------------------------------
// A buffer resource covers [base, base + bytes); loads outside it return 0 and
// stores outside it are dropped by the hardware, so ragged tails need no
// branches, and a lane whose offset is kOffNone never touches memory.  The
// per-token offset is wave-uniform and lives in an SGPR (soffset).
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer descriptor
constexpr uint32_t kOffNone = 0x80000000u;   // voffset that is out of range for every buffer here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                             static_cast<int>(kRsrcWord3));
}

template <typename TIn>
struct BufLd;

template <>
struct BufLd<float> {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float at(Rsrc r, uint32_t voff, uint32_t soff) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
};

template <>
struct BufLd<uint16_t> {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float at(Rsrc r, uint32_t voff, uint32_t soff) {
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0)) << 16);
    }
};

// Output stores stream: nothing here reads them back, so they are marked
// non-temporal (sc0 nt) and do not displace the inputs and carries in L2.
#ifndef WKV_STORE_AUX
#define WKV_STORE_AUX 3
#endif

__device__ __forceinline__ void buf_store(float v, Rsrc r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, WKV_STORE_AUX);
}

// Cache policies of the buffer -> LDS copies of streamed inputs.  kStageKeep
// (the default policy) for inputs that a later call reads again: the inputs of
// a forward that saves states for its backward, which reads them next and finds
// part of them in the Infinity Cache.  kStageLast (non-temporal) for the last
// read of an input: the backwards' inputs and saved states, and the inputs of a
// forward that saves no states.  Measured at B=8 T=1024 C=4096 bf16,
// forward then backward over three rotated operand sets, builds interleaved in
// one process: backward 100.2 -> 94.8 us with its copies non-temporal; a
// non-temporal forward as well left that backward 107.5 us (the RWKV-5
// training step likewise: its backward 292 -> 304 us), so forwards keep the
// default although alone they run 2-7 % faster non-temporal.
constexpr int kStageKeep = 0;
constexpr int kStageLast = 2;

// Asynchronous copy of one input's L token rows x 64 channels (rows row0..
// of a buffer whose rows are C elements, channels c0..c0+63) into LDS laid out
// [L][64].  Each lane moves 16 bytes (buffer_load ... lds); one instruction
// fills 1 KB of LDS, and a lane's 16 bytes land at the instruction's LDS base
// + 16 * lane, which is exactly the [token][channel] order.  Chunks at or past
// channel C, or past the buffer's end, arrive as zeros.  Needs C * sizeof(TIn)
// to be a multiple of 16 (no chunk straddles C) and a 16-byte-aligned buffer.
// The copy is tracked by vmcnt only, not by the compiler: its consumer waits
// explicitly before reading the LDS rows.
template <typename TIn, int L, int Aux>
__device__ __forceinline__ void stage_rows(Rsrc r, TIn (*dst)[64], int64_t row0, int64_t c0, int64_t C, int lane) {
    constexpr int ES = sizeof(TIn);
    constexpr int LPR = 64 * ES / 16;  // lanes per row
    constexpr int RPI = 64 / LPR;      // rows per instruction
    static_assert(L % RPI == 0, "whole instructions of rows");
    const int q = lane % LPR;
    const bool ok = c0 + q * (16 / ES) < C;
#pragma unroll
    for (int i = 0; i < L / RPI; ++i) {
        const int64_t j = row0 + i * RPI + lane / LPR;
        const uint32_t voff = ok ? static_cast<uint32_t>((j * C + c0) * ES + q * 16) : kOffNone;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&dst[i * RPI][0], 16, voff,
                                                 0, 0, Aux);
    }
}

// Waits on this wave's outstanding copies and loads (before reading staged
// rows), and on its LDS reads (before a copy may overwrite them).  As asm
// statements they also keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wait_staged() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same where at least N vector memory instructions were issued after the copies: the counter
// drops in issue order, so this waits for the copies without waiting for the N later ones (the
// previous block's output stores) to complete.
template <int N>
__device__ __forceinline__ void wait_staged_before() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One input over L tokens of a lane (token j at soffset j * row), held in
// registers: bf16 values two to a register, float32 values one each.
template <typename TIn, int L>
struct Chunk1;

template <int L>
struct Chunk1<uint16_t, L> {
    uint32_t pk[(L + 1) / 2];
    __device__ __forceinline__ void load(Rsrc r, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; j += 2) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff, j * row, 0);
            const uint32_t hi = j + 1 < L ? __builtin_amdgcn_raw_buffer_load_b16(r, voff, (j + 1) * row, 0) : 0u;
            pk[j / 2] = lo | (hi << 16);
        }
    }
    // from a [L][64] block staged in LDS, lane = channel
    __device__ __forceinline__ void load_lds(const uint16_t (*x)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; j += 2) {
            const uint32_t lo = x[j][lane];
            const uint32_t hi = j + 1 < L ? static_cast<uint32_t>(x[j + 1][lane]) : 0u;
            pk[j / 2] = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ float at(int j) const {
        return (j & 1) ? __uint_as_float(pk[j / 2] & 0xffff0000u) : __uint_as_float(pk[j / 2] << 16);
    }
};

template <int L>
struct Chunk1<float, L> {
    float x[L];
    __device__ __forceinline__ void load(Rsrc r, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; ++j) x[j] = BufLd<float>::at(r, voff, j * row);
    }
    __device__ __forceinline__ void load_lds(const float (*s)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; ++j) x[j] = s[j][lane];
    }
    __device__ __forceinline__ float at(int j) const { return x[j]; }
};

// Receptance gate ("RWKV（Receptance Weighted Key Value）概念", section 3.2:
// out = sigmoid(r) wkv).  t = e^{-r}; sigmoid(r) = 1/(1+t) and
// 1 - sigmoid(r) = t/(1+t), formed without cancellation on either side.
struct Gate {
    float s, om;  // sigmoid(r), 1 - sigmoid(r)
};

__device__ __forceinline__ Gate gate_of(float r) {
    const float t = ex2(-r * kL2E);
    const float s = rcp(1.f + t);
    return Gate{s, t > 1.f ? 1.f - s : t * s};
}

// ---- per-channel constants -------------------------------------------------
struct Chan {
    double dd;       // e^{-w}
    float dhi, dlo;  // e^{-w} = dhi + dlo (to ~2^-48 relative)
    float u2;        // u * log2(e)
};

__device__ __forceinline__ Chan make_chan(float w, float u) {
    Chan ch;
    ch.dd = exp(-static_cast<double>(w));
    ch.dhi = static_cast<float>(ch.dd);
    ch.dlo = static_cast<float>(ch.dd - static_cast<double>(ch.dhi));
    ch.u2 = fmaf(u, kL2E, u * kL2E_lo);
    return ch;
}

// x^N by repeated squaring (N a compile-time count: a few float64 multiplies
// instead of another exp; relative error ~N 2^-53).
template <int N>
__device__ __forceinline__ double ipow(double x) {
    double r = 1.0;
#pragma unroll
    for (int n = N; n > 0; n >>= 1) {
        if (n & 1) r *= x;
        x *= x;
    }
    return r;
}

// ---- keys -----------------------------------------------------------------------
constexpr float kNMax = 4194304.0f;  // |n| clamp (2^22): keys beyond |k| ~ 2.9e6 saturate

struct Key {
    float em;  // 2^f, f = k log2 e - n
    float f;
    int n;
};

__device__ __forceinline__ Key key_split(float k) {
    const float n = __builtin_amdgcn_fmed3f(__builtin_rintf(k * kL2E), -kNMax, kNMax);
    const float f = fmaf(k, kL2E_lo, fmaf(k, kL2E, -n));
    return Key{ex2(f), f, static_cast<int>(n)};
}

// The same split for a key already known to satisfy |k log2 e| < kNMax.
__device__ __forceinline__ Key key_split_bounded(float k) {
    const float n = __builtin_rintf(k * kL2E);
    const float f = fmaf(k, kL2E_lo, fmaf(k, kL2E, -n));
    return Key{ex2(f), f, static_cast<int>(n)};
}

// ---- lane state ---------------------------------------------------------------
constexpr int kSEmpty = -(1 << 29);  // scale of the empty state (a = b = 0)
// Fixed-scale paths hold every denominator they divide by at or above this
// (relative to their scale); a wave where one falls below redoes its work on
// the general path.  Terms that underflow next to such a denominator are
// below float32 resolution anyway.
constexpr float kTiny = 0x1p-100f;

struct St {
    float a, b;  // A = a 2^s, B = b 2^s
    int s;
};

__device__ __forceinline__ St empty_state() { return St{0.f, 0.f, kSEmpty}; }

// Move the scale to s' = max(n, s + E(b)), b < 2^E(b): afterwards b < 1 and
// the new weight em 2^(n - s') <= 2^1/2.  Exact (powers of two).
__device__ __forceinline__ void rescale(St& st, int n) {
    const int lvl = st.b > 0.f ? st.s + __builtin_amdgcn_frexp_expf(st.b) : kSEmpty;
    const int sn = max(lvl, n);
    st.a = ldx(st.a, st.s - sn);
    st.b = ldx(st.b, st.s - sn);
    st.s = sn;
}

// Rescale first when the new weight or b is out of range; the three
// conditions are folded into one mask so the rare rescale costs a single
// branch per token.  Returns the weight e = e^k / 2^s.
__device__ __forceinline__ float key_weight(St& st, const Key& kk) {
    const bool out = (kk.n - st.s > static_cast<int>(kBig)) | !(st.b >= kLo) | (st.b > kHi);
    if (__builtin_expect(out, 0)) rescale(st, kk.n);
    return ldx(kk.em, kk.n - st.s);
}

// log2 of the weight relative to 2^s (rounded; used only to normalise outputs).
__device__ __forceinline__ float key_log2(const St& st, const Key& kk) {
    return static_cast<float>(kk.n - st.s) + kk.f;
}

// Output of one token from the state before it (robust to any u):
// z = x + u2 is the log2 weight of the current token relative to 2^s.
struct Out {
    float y;
    float co;  // weight of the history in the normalised fraction (<= 1)
    float cn;  // weight of the current token (<= 1)
    float r;   // 1 / (b co + cn)
};

__device__ __forceinline__ Out token_out(const St& st, float x, float v, const Chan& ch) {
    const float z = x + ch.u2;
    const float ez = ex2(-fabsf(z));
    const bool zp = z > 0.f;
    Out o;
    o.co = zp ? ez : 1.f;
    o.cn = zp ? 1.f : ez;
    const float D = fmaf(st.b, o.co, o.cn);
    const float N = fmaf(st.a, o.co, o.cn * v);
    o.r = rcp(D);
    o.y = N * o.r;
    return o;
}

// Output of one token when |u| is small enough that the current-token weight
// e^{u} e cannot overflow (|u| <= kFastU with e <= 2^32): one multiply instead
// of the normalised two-branch form.
constexpr float kFastU = 40.0f;

__device__ __forceinline__ float token_out_fast(const St& st, float e, float v, float eu) {
    const float E = e * eu;
    return fmaf(E, v, st.a) * rcp(st.b + E);
}

// Decay-and-add of one token with weight e: A <- d A + e v, B <- d B + e, d = dhi + dlo.
__device__ __forceinline__ void token_add(St& st, float e, float v, const Chan& ch) {
    const float ev = e * v;
    st.a = fmaf(ch.dhi, st.a, fmaf(ch.dlo, st.a, ev));
    st.b = fmaf(ch.dhi, st.b, fmaf(ch.dlo, st.b, e));
}

}  // namespace wkv
