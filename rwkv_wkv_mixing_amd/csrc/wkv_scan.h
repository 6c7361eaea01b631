// Chunk-level combine of WKV states and the decoupled look-back protocol that
// passes carries between workgroups along time.
//
// Chunkwise-parallel execution ("RWKV模型深度研究报告", section 1.4.1: split the
// sequence into chunks, compute inside each chunk in parallel, pass state
// between chunks; "RWKV（Receptance Weighted Key Value）概念", section 3.4:
// parallel prefix scan).  A chunk of n tokens run from the empty state yields a
// summary S with  state_after = d^n * state_before + S  (the recurrence is a
// first-order linear one with a constant coefficient, so this map is
// associative).
#pragma once

#include "wkv_device.h"

namespace wkv {

// Combine a state X (at the start of an n-token interval) with the summary S
// of that interval; D = d^n in double, applied as a float32 hi + lo product.
// The result keeps X's scale unless the summary would not fit (lazy
// rescale).  Scales are integers, so bringing both terms to the common scale
// is exact and the only roundings are the decay product and the final sums.
__device__ __forceinline__ St combine(const St& X, const St& S, double D) {
    const float Dhi = static_cast<float>(D);
    const float Dlo = static_cast<float>(D - static_cast<double>(Dhi));
    const float xa = fmaf(Dhi, X.a, Dlo * X.a);
    const float xb = fmaf(Dhi, X.b, Dlo * X.b);
    if (!(S.b > 0.f)) return St{xa, xb, X.s};
    if (!(xb > 0.f)) return S;
    int sn = X.s;
    const int ls = S.s + __builtin_amdgcn_frexp_expf(S.b);  // S.b 2^S.s < 2^ls
    if ((ls > X.s + static_cast<int>(kBig)) | (xb < kLo) | (xb > kHi))
        sn = max(X.s + __builtin_amdgcn_frexp_expf(xb), ls);
    return St{ldx(xa, X.s - sn) + ldx(S.a, S.s - sn), ldx(xb, X.s - sn) + ldx(S.b, S.s - sn), sn};
}

// ---- the decode-step state (a, b, p), A = a e^p, B = b e^p ---------------------
// Conversions to and from the lane state (a, b, s), A = a 2^s.  The integer
// and fractional parts of p log2 e are split in float64; the factor 2^frac is
// one float32 exp2 applied to a and b alike, so a/b is unchanged and B carries
// one float32 rounding.
__device__ __forceinline__ St state_from_abp(float a, float b, float p) {
    if (!(b > 0.f)) return empty_state();  // the empty state (b = 0), whatever p
    const double q = static_cast<double>(p) * 1.4426950408889634;
    const double n = floor(fmax(q, -1.0e9));
    const float f = ex2(static_cast<float>(q - n));
    return St{a * f, b * f, static_cast<int>(n)};
}

__device__ __forceinline__ void state_to_abp(const St& st, float& a, float& b, float& p) {
    if (!(st.b > 0.f)) {
        a = 0.f;
        b = 0.f;
        p = -1e38f;
        return;
    }
    const double pd = static_cast<double>(st.s) * 0.6931471805599453;
    const float pf = static_cast<float>(pd);
    // fold the rounding of p into a, b: e^{pd - pf} = 2^{(pd - pf) log2 e}
    const float c = ex2(static_cast<float>((pd - static_cast<double>(pf)) * 1.4426950408889634));
    a = st.a * c;
    b = st.b * c;
    p = pf;
}

// Barrier for LDS traffic only: outstanding global loads (prefetches) and
// stores stay in flight across it.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- carries between workgroups --------------------------------------------------
// A chained scan along time: the workgroup of time block j waits for the
// inclusive state of block j-1 of the same tile and publishes its own.  Each
// (tile, block, lane) slot is 16 bytes (a, b, s bits, status) written with ONE
// 16-byte store and polled with 16-byte loads, both with the system-coherent
// cache policy (sc0 sc1), which bypasses the per-XCD L2s.  So no release or
// acquire fence is needed: such fences would write back or invalidate the
// whole L2 of the XCD on every exchange, which the bandwidth-bound stream of
// outputs from the other workgroups cannot afford.  Status 0 means "not yet";
// slots are zeroed by a small kernel before each launch.  Always taking block
// j-1's state (never a look-back over several aggregates) keeps the rounding,
// and therefore the result, independent of timing.
constexpr int kCoherent = 1 | 16;          // sc0 | sc1
constexpr uint32_t kSpinLimit = 1u << 22;  // bounded wait: a broken protocol cannot hang

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void publish_state(Rsrc r, uint32_t off, const St& st) {
    const f32x4 v = {st.a, st.b, __int_as_float(st.s), __uint_as_float(1u)};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}

// Wait for the state published at `off`; after kSpinLimit polls give up,
// set *error and return the empty state (results are then invalid, but every
// wave terminates).
__device__ __forceinline__ St wait_state(Rsrc r, uint32_t off, uint32_t* error) {
    for (uint32_t it = 0; it < kSpinLimit; ++it) {
        const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
        if (__float_as_uint(v.w) != 0u) return St{v.x, v.y, __float_as_int(v.z)};
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return empty_state();
}

}  // namespace wkv
