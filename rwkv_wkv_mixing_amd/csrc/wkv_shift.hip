// Token-shift mix: the per-channel mix of each token's input with the previous
// token's that feeds the time-mixing (and channel-mixing) projections
// ("RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section "关键设计 1：
// Token Shift - 给并行投影注入前一时刻"; "RWKV（Receptance Weighted Key Value）
// 概念", section 3.3):
//     out_j[b, t, c] = mu_j[c] x[b, t, c] + (1 - mu_j[c]) x[b, t-1, c],  j < M
// with x[b, -1] the carried previous input (the state tuple's x) or zero.
//
// Pure streaming work with a one-token halo.  A thread owns one vector of V
// channels (8 or 16 bytes of x) over a run of RUN consecutive tokens, so x is
// read once (plus one halo token per run) and the M outputs leave from
// registers.  A 256-thread block is CV vectors wide and 256 / CV runs deep;
// each wave instruction covers whole 128-byte lines of one or two token rows.
// The mix is evaluated as xs + mu (x - xs): one subtraction, one fma.
//
// Backward, for L = sum_j <g_j, out_j>:
//     dx_t    = sum_j mu_j g_j,t + (1 - mu_j) g_j,t+1       (no t+1 term at T-1)
//     dmu_j   = sum_{b,t} g_j,t (x_t - x_{t-1})
//     dx_prev = sum_j (1 - mu_j) g_j,0
// A thread walks its run from the last token to the first, carrying g_{t+1}
// and x_t in registers.  dmu is summed per thread, then over the block's runs
// in LDS, then over blocks by shift_reduce_kernel, each stage in a fixed
// order, so results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_launch.h"

namespace wkv {
namespace {

// Launch shapes (measured on MI355X with operands cold in HBM): the forward writes three times what it reads and prefers
// wide blocks of short runs; the backward holds M + 1 inputs per token and
// prefers 8-byte bf16 vectors (fewer registers, more waves) and long runs.
#ifndef WKV_SHIFT_FWD_CV
#define WKV_SHIFT_FWD_CV 64
#endif
#ifndef WKV_SHIFT_FWD_RUN
#define WKV_SHIFT_FWD_RUN 16
#endif
#ifndef WKV_SHIFT_FWD_VBF
#define WKV_SHIFT_FWD_VBF 4
#endif
#ifndef WKV_SHIFT_BWD_CV
#define WKV_SHIFT_BWD_CV 64  // with the non-temporal loads: 76.0 us against 78.2 at 32 (B=8 T=1024 C=4096 M=3)
#endif
#ifndef WKV_SHIFT_BWD_RUN
#define WKV_SHIFT_BWD_RUN 32
#endif
#ifndef WKV_SHIFT_BWD_VBF
#define WKV_SHIFT_BWD_VBF 4
#endif
#ifndef WKV_SHIFT_NT
#define WKV_SHIFT_NT 1
#endif

constexpr int kThreads = 256;

// V channels per thread, CV vectors per block, TC = 256 / CV runs of RUN
// tokens per block.
template <int V_, int CV_, int RUN_>
struct Layout {
    static constexpr int V = V_;
    static constexpr int CV = CV_;
    static constexpr int TC = kThreads / CV_;
    static constexpr int RUN = RUN_;
    static constexpr int BLOCK_T = TC * RUN_;
};
template <int V>
using FwdLay = Layout<V, WKV_SHIFT_FWD_CV, WKV_SHIFT_FWD_RUN>;
template <int V>
using BwdLay = Layout<V, WKV_SHIFT_BWD_CV, WKV_SHIFT_BWD_RUN>;

template <typename T>
__device__ __forceinline__ void st_out(T v, T* p) {
    if constexpr (WKV_SHIFT_NT) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

// A load with the non-temporal hint (NT) or the default policy.  The backward is the last reader
// of x and of the output gradients, so it reads them non-temporal (85.0 -> 81.7 us at B=8 T=1024
// C=4096 M=3, bf16); the forward's x keeps the default policy, since the backward reads it again.
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// V elements of TIn widened to float32 (bf16: exact) and narrowed back
// (bf16: round to nearest even, one v_cvt_pk_bf16_f32 per pair).
template <typename TIn, int V>
struct Pack;

template <>
struct Pack<float, 4> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const float* __restrict__ p, int64_t i, float (&f)[4]) {
        const f4 r = ld<NT>(reinterpret_cast<const f4*>(p + i));
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
    static __device__ __forceinline__ void store(float* __restrict__ p, int64_t i, const float (&f)[4]) {
        const f4 r = {f[0], f[1], f[2], f[3]};
        st_out(r, reinterpret_cast<f4*>(p + i));
    }
};

template <>
struct Pack<float, 1> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const float* __restrict__ p, int64_t i, float (&f)[1]) { f[0] = ld<NT>(p + i); }
    static __device__ __forceinline__ void store(float* __restrict__ p, int64_t i, const float (&f)[1]) {
        st_out(f[0], p + i);
    }
};

template <>
struct Pack<uint16_t, 8> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t i, float (&f)[8]) {
        const u4 r = ld<NT>(reinterpret_cast<const u4*>(p + i));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(r[q] << 16);
            f[2 * q + 1] = __uint_as_float(r[q] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* __restrict__ p, int64_t i, const float (&f)[8]) {
        u4 r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f2 pr = {f[2 * q], f[2 * q + 1]};
            r[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2));
        }
        st_out(r, reinterpret_cast<u4*>(p + i));
    }
};

template <>
struct Pack<uint16_t, 4> {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    template <bool NT = false>
    static __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t i, float (&f)[4]) {
        const u2 r = ld<NT>(reinterpret_cast<const u2*>(p + i));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f[2 * q] = __uint_as_float(r[q] << 16);
            f[2 * q + 1] = __uint_as_float(r[q] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* __restrict__ p, int64_t i, const float (&f)[4]) {
        u2 r;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const f2 pr = {f[2 * q], f[2 * q + 1]};
            r[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf2));
        }
        st_out(r, reinterpret_cast<u2*>(p + i));
    }
};

template <>
struct Pack<uint16_t, 1> {
    template <bool NT = false>
    static __device__ __forceinline__ void load(const uint16_t* __restrict__ p, int64_t i, float (&f)[1]) {
        f[0] = __uint_as_float(static_cast<uint32_t>(ld<NT>(p + i)) << 16);
    }
    static __device__ __forceinline__ void store(uint16_t* __restrict__ p, int64_t i, const float (&f)[1]) {
        st_out(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f[0])), p + i);
    }
};

// float32 outputs of the backward: V floats (V = 8 as two 16-byte stores)
template <int V>
__device__ __forceinline__ void store_f32(float* __restrict__ p, int64_t i, const float (&f)[V]) {
    if constexpr (V == 1) {
        Pack<float, 1>::store(p, i, f);
    } else {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            const float q[4] = {f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]};
            Pack<float, 4>::store(p, i + 4 * h, q);
        }
    }
}

template <int V>
__device__ __forceinline__ void load_f32(const float* __restrict__ p, int64_t i, float (&f)[V]) {
    if constexpr (V == 1) {
        f[0] = p[i];
    } else {
#pragma unroll
        for (int h = 0; h < V / 4; ++h) {
            float q[4];
            Pack<float, 4>::load(p, i + 4 * h, q);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * h + e] = q[e];
        }
    }
}

// Position of a thread: batch row b, first channel c, first token t0 of its
// run, its run index within the block, and how many tokens the run holds.
struct Where {
    int64_t b, c, t0, tb;
    int run, n;
    bool active;
};

template <class Lay>
__device__ __forceinline__ Where where(const ShiftArgs& P) {
    constexpr int V = Lay::V, CV = Lay::CV, RUN = Lay::RUN;
    const int64_t ncb = (P.C / V + CV - 1) / CV;
    const int64_t ntb = (P.T + Lay::BLOCK_T - 1) / Lay::BLOCK_T;
    int64_t blk = blockIdx.x;
    const int64_t cb = blk % ncb;
    blk /= ncb;
    Where w;
    w.tb = blk % ntb;
    w.b = blk / ntb;
    w.run = threadIdx.x / CV;
    w.c = (cb * CV + threadIdx.x % CV) * V;
    w.t0 = w.tb * Lay::BLOCK_T + int64_t{w.run} * RUN;
    const int64_t left = P.T - w.t0;
    w.n = left < RUN ? static_cast<int>(left) : RUN;
    w.active = w.c < P.C && w.n > 0;
    return w;
}

template <typename TIn, int V>
__device__ __forceinline__ void load_prev(const ShiftArgs& P, const Where& w, float (&xp)[V]) {
    const TIn* __restrict__ x = static_cast<const TIn*>(P.x);
    if (w.t0 > 0) {
        Pack<TIn, V>::load(x, (w.b * P.T + w.t0 - 1) * P.C + w.c, xp);
    } else if (P.x_prev) {
        Pack<TIn, V>::load(static_cast<const TIn*>(P.x_prev), w.b * P.C + w.c, xp);
    } else {
#pragma unroll
        for (int e = 0; e < V; ++e) xp[e] = 0.f;
    }
}

template <typename TIn, class Lay, int M>
__global__ __launch_bounds__(kThreads) void shift_fwd_kernel(ShiftArgs P) {
    constexpr int V = Lay::V, kRun = Lay::RUN;
    const Where w = where<Lay>(P);
    if (!w.active) return;
    const TIn* __restrict__ x = static_cast<const TIn*>(P.x);
    TIn* __restrict__ out = static_cast<TIn*>(P.out);
    const int64_t N = P.B * P.T * P.C;
    float mu[M][V];
#pragma unroll
    for (int j = 0; j < M; ++j) load_f32<V>(P.mu, j * P.C + w.c, mu[j]);
    float prev[V];
    load_prev<TIn, V>(P, w, prev);
    const int64_t base = (w.b * P.T + w.t0) * P.C + w.c;
    auto token = [&](int i) {
        float cur[V];
        Pack<TIn, V>::load(x, base + i * P.C, cur);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = __builtin_fmaf(mu[j][e], cur[e] - prev[e], prev[e]);
            Pack<TIn, V>::store(out, j * N + base + i * P.C, o);
        }
#pragma unroll
        for (int e = 0; e < V; ++e) prev[e] = cur[e];
    };
    if (w.n == kRun) {
#pragma unroll
        for (int i = 0; i < kRun; ++i) token(i);
    } else {
        for (int i = 0; i < w.n; ++i) token(i);
    }
}

template <typename TIn, class Lay, int M>
__global__ __launch_bounds__(kThreads) void shift_bwd_kernel(ShiftArgs P) {
    constexpr int V = Lay::V, kRun = Lay::RUN, kCV = Lay::CV, kTC = Lay::TC;
    __shared__ float part[kTC][kCV * V * M];
    const Where w = where<Lay>(P);
    const int64_t N = P.B * P.T * P.C;
    float acc[M][V];
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[j][e] = 0.f;
    if (w.active) {
        const TIn* __restrict__ x = static_cast<const TIn*>(P.x);
        const TIn* __restrict__ g = static_cast<const TIn*>(P.g);
        float mu[M][V];
#pragma unroll
        for (int j = 0; j < M; ++j) load_f32<V>(P.mu, j * P.C + w.c, mu[j]);
        const int64_t base = (w.b * P.T + w.t0) * P.C + w.c;
        // g_{t+1} after the run's last token (zero at the sequence end), and x_t
        float gn[M][V], xc[V];
        const bool tail = w.t0 + w.n < P.T;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            if (tail) {
                Pack<TIn, V>::template load<true>(g, j * N + base + w.n * P.C, gn[j]);
            } else {
#pragma unroll
                for (int e = 0; e < V; ++e) gn[j][e] = 0.f;
            }
        }
        Pack<TIn, V>::template load<true>(x, base + (w.n - 1) * P.C, xc);
        auto token = [&](int i) {  // token t0 + i, walking backwards
            float xp[V], gc[M][V], dx[V];
            if (i > 0) {
                Pack<TIn, V>::template load<true>(x, base + (i - 1) * P.C, xp);
            } else {
                load_prev<TIn, V>(P, w, xp);
            }
#pragma unroll
            for (int j = 0; j < M; ++j) Pack<TIn, V>::template load<true>(g, j * N + base + i * P.C, gc[j]);
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    s = __builtin_fmaf(mu[j][e], gc[j][e], s);
                    s = __builtin_fmaf(1.f - mu[j][e], gn[j][e], s);
                    acc[j][e] = __builtin_fmaf(gc[j][e], xc[e] - xp[e], acc[j][e]);
                    gn[j][e] = gc[j][e];
                }
                dx[e] = s;
                xc[e] = xp[e];
            }
            store_f32<V>(P.dx, base + i * P.C, dx);
        };
        // four tokens per iteration: their 4 (M + 1) loads issue together
        // without holding a whole run of inputs in registers
        if (w.n == kRun) {
#pragma unroll 4
            for (int i = kRun - 1; i >= 0; --i) token(i);
        } else {
            for (int i = w.n - 1; i >= 0; --i) token(i);
        }
        if (w.t0 == 0 && P.dx_prev) {  // gn now holds g_0
            float dp[V];
#pragma unroll
            for (int e = 0; e < V; ++e) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < M; ++j) s = __builtin_fmaf(1.f - mu[j][e], gn[j][e], s);
                dp[e] = s;
            }
            store_f32<V>(P.dx_prev, w.b * P.C + w.c, dp);
        }
    }
    // block partial of dmu: runs summed in order 0..kTC-1
    const int cv = threadIdx.x % kCV;
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) part[w.run][(j * kCV + cv) * V + e] = acc[j][e];
    __syncthreads();
    const int64_t ncb = (P.C / V + kCV - 1) / kCV;
    const int64_t cb = blockIdx.x % ncb;
    const int64_t row = w.b * ((P.T + Lay::BLOCK_T - 1) / Lay::BLOCK_T) + w.tb;
    for (int q = threadIdx.x; q < kCV * V * M; q += kThreads) {
        const int j = q / (kCV * V);
        const int64_t c = cb * kCV * V + q % (kCV * V);
        if (c >= P.C) continue;
        float s = part[0][q];
#pragma unroll
        for (int r = 1; r < kTC; ++r) s += part[r][q];
        P.ws[(row * M + j) * P.C + c] = s;
    }
}

// dmu[j, c] = sum over the block rows (b, tb) in order of the partials.
__global__ __launch_bounds__(kThreads) void shift_reduce_kernel(const float* __restrict__ ws, int64_t rows,
                                                                 int64_t MC, float* __restrict__ dmu) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (q >= MC) return;
    // loads of 16 rows issue together; the sum keeps the row order
    float s = 0.f;
    int64_t r = 0;
    for (; r + 16 <= rows; r += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = ws[(r + i) * MC + q];
#pragma unroll
        for (int i = 0; i < 16; ++i) s += v[i];
    }
    for (; r < rows; ++r) s += ws[r * MC + q];
    dmu[q] = s;
}

__global__ void shift_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

template <class Lay>
int64_t shift_blocks(const ShiftArgs& a) {
    return a.B * ((a.T + Lay::BLOCK_T - 1) / Lay::BLOCK_T) * ((a.C / Lay::V + Lay::CV - 1) / Lay::CV);
}

template <typename TIn, class Lay, int M>
hipError_t launch_fwd_tvm(const ShiftArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((shift_fwd_kernel<TIn, Lay, M>), dim3(static_cast<unsigned>(shift_blocks<Lay>(a))),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename TIn, class Lay, int M>
hipError_t launch_bwd_tvm(const ShiftArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((shift_bwd_kernel<TIn, Lay, M>), dim3(static_cast<unsigned>(shift_blocks<Lay>(a))),
                       dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t MC = a.M * a.C;
    hipLaunchKernelGGL(shift_reduce_kernel, dim3(static_cast<unsigned>((MC + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, a.ws, shift_partial_rows(a.B, a.T), MC, a.dmu);
    return hipGetLastError();
}

template <typename TIn, int V, bool Bwd>
hipError_t launch_m(const ShiftArgs& a, hipStream_t s) {
    if constexpr (Bwd) {
        switch (a.M) {
            case 1: return launch_bwd_tvm<TIn, BwdLay<V>, 1>(a, s);
            case 2: return launch_bwd_tvm<TIn, BwdLay<V>, 2>(a, s);
            case 3: return launch_bwd_tvm<TIn, BwdLay<V>, 3>(a, s);
            default: return launch_bwd_tvm<TIn, BwdLay<V>, 4>(a, s);
        }
    } else {
        switch (a.M) {
            case 1: return launch_fwd_tvm<TIn, FwdLay<V>, 1>(a, s);
            case 2: return launch_fwd_tvm<TIn, FwdLay<V>, 2>(a, s);
            case 3: return launch_fwd_tvm<TIn, FwdLay<V>, 3>(a, s);
            default: return launch_fwd_tvm<TIn, FwdLay<V>, 4>(a, s);
        }
    }
}

template <bool Bwd>
hipError_t launch_shift(const ShiftArgs& a, hipStream_t s) {
    constexpr int VB = Bwd ? WKV_SHIFT_BWD_VBF : WKV_SHIFT_FWD_VBF;
    if (a.bf16) return a.vec ? launch_m<uint16_t, VB, Bwd>(a, s) : launch_m<uint16_t, 1, Bwd>(a, s);
    return a.vec ? launch_m<float, 4, Bwd>(a, s) : launch_m<float, 1, Bwd>(a, s);
}

}  // namespace

int64_t shift_partial_rows(int64_t B, int64_t T) {
    return B * ((T + BwdLay<1>::BLOCK_T - 1) / BwdLay<1>::BLOCK_T);
}

int shift_vector_width(bool bf16, bool bwd) {
    return bf16 ? (bwd ? WKV_SHIFT_BWD_VBF : WKV_SHIFT_FWD_VBF) : 4;
}

hipError_t launch_shift_fwd(const ShiftArgs& a, hipStream_t stream) { return launch_shift<false>(a, stream); }

hipError_t launch_shift_bwd(const ShiftArgs& a, hipStream_t stream) { return launch_shift<true>(a, stream); }

hipError_t launch_shift_zero(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(shift_zero_kernel, dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace wkv
