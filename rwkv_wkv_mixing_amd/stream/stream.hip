// Streaming kernels that measure what HBM delivers to a kernel on this chip:
// the practical ceiling against which the WKV kernels' rates are read.
//
// Each launch reads NR arrays and writes NW arrays of n 16-byte vectors,
// elementwise (out_j[i] = xor of the in_r[i], plus j + 1), with grid-stride
// loops.  A thread issues U independent 16-byte vectors per array and
// iteration before using any of them (multi-issue), and loads and stores may
// carry the non-temporal hint.  The read-only form keeps its loads alive
// through a store that depends on the data and never happens for the zero
// inputs the measurement uses.
//
// Not part of the operator library: built as its own librwkv_stream.so and
// used only by the benchmark's ceiling measurement.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct StreamArgs {
    const u32x4* in[4];
    u32x4* out[4];
    int64_t n;  // 16-byte vectors per array
    u32x4* sink;
};

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <int NR, int NW, int U, bool NT>
__global__ void __launch_bounds__(1024) stream_kernel(StreamArgs a) {
    const int64_t bd = blockDim.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * bd * U;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * bd * U + threadIdx.x; base < a.n; base += stride) {
        u32x4 x[U];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t i = base + q * bd;
            u32x4 s = {0u, 0u, 0u, 0u};
            if (i < a.n) {
#pragma unroll
                for (int r = 0; r < NR; ++r) s ^= ld<NT>(a.in[r] + i);
            }
            x[q] = s;
        }
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int64_t i = base + q * bd;
            if (i < a.n) {
#pragma unroll
                for (int w = 0; w < NW; ++w) st<NT>(a.out[w] + i, x[q] + static_cast<uint32_t>(w + 1));
            }
            acc ^= x[q];
        }
    }
    if (NW == 0 && (acc.x | acc.y | acc.z | acc.w) == 0x9e3779b9u) a.sink[threadIdx.x] = acc;
}

typedef void (*Kern)(StreamArgs);

template <int NR, int NW, int U>
Kern pick(bool nt) {
    return nt ? stream_kernel<NR, NW, U, true> : stream_kernel<NR, NW, U, false>;
}

template <int NR, int NW>
Kern pick_u(int u, bool nt) {
    switch (u) {
        case 1: return pick<NR, NW, 1>(nt);
        case 2: return pick<NR, NW, 2>(nt);
        case 4: return pick<NR, NW, 4>(nt);
        default: return nullptr;
    }
}

Kern select(int nr, int nw, int u, bool nt) {
    if (nr == 1 && nw == 0) return pick_u<1, 0>(u, nt);
    if (nr == 0 && nw == 1) return pick_u<0, 1>(u, nt);
    if (nr == 1 && nw == 1) return pick_u<1, 1>(u, nt);
    if (nr == 3 && nw == 4) return pick_u<3, 4>(u, nt);
    if (nr == 1 && nw == 3) return pick_u<1, 3>(u, nt);
    if (nr == 2 && nw == 1) return pick_u<2, 1>(u, nt);
    if (nr == 3 && nw == 2) return pick_u<3, 2>(u, nt);
    return nullptr;
}

}  // namespace

// Launch one streaming pass on `stream`.  in[0..nr-1] and out[0..nw-1] are
// device arrays of n16 16-byte vectors each (16-byte aligned); sink holds
// `block` vectors.  Supported (nr, nw): (1,0) (0,1) (1,1) (3,4) (1,3) (2,1)
// (3,2); unroll 1, 2 or 4; block <= 1024.  Returns 0, or -1 for an
// unsupported combination, or the HIP error code of the launch.
extern "C" int wkv_stream_launch(int nr, int nw, int unroll, int nt, int grid, int block, const void* const* in,
                                 void* const* out, int64_t n16, void* sink, void* stream) {
    const Kern k = select(nr, nw, unroll, nt != 0);
    if (k == nullptr || grid <= 0 || block <= 0 || block > 1024 || nr > 4 || nw > 4) return -1;
    StreamArgs a{};
    for (int r = 0; r < nr; ++r) a.in[r] = static_cast<const u32x4*>(in[r]);
    for (int w = 0; w < nw; ++w) a.out[w] = static_cast<u32x4*>(out[w]);
    a.n = n16;
    a.sink = static_cast<u32x4*>(sink);
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(grid)), dim3(static_cast<unsigned>(block)), 0,
                       static_cast<hipStream_t>(stream), a);
    return static_cast<int>(hipGetLastError());
}
