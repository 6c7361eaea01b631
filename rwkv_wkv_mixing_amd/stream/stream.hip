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

struct TileArgs {
    const uint16_t* in[4];
    float* out[4];
    int B, T, C, ld;
};

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

// The tiled access order of the WKV tile kernels, without their arithmetic: one workgroup per
// 64-channel tile of one batch row walks the sequence in blocks of W x L tokens.  Each wave copies
// its L rows of the NR bf16 inputs into LDS by 16-byte buffer -> LDS copies (issued once the
// previous block is read, as the kernels do), reads its channel back, and stores NW float32
// outputs per token, one 4-byte store per lane.  [B, T, C] arrays, channel fastest, rows ld >= C
// elements apart (ld = C is the dense layout the WKV calls take; a larger ld shows what the row
// stride alone costs).
using Rsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ Rsrc rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

template <int NR, int NW, int W, int L>
__global__ void __launch_bounds__(64 * W) tile_pattern_kernel(TileArgs a) {
    static_assert(L % 8 == 0, "8 rows of 128 bytes per copy instruction");
    __shared__ uint16_t st[W][NR][L][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nct = a.C / 64;
    const int b = blockIdx.x / nct, c0 = (blockIdx.x % nct) * 64;
    const int nblk = a.T / (L * W);
    auto stage = [&](int blk) {
        const int64_t row0 = (static_cast<int64_t>(b) * a.T + static_cast<int64_t>(blk) * L * W + wave * L) * a.ld;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const Rsrc rs = rsrc(a.in[r] + row0, static_cast<uint32_t>(L * a.ld * 2));
#pragma unroll
            for (int i = 0; i < L / 8; ++i) {
                const int j = i * 8 + lane / 8;
                const uint32_t off = static_cast<uint32_t>((j * a.ld + c0) * 2 + (lane % 8) * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&st[wave][r][i * 8][0],
                                                         16, off, 0, 0, 0);
            }
        }
    };
    float acc = 0.f;
    stage(0);
    for (int blk = 0; blk < nblk; ++blk) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        float x[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            x[j] = 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r) x[j] += __uint_as_float(static_cast<uint32_t>(st[wave][r][j][lane]) << 16);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (blk + 1 < nblk) stage(blk + 1);
        const int64_t row0 = (static_cast<int64_t>(b) * a.T + static_cast<int64_t>(blk) * L * W + wave * L) * a.ld;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const Rsrc ro = rsrc(a.out[w] + row0, static_cast<uint32_t>(L * a.ld * 4));
#pragma unroll
            for (int j = 0; j < L; ++j) {
                acc = fmaf(acc, 0.5f, x[j]);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), ro, static_cast<uint32_t>((c0 + lane) * 4),
                                                      j * a.ld * 4, 3);
            }
        }
    }
}

}  // namespace

// Launch one pass of the tile kernels' access order: (nr, nw) = (2, 1) as the forward (k, v in, y
// out; 8 waves x 16 tokens per block) or (3, 2) as the backward (k, v, gy in, dk, dv out; 4 waves x
// 16 tokens).  in[]: bf16 [B, T, ld]; out[]: float32 [B, T, ld], of which channels 0 .. C - 1 are
// read and written.  Needs C a multiple of 64, ld >= C and T a multiple of the block length (128 or
// 64).  Returns 0, -1 for an unsupported shape, or the HIP error code.
extern "C" int wkv_tile_pattern_launch(int nr, int nw, const void* const* in, void* const* out, int B, int T, int C,
                                       int ld, void* stream) {
    TileArgs a{};
    for (int r = 0; r < nr && r < 4; ++r) a.in[r] = static_cast<const uint16_t*>(in[r]);
    for (int w = 0; w < nw && w < 4; ++w) a.out[w] = static_cast<float*>(out[w]);
    a.B = B;
    a.T = T;
    a.C = C;
    a.ld = ld;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (B <= 0 || C <= 0 || C % 64 != 0 || ld < C || static_cast<int64_t>(T) * ld * 4 > 0x7fffffff) return -1;
    const dim3 grid(static_cast<unsigned>(B * (C / 64)));
    if (nr == 2 && nw == 1 && T > 0 && T % 128 == 0)
        hipLaunchKernelGGL((tile_pattern_kernel<2, 1, 8, 16>), grid, dim3(512), 0, s, a);
    else if (nr == 3 && nw == 2 && T > 0 && T % 64 == 0)
        hipLaunchKernelGGL((tile_pattern_kernel<3, 2, 4, 16>), grid, dim3(256), 0, s, a);
    else
        return -1;
    return static_cast<int>(hipGetLastError());
}

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
