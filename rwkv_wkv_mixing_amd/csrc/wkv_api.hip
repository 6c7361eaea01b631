// C ABI of the WKV library (declared in include/wkv.h): argument validation,
// workspace sizing, path selection and kernel launches.  Every check runs on
// the host before any HIP call, so invalid calls never touch the device.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "wkv.h"
#include "wkv_launch.h"

namespace {

std::atomic<uint32_t> g_spin_limit{1u << 22};

thread_local char g_hip_msg[256] = "";

wkv_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return WKV_OK;
    snprintf(g_hip_msg, sizeof(g_hip_msg), "%s (%d)", hipGetErrorString(e), static_cast<int>(e));
    return WKV_EHIP;
}

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
    int64_t t;
    if (__builtin_mul_overflow(a, b, &t)) return false;
    if (__builtin_mul_overflow(t, c, out)) return false;
    return true;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dtype_ok(int dt) { return dt == WKV_F32 || dt == WKV_BF16; }

size_t in_size(int dt) { return dt == WKV_BF16 ? 2 : 4; }

// Largest lane count the 1-D grids index: blocks of 256 threads, grid.x < 2^31.
constexpr int64_t kMaxLanes = (int64_t{1} << 31) * 256 - 1;

struct Plan {
    wkv_status_t st;
    size_t ws_bytes;
    int64_t N;
    int64_t nblk;
};

Plan plan(int op, int64_t B, int64_t T, int64_t C, int dt) {
    Plan p{WKV_OK, 0, 0, 0};
    if (B < 0 || T < 0 || C < 0) return Plan{WKV_EINVAL, 0, 0, 0};
    if (!dtype_ok(dt)) return Plan{WKV_EDTYPE, 0, 0, 0};
    if (op != WKV_OP_FORWARD && op != WKV_OP_BACKWARD) return Plan{WKV_EDTYPE, 0, 0, 0};
    if (!mul3(B, T, C, &p.N)) return Plan{WKV_ESIZE, 0, 0, 0};
    int64_t bytes;
    if (__builtin_mul_overflow(p.N, int64_t{16}, &bytes)) return Plan{WKV_ESIZE, 0, 0, 0};
    int64_t lanes;
    if (__builtin_mul_overflow(B, C, &lanes) || lanes > kMaxLanes) return Plan{WKV_ESIZE, 0, 0, 0};
    p.nblk = (T + wkv::kCkptLen - 1) / wkv::kCkptLen;
    if (op == WKV_OP_BACKWARD && p.N > 0) p.ws_bytes = wkv::bwd_chunk_workspace_bytes(B, T, C);
    if (op == WKV_OP_FORWARD && p.N > 0) p.ws_bytes = wkv::fwd_chunk_workspace_bytes(B, T, C);
    if (p.ws_bytes == SIZE_MAX) return Plan{WKV_ESIZE, 0, 0, 0};
    return p;
}

struct ShiftPlan {
    wkv_status_t st;
    int64_t N;
    size_t ws_bytes;
};

ShiftPlan shift_plan(int64_t B, int64_t T, int64_t C, int64_t M, int dt) {
    if (B < 0 || T < 0 || C < 0 || M < 1 || M > 4) return ShiftPlan{WKV_EINVAL, 0, 0};
    if (!dtype_ok(dt)) return ShiftPlan{WKV_EDTYPE, 0, 0};
    ShiftPlan p{WKV_OK, 0, 0};
    int64_t bytes, rows_c, ws;
    if (!mul3(B, T, C, &p.N) || !mul3(p.N, M, 4, &bytes)) return ShiftPlan{WKV_ESIZE, 0, 0};
    // grid: at most one block per (row of partials, channel), below 2^31 blocks
    const int64_t rows = wkv::shift_partial_rows(B, T);
    if (__builtin_mul_overflow(rows, C, &rows_c) || rows_c >= (int64_t{1} << 31)) return ShiftPlan{WKV_ESIZE, 0, 0};
    if (!mul3(rows_c, M, 4, &ws)) return ShiftPlan{WKV_ESIZE, 0, 0};
    p.ws_bytes = static_cast<size_t>(ws);
    return p;
}

// T == 0 through carried state: the handed-on state is the given one, so its gradient passes back,
// from the representation at p_out to that at p_in (zeros for an empty given state).
__global__ void state_grad_passthrough_kernel(int64_t n, const float* a_in, const float* b_in, const float* p_in,
                                              const float* ga_out, const float* gb_out, const float* p_out,
                                              float* ga_in, float* gb_in, float* gp_in) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double ga = 0.0, gb = 0.0;
    if (ga_out != nullptr && b_in[i] > 0.f && p_out[i] > -1e30f) {
        const double f = exp(static_cast<double>(p_in[i]) - static_cast<double>(p_out[i]));
        ga = ga_out[i] * f;
        gb = gb_out[i] * f;
    }
    ga_in[i] = static_cast<float>(ga);
    gb_in[i] = static_cast<float>(gb);
    gp_in[i] = static_cast<float>(fma(static_cast<double>(a_in[i]), ga, static_cast<double>(b_in[i]) * gb));
}

__global__ void zero2_kernel(int64_t n, float* a, float* b) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) {
        a[i] = 0.f;
        b[i] = 0.f;
    }
}

}  // namespace

uint32_t wkv::spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

extern "C" {

size_t wkv_workspace_bytes(int op, int64_t B, int64_t T, int64_t C, int in_dtype) {
    const Plan p = plan(op, B, T, C, in_dtype);
    return p.st == WKV_OK ? p.ws_bytes : 0;
}

size_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0) return 0;
    const int64_t nblk = (T + wkv::kCkptLen - 1) / wkv::kCkptLen;
    int64_t n;
    if (!mul3(B, nblk, C, &n)) return 0;
    if (__builtin_mul_overflow(n, int64_t{12}, &n)) return 0;
    return static_cast<size_t>(n);
}

}  // extern "C"

// Scratch of wkv_forward_state_noalloc, one copy per GPU the library runs on, held until the process
// ends.  Static storage: zero when the code object loads, which is all the workspace protocol needs
// before a first call (the last workgroup of every call returns the header to zero, and carry slots
// are tagged with the call's generation).  Host code never passes `scratch` itself to a kernel: its
// device address, taken once per device, is kept in g_scratch_ptr.
constexpr size_t kStaticScratchBytes = WKV_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, its address looked up on the first use on that device.
hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (ptr == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return hipSuccess;
}

// wkv_forward_state on the caller's workspace, or (use_static) on this device's static scratch.
wkv_status_t forward_state(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w, const float* u,
                           const void* k, const void* v, float* y, const float* a_in, const float* b_in,
                           const float* p_in, float* a_out, float* b_out, float* p_out, void* ckpt,
                           void* workspace, size_t workspace_bytes, bool use_static, void* hip_stream) {
    const Plan p = plan(WKV_OP_FORWARD, B, T, C, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (use_static && p.ws_bytes > kStaticScratchBytes) return WKV_ESCRATCH;
    const bool sin = a_in || b_in || p_in, sout = a_out || b_out || p_out;
    if ((sin && !(a_in && b_in && p_in)) || (sout && !(a_out && b_out && p_out))) return WKV_EINVAL;
    if ((sin && (!aligned(a_in, 4) || !aligned(b_in, 4) || !aligned(p_in, 4))) ||
        (sout && (!aligned(a_out, 4) || !aligned(b_out, 4) || !aligned(p_out, 4))))
        return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    wkv::FwdArgs a{B, T, C, in_dtype == WKV_BF16, w, u, k, v, y, ckpt, p.nblk, workspace, workspace_bytes};
    a.a_in = a_in; a.b_in = b_in; a.p_in = p_in;
    a.a_out = a_out; a.b_out = b_out; a.p_out = p_out;
    if (p.N == 0) return T == 0 ? hip_status(wkv::launch_state_passthrough(a, stream)) : WKV_OK;
    if (!w || !u || !k || !v || !y) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(y, 4) || !aligned(k, es) || !aligned(v, es) ||
        (ckpt && !aligned(ckpt, 4)))
        return WKV_EALIGN;
    if (use_static && p.ws_bytes > 0) {
        const hipError_t e = static_scratch(&a.ws);
        if (e != hipSuccess) return hip_status(e);
        a.ws_bytes = kStaticScratchBytes;
    } else if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256))) {
        return WKV_EWORKSPACE;
    }
    return hip_status(wkv::launch_fwd_chunk(a, stream));
}

}  // namespace

extern "C" {

wkv_status_t wkv_forward_state(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                               const float* u, const void* k, const void* v, float* y,
                               const float* a_in, const float* b_in, const float* p_in, float* a_out,
                               float* b_out, float* p_out, void* ckpt, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
    return forward_state(B, T, C, in_dtype, w, u, k, v, y, a_in, b_in, p_in, a_out, b_out, p_out, ckpt, workspace,
                         workspace_bytes, false, hip_stream);
}

wkv_status_t wkv_forward_state_noalloc(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                                       const float* u, const void* k, const void* v, float* y,
                                       const float* a_in, const float* b_in, const float* p_in, float* a_out,
                                       float* b_out, float* p_out, void* ckpt, void* hip_stream) {
    return forward_state(B, T, C, in_dtype, w, u, k, v, y, a_in, b_in, p_in, a_out, b_out, p_out, ckpt, nullptr, 0,
                         true, hip_stream);
}

wkv_status_t wkv_forward_gated(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                               const float* u, const void* k, const void* v, const void* r, float* out,
                               void* ckpt, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const Plan p = plan(WKV_OP_FORWARD, B, T, C, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (p.N == 0) return WKV_OK;
    if (!w || !u || !k || !v || !r || !out) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(out, 4) || !aligned(k, es) || !aligned(v, es) ||
        !aligned(r, es) || (ckpt && !aligned(ckpt, 4)))
        return WKV_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256)))
        return WKV_EWORKSPACE;
    wkv::FwdArgs a{B, T, C, in_dtype == WKV_BF16, w, u, k, v, out, ckpt, p.nblk, workspace, workspace_bytes};
    a.r = r;
    return hip_status(wkv::launch_fwd_chunk(a, static_cast<hipStream_t>(hip_stream)));
}

wkv_status_t wkv_forward(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                         const float* u, const void* k, const void* v, float* y, void* ckpt,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
    return wkv_forward_state(B, T, C, in_dtype, w, u, k, v, y, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, ckpt, workspace, workspace_bytes, hip_stream);
}

wkv_status_t wkv_backward(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                          const float* u, const void* k, const void* v, const void* gy,
                          float* dk, float* dv, float* dw, float* du, const void* ckpt,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    const Plan p = plan(WKV_OP_BACKWARD, B, T, C, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (C == 0) return WKV_OK;
    if (!dw || !du) return WKV_EINVAL;
    if (!aligned(dw, 4) || !aligned(du, 4)) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p.N == 0) {  // empty sums: dw = du = 0
        hipLaunchKernelGGL(zero2_kernel, dim3(static_cast<unsigned>((C + 255) / 256)), dim3(256), 0,
                           stream, C, dw, du);
        return hip_status(hipGetLastError());
    }
    if (!w || !u || !k || !v || !gy || !dk || !dv) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(dk, 4) || !aligned(dv, 4) ||
        !aligned(k, es) || !aligned(v, es) || !aligned(gy, es) || (ckpt && !aligned(ckpt, 4)))
        return WKV_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256)))
        return WKV_EWORKSPACE;
    wkv::BwdArgs a{B, T, C, in_dtype == WKV_BF16, w, u, k, v, gy, dk, dv, dw, du, ckpt, p.nblk,
                   workspace, workspace_bytes};
    return hip_status(wkv::launch_bwd_chunk(a, stream));
}

wkv_status_t wkv_backward_state(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                                const float* u, const void* k, const void* v, const void* gy,
                                const float* a_in, const float* b_in, const float* p_in, const float* ga_out,
                                const float* gb_out, const float* p_out, float* dk, float* dv, float* dw,
                                float* du, float* ga_in, float* gb_in, float* gp_in, const void* ckpt,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
    const Plan p = plan(WKV_OP_BACKWARD, B, T, C, in_dtype);
    if (p.st != WKV_OK) return p.st;
    const bool sin = a_in || b_in || p_in, sout = ga_out || gb_out || p_out, gin = ga_in || gb_in || gp_in;
    if ((sin && !(a_in && b_in && p_in)) || (sout && !(ga_out && gb_out && p_out)) ||
        (gin && !(ga_in && gb_in && gp_in)) || (gin && !sin))
        return WKV_EINVAL;
    const float* st4[9] = {a_in, b_in, p_in, ga_out, gb_out, p_out, ga_in, gb_in, gp_in};
    for (const float* q : st4)
        if (q && !aligned(q, 4)) return WKV_EALIGN;
    if (C == 0) return WKV_OK;
    if (!dw || !du) return WKV_EINVAL;
    if (!aligned(dw, 4) || !aligned(du, 4)) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p.N == 0) {  // empty sums: dw = du = 0; with T == 0 the state's gradient passes back
        hipLaunchKernelGGL(zero2_kernel, dim3(static_cast<unsigned>((C + 255) / 256)), dim3(256), 0,
                           stream, C, dw, du);
        hipError_t e = hipGetLastError();
        const int64_t n = B * C;
        if (e == hipSuccess && gin && n > 0) {
            hipLaunchKernelGGL(state_grad_passthrough_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                               0, stream, n, a_in, b_in, p_in, ga_out, gb_out, p_out, ga_in, gb_in, gp_in);
            e = hipGetLastError();
        }
        return hip_status(e);
    }
    if (!w || !u || !k || !v || !gy || !dk || !dv) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(dk, 4) || !aligned(dv, 4) ||
        !aligned(k, es) || !aligned(v, es) || !aligned(gy, es) || (ckpt && !aligned(ckpt, 4)))
        return WKV_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256)))
        return WKV_EWORKSPACE;
    wkv::BwdArgs a{B, T, C, in_dtype == WKV_BF16, w, u, k, v, gy, dk, dv, dw, du, ckpt, p.nblk,
                   workspace, workspace_bytes};
    a.a_in = a_in; a.b_in = b_in; a.p_in = p_in;
    a.ga_out = ga_out; a.gb_out = gb_out; a.p_out = p_out;
    a.ga_in = ga_in; a.gb_in = gb_in; a.gp_in = gp_in;
    return hip_status(wkv::launch_bwd_chunk(a, stream));
}

wkv_status_t wkv_backward_gated(int64_t B, int64_t T, int64_t C, int in_dtype, const float* w,
                                const float* u, const void* k, const void* v, const void* r,
                                const void* gout, float* dk, float* dv, float* dr, float* dw, float* du,
                                const void* ckpt, void* workspace, size_t workspace_bytes, void* hip_stream) {
    const Plan p = plan(WKV_OP_BACKWARD, B, T, C, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (C == 0) return WKV_OK;
    if (!dw || !du) return WKV_EINVAL;
    if (!aligned(dw, 4) || !aligned(du, 4)) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p.N == 0) {  // empty sums: dw = du = 0
        hipLaunchKernelGGL(zero2_kernel, dim3(static_cast<unsigned>((C + 255) / 256)), dim3(256), 0,
                           stream, C, dw, du);
        return hip_status(hipGetLastError());
    }
    if (!w || !u || !k || !v || !r || !gout || !dk || !dv || !dr) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(dk, 4) || !aligned(dv, 4) || !aligned(dr, 4) ||
        !aligned(k, es) || !aligned(v, es) || !aligned(r, es) || !aligned(gout, es) || (ckpt && !aligned(ckpt, 4)))
        return WKV_EALIGN;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256)))
        return WKV_EWORKSPACE;
    wkv::BwdArgs a{B, T, C, in_dtype == WKV_BF16, w, u, k, v, gout, dk, dv, dw, du, ckpt, p.nblk,
                   workspace, workspace_bytes};
    a.r = r;
    a.dr = dr;
    return hip_status(wkv::launch_bwd_chunk(a, stream));
}

wkv_status_t wkv_step(int64_t L, int64_t B, int64_t C, int in_dtype, const float* w,
                      const float* u, const void* k, const void* v, float* y, float* a, float* b,
                      float* p, void* hip_stream) {
    if (L < 0 || B < 0 || C < 0) return WKV_EINVAL;
    if (!dtype_ok(in_dtype)) return WKV_EDTYPE;
    int64_t n;
    if (!mul3(L, B, C, &n)) return WKV_ESIZE;
    int64_t bytes;
    if (__builtin_mul_overflow(n, int64_t{16}, &bytes) || n > kMaxLanes) return WKV_ESIZE;
    if (n == 0) return WKV_OK;
    if (!w || !u || !k || !v || !y || !a || !b || !p) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(y, 4) || !aligned(a, 4) || !aligned(b, 4) ||
        !aligned(p, 4) || !aligned(k, es) || !aligned(v, es))
        return WKV_EALIGN;
    const bool vec4 = (C % 4 == 0) && aligned(w, 16) && aligned(u, 16) && aligned(y, 16) &&
                      aligned(a, 16) && aligned(b, 16) && aligned(p, 16) && aligned(k, 4 * es) &&
                      aligned(v, 4 * es);
    wkv::StepArgs s{L, B, C, in_dtype == WKV_BF16, vec4, w, u, k, v, y, a, b, p};
    return hip_status(wkv::launch_step(s, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"

namespace {

// Shared argument checks of the RWKV-5 calls; fills the (batch row, head) count,
// the state element count and the workspace of the backward.
struct Wkv5Plan {
    wkv_status_t st;
    int64_t bh, ns;
    size_t ckpt_bytes, ws_bytes;
};

Wkv5Plan wkv5_plan(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype) {
    Wkv5Plan p{WKV_OK, 0, 0, 0, 0};
    if (B < 0 || T < 0 || H < 0 || N != 64) return Wkv5Plan{WKV_EINVAL, 0, 0, 0, 0};
    if (!dtype_ok(in_dtype)) return Wkv5Plan{WKV_EDTYPE, 0, 0, 0, 0};
    if (in_dtype != WKV_BF16) return Wkv5Plan{WKV_EDTYPE, 0, 0, 0, 0};  // the products run on bf16 operands
    int64_t n, bytes, ck;
    if (!mul3(B, T, H, &n) || __builtin_mul_overflow(n, int64_t{64 * 4}, &bytes)) return Wkv5Plan{WKV_ESIZE, 0, 0, 0, 0};
    if (__builtin_mul_overflow(B, H, &p.bh) || p.bh >= (int64_t{1} << 31)) return Wkv5Plan{WKV_ESIZE, 0, 0, 0, 0};
    if (__builtin_mul_overflow(p.bh, int64_t{64 * 64}, &p.ns)) return Wkv5Plan{WKV_ESIZE, 0, 0, 0, 0};
    // one chunk's rows must fit a buffer resource: 64 rows of C = 64 H float32
    if (H > 0 && 64 * 64 * H * 4 >= (int64_t{1} << 32)) return Wkv5Plan{WKV_ESIZE, 0, 0, 0, 0};
    // backward workspace: the bf16 state before every 64-token chunk, then 2 x 64
    // float32 partial sums (dw, du) per (batch row, head)
    const int64_t nch = (T + 63) / 64;
    if (!mul3(p.bh, nch, 64 * 64 * 2, &ck) || ck > (int64_t{1} << 60)) return Wkv5Plan{WKV_ESIZE, 0, 0, 0, 0};
    p.ckpt_bytes = (static_cast<size_t>(ck) + 255) / 256 * 256;
    p.ws_bytes = T > 0 ? static_cast<size_t>(p.bh) * 2 * 64 * 4 : 0;  // without the chunk-start states
    return p;
}

}  // namespace

extern "C" {

size_t wkv5_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t N) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, WKV_BF16);
    return p.st == WKV_OK ? p.ckpt_bytes : 0;
}

}  // extern "C"

namespace {

// The time split of a matrix-state forward (few (batch row, head) pairs): a state-only pass over every
// segment from the zero state, the chain of the segments' start states, then the outputs of every
// segment from its start.  ws holds [BH, nseg, 64, 64] local end states, the same for the start
// states, and (RWKV-6) [BH, nseg, 64] summed rates.
template <class A, hipError_t (*Launch)(const A&, hipStream_t)>
hipError_t run_split(const A& a, bool per_token, const float* w5, int64_t nseg, int64_t cps, void* ws,
                     hipStream_t stream) {
    const int64_t bh = a.B * a.H;
    float* loc = static_cast<float*>(ws);
    float* start = loc + bh * nseg * 64 * 64;
    float* rates = start + bh * nseg * 64 * 64;
    A p1 = a;  // state-only, from the zero state, each segment's end state into loc
    p1.o = nullptr;
    p1.s_in = nullptr;
    p1.s_out = loc;
    p1.ckpt = nullptr;
    p1.nseg = nseg;
    p1.cps = cps;
    p1.seg_rates = per_token ? rates : nullptr;
    hipError_t e = Launch(p1, stream);
    if (e != hipSuccess) return e;
    const wkv::SegChainArgs c{bh, a.H, a.T, nseg, cps, per_token ? nullptr : w5, per_token ? rates : nullptr,
                              a.s_in, loc, start, a.s_out};
    e = wkv::launch_seg_chain(c, stream);
    if (e != hipSuccess) return e;
    A p3 = a;  // the outputs (and saved states) of every segment from its start
    p3.s_in = start;
    p3.s_out = nullptr;
    p3.nseg = nseg;
    p3.cps = cps;
    p3.seg_rates = nullptr;
    return Launch(p3, stream);
}

size_t split_bytes(int64_t B, int64_t T, int64_t H, int64_t* nseg, int64_t* cps, int64_t max_bh = 255) {
    *nseg = wkv::wkv56_segments(B * H, T, cps, max_bh);
    if (*nseg <= 1) return 0;
    return static_cast<size_t>(B * H * *nseg) * (2 * 64 * 64 + 64) * 4;
}

// The matrix-state backwards' workspace: the dw / du partials of every (segment, batch row, head);
// with a time split, the forward split's [BH, nseg, 64, 64] x 2 + [BH, nseg, 64] region (local and
// chained adjoints and summed rates; a recompute of the chunk-start states uses it first); without a
// ckpt, the recomputed chunk-start states.  Every offset is a multiple of 256 bytes.
struct BwdLayout {
    int64_t nseg = 1, cps = 0;
    size_t split_off = 0, ckpt_off = 0, total = 0;
};

BwdLayout bwd_layout(const Wkv5Plan& p, int64_t B, int64_t T, int64_t H, bool split, bool have_ckpt) {
    BwdLayout l;
    const size_t sb = split ? split_bytes(B, T, H, &l.nseg, &l.cps, 256) : 0;
    if (sb == 0) l.nseg = 1;
    l.split_off = p.ws_bytes * static_cast<size_t>(l.nseg);
    l.ckpt_off = l.split_off + sb;
    l.total = l.ckpt_off + (have_ckpt ? 0 : p.ckpt_bytes);
    return l;
}

// The backward splits up to 256 pairs, the forward below 256: the recompute of the chunk-start
// states takes the forward's own rule, so its states are the bits a forward given a workspace saves.
bool recompute_split(const BwdLayout& l, int64_t B, int64_t H) { return l.nseg > 1 && B * H < 256; }

// A backward with a time split (nseg > 1): every segment's local adjoint, the chain of the adjoints
// after the segments (last first, from ds_out), then the backward of every segment from its own.
template <class BA, hipError_t (*Launch)(const BA&, hipStream_t)>
hipError_t run_bwd(BA ba, const BwdLayout& l, bool per_token, void* ws, hipStream_t stream) {
    if (l.nseg > 1) {
        const int64_t bh = ba.B * ba.H;
        float* loc = reinterpret_cast<float*>(static_cast<char*>(ws) + l.split_off);
        float* gend = loc + bh * l.nseg * 64 * 64;
        float* rates = gend + bh * l.nseg * 64 * 64;
        const wkv::AdjLocalArgs al{ba.B, ba.T, ba.H, l.nseg, l.cps, ba.w, per_token, ba.r, ba.go, loc, rates};
        hipError_t e = wkv::launch_adj_local(al, stream);
        if (e != hipSuccess) return e;
        wkv::SegChainArgs c{bh, ba.H, ba.T, l.nseg, l.cps, per_token ? nullptr : ba.w, per_token ? rates : nullptr,
                            ba.ds_out, loc, gend, nullptr};
        c.reverse = 1;
        e = wkv::launch_seg_chain(c, stream);
        if (e != hipSuccess) return e;
        ba.nseg = l.nseg;
        ba.cps = l.cps;
        ba.gstart = gend;
    }
    return Launch(ba, stream);
}

}  // namespace

extern "C" {

size_t wkv5_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, WKV_BF16);
    if (p.st != WKV_OK || p.bh == 0) return 0;
    int64_t nseg, cps;
    return split_bytes(B, T, H, &nseg, &cps);
}

size_t wkv6_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N) {
    return wkv5_forward_workspace_bytes(B, T, H, N);
}

wkv_status_t wkv5_forward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype, const float* w,
                          const float* u, const void* r, const void* k, const void* v, float* o,
                          const float* s_in, float* s_out, void* ckpt, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, in_dtype);
    if (p.st != WKV_OK) return p.st;
    const int64_t ns = p.ns;
    if (p.bh == 0) return WKV_OK;
    if ((s_in && !aligned(s_in, 4)) || (s_out && !aligned(s_out, 4))) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (T == 0) return hip_status(wkv::launch_wkv5_state_copy(s_in, s_out, ns, stream));
    if (!w || !u || !r || !k || !v || !o) return WKV_EINVAL;
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(o, 4) || !aligned(r, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        (ckpt && !aligned(ckpt, 16)))
        return WKV_EALIGN;
    int64_t nseg = 1, cps = 0;
    const size_t need = split_bytes(B, T, H, &nseg, &cps);
    if (workspace && (workspace_bytes < need || !aligned(workspace, 256))) return WKV_EWORKSPACE;
    wkv::Wkv5Args a{B, T, H, w, u, static_cast<const uint16_t*>(r), static_cast<const uint16_t*>(k),
                    static_cast<const uint16_t*>(v), o, s_in, s_out};
    a.ckpt = static_cast<uint16_t*>(ckpt);
    if (workspace && nseg > 1)
        return hip_status(run_split<wkv::Wkv5Args, wkv::launch_wkv5_fwd>(a, false, w, nseg, cps, workspace, stream));
    return hip_status(wkv::launch_wkv5_fwd(a, stream));
}

wkv_status_t wkv6_forward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype, const float* w,
                          const float* u, const void* r, const void* k, const void* v, float* o,
                          const float* s_in, float* s_out, void* ckpt, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (p.bh == 0) return WKV_OK;
    if ((s_in && !aligned(s_in, 4)) || (s_out && !aligned(s_out, 4))) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (T == 0) return hip_status(wkv::launch_wkv5_state_copy(s_in, s_out, p.ns, stream));
    if (!w || !u || !r || !k || !v || !o) return WKV_EINVAL;
    if (!aligned(w, 16) || !aligned(u, 4) || !aligned(o, 4) || !aligned(r, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        (ckpt && !aligned(ckpt, 16)))
        return WKV_EALIGN;
    int64_t nseg = 1, cps = 0;
    const size_t need = split_bytes(B, T, H, &nseg, &cps);
    if (workspace && (workspace_bytes < need || !aligned(workspace, 256))) return WKV_EWORKSPACE;
    wkv::Wkv6Args a{B, T, H, w, u, static_cast<const uint16_t*>(r), static_cast<const uint16_t*>(k),
                    static_cast<const uint16_t*>(v), o, s_in, s_out};
    a.ckpt = static_cast<uint16_t*>(ckpt);
    if (workspace && nseg > 1)
        return hip_status(run_split<wkv::Wkv6Args, wkv::launch_wkv6_fwd>(a, true, nullptr, nseg, cps, workspace, stream));
    return hip_status(wkv::launch_wkv6_fwd(a, stream));
}

size_t wkv5_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N, int flags) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, WKV_BF16);
    if (p.st != WKV_OK || p.ws_bytes == 0) return 0;
    return bwd_layout(p, B, T, H, !(flags & WKV_WS_NO_SPLIT), (flags & WKV_WS_HAVE_CKPT) != 0).total;
}

wkv_status_t wkv5_backward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype, const float* w,
                           const float* u, const void* r, const void* k, const void* v, const void* go,
                           const float* s_in, const float* ds_out, float* dr, float* dk, float* dv, float* dw,
                           float* du, float* ds_in, const void* ckpt, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (H == 0) return WKV_OK;
    if (!dw || !du) return WKV_EINVAL;
    if (!aligned(dw, 4) || !aligned(du, 4) || (ds_in && !aligned(ds_in, 4))) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (ds_out && !aligned(ds_out, 4)) return WKV_EALIGN;
    if (B == 0 || T == 0) {  // empty sums: dw = du = 0, and dS0 = dS_T
        const int64_t nc = H * 64;
        hipLaunchKernelGGL(zero2_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, stream, nc,
                           dw, du);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && ds_in != nullptr) e = wkv::launch_wkv5_state_copy(ds_out, ds_in, p.ns, stream);
        return hip_status(e);
    }
    if (!w || !u || !r || !k || !v || !go || !dr || !dk || !dv) return WKV_EINVAL;
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(dr, 4) || !aligned(dk, 4) || !aligned(dv, 4) ||
        (s_in && !aligned(s_in, 4)) || !aligned(r, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(go, 16) ||
        (ckpt && !aligned(ckpt, 16)))
        return WKV_EALIGN;
    if (!workspace || !aligned(workspace, 256)) return WKV_EWORKSPACE;
    const BwdLayout full = bwd_layout(p, B, T, H, true, ckpt != nullptr);
    const BwdLayout l = workspace_bytes >= full.total ? full : bwd_layout(p, B, T, H, false, ckpt != nullptr);
    if (workspace_bytes < l.total) return WKV_EWORKSPACE;
    auto* part = static_cast<float*>(workspace);
    void* split_ws = static_cast<char*>(workspace) + l.split_off;
    const auto* r16 = static_cast<const uint16_t*>(r);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const uint16_t* states = static_cast<const uint16_t*>(ckpt);
    if (ckpt == nullptr) {  // the states before every chunk, recomputed by a state-only forward pass
        auto* tmp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + l.ckpt_off);
        wkv::Wkv5Args fa{B, T, H, w, u, r16, k16, v16, nullptr, s_in, nullptr};
        fa.ckpt = tmp;
        hipError_t e = recompute_split(l, B, H)
                           ? run_split<wkv::Wkv5Args, wkv::launch_wkv5_fwd>(fa, false, w, l.nseg, l.cps, split_ws, stream)
                           : wkv::launch_wkv5_fwd(fa, stream);
        if (e != hipSuccess) return hip_status(e);
        states = tmp;
    }
    wkv::Wkv5BwdArgs ba{B, T, H, w, u, r16, k16, v16, static_cast<const uint16_t*>(go), states, ds_out,
                        dr, dk, dv, part, dw, du, ds_in};
    return hip_status(run_bwd<wkv::Wkv5BwdArgs, wkv::launch_wkv5_bwd>(ba, l, false, workspace, stream));
}

size_t wkv6_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t N) { return wkv5_ckpt_bytes(B, T, H, N); }

size_t wkv6_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N, int flags) {
    return wkv5_backward_workspace_bytes(B, T, H, N, flags);
}

wkv_status_t wkv6_backward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype, const float* w,
                           const float* u, const void* r, const void* k, const void* v, const void* go,
                           const float* s_in, const float* ds_out, float* dr, float* dk, float* dv, float* dw,
                           float* du, float* ds_in, const void* ckpt, void* workspace, size_t workspace_bytes,
                           void* hip_stream) {
    const Wkv5Plan p = wkv5_plan(B, T, H, N, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (H == 0) return WKV_OK;
    if (!du) return WKV_EINVAL;
    if (!aligned(du, 4) || (ds_in && !aligned(ds_in, 4)) || (ds_out && !aligned(ds_out, 4))) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (B == 0 || T == 0) {  // empty sum: du = 0, and dS0 = dS_T (dw has no elements)
        hipError_t e = wkv::launch_shift_zero(du, H * 64, stream);
        if (e == hipSuccess && ds_in != nullptr) e = wkv::launch_wkv5_state_copy(ds_out, ds_in, p.ns, stream);
        return hip_status(e);
    }
    if (!w || !u || !r || !k || !v || !go || !dr || !dk || !dv || !dw) return WKV_EINVAL;
    if (!aligned(w, 16) || !aligned(u, 4) || !aligned(dr, 4) || !aligned(dk, 4) || !aligned(dv, 4) ||
        !aligned(dw, 4) || (s_in && !aligned(s_in, 4)) || !aligned(r, 16) || !aligned(k, 16) || !aligned(v, 16) ||
        !aligned(go, 16) || (ckpt && !aligned(ckpt, 16)))
        return WKV_EALIGN;
    if (!workspace || !aligned(workspace, 256)) return WKV_EWORKSPACE;
    const BwdLayout full = bwd_layout(p, B, T, H, true, ckpt != nullptr);
    const BwdLayout l = workspace_bytes >= full.total ? full : bwd_layout(p, B, T, H, false, ckpt != nullptr);
    if (workspace_bytes < l.total) return WKV_EWORKSPACE;
    auto* part = static_cast<float*>(workspace);
    void* split_ws = static_cast<char*>(workspace) + l.split_off;
    const auto* r16 = static_cast<const uint16_t*>(r);
    const auto* k16 = static_cast<const uint16_t*>(k);
    const auto* v16 = static_cast<const uint16_t*>(v);
    const uint16_t* states = static_cast<const uint16_t*>(ckpt);
    if (ckpt == nullptr) {  // the states before every chunk, recomputed by a state-only forward pass
        auto* tmp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + l.ckpt_off);
        wkv::Wkv6Args fa{B, T, H, w, u, r16, k16, v16, nullptr, s_in, nullptr};
        fa.ckpt = tmp;
        hipError_t e = recompute_split(l, B, H)
                           ? run_split<wkv::Wkv6Args, wkv::launch_wkv6_fwd>(fa, true, nullptr, l.nseg, l.cps, split_ws, stream)
                           : wkv::launch_wkv6_fwd(fa, stream);
        if (e != hipSuccess) return hip_status(e);
        states = tmp;
    }
    wkv::Wkv6BwdArgs ba{B, T, H, w, u, r16, k16, v16, static_cast<const uint16_t*>(go), states, ds_out,
                        dr, dk, dv, dw, part, du, ds_in};
    return hip_status(run_bwd<wkv::Wkv6BwdArgs, wkv::launch_wkv6_bwd>(ba, l, true, workspace, stream));
}

size_t wkv_token_shift_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t M) {
    const ShiftPlan p = shift_plan(B, T, C, M, WKV_F32);
    return p.st == WKV_OK ? p.ws_bytes : 0;
}

wkv_status_t wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, int in_dtype, const float* mu,
                             const void* x, const void* x_prev, void* out, void* hip_stream) {
    const ShiftPlan p = shift_plan(B, T, C, M, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (p.N == 0) return WKV_OK;
    if (!mu || !x || !out) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(mu, 4) || !aligned(x, es) || !aligned(out, es) || (x_prev && !aligned(x_prev, es)))
        return WKV_EALIGN;
    const bool bf = in_dtype == WKV_BF16;
    wkv::ShiftArgs a{B, T, C, M, bf, false, mu, x, x_prev, out, nullptr, nullptr, nullptr, nullptr, nullptr};
    a.vec = C % wkv::shift_vector_width(bf, false) == 0 && aligned(mu, 16) && aligned(x, 16) && aligned(out, 16) &&
            (!x_prev || aligned(x_prev, 16));
    return hip_status(wkv::launch_shift_fwd(a, static_cast<hipStream_t>(hip_stream)));
}

wkv_status_t wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, int in_dtype,
                                      const float* mu, const void* x, const void* x_prev, const void* gout,
                                      float* dx, float* dmu, float* dx_prev, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
    const ShiftPlan p = shift_plan(B, T, C, M, in_dtype);
    if (p.st != WKV_OK) return p.st;
    if (C == 0) return WKV_OK;
    if (!dmu) return WKV_EINVAL;
    if (!aligned(dmu, 4) || (dx_prev && !aligned(dx_prev, 4))) return WKV_EALIGN;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (p.N == 0) {  // empty sums: dmu = 0, and no token reads the previous input
        hipError_t e = wkv::launch_shift_zero(dmu, M * C, stream);
        if (e == hipSuccess && dx_prev) e = wkv::launch_shift_zero(dx_prev, B * C, stream);
        return hip_status(e);
    }
    if (!mu || !x || !gout || !dx) return WKV_EINVAL;
    const size_t es = in_size(in_dtype);
    if (!aligned(mu, 4) || !aligned(x, es) || !aligned(gout, es) || !aligned(dx, 4) ||
        (x_prev && !aligned(x_prev, es)))
        return WKV_EALIGN;
    if (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 256)) return WKV_EWORKSPACE;
    const bool bf = in_dtype == WKV_BF16;
    wkv::ShiftArgs a{B, T, C, M, bf, false, mu, x, x_prev, nullptr, gout, dx, dmu, dx_prev,
                     static_cast<float*>(workspace)};
    a.vec = C % wkv::shift_vector_width(bf, true) == 0 && aligned(mu, 16) && aligned(x, 16) && aligned(gout, 16) &&
            aligned(dx, 16) && (!x_prev || aligned(x_prev, 16)) && (!dx_prev || aligned(dx_prev, 16));
    return hip_status(wkv::launch_shift_bwd(a, stream));
}

const char* wkv_status_str(wkv_status_t s) {
    switch (s) {
        case WKV_OK: return "ok";
        case WKV_EINVAL: return "invalid argument (negative dimension or NULL pointer)";
        case WKV_EDTYPE: return "unknown dtype or op";
        case WKV_ESIZE: return "size overflow or beyond kernel indexing limits";
        case WKV_EALIGN: return "pointer not aligned to its element size";
        case WKV_EWORKSPACE: return "workspace missing or too small";
        case WKV_EHIP: return "HIP launch failed";
        case WKV_ETIMEOUT: return "a wait between workgroups gave up (outputs invalid), or the workspace was not "
                                  "zero-filled before its first use";
        case WKV_ESCRATCH: return "the problem needs more scratch memory than the library's static buffer holds";
        default: return "unknown status";
    }
}

wkv_status_t wkv_workspace_status(const void* workspace, size_t workspace_bytes, int clear, void* hip_stream) {
    if (!workspace) return WKV_EINVAL;
    if (workspace_bytes < 8 || !aligned(workspace, 256)) return WKV_EWORKSPACE;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    const char* err = static_cast<const char*>(workspace) + offsetof(wkv::CallHdrLayout, error);
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, err, sizeof(word), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e == hipSuccess && clear && word != 0u) {
        const uint32_t zero = 0u;
        e = hipMemcpyAsync(const_cast<char*>(err), &zero, sizeof(zero), hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
    }
    if (e != hipSuccess) return hip_status(e);
    return word == 0u ? WKV_OK : WKV_ETIMEOUT;
}

uint32_t wkv_debug_spin_limit(uint32_t polls) { return g_spin_limit.exchange(polls, std::memory_order_relaxed); }

const char* wkv_last_hip_error(void) { return g_hip_msg; }

const char* wkv_version(void) { return "0.1.0"; }

}  // extern "C"
