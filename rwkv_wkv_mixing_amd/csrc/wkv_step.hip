// Recurrent-mode (decode) step: one token for L x B independent WKV states.
//
// "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section "关键设计 4"
// (output read from the previous state, then decay-and-add).  The state is
// (a, b, p) with A = a e^p, B = b e^p.  As in the sequence kernels, the
// exponent p only moves on a rescale (a new key more than e^22 above it, or
// b outside [2^-32, 2^32]), where it jumps to the running max
// max(k, p + ln b); the decay itself is applied to (a, b) as a product with
// e^{-w} split into float32 hi + lo parts, so no per-token rounding of p - w
// acts as a systematic change of w.
//
// Memory-bound: 32 bytes per lane for bf16 inputs (read a, b, p, k, v; write
// y, a, b, p).  A thread owns a group of 4 channels (or 1) of one layer for
// `spt` consecutive streams, so the per-channel constants (including the
// float64 exp that splits e^{-w}) are computed once per group and every
// access of a wavefront is one contiguous row segment.  spt is chosen at
// launch: up to kMaxStreamsPerThread while that still leaves kThreadsPerCu
// threads per CU.  Measured at 32 layers x 256 streams x 4096 channels: one
// stream per thread (the grid then covers every group once) takes 194 us
// against 214 us for 16 streams per thread (2,048 threads per CU) and 207 us
// for 4: the per-group constants cost nothing beside the memory traffic, while
// a thread walking several streams has one stream's loads in flight at a time.
#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkv {

constexpr int64_t kMaxStreamsPerThread = 16;
constexpr int64_t kThreadsPerCu = 32768;
constexpr float kRescaleX = 22.0f;  // e^22 ~ 2^32

struct StepChan {
    float dhi, dlo, u;
};

__device__ __forceinline__ StepChan step_chan(float w, float u) {
    StepChan c;
    const double dd = exp(-static_cast<double>(w));
    c.dhi = static_cast<float>(dd);
    c.dlo = static_cast<float>(dd - static_cast<double>(c.dhi));
    c.u = u;
    return c;
}

// One token on one lane; a, b, p updated in place, returns y.
__device__ __forceinline__ float step_lane(const StepChan& ch, float k, float v, float& a, float& b,
                                           float& p) {
    p = fmaxf(p, -1e38f);  // -inf (empty) behaves as the finite sentinel
    float x = k - p;
    if (x > kRescaleX || !(b >= kLo) || b > kHi) {
        const float lvl = b > 0.f ? p + __logf(b) : -INFINITY;
        const float pn = fmaxf(lvl, k);
        const float f = ex2((p - pn) * kL2E);
        a *= f;
        b *= f;
        p = pn;
        x = k - p;
    }
    // output from the state before the token; z = log weight of the token
    const float z = x + ch.u;
    const float az = fabsf(z);
    const float ez = ex2(-fmaf(az, kL2E, az * kL2E_lo));
    const bool zp = z > 0.f;
    const float co = zp ? ez : 1.f;
    const float cn = zp ? 1.f : ez;
    const float y = fmaf(a, co, cn * v) * rcp(fmaf(b, co, cn));
    // decay-and-add
    const float e = ex2(fmaf(x, kL2E, x * kL2E_lo));
    a = fmaf(ch.dhi, a, fmaf(ch.dlo, a, e * v));
    b = fmaf(ch.dhi, b, fmaf(ch.dlo, b, e));
    return y;
}

template <typename TIn>
__global__ void __launch_bounds__(256) step_kernel_scalar(int64_t L, int64_t B, int64_t C,
                                                          int64_t nbt, int64_t spt,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ u,
                                                          const TIn* __restrict__ k,
                                                          const TIn* __restrict__ v,
                                                          float* __restrict__ y, float* a,
                                                          float* b, float* p) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= L * nbt * C) return;
    const int64_t c = t % C;
    const int64_t bt = (t / C) % nbt;
    const int64_t l = t / (C * nbt);
    const StepChan ch = step_chan(w[l * C + c], u[l * C + c]);
    const int64_t b_end = (bt + 1) * spt < B ? (bt + 1) * spt : B;
    for (int64_t s = bt * spt; s < b_end; ++s) {
        const int64_t i = (l * B + s) * C + c;
        float aa = a[i], bb = b[i], pp = p[i];
        y[i] = step_lane(ch, Ld<TIn>::at(k, i), Ld<TIn>::at(v, i), aa, bb, pp);
        a[i] = aa;
        b[i] = bb;
        p[i] = pp;
    }
}

template <typename TIn>
struct Vec4In;
// Group g's 4 inputs, read with the non-temporal hint: a token's k and v are read once (the state,
// read again by the next step, keeps the default policy).  216.4 -> 213.0 us at 32 layers x 256
// streams x 4096 channels, bf16.
template <>
struct Vec4In<float> {
    typedef float nf4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ void load(const float* p, int64_t g, float out[4]) {
        const nf4 r = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p) + g);
        out[0] = r.x; out[1] = r.y; out[2] = r.z; out[3] = r.w;
    }
};
template <>
struct Vec4In<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, int64_t g, float out[4]) {
        const uint64_t r = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p) + g);  // 4 bf16
        const uint32_t lo = static_cast<uint32_t>(r), hi = static_cast<uint32_t>(r >> 32);
        out[0] = __uint_as_float(lo << 16);
        out[1] = __uint_as_float(lo & 0xffff0000u);
        out[2] = __uint_as_float(hi << 16);
        out[3] = __uint_as_float(hi & 0xffff0000u);
    }
};

// 4 channels per thread: C % 4 == 0, float pointers 16-byte aligned, k and v
// aligned to 4 elements.
template <typename TIn>
__global__ void __launch_bounds__(256) step_kernel_vec4(int64_t L, int64_t B, int64_t C,
                                                        int64_t nbt, int64_t spt,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ u,
                                                        const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v,
                                                        float* __restrict__ y, float* a,
                                                        float* b, float* p) {
    using V = Vec4In<TIn>;
    const int64_t C4 = C / 4;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= L * nbt * C4) return;
    const int64_t c4 = t % C4;
    const int64_t bt = (t / C4) % nbt;
    const int64_t l = t / (C4 * nbt);
    const float4 w4 = reinterpret_cast<const float4*>(w)[l * C4 + c4];
    const float4 u4 = reinterpret_cast<const float4*>(u)[l * C4 + c4];
    const StepChan ch[4] = {step_chan(w4.x, u4.x), step_chan(w4.y, u4.y), step_chan(w4.z, u4.z),
                            step_chan(w4.w, u4.w)};
    const int64_t b_end = (bt + 1) * spt < B ? (bt + 1) * spt : B;
    for (int64_t s = bt * spt; s < b_end; ++s) {
        const int64_t g = (l * B + s) * C4 + c4;
        float kf[4], vf[4];
        V::load(k, g, kf);
        V::load(v, g, vf);
        const float4 a4 = reinterpret_cast<const float4*>(a)[g];
        const float4 b4 = reinterpret_cast<const float4*>(b)[g];
        const float4 p4 = reinterpret_cast<const float4*>(p)[g];
        float aa[4] = {a4.x, a4.y, a4.z, a4.w};
        float bb[4] = {b4.x, b4.y, b4.z, b4.w};
        float pp[4] = {p4.x, p4.y, p4.z, p4.w};
        float yo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) yo[j] = step_lane(ch[j], kf[j], vf[j], aa[j], bb[j], pp[j]);
        reinterpret_cast<float4*>(y)[g] = make_float4(yo[0], yo[1], yo[2], yo[3]);
        reinterpret_cast<float4*>(a)[g] = make_float4(aa[0], aa[1], aa[2], aa[3]);
        reinterpret_cast<float4*>(b)[g] = make_float4(bb[0], bb[1], bb[2], bb[3]);
        reinterpret_cast<float4*>(p)[g] = make_float4(pp[0], pp[1], pp[2], pp[3]);
    }
}

template <typename TIn>
hipError_t launch_step_t(const StepArgs& s, hipStream_t stream) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t groups = s.L * s.B * (s.vec4 ? s.C / 4 : s.C);  // (layer, stream, channel group) items
    int64_t spt = groups / (static_cast<int64_t>(ncu) * kThreadsPerCu);
    spt = spt < 1 ? 1 : (spt > kMaxStreamsPerThread ? kMaxStreamsPerThread : spt);
    const int64_t nbt = (s.B + spt - 1) / spt;
    if (s.vec4) {
        const int64_t threads = s.L * nbt * (s.C / 4);
        hipLaunchKernelGGL(step_kernel_vec4<TIn>, dim3(static_cast<unsigned>((threads + 255) / 256)),
                           dim3(256), 0, stream, s.L, s.B, s.C, nbt, spt, s.w, s.u,
                           static_cast<const TIn*>(s.k), static_cast<const TIn*>(s.v), s.y, s.a,
                           s.b, s.p);
    } else {
        const int64_t threads = s.L * nbt * s.C;
        hipLaunchKernelGGL(step_kernel_scalar<TIn>,
                           dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream,
                           s.L, s.B, s.C, nbt, spt, s.w, s.u, static_cast<const TIn*>(s.k),
                           static_cast<const TIn*>(s.v), s.y, s.a, s.b, s.p);
    }
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs& s, hipStream_t stream) {
    return s.bf16 ? launch_step_t<uint16_t>(s, stream) : launch_step_t<float>(s, stream);
}

}  // namespace wkv
