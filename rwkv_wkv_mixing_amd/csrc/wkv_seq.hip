// Lane-sequential WKV kernels: one thread per (b, c) lane walks all T tokens.
//
// These are the reference-shaped GPU kernels (simple, general, any shape):
//   fwd_seq   forward, optionally saving block-start states (ckpt);
//   bwd_seq   backward in two sweeps over each lane, with per-token forward
//             quantities staged in the caller's workspace;
//   reduce_dwdu  fixed-order sum of per-lane dw/du partials over b.
// Consecutive threads take consecutive channels, so every per-token load and
// store of a wavefront is one contiguous 64-channel run of a [B, T, C] row.
#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkv {

template <typename TIn>
__global__ void __launch_bounds__(256) fwd_seq_kernel(int64_t B, int64_t T, int64_t C,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ u,
                                                      const TIn* __restrict__ k,
                                                      const TIn* __restrict__ v,
                                                      float* __restrict__ y,
                                                      float* __restrict__ ckpt, int64_t nblk) {
    const int64_t lane = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (lane >= B * C) return;
    const int64_t b = lane / C, c = lane - b * C;
    const Chan ch = make_chan(w[c], u[c]);
    St st = empty_state();
    const int64_t base = b * T * C + c;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t i = base + t * C;
        if (ckpt != nullptr && (t % kCkptLen) == 0) {
            float* cp = ckpt + ((b * nblk + t / kCkptLen) * 3) * C + c;
            cp[0] = st.a;
            cp[C] = st.b;
            cp[2 * C] = st.s;
        }
        const float kk = Ld<TIn>::at(k, i);
        const float vv = Ld<TIn>::at(v, i);
        const float x = key_offset(st, kk);
        y[i] = token_out(st, x, vv, ch).y;
        token_update(st, x, vv, ch);
    }
}

// Backward, two sweeps per lane (derivation: gradient of the section-3.2 sum
// of "RWKV（Receptance Weighted Key Value）概念"; see the float64 oracle).
//
// Forward sweep, in MEAN form: the state is the history mean m = A/B, the
// scaled denominator b = B/2^s and the scale s.  Per token, with
// delta = v - m, pi = e^{u+k}/D, rho = 2^s/D, lam = e^k/B_t, lamc = 1 - lam:
//     y = m + pi delta,   v - y = (1 - pi) delta,   m_t = m + lam delta.
// Differences of outputs are carried through these increments rather than
// formed from rounded outputs: where one token dominates, every later y_s
// rounds to the same float32 value, but y_s - m_t stays exact this way.
//
// Reverse sweep (decay again applied as the split product dhi + dlo: these
// sums cancel strongly, and a single rounded d would weight a token s - t
// steps away with a relative error of (s - t) 2^-24):
// G_t = sum_{s>t} gy_s d^{s-1-t} / D_s and, instead
// of H_t = sum gy_s y_s d^{s-1-t} / D_s, the centred J_t = H_t - m_t G_t
// (and J'_t = H'_t - m_t G'_t), all scaled by 2^{s_t}:
//     G_{t-1}  = d G_t + gy_t rho_t
//     J_{t-1}  = d (J_t + lam_t delta_t G_t) + gy_t rho_t pi_t delta_t
//     G'_{t-1} = d (G'_t + G_t)
//     J'_{t-1} = d (J'_t + J_t + lam_t delta_t (G'_t + G_t))
// and, with e_t = e^{k_t}/2^{s_t}, v_t - m_t = lamc_t delta_t:
//     dv_t = gy_t pi_t + e_t G_t
//     dk_t = gy_t pi_t (v_t - y_t) + e_t ((v_t - m_t) G_t - J_t)
//     du  += gy_t pi_t (v_t - y_t),    dw -= e_t ((v_t - m_t) G'_t - J'_t).
struct MeanStep {
    float y, delta, pi, pic, rho, lam, lamc;
};

// One token of the mean-form forward; updates (m, b, s) and returns the
// per-token quantities the reverse sweep needs.
__device__ __forceinline__ MeanStep mean_token(float& m, float& b, float& s, float k, float v,
                                               const Chan& ch) {
    float x = fmaf(k, kL2E, -s);
    if (x > kBig || !(b >= kLo) || b > kHi) {
        const float lvl = b > 0.f ? s + lg2(b) : -INFINITY;
        const float sn = fmaxf(lvl, k * kL2E);
        b *= ex2(s - sn);
        s = sn;
        x = fmaf(k, kL2E, -s);
    }
    const float z = x + ch.u2;
    const float ez = ex2(-fabsf(z));
    const bool zp = z > 0.f;
    const float co = zp ? ez : 1.f;
    const float cn = zp ? 1.f : ez;
    const float r = rcp(fmaf(b, co, cn));
    MeanStep o;
    o.pi = cn * r;
    o.rho = co * r;
    o.pic = o.rho * b;  // 1 - pi, without cancellation
    o.delta = v - m;
    o.y = fmaf(o.pi, o.delta, m);
    const float e = ex2(x);
    const float db = fmaf(ch.dhi, b, ch.dlo * b);
    b = db + e;
    const float rb = rcp(fmaxf(b, 1e-37f));  // b = 0 only if both terms underflow
    o.lam = e * rb;
    o.lamc = db * rb;  // 1 - lam, without cancellation
    m = fmaf(o.lam, o.delta, m);
    return o;
}

template <typename TIn>
__global__ void __launch_bounds__(256) bwd_seq_kernel(int64_t B, int64_t T, int64_t C,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ u,
                                                      const TIn* __restrict__ k,
                                                      const TIn* __restrict__ v,
                                                      const TIn* __restrict__ gy,
                                                      float* __restrict__ dk,
                                                      float* __restrict__ dv,
                                                      float* __restrict__ ws, int64_t N,
                                                      float* __restrict__ part_dw,
                                                      float* __restrict__ part_du) {
    const int64_t lane = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (lane >= B * C) return;
    const int64_t b = lane / C, c = lane - b * C;
    const Chan ch = make_chan(w[c], u[c]);
    const int64_t base = b * T * C + c;
    float* s_delta = ws;
    float* s_pi = s_delta + N;
    float* s_pic = s_pi + N;
    float* s_rho = s_pic + N;
    float* s_lam = s_rho + N;
    float* s_lamc = s_lam + N;
    float* s_s = s_lamc + N;
    float m = 0.f, bb = 0.f, sc = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t i = base + t * C;
        const MeanStep o = mean_token(m, bb, sc, Ld<TIn>::at(k, i), Ld<TIn>::at(v, i), ch);
        s_delta[i] = o.delta;
        s_pi[i] = o.pi;
        s_pic[i] = o.pic;
        s_rho[i] = o.rho;
        s_lam[i] = o.lam;
        s_lamc[i] = o.lamc;
        s_s[i] = sc;
    }
    float G = 0.f, J = 0.f, Gp = 0.f, Jp = 0.f, acc_dw = 0.f, acc_du = 0.f;
    float s_next = s_s[base + (T - 1) * C];
    for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t i = base + t * C;
        const float s_t = s_next;
        const float g = Ld<TIn>::at(gy, i);
        const float dl = s_delta[i];
        const float pi = s_pi[i];
        const float e = ex2(fmaf(Ld<TIn>::at(k, i), kL2E, -s_t));
        const float vm = s_lamc[i] * dl;
        const float vy = s_pic[i] * dl;
        const float gpi = g * pi;
        dv[i] = fmaf(e, G, gpi);
        dk[i] = fmaf(gpi, vy, e * fmaf(vm, G, -J));
        acc_du = fmaf(gpi, vy, acc_du);
        acc_dw = fmaf(e, fmaf(vm, Gp, -Jp), acc_dw);
        const float ld = s_lam[i] * dl;
        const float gr = g * s_rho[i];
        const float GG = Gp + G;
        const float tJp = fmaf(ld, GG, Jp + J);
        Jp = fmaf(ch.dhi, tJp, ch.dlo * tJp);
        Gp = fmaf(ch.dhi, GG, ch.dlo * GG);
        const float tJ = fmaf(ld, G, J);
        J = fmaf(ch.dhi, tJ, fmaf(ch.dlo, tJ, gr * (pi * dl)));
        G = fmaf(ch.dhi, G, fmaf(ch.dlo, G, gr));
        if (t > 0) {
            s_next = s_s[i - C];
            if (s_next != s_t) {
                const float f = ex2(s_next - s_t);
                G *= f;
                J *= f;
                Gp *= f;
                Jp *= f;
            }
        }
    }
    part_dw[lane] = -acc_dw;
    part_du[lane] = acc_du;
}

// dw[c] = sum_b part_dw[b, c] (same for du), summed in increasing b.
__global__ void __launch_bounds__(256) reduce_dwdu_kernel(int64_t B, int64_t C,
                                                          const float* __restrict__ part_dw,
                                                          const float* __restrict__ part_du,
                                                          float* __restrict__ dw,
                                                          float* __restrict__ du) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (c >= C) return;
    float sw = 0.f, su = 0.f;
    for (int64_t b = 0; b < B; ++b) {
        sw += part_dw[b * C + c];
        su += part_du[b * C + c];
    }
    dw[c] = sw;
    du[c] = su;
}

constexpr int64_t kSeqStaged = 7;  // per-token floats staged by bwd_seq

static inline unsigned blocks_for(int64_t n, int threads) {
    return static_cast<unsigned>((n + threads - 1) / threads);
}

template <typename TIn>
hipError_t launch_fwd_seq_t(const FwdArgs& a, hipStream_t stream) {
    const int64_t lanes = a.B * a.C;
    hipLaunchKernelGGL(fwd_seq_kernel<TIn>, dim3(blocks_for(lanes, 256)), dim3(256), 0, stream,
                       a.B, a.T, a.C, a.w, a.u, static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.y, static_cast<float*>(a.ckpt), a.nblk);
    return hipGetLastError();
}

hipError_t launch_fwd_seq(const FwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_fwd_seq_t<uint16_t>(a, stream) : launch_fwd_seq_t<float>(a, stream);
}

template <typename TIn>
hipError_t launch_bwd_seq_t(const BwdArgs& a, hipStream_t stream) {
    const int64_t lanes = a.B * a.C;
    const int64_t N = lanes * a.T;
    float* ws = static_cast<float*>(a.ws);
    float* part_dw = ws + kSeqStaged * N;
    float* part_du = part_dw + lanes;
    hipLaunchKernelGGL(bwd_seq_kernel<TIn>, dim3(blocks_for(lanes, 256)), dim3(256), 0, stream,
                       a.B, a.T, a.C, a.w, a.u, static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), static_cast<const TIn*>(a.gy), a.dk, a.dv,
                       ws, N, part_dw, part_du);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_dwdu_kernel, dim3(blocks_for(a.C, 256)), dim3(256), 0, stream, a.B,
                       a.C, part_dw, part_du, a.dw, a.du);
    return hipGetLastError();
}

size_t bwd_seq_workspace_bytes(int64_t B, int64_t T, int64_t C) {
    return static_cast<size_t>(kSeqStaged * B * T * C + 2 * B * C) * sizeof(float);
}

hipError_t launch_bwd_seq(const BwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_bwd_seq_t<uint16_t>(a, stream) : launch_bwd_seq_t<float>(a, stream);
}

}  // namespace wkv
