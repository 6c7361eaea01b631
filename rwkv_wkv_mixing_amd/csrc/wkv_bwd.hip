// Chunked (time-split) WKV backward for gfx950.
//
// Gradients of L = sum gy * y, derived by differentiating the weighted sum of
// "RWKV（Receptance Weighted Key Value）概念", section 3.2 (the pages print no
// backward; the float64 oracle documents the formulas).  The forward is
// recomputed on chip from the block-start states the forward saved every
// kCkptLen tokens, in the mean form (history mean m = A/B) so that output
// differences never come from rounded outputs:
//     delta = v - m,  pi = e^{u+k}/D,  rho = 2^s/D,  lam = e^k/B_t,  m_t = m + lam delta.
// The per-token reverse accumulators, scaled by 2^{s}, run in float32
// (float64 when built with WKV_BWD_ACC_F64=1, which measured no better once
// the states were exact); the span maps, their composition and the carries
// between workgroups are float64.  At a dominant token the gradient sums
// ~10^2 signed terms of order one whose total can be ~10^-3 of that; what
// keeps those terms consistent with each other is the exact integer-scale
// arithmetic of the lane state and a key weight formed the same way in every
// pass (k log2 e in two words, scaled by an integer power of two).  The
// accumulators are
//     G_{t-1}  = d G_t + gy_t rho_t
//     J_{t-1}  = d (J_t + lam_t delta_t G_t) + gy_t rho_t pi_t delta_t     (J = H - m G)
//     G'_{t-1} = d (G'_t + G_t)
//     J'_{t-1} = d (J'_t + J_t + lam_t delta_t (G'_t + G_t))
// and with e_t = e^{k_t}/2^{s_t}:
//     dv_t = gy_t pi_t + e_t G_t
//     dk_t = gy_t pi_t (1 - pi_t) delta_t + e_t ((1 - lam_t) delta_t G_t - J_t)
// (1 - pi and 1 - lam are formed as rho b and d b / B_t, never by subtraction)
//     du  += gy_t pi_t (1 - pi_t) delta_t,   dw -= e_t ((1 - lam_t) delta_t G'_t - J'_t).
//
// Work decomposition: as the forward, a workgroup owns 64 channels x W*L
// tokens, wave i owns L tokens.  The reverse carry (G, J, G', J') through n
// tokens is the affine map
//     C_start = d^n [[1,0,0,0],[S,1,0,0],[n,0,1,0],[nS,n,S,1]] C_end + c0,
//     S = sum lam_t delta_t,   c0 = sum_u d^u gr_u (1, P_u + pi_u delta_u, u, u (P_u + pi_u delta_u))
// (gr_u = gy_u rho_u, P_u = sum_{t<u} lam_t delta_t, u counted from the span's
// first token).  This form is closed under composition (n and S add), and its
// offset accumulates in forward time during the recompute, so each wave
// summarises its span without an extra reverse sweep.  Waves compose the maps
// of the later waves through LDS; blocks are chained backward in time through
// the same coherent 32-byte slots as the forward's carries.  dw and du are
// per-block partial sums, reduced over batch rows and blocks in a fixed order.
#include "wkv_launch.h"
#include "wkv_scan.h"

namespace wkv {

struct BwdChunk {
    int64_t B, T, C;
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    const void* gy;
    float* dk;
    float* dv;
    const float* ckpt;
    int64_t nblk_ck;
    int64_t nct, ntiles, nblocks;
    CallHdr* hdr;          // workspace header: error word, finished streams, generation (time-split kernel)
    StreamCtr* sc;         // [kMaxStreams] ticket streams (time-split kernel)
    int64_t nstream;       // streams in use; divides ntiles
    uint32_t spin;         // polls before a carry wait gives up
    uint32_t* fold;        // [kFoldLines][16]: workgroups of the channel tiles ct = q mod kFoldLines that have stored their partials
    int64_t npb;           // partial rows per tile: time blocks (time-split kernel) or 1 (whole-tile)
    float* dw;             // [C] outputs, written by the last workgroup of each channel tile
    float* du;
    float* carry;          // [ntiles][nblocks][64][12]: G, J, G', J' as hi/lo pairs, scale, 3 status words
    uint32_t carry_bytes;
    float* part;           // [ntiles][nblocks][2][64]: dw, du partial sums
    const void* r;         // receptance [B, T, C] (gated kernels; gy is then the gradient of sigmoid(r) y)
    float* dr;             // [B, T, C] gradient of r (gated kernels)
    // backward through carried state (St kernels), each [B, C] or NULL: the state given before the
    // first token (a, b, p), the gradient (ga, gb) of the state handed on after the last token at the
    // p the forward wrote, and the gradients of the given state
    const float* a_in;
    const float* b_in;
    const float* p_in;
    const float* ga_out;
    const float* gb_out;
    const float* p_out;
    float* ga_in;
    float* gb_in;
    float* gp_in;
};

// Reverse carry at log2-scale sg: the true G is G * 2^{-sg}.
struct RCarry {
    double G, J, Gp, Jp;
    int sg;
};

// Affine reverse map of a span of n tokens (n = 0: identity).
struct RMap {
    double D;     // d^n
    double S;
    double c[4];  // offset, at scale so
    float n;
    int so;
};

__device__ __forceinline__ RMap rmap_identity() {
    RMap m;
    m.D = 1.0;
    m.S = 0.0;
    m.c[0] = m.c[1] = m.c[2] = m.c[3] = 0.0;
    m.n = 0.f;
    m.so = 0;
    return m;
}

__device__ __forceinline__ RCarry rapply(const RMap& m, const RCarry& X) {
    if (m.n == 0.f) return X;
    const double f = ldexp(m.D, m.so - X.sg);
    const double n = m.n, S = m.S;
    RCarry r;
    r.G = fma(f, X.G, m.c[0]);
    r.J = fma(f, fma(S, X.G, X.J), m.c[1]);
    r.Gp = fma(f, fma(n, X.G, X.Gp), m.c[2]);
    r.Jp = fma(f, fma(n * S, X.G, fma(n, X.J, fma(S, X.Gp, X.Jp))), m.c[3]);
    r.sg = m.so;
    return r;
}

// a spans the tokens just before those of b.
__device__ __forceinline__ RMap rcompose(const RMap& a, const RMap& b) {
    if (b.n == 0.f) return a;
    if (a.n == 0.f) return b;
    const RCarry cb = rapply(a, RCarry{b.c[0], b.c[1], b.c[2], b.c[3], b.so});
    RMap r;
    r.D = a.D * b.D;
    r.n = a.n + b.n;
    r.S = a.S + b.S;
    r.c[0] = cb.G;
    r.c[1] = cb.J;
    r.c[2] = cb.Gp;
    r.c[3] = cb.Jp;
    r.so = a.so;
    return r;
}

// A carry crosses workgroups as float hi + lo pairs (about 48 significant
// bits) in three 16-byte slots, each with its own status word, since the
// three stores may become visible in any order.
__device__ __forceinline__ float hi_of(double x) { return static_cast<float>(x); }
__device__ __forceinline__ float lo_of(double x) {
    return static_cast<float>(x - static_cast<double>(static_cast<float>(x)));
}
__device__ __forceinline__ double join(float hi, float lo) {
    return static_cast<double>(hi) + static_cast<double>(lo);
}

constexpr uint32_t kCarrySlot = 48;

__device__ __forceinline__ void publish_carry(Rsrc r, uint32_t off, const RCarry& c, uint32_t tag) {
    const float one = __uint_as_float(tag);
    const f32x4 v0 = {hi_of(c.G), lo_of(c.G), hi_of(c.J), one};
    const f32x4 v1 = {lo_of(c.J), hi_of(c.Gp), lo_of(c.Gp), one};
    const f32x4 v2 = {hi_of(c.Jp), lo_of(c.Jp), __int_as_float(c.sg), one};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v0), r, off, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v1), r, off + 16, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v2), r, off + 32, 0, kCoherent);
}

__device__ __forceinline__ RCarry wait_carry(Rsrc r, uint32_t off, uint32_t tag, uint32_t spin, CallHdr* h) {
    for (uint32_t it = 0; it < spin; ++it) {
        const f32x4 v0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
        const f32x4 v1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kCoherent));
        const f32x4 v2 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 32, 0, kCoherent));
        if ((__float_as_uint(v0.w) == tag) & (__float_as_uint(v1.w) == tag) & (__float_as_uint(v2.w) == tag))
            return RCarry{join(v0.x, v0.y), join(v0.z, v1.x), join(v1.y, v1.z), join(v2.x, v2.y),
                          __float_as_int(v2.z)};
        __builtin_amdgcn_s_sleep(1);
    }
    hdr_flag(h, kErrWait);
    return RCarry{0.0, 0.0, 0.0, 0.0, 0};
}

template <typename TIn, int L>
struct KvChunk;

template <int L>
struct KvChunk<uint16_t, L> {
    uint32_t kv[L];
    __device__ __forceinline__ void load(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rk, voff, j * row, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rv, voff, j * row, 0);
            kv[j] = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ void load_lds(const uint16_t (*k)[64], const uint16_t (*v)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; ++j) kv[j] = static_cast<uint32_t>(k[j][lane]) | (static_cast<uint32_t>(v[j][lane]) << 16);
    }
    __device__ __forceinline__ float k(int j) const { return __uint_as_float(kv[j] << 16); }
    __device__ __forceinline__ float v(int j) const { return __uint_as_float(kv[j] & 0xffff0000u); }
};

template <int L>
struct KvChunk<float, L> {
    float kk[L], vv[L];
    __device__ __forceinline__ void load(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            kk[j] = BufLd<float>::at(rk, voff, j * row);
            vv[j] = BufLd<float>::at(rv, voff, j * row);
        }
    }
    __device__ __forceinline__ void load_lds(const float (*k)[64], const float (*v)[64], int lane) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            kk[j] = k[j][lane];
            vv[j] = v[j][lane];
        }
    }
    __device__ __forceinline__ float k(int j) const { return kk[j]; }
    __device__ __forceinline__ float v(int j) const { return vv[j]; }
};

// ---- lane recompute in the mean form -------------------------------------------
// History state (m, b, s): m = A / B, B = b 2^s.
struct MSt {
    float m, b;
    int s;
};

// What the reverse sweep needs of one token, at the token's scale s:
// pi = e^{u+k}/D, rho = 2^s/D, e = e^k/2^s, vy = (1-pi)(v-m), vm = (1-lam)(v-m),
// ld = lam (v-m), pd = pi (v-m), lam = e^k/B_t.
struct TokQ {
    float pi, rho, e, vy, vm, ld, pd;
};

// One token of the general path: lazy exact rescale, current-token
// normalisation valid for any u (z = log2 of its weight relative to 2^s).
__device__ __forceinline__ TokQ mean_step(MSt& st, float k, float v, const Chan& ch, float eu, bool fast_out) {
    const Key kk = key_split(k);
    const bool out = (kk.n - st.s > static_cast<int>(kBig)) | !(st.b >= kLo) | (st.b > kHi);
    if (out) {
        const int lvl = st.b > 0.f ? st.s + __builtin_amdgcn_frexp_expf(st.b) : kSEmpty;
        const int sn = max(lvl, kk.n);
        st.b = ldx(st.b, st.s - sn);
        st.s = sn;
    }
    const float e = ldx(kk.em, kk.n - st.s);
    float pi, rho;
    if (fast_out) {
        const float E = e * eu;
        rho = rcp(st.b + E);
        pi = E * rho;
    } else {
        const float z = static_cast<float>(kk.n - st.s) + kk.f + ch.u2;
        const float ez = ex2(-fabsf(z));
        const float co = z > 0.f ? ez : 1.f;
        const float cn = z > 0.f ? 1.f : ez;
        const float r = rcp(fmaf(st.b, co, cn));
        pi = cn * r;
        rho = co * r;
    }
    TokQ q;
    const float dl = v - st.m;
    q.pi = pi;
    q.rho = rho;
    q.e = e;
    q.vy = (rho * st.b) * dl;  // (1 - pi) delta without the subtraction
    const float db = fmaf(ch.dhi, st.b, ch.dlo * st.b);
    st.b = db + e;
    const float rb = rcp(fmaxf(st.b, 1e-37f));
    q.ld = (e * rb) * dl;
    q.vm = (db * rb) * dl;  // (1 - lam) delta without the subtraction
    q.pd = pi * dl;
    st.m += q.ld;
    return q;
}

// Per-token running sums of the fast path: float32, or float64 when built with
// WKV_BWD_ACC_F64=1.
#ifndef WKV_BWD_ACC_F64
#define WKV_BWD_ACC_F64 0
#endif
#if WKV_BWD_ACC_F64
using acc_t = double;
#else
using acc_t = float;
#endif

// x * d with d = dhi + dlo (float32: two FMAs, ~2^-48 relative) or d in float64.
struct Decay {
    float dhi, dlo;
    double dd;
    __device__ __forceinline__ float mul(float x) const { return fmaf(dhi, x, dlo * x); }
    __device__ __forceinline__ double mul(double x) const { return dd * x; }
};


#ifndef WKV_BWD_OCC
#define WKV_BWD_OCC 1  // minimum waves per SIMD asked of the register allocator
#endif

// ---- one wave's span of L tokens ----------------------------------------------
// Where a span's data lives for one lane.
struct SpanGeo {
    Rsrc rk, rv, rg, rr, rdk, rdv, rdr;
    uint32_t vin, vout, row_in, row_out;
    const float* ck;  // saved state at the span start, or nullptr
};

// Geometry of wave `wave`'s span in time block `blk` of batch row b (W L tokens
// per block).  Tokens past T read as zeros and their stores are dropped.
template <typename TIn, int L, int W>
__device__ __forceinline__ SpanGeo span_geo(const BwdChunk& P, int64_t b, int64_t c, bool cok, int64_t blk, int wave) {
    constexpr int ES = BufLd<TIn>::kBytes;
    const int64_t tb0 = blk * (int64_t)(L * W);
    const int64_t t0 = tb0 + (int64_t)wave * L;
    const int64_t blk_tokens = (P.T - tb0) < (int64_t)(L * W) ? (P.T - tb0) : (int64_t)(L * W);
    const int64_t row0 = (b * P.T + tb0) * P.C;
    const uint32_t nin = (uint32_t)(blk_tokens * P.C * ES), nout = (uint32_t)(blk_tokens * P.C * 4);
    SpanGeo g;
    g.rk = make_rsrc(static_cast<const TIn*>(P.k) + row0, nin);
    g.rv = make_rsrc(static_cast<const TIn*>(P.v) + row0, nin);
    g.rg = make_rsrc(static_cast<const TIn*>(P.gy) + row0, nin);
    g.rdk = make_rsrc(P.dk + row0, nout);
    g.rdv = make_rsrc(P.dv + row0, nout);
    g.rr = P.r != nullptr ? make_rsrc(static_cast<const TIn*>(P.r) + row0, nin) : make_rsrc(nullptr, 0);
    g.rdr = P.dr != nullptr ? make_rsrc(P.dr + row0, nout) : make_rsrc(nullptr, 0);
    const uint32_t lin = cok ? (uint32_t)((int64_t)wave * L * P.C + c) : kOffNone;
    g.vin = cok ? lin * ES : kOffNone;
    g.vout = cok ? lin * 4 : kOffNone;
    g.row_in = (uint32_t)(P.C * ES);
    g.row_out = (uint32_t)(P.C * 4);
    g.ck = (cok && t0 < P.T) ? P.ckpt + ((b * P.nblk_ck + t0 / kCkptLen) * 3) * P.C + c : nullptr;
    return g;
}

// The inputs k, v, gy (and, NI = 4, the gate's r) of one time block staged in LDS:
// [wave][input][token][channel].
template <typename TIn, int L, int W, int NI = 3>
struct BwdStage {
    TIn x[W][NI][L][64];
};

// Start the asynchronous copies of wave `wave`'s span of k, v, gy (and r) into LDS.
template <typename TIn, int L, int W, int NI>
__device__ __forceinline__ void stage_span(BwdStage<TIn, L, W, NI>& st, const SpanGeo& g, int wave, int lane,
                                           int64_t c0, int64_t C) {
    stage_rows<TIn, L, kStageLast>(g.rk, st.x[wave][0], int64_t{wave} * L, c0, C, lane);
    stage_rows<TIn, L, kStageLast>(g.rv, st.x[wave][1], int64_t{wave} * L, c0, C, lane);
    stage_rows<TIn, L, kStageLast>(g.rg, st.x[wave][2], int64_t{wave} * L, c0, C, lane);
    if constexpr (NI == 4) stage_rows<TIn, L, kStageLast>(g.rr, st.x[wave][3], int64_t{wave} * L, c0, C, lane);
}

// A span's inputs, loaded ahead of use (gy holds the output gradient; with
// the gate, r too).
template <typename TIn, int L, bool Gated>
struct SpanIn {
    KvChunk<TIn, L> kv;
    Chunk1<TIn, L> gy;
    float a0, b0, s0;
    __device__ __forceinline__ void load(const SpanGeo& g, int64_t C) {
        kv.load(g.rk, g.rv, g.vin, g.row_in);
        gy.load(g.rg, g.vin, g.row_in);
        load_ck(g, C);
    }
    __device__ __forceinline__ void load_ck(const SpanGeo& g, int64_t C) {
        a0 = 0.f;
        b0 = 0.f;
        s0 = static_cast<float>(kSEmpty);
        if (g.ck != nullptr) {
            a0 = g.ck[0];
            b0 = g.ck[C];
            s0 = g.ck[2 * C];
        }
    }
    template <int W, int NI>
    __device__ __forceinline__ void load_lds(const BwdStage<TIn, L, W, NI>& st, int wave, int lane) {
        kv.load_lds(st.x[wave][0], st.x[wave][1], lane);
        gy.load_lds(st.x[wave][2], lane);
    }
};

// Forward recompute of a span, its reverse map, and (fast path) the per-token
// products of the reverse sweep: gpi = gy pi, gvy = gy pi vy, gr = gy rho,
// grpd = gy rho pd, e, vm, ld.  Gated: gy = gout sigmoid(r) and the recompute
// also writes dr = gout y sigmoid(r) (1 - sigmoid(r)), y = m + pi (v - m).
// The gradient of the state a backward through carried state hands on, as gradients of the plain
// sums: gA = ga 2^{-s}, gB = gb 2^{-s} (zero: no gradient).
struct Seed {
    float ga = 0.f, gb = 0.f;
    int s = 0;
};

// Largest scale step of the backward's fast path (Span::recompute): keys then weigh at most 2^60,
// e^u at most 2^58 more, and the span's sums of key weights at most 17 * 2^60, inside float32.
constexpr int kMaxShift = 60;

template <typename TIn, int L, bool Gated>
struct Span {
    float gpi[L], gvy[L], gr[L], grpd[L], e[L], vm[L], ld[L];
    acc_t Psum, Gs, Js, Gps, Jps;
    float du;
    int so;     // scale of the map offsets (and of the whole fast-path sweep)
    bool fast;  // wave-uniform
    MSt x0;
    float mT;  // the mean after the span's last token (the handed-on state's, in the span ending at T)

    // rg: the gate's inputs of the span (used when Gated; not part of SpanIn so
    // that the whole-tile kernel does not double-buffer them)
    //
    // Inj (backward through carried state, the span holding token T as its token tcut, 0 < tcut < L):
    // the tokens from T on read as zeros (gy = 0 included) and add nothing; the handed-on state's
    // gradient sd joins as the reverse seed of token tcut, so that the carry before that token is
    // (G, J) = (gA, -gB - m_T gA) with m_T the mean before it.  Through gr and grpd it reaches the
    // map's offsets and the reverse sweep without further code.
    template <bool Inj = false>
    __device__ __forceinline__ void recompute(const SpanIn<TIn, L, Gated>& in, const Chunk1<TIn, L>& rg,
                                              const SpanGeo& g, const Chan& ch, float eu, const Decay& dec,
                                              bool fast_out, int tcut = 0, const Seed& sd = Seed{}) {
        x0.s = static_cast<int>(in.s0);
        x0.b = in.b0;
        x0.m = in.b0 > 0.f ? in.a0 / in.b0 : 0.f;
        // fixed span scale: the larger of the history level and the largest key
        float kmax = -INFINITY, kmin = INFINITY;
#pragma unroll
        for (int j = 0; j < L; ++j) {
            kmax = fmaxf(kmax, in.kv.k(j));
            kmin = fminf(kmin, in.kv.k(j));
        }
        const int lvl0 = x0.b > 0.f ? x0.s + __builtin_amdgcn_frexp_expf(x0.b) : kSEmpty;
        const int sc = max(lvl0, key_split(kmax).n);
        // Every denominator of the fast path is at least min_j e^{k_j} min(e^u, 1) (D_t >=
        // e^{u+k_t}, B_t >= e^{k_t}).  Where that bound lies more than 2^96 below 2^sc (a key spike
        // beside a very small key in a fast-decaying channel) the lane carries its span 2^shift
        // higher, at the scale so = sc - shift: each key weight is the same exact fraction times an
        // exact power of two, and the denominators stay above kTiny.  Otherwise the wave would take
        // the general path, whose per-token recomputation re-reads the span's inputs O(L^2) times:
        // two such waves among 32,768 held a whole call back by a fifth.  Only where every key
        // weight is a normal float at 2^sc already (the shift is then exact, and no key that the
        // wider range would hold has been flushed to zero); wider spans keep the general path.
        const float xlo = fmaf(kmin, kL2E, -static_cast<float>(sc));
        const float lo = xlo + fminf(ch.u2, 0.f);
        const int shift = (lo < -96.f) & (xlo >= -125.f) ? min(static_cast<int>(-96.f - lo) + 1, kMaxShift) : 0;
        const bool keys_ok = kmax * kL2E < kNMax;
        fast = fast_out && __all(keys_ok);
        Psum = Gs = Js = Gps = Jps = 0;
        du = 0.f;
        so = sc - shift;
        if (fast) {
            float m = x0.m;
            float bb = ldx(x0.b, x0.s - so);
            float dmin = INFINITY;  // smallest denominator (D_t and B_t) used
            const float scf = static_cast<float>(sc);
            acc_t dp = 1;
            float xg = 0.f, xb = 0.f;  // Inj: gA and gB at the span's scale
            if (Inj && tcut > 0) {
                xg = ldx(sd.ga, so - sd.s);
                xb = ldx(sd.gb, so - sd.s);
            }
#pragma unroll
            for (int j = 0; j < L; ++j) {
                // e = e^k / 2^so.  For the key that sets the scale fma(k, log2 e,
                // -sc) is exactly the key split's fraction, so the weight is
                // bit-equal to the forward's (times 2^shift); a key D binades below the span's
                // scale is rounded to ~D 2^-24 relative while its share of every
                // denominator here is ~2^-D (the forward's saved states, where
                // such a key might dominate later, use the exact split)
                const float kj = in.kv.k(j);
                const float ej = ldx(ex2(fmaf(kj, kL2E_lo, fmaf(kj, kL2E, -scf))), shift);
                const float E = ej * eu;
                const float den = bb + E;
                dmin = fminf(dmin, den);
                const float r = rcp(den);
                const float pi = E * r;
                const float dl = in.kv.v(j) - m;
                const float vy = (r * bb) * dl;
                const float db = fmaf(ch.dhi, bb, ch.dlo * bb);
                bb = db + ej;
                dmin = fminf(dmin, bb);  // B_t, the denominator of lam
                const float rb = rcp(bb);
                const float ldj = (ej * rb) * dl;
                float gj = in.gy.at(j);
                if (Gated) {
                    const Gate gt = gate_of(rg.at(j));
                    buf_store(gj * fmaf(pi, dl, m) * gt.s * gt.om, g.rdr, g.vout, j * g.row_out);
                    gj *= gt.s;
                }
                const float gpij = gj * pi;
                float grj = gj * r;
                float grpdj = grj * (pi * dl);
                if (Inj && j == tcut) {  // wave-uniform (tcut 0: no seed in this span)
                    grj += xg;
                    grpdj -= fmaf(m, xg, xb);
                }
                gpi[j] = gpij;
                gvy[j] = gpij * vy;
                gr[j] = grj;
                grpd[j] = grpdj;
                e[j] = ej;
                vm[j] = (db * rb) * dl;
                ld[j] = ldj;
                m += ldj;
                du = fmaf(gpij, vy, du);
                const acc_t q = dp * static_cast<acc_t>(grj);
                const acc_t t1 = fma(q, Psum, dp * static_cast<acc_t>(grpd[j]));
                Gs += q;
                Js += t1;
                Gps = fma(q, static_cast<acc_t>(j), Gps);
                Jps = fma(t1, static_cast<acc_t>(j), Jps);
                Psum += static_cast<acc_t>(ldj);
                dp = dec.mul(dp);
            }
            fast = __all(dmin >= kTiny);
            mT = m;
        }
        if (!fast) {
            // general path: per-token rescales, inputs re-read one token at a
            // time; the map is kept at the scale of the span's first token
            Psum = Gs = Js = Gps = Jps = 0;
            du = 0.f;
            MSt st = x0;
            double dpd = 1.0;
#pragma unroll 1
            for (int j = 0; j < L; ++j) {
                const int s_before = st.s;
                const float m_before = st.m;
                const TokQ q = mean_step(st, BufLd<TIn>::at(g.rk, g.vin, j * g.row_in),
                                         BufLd<TIn>::at(g.rv, g.vin, j * g.row_in), ch, eu, fast_out);
                if (j == 0)
                    so = st.s;
                else if (st.s != s_before)
                    dpd = ldexp(dpd, s_before - st.s);
                float gj = BufLd<TIn>::at(g.rg, g.vin, j * g.row_in);
                if (Gated) {
                    const Gate gt = gate_of(BufLd<TIn>::at(g.rr, g.vin, j * g.row_in));
                    buf_store(gj * (m_before + q.pd) * gt.s * gt.om, g.rdr, g.vout, j * g.row_out);
                    gj *= gt.s;
                }
                const double grj = static_cast<double>(gj * q.rho);
                const double qq = dpd * grj;
                double t1 = qq * (static_cast<double>(Psum) + static_cast<double>(q.pd));
                double qi = qq;
                if (Inj && tcut > 0 && j == tcut) {  // the seed at this token's scale
                    const double xg = ldexp(static_cast<double>(sd.ga), st.s - sd.s);
                    const double xb = ldexp(static_cast<double>(sd.gb), st.s - sd.s);
                    qi += dpd * xg;
                    t1 += dpd * (xg * static_cast<double>(Psum) - fma(static_cast<double>(m_before), xg, xb));
                }
                Gs += static_cast<acc_t>(qi);
                Js += static_cast<acc_t>(t1);
                Gps += static_cast<acc_t>(qi * j);
                Jps += static_cast<acc_t>(t1 * j);
                Psum += static_cast<acc_t>(q.ld);
                du = fmaf(gj * q.pi, q.vy, du);
                dpd *= dec.dd;
            }
            mT = st.m;
        }
    }

    // Reverse sweep from the carry at the span's end: writes dk, dv and
    // returns this span's part of -dw.
    //
    // St: tcut and sd as recompute's (the general path, which recomputes every token, seeds token
    // tcut again here).
    template <bool St = false>
    __device__ __forceinline__ float reverse(const RCarry& C, const SpanGeo& g, const Chan& ch, float eu,
                                             const Decay& dec, bool fast_out, int tcut = 0,
                                             const Seed& sd = Seed{}) const {
        float acc_dw = 0.f;
        if (fast) {
            acc_t G = static_cast<acc_t>(ldexp(C.G, so - C.sg)), J = static_cast<acc_t>(ldexp(C.J, so - C.sg));
            acc_t Gp = static_cast<acc_t>(ldexp(C.Gp, so - C.sg)), Jp = static_cast<acc_t>(ldexp(C.Jp, so - C.sg));
#pragma unroll
            for (int j = L - 1; j >= 0; --j) {
                const float ej = e[j], vmj = vm[j];
                buf_store(fmaf(ej, static_cast<float>(G), gpi[j]), g.rdv, g.vout, j * g.row_out);
                buf_store(fmaf(ej, static_cast<float>(fma(static_cast<acc_t>(vmj), G, -J)), gvy[j]), g.rdk, g.vout,
                          j * g.row_out);
                acc_dw = fmaf(ej, static_cast<float>(fma(static_cast<acc_t>(vmj), Gp, -Jp)), acc_dw);
                const acc_t ldj = static_cast<acc_t>(ld[j]);
                const acc_t GG = Gp + G;
                Jp = dec.mul(fma(ldj, GG, Jp + J));
                Gp = dec.mul(GG);
                J = dec.mul(fma(ldj, G, J)) + static_cast<acc_t>(grpd[j]);
                G = dec.mul(G) + static_cast<acc_t>(gr[j]);
            }
        } else {
            // general path, without per-token arrays: token t's quantities come
            // from a recompute over the span's first t + 1 tokens
            double G = C.G, J = C.J, Gp = C.Gp, Jp = C.Jp;
            int sg = C.sg;
#pragma unroll 1
            for (int t = L - 1; t >= 0; --t) {
                MSt st = x0;
#pragma unroll 1
                for (int j = 0; j < t; ++j)
                    (void)mean_step(st, BufLd<TIn>::at(g.rk, g.vin, j * g.row_in),
                                    BufLd<TIn>::at(g.rv, g.vin, j * g.row_in), ch, eu, fast_out);
                const float m_before = st.m;
                const TokQ q = mean_step(st, BufLd<TIn>::at(g.rk, g.vin, t * g.row_in),
                                         BufLd<TIn>::at(g.rv, g.vin, t * g.row_in), ch, eu, fast_out);
                float gt = BufLd<TIn>::at(g.rg, g.vin, t * g.row_in);
                if (Gated) gt *= gate_of(BufLd<TIn>::at(g.rr, g.vin, t * g.row_in)).s;
                const int ds = st.s - sg;  // bring the carry to this token's scale
                G = ldexp(G, ds);
                J = ldexp(J, ds);
                Gp = ldexp(Gp, ds);
                Jp = ldexp(Jp, ds);
                sg = st.s;
                const float gpit = gt * q.pi;
                buf_store(fmaf(q.e, static_cast<float>(G), gpit), g.rdv, g.vout, t * g.row_out);
                buf_store(fmaf(gpit, q.vy, q.e * static_cast<float>(fma(static_cast<double>(q.vm), G, -J))), g.rdk,
                          g.vout, t * g.row_out);
                acc_dw = fmaf(q.e, static_cast<float>(fma(static_cast<double>(q.vm), Gp, -Jp)), acc_dw);
                const double grt = static_cast<double>(gt * q.rho), ldt = q.ld;
                const double GG = Gp + G;
                Jp = dec.dd * fma(ldt, GG, Jp + J);
                Gp = dec.dd * GG;
                J = fma(dec.dd, fma(ldt, G, J), grt * static_cast<double>(q.pd));
                G = fma(dec.dd, G, grt);
                if (St && tcut > 0 && t == tcut) {  // the carry before token tcut: the seed (G, J were zero)
                    const double xg = ldexp(static_cast<double>(sd.ga), sg - sd.s);
                    const double xb = ldexp(static_cast<double>(sd.gb), sg - sd.s);
                    G += xg;
                    J -= fma(static_cast<double>(m_before), xg, xb);
                }
            }
        }
        return acc_dw;
    }
};

template <int W>
struct BwdShared {
    double mapd[W][5][64];  // S, c0..c3 of each wave's span
    float mapn[W][64];
    int maps[W][64];
    double cin[4][64];      // carry at the block's end
    int cin_s[64];
    float red[W][2][64];
    uint32_t ticket;
};

// x: added to the span's offsets (St: the handed-on state's carry carried back to the span's start).
template <int W, typename TIn, int L, bool Gated>
__device__ __forceinline__ void put_map(BwdShared<W>& sm, int wave, int lane, const Span<TIn, L, Gated>& sp,
                                        const RCarry* x = nullptr) {
    sm.mapn[wave][lane] = static_cast<float>(L);
    sm.maps[wave][lane] = sp.so;
    sm.mapd[wave][0][lane] = static_cast<double>(sp.Psum);
    if (x == nullptr) {
        sm.mapd[wave][1][lane] = static_cast<double>(sp.Gs);
        sm.mapd[wave][2][lane] = static_cast<double>(sp.Js);
        sm.mapd[wave][3][lane] = static_cast<double>(sp.Gps);
        sm.mapd[wave][4][lane] = static_cast<double>(sp.Jps);
    } else {
        sm.mapd[wave][1][lane] = static_cast<double>(sp.Gs) + x->G;
        sm.mapd[wave][2][lane] = static_cast<double>(sp.Js) + x->J;
        sm.mapd[wave][3][lane] = static_cast<double>(sp.Gps) + x->Gp;
        sm.mapd[wave][4][lane] = static_cast<double>(sp.Jps) + x->Jp;
    }
}

template <int W>
__device__ __forceinline__ RMap get_map(const BwdShared<W>& sm, int i, int lane, double dL) {
    RMap r;
    r.n = sm.mapn[i][lane];
    r.so = sm.maps[i][lane];
    r.S = sm.mapd[i][0][lane];
    r.c[0] = sm.mapd[i][1][lane];
    r.c[1] = sm.mapd[i][2][lane];
    r.c[2] = sm.mapd[i][3][lane];
    r.c[3] = sm.mapd[i][4][lane];
    r.D = dL;
    return r;
}

// dw, du of a workgroup: fixed-order sum over its waves into part[slot], then
// the fold over the channel tiles' workgroups.  The channel tiles ct with the
// same q = ct mod kFoldLines share fold line q (one 64-byte line in the
// workspace's fixed prefix, wkv_scan.h).  Each of their workgroups stores its
// partials with system-coherent stores, waits for them to complete, then
// counts itself on line q; the one that counts last sums, for each of the
// line's channel tiles, that tile's partials in the fixed order (batch row,
// time block) with coherent loads, writes dw and du, and returns the count to
// zero (so a workspace needs zeros before its first call only).  The order of
// each sum does not depend on which workgroup finishes last: results are
// bitwise reproducible.
template <int W>
__device__ __forceinline__ void put_partials(BwdShared<W>& sm, const BwdChunk& P, int64_t b, int64_t ct,
                                             int64_t blk, int wave, int lane, float ndw, float du) {
    sm.red[wave][0][lane] = -ndw;
    sm.red[wave][1][lane] = du;
    lds_sync();
    if (wave != 0) return;
    float sw = 0.f, su = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        sw += sm.red[i][0][lane];
        su += sm.red[i][1][lane];
    }
    const int64_t rows = P.B * P.npb;  // partial rows per channel tile
    const uint32_t row_bytes = 2 * 64 * 4;
    const Rsrc rp = make_rsrc(P.part, static_cast<uint32_t>(P.ntiles * P.npb) * row_bytes);
    auto row_off = [&](int64_t c_t, int64_t bb, int64_t jb) {
        return static_cast<uint32_t>(((bb * P.nct + c_t) * P.npb + jb) * row_bytes + lane * 4);
    };
    const uint32_t off = row_off(ct, b, blk);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sw), rp, off, 0, kCoherent);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(su), rp, off + 64 * 4, 0, kCoherent);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int64_t q = ct % kFoldLines;
    const int64_t nq = (P.nct - q + kFoldLines - 1) / kFoldLines;  // channel tiles on line q
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(P.fold + 16 * q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev + 1 != static_cast<uint32_t>(rows * nq)) return;
    // last of the line's workgroups: per channel tile, a fixed-order sum, 8 rows' loads in flight at a time
    for (int64_t c_t = q; c_t < P.nct; c_t += kFoldLines) {
        float tw = 0.f, tu = 0.f;
        int64_t r = 0;
        for (; r + 8 <= rows; r += 8) {
            float w8[8], u8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t bb = (r + i) / P.npb, jb = (r + i) - bb * P.npb;
                const uint32_t o = row_off(c_t, bb, jb);
                w8[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, o, 0, kCoherent));
                u8[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, o + 64 * 4, 0, kCoherent));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                tw += w8[i];
                tu += u8[i];
            }
        }
        for (; r < rows; ++r) {
            const int64_t bb = r / P.npb, jb = r - bb * P.npb;
            const uint32_t o = row_off(c_t, bb, jb);
            tw += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, o, 0, kCoherent));
            tu += __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, o + 64 * 4, 0, kCoherent));
        }
        const int64_t c = c_t * 64 + lane;
        if (c < P.C) {
            P.dw[c] = tw;
            P.du[c] = tu;
        }
    }
    if (lane == 0) __hip_atomic_store(P.fold + 16 * q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- backward through carried state (St kernels) --------------------------------
constexpr double kL2Ed = 1.4426950408889634;  // log2(e)

// The handed-on state's gradient (ga, gb) at the p_T the forward wrote, as gradients of the plain
// sums (A_T, B_T): gA = ga e^{-p_T} = ga 2^{-q}, q = p_T log2 e, split as (ga 2^{n - q}) 2^{-n}.
__device__ __forceinline__ Seed load_seed(const BwdChunk& P, int64_t i, bool cok) {
    Seed sd;
    if (!cok || P.ga_out == nullptr) return sd;
    const float pT = P.p_out[i];
    if (!(pT > -1e30f)) return sd;  // an empty handed-on state
    const double q = static_cast<double>(pT) * kL2Ed;
    const double n = rint(q);
    const float f = ex2(static_cast<float>(n - q));
    sd.ga = P.ga_out[i] * f;
    sd.gb = P.gb_out[i] * f;
    sd.s = static_cast<int>(n);
    return sd;
}

// A span ending exactly at T: the seed as the carry at its end, (G, J) = (gA, -gB - m_T gA) at the
// span's scale, and that carry taken back to the span's start by the span's own map without its
// offsets (added to the offsets, so earlier spans and blocks receive it).
template <typename TIn, int L, bool Gated>
__device__ __forceinline__ RCarry end_seed(const Span<TIn, L, Gated>& sp, const Seed& sd, double dL, RCarry* back) {
    const double xg = ldexp(static_cast<double>(sd.ga), sp.so - sd.s);
    const double xb = ldexp(static_cast<double>(sd.gb), sp.so - sd.s);
    const RCarry X{xg, -fma(static_cast<double>(sp.mT), xg, xb), 0.0, 0.0, sp.so};
    RMap m = rmap_identity();
    m.D = dL;
    m.S = static_cast<double>(sp.Psum);
    m.n = static_cast<float>(L);
    m.so = sp.so;
    *back = rapply(m, X);
    return X;
}

// C + X (X's scale brought to C's).
__device__ __forceinline__ RCarry add_carry(const RCarry& C, const RCarry& X) {
    const int d = C.sg - X.sg;
    return RCarry{C.G + ldexp(X.G, d), C.J + ldexp(X.J, d), C.Gp + ldexp(X.Gp, d), C.Jp + ldexp(X.Jp, d), C.sg};
}

// The gradients of the given state (a, b, p) from the reverse carry C0 before the first token and
// the history mean m0: for the plain sums dA = G and dB = -(J + m0 G), so ga = e^p dA, gb = e^p dB
// and gp = a ga + b gb = -B J (B = b e^p).  Returns the history's part of dw, B J' (its decay before
// every token).  An empty given state (b <= 0) is a constant: zeros.
__device__ __forceinline__ float state_grads(const BwdChunk& P, int64_t i, bool cok, const RCarry& C0, float m0) {
    if (!cok || P.a_in == nullptr) return 0.f;
    const float bi = P.b_in[i];
    float ga = 0.f, gb = 0.f, gp = 0.f, hist = 0.f;
    if (bi > 0.f) {
        const double f = exp2(static_cast<double>(P.p_in[i]) * kL2Ed - static_cast<double>(C0.sg));
        ga = static_cast<float>(C0.G * f);
        gb = static_cast<float>(-fma(static_cast<double>(m0), C0.G, C0.J) * f);
        gp = static_cast<float>(-static_cast<double>(bi) * C0.J * f);
        hist = static_cast<float>(static_cast<double>(bi) * C0.Jp * f);
    }
    if (P.ga_in != nullptr) {
        P.ga_in[i] = ga;
        P.gb_in[i] = gb;
        P.gp_in[i] = gp;
    }
    return hist;
}

// St: T - t0 for the span of wave `wave` in time block blk that holds token T-1 (1..L: token T is
// its token tcut, or its end when tcut = L), else 0.
template <int L, int W>
__device__ __forceinline__ int span_cut(int64_t T, int64_t blk, int wave) {
    const int64_t left = T - (blk * static_cast<int64_t>(L * W) + static_cast<int64_t>(wave) * L);
    return (left > 0 && left <= L) ? static_cast<int>(left) : 0;
}

// One span's recompute, with the seed where the span holds token T (St).
template <bool St, typename TIn, int L, bool Gated>
__device__ __forceinline__ void span_recompute(Span<TIn, L, Gated>& sp, const SpanIn<TIn, L, Gated>& in,
                                               const Chunk1<TIn, L>& rg, const SpanGeo& g, const Chan& ch, float eu,
                                               const Decay& dec, bool fast_out, int tcut, const Seed& sd) {
    sp.template recompute<St>(in, rg, g, ch, eu, dec, fast_out, tcut < L ? tcut : 0, sd);
}

// Time-split backward: one workgroup per (tile, time block); blocks are
// chained backward in time through the coherent carry slots.  St: through
// carried state (the handed-on state's gradient joins at token T; block 0
// returns the given state's gradients and adds the history's part of dw).
template <typename TIn, int L, int W, bool Gated, bool St = false>
__global__ void __launch_bounds__(64 * W, WKV_BWD_OCC) bwd_chunk_kernel(BwdChunk P) {
    __shared__ BwdShared<W> sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // stream j = blockIdx mod K hands out the time blocks of its tiles j, j + K, ..
    // last-in-time first (wkv_scan.h), so the awaited block is already running
    const int64_t j = blockIdx.x % P.nstream;
    const int64_t per = P.ntiles / P.nstream;  // tiles per stream
    int64_t tile = blockIdx.x, rblk = 0;
    uint32_t tag = 0, done_before = 0;
    if (P.nblocks > 1) {
        if (threadIdx.x == 0) {
            sm.ticket = stream_ticket(P.sc + j);
            if (sm.ticket >= per * P.nblocks) hdr_flag(P.hdr, kErrTicket);  // a workspace not zeroed before first use
        }
        __syncthreads();
        const int64_t k = sm.ticket;
        if (wave == 0) tag = stream_tag(P.sc + j);  // the carry wave's
        if (k >= per * P.nblocks) {  // uniform per workgroup: nothing to compute
            if (wave == 0)
                stream_finish(P.hdr, P.sc, j, stream_count(P.sc, j, lane), static_cast<uint32_t>(per * P.nblocks),
                              static_cast<uint32_t>(P.nstream), tag, lane);
            return;
        }
        rblk = k / per;
        tile = j + P.nstream * (k - rblk * per);
    }
    const int64_t blk = P.nblocks - 1 - rblk;
    const int64_t b = tile / P.nct;
    const int64_t c = (tile - b * P.nct) * 64 + lane;
    const bool cok = c < P.C;
    const float wc = cok ? P.w[c] : 0.f;
    const float uc = cok ? P.u[c] : 0.f;
    const Chan ch = make_chan(wc, uc);
    const bool fast_out = __all((fabsf(uc) <= kFastU) & (wc >= 0.f));
    const float eu = ex2(ch.u2);
    const Decay dec{ch.dhi, ch.dlo, ch.dd};
    const double dL = ipow<L>(ch.dd);

    const SpanGeo g = span_geo<TIn, L, W>(P, b, c, cok, blk, wave);
    SpanIn<TIn, L, Gated> in;
    in.load(g, P.C);
    Chunk1<TIn, L> rg;
    if (Gated) rg.load(g.rr, g.vin, g.row_in);
    Span<TIn, L, Gated> sp;
    const int tcut = St ? span_cut<L, W>(P.T, blk, wave) : 0;
    const Seed sd = (St && tcut > 0) ? load_seed(P, b * P.C + c, cok) : Seed{};
    span_recompute<St>(sp, in, rg, g, ch, eu, dec, fast_out, tcut, sd);
    RCarry X{0.0, 0.0, 0.0, 0.0, 0};  // St, the span ending at T: the seed at its end
    if (St && tcut == L) {  // wave-uniform
        RCarry back;
        X = end_seed(sp, sd, dL, &back);
        put_map(sm, wave, lane, sp, &back);
    } else {
        put_map(sm, wave, lane, sp);
    }
    lds_sync();

    RMap suf = rmap_identity();
    for (int i = W - 1; i > wave; --i) suf = rcompose(get_map(sm, i, lane, dL), suf);
    float hist = 0.f;
    if (wave == 0) {
        RCarry cin{0.0, 0.0, 0.0, 0.0, 0};
        if (P.nblocks > 1) {
            const Rsrc rc = make_rsrc(P.carry, P.carry_bytes);
            const uint32_t slot = (uint32_t)(((tile * P.nblocks + blk) * 64 + lane) * kCarrySlot);
            if (blk < P.nblocks - 1) cin = wait_carry(rc, slot + 64 * kCarrySlot, tag, P.spin, P.hdr);  // block blk+1
            if (blk > 0) publish_carry(rc, slot, rapply(rcompose(get_map(sm, 0, lane, dL), suf), cin), tag);
            done_before = stream_count(P.sc, j, lane);
        }
        if (St && blk == 0)  // the carry before the first token
            hist = state_grads(P, b * P.C + c, cok, rapply(rcompose(get_map(sm, 0, lane, dL), suf), cin), sp.x0.m);
        sm.cin[0][lane] = cin.G;
        sm.cin[1][lane] = cin.J;
        sm.cin[2][lane] = cin.Gp;
        sm.cin[3][lane] = cin.Jp;
        sm.cin_s[lane] = cin.sg;
    }
    lds_sync();
    RCarry C = rapply(suf, RCarry{sm.cin[0][lane], sm.cin[1][lane], sm.cin[2][lane], sm.cin[3][lane],
                                  sm.cin_s[lane]});
    if (St && tcut == L) C = add_carry(C, X);
    const float ndw = sp.template reverse<St>(C, g, ch, eu, dec, fast_out, tcut < L ? tcut : 0, sd) - hist;
    const int64_t ct = tile - b * P.nct;
    put_partials(sm, P, b, ct, blk, wave, lane, ndw, sp.du);
    if (P.nblocks > 1 && wave == 0)  // the carry wave
        stream_finish(P.hdr, P.sc, j, done_before, static_cast<uint32_t>(per * P.nblocks),
                      static_cast<uint32_t>(P.nstream), tag, lane);
}

// Whole-tile backward: one workgroup walks all time blocks of its tile from
// the last to the first, keeping the carry in LDS (no cross-workgroup
// exchange).  Used when there are enough tiles to fill the GPU.
//
// Staged: while a block is computed, the next block's k, v, gy (and, gated with
// bf16 inputs, r) stream into LDS by asynchronous buffer -> LDS copies
// (stage_span), and its saved state
// into three registers, so the loads overlap the arithmetic without holding
// a second block in registers.  Each wave copies and reads only its own span,
// so the waits are per wave: wait_staged() before reading a block from LDS,
// and wait_lds_reads() after, before the next copy may overwrite it.
//
// St: through carried state, as the time-split kernel.
template <typename TIn, int L, int W, bool Gated, bool Staged, bool St = false>
__global__ void __launch_bounds__(64 * W, WKV_BWD_OCC) bwd_tile_kernel(BwdChunk P) {
    // r joins the staged inputs when it is bf16 (as float32 it would cost the second workgroup per CU)
    constexpr int kNI = (Gated && sizeof(TIn) == 2) ? 4 : 3;
    __shared__ BwdShared<W> sm;
    __shared__ BwdStage<TIn, L, W, kNI> stage;  // referenced (and allocated) only when Staged
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / P.nct;
    const int64_t c = (tile - b * P.nct) * 64 + lane;
    const bool cok = c < P.C;
    const float wc = cok ? P.w[c] : 0.f;
    const float uc = cok ? P.u[c] : 0.f;
    const Chan ch = make_chan(wc, uc);
    const bool fast_out = __all((fabsf(uc) <= kFastU) & (wc >= 0.f));
    const float eu = ex2(ch.u2);
    const Decay dec{ch.dhi, ch.dlo, ch.dd};
    const double dL = ipow<L>(ch.dd);

    RCarry cin{0.0, 0.0, 0.0, 0.0, 0};  // carry at the current block's end (same in every wave)
    float ndw = 0.f, du = 0.f;
    float m0 = 0.f;  // St: the mean at the span's start (at the end of the loop: before the first token)
    SpanIn<TIn, L, Gated> cur, nxt;  // nxt: only the next block's saved state (Staged)
    const int64_t c0 = (tile - b * P.nct) * 64;
    if constexpr (Staged) {
        const SpanGeo g0 = span_geo<TIn, L, W>(P, b, c, cok, P.nblocks - 1, wave);
        stage_span(stage, g0, wave, lane, c0, P.C);
        nxt.load_ck(g0, P.C);
    }
    for (int64_t blk = P.nblocks - 1; blk >= 0; --blk) {
        const SpanGeo g = span_geo<TIn, L, W>(P, b, c, cok, blk, wave);
        Chunk1<TIn, L> rg;
        if constexpr (Staged) {
            // after the first block, every path issued at least the 2 L dv, dk stores of the
            // previous block after this block's copies
            if (blk == P.nblocks - 1)
                wait_staged();
            else
                wait_staged_before<2 * L>();
            cur.load_lds(stage, wave, lane);
            if constexpr (kNI == 4) rg.load_lds(stage.x[wave][3], lane);
            cur.a0 = nxt.a0;
            cur.b0 = nxt.b0;
            cur.s0 = nxt.s0;
            wait_lds_reads();
            if (blk > 0) {
                const SpanGeo gn = span_geo<TIn, L, W>(P, b, c, cok, blk - 1, wave);
                stage_span(stage, gn, wave, lane, c0, P.C);
                nxt.load_ck(gn, P.C);
            }
        } else {
            cur.load(g, P.C);
        }
        if constexpr (Gated && !(Staged && kNI == 4)) rg.load(g.rr, g.vin, g.row_in);
        Span<TIn, L, Gated> sp;
        const int tcut = St ? span_cut<L, W>(P.T, blk, wave) : 0;
        const Seed sd = (St && tcut > 0) ? load_seed(P, b * P.C + c, cok) : Seed{};
        span_recompute<St>(sp, cur, rg, g, ch, eu, dec, fast_out, tcut, sd);
        du += sp.du;
        RCarry X{0.0, 0.0, 0.0, 0.0, 0};  // St, the span ending at T: the seed at its end
        if (St && tcut == L) {  // wave-uniform: the last block only
            RCarry back;
            X = end_seed(sp, sd, dL, &back);
            put_map(sm, wave, lane, sp, &back);
        } else {
            put_map(sm, wave, lane, sp);
        }
        if constexpr (St) m0 = sp.x0.m;
        lds_sync_lgkm();
        RMap suf = rmap_identity();
        for (int i = W - 1; i > wave; --i) suf = rcompose(get_map(sm, i, lane, dL), suf);
        if (wave == 0) {
            const RCarry out = rapply(rcompose(get_map(sm, 0, lane, dL), suf), cin);
            sm.cin[0][lane] = out.G;
            sm.cin[1][lane] = out.J;
            sm.cin[2][lane] = out.Gp;
            sm.cin[3][lane] = out.Jp;
            sm.cin_s[lane] = out.sg;
        }
        RCarry C = rapply(suf, cin);
        if (St && tcut == L) C = add_carry(C, X);
        ndw += sp.template reverse<St>(C, g, ch, eu, dec, fast_out, tcut < L ? tcut : 0, sd);
        lds_sync_lgkm();
        cin = RCarry{sm.cin[0][lane], sm.cin[1][lane], sm.cin[2][lane], sm.cin[3][lane], sm.cin_s[lane]};
    }
    if constexpr (St) {  // cin is the carry before the first token, m0 wave 0's history mean there
        if (wave == 0) ndw -= state_grads(P, b * P.C + c, cok, cin, m0);
    }
    put_partials(sm, P, b, tile - b * P.nct, 0, wave, lane, ndw, du);
}

namespace {
#ifndef WKV_BWD_L
#define WKV_BWD_L 16
#endif
#ifndef WKV_BWD_W
#define WKV_BWD_W 8
#endif
#ifndef WKV_BWD_TILE_W
#define WKV_BWD_TILE_W 4
#endif
#ifndef WKV_BWD_STAGE
#define WKV_BWD_STAGE 1  // whole-tile backward: stage each next block's inputs in LDS
#endif
constexpr int kBwdL = WKV_BWD_L;
constexpr int kBwdW = WKV_BWD_W;        // waves per workgroup, time-split kernel
constexpr int kBwdTileW = WKV_BWD_TILE_W;  // waves per workgroup, whole-tile kernel
static_assert(kBwdL % kCkptLen == 0, "backward spans must start on saved forward states");

struct BwdLayout {
    int64_t nct, ntiles, nblocks, nblk_ck;
    size_t off_carry, carry_bytes, off_part, off_ckpt, ckpt_bytes, bytes;
};

BwdLayout bwd_layout(int64_t B, int64_t T, int64_t C) {
    BwdLayout l{};
    l.nct = (C + 63) / 64;
    l.ntiles = B * l.nct;
    l.nblocks = (T + kBwdL * kBwdW - 1) / (kBwdL * kBwdW);
    l.nblk_ck = (T + kCkptLen - 1) / kCkptLen;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    // the counters' fixed prefix (wkv_scan.h), then the carries between workgroups at the same
    // fixed offset for every shape, shared with the forward that recomputes the saved states when
    // none are given (it runs first, and its carries are dead once it ends), then the dw, du
    // partials and the recomputed states
    const size_t fwd_ws = fwd_chunk_workspace_bytes(B, T, C);
    const size_t fwd_carry = fwd_ws > kWsPrefix ? fwd_ws - kWsPrefix : 0;
    l.off_carry = kWsPrefix;
    l.carry_bytes = l.nblocks > 1 ? static_cast<size_t>(l.ntiles * l.nblocks * 64) * kCarrySlot : 0;
    size_t off = up(l.off_carry + (fwd_ws == SIZE_MAX ? 0 : (l.carry_bytes > fwd_carry ? l.carry_bytes : fwd_carry)));
    l.off_part = off;
    off = up(off + static_cast<size_t>(l.ntiles * l.nblocks * 2 * 64) * 4);
    l.off_ckpt = off;
    l.ckpt_bytes = static_cast<size_t>(B * l.nblk_ck * C) * 12;
    l.bytes = off + l.ckpt_bytes;
    // carries and partials are addressed through 32-bit buffer resources
    if (l.carry_bytes > 0xffffffffull || static_cast<size_t>(l.ntiles * l.nblocks) * 512 > 0xffffffffull ||
        fwd_ws == SIZE_MAX)
        l.bytes = SIZE_MAX;
    return l;
}
}  // namespace

size_t bwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t C) { return bwd_layout(B, T, C).bytes; }

template <typename TIn>
hipError_t launch_bwd_chunk_t(const BwdArgs& a, hipStream_t stream) {
    const BwdLayout l = bwd_layout(a.B, a.T, a.C);
    char* ws = static_cast<char*>(a.ws);
    const float* ckpt = static_cast<const float*>(a.ckpt);
    const bool st = a.a_in != nullptr || a.ga_out != nullptr || a.ga_in != nullptr;  // through carried state
    if (ckpt == nullptr) {  // recompute the block-start states with the forward (no y written)
        FwdArgs f{a.B, a.T, a.C, a.bf16, a.w, a.u, a.k, a.v, nullptr, ws + l.off_ckpt, l.nblk_ck,
                  ws, l.off_part};
        f.a_in = a.a_in;
        f.b_in = a.b_in;
        f.p_in = a.p_in;
        const hipError_t e = launch_fwd_chunk(f, stream);
        if (e != hipSuccess) return e;
        ckpt = reinterpret_cast<const float*>(ws + l.off_ckpt);
    }
    BwdChunk P{};
    P.B = a.B; P.T = a.T; P.C = a.C;
    P.w = a.w; P.u = a.u; P.k = a.k; P.v = a.v; P.gy = a.gy;
    P.dk = a.dk; P.dv = a.dv;
    P.ckpt = ckpt;
    P.nblk_ck = l.nblk_ck;
    P.nct = l.nct; P.ntiles = l.ntiles;
    P.part = reinterpret_cast<float*>(ws + l.off_part);
    P.r = a.r;
    P.dr = a.dr;
    P.fold = reinterpret_cast<uint32_t*>(ws + kWsFoldOff);
    P.dw = a.dw;
    P.du = a.du;
    P.hdr = reinterpret_cast<CallHdr*>(ws);
    P.sc = reinterpret_cast<StreamCtr*>(ws + kWsStreamOff);
    P.nstream = 1;
    P.spin = spin_limit();
    P.a_in = a.a_in; P.b_in = a.b_in; P.p_in = a.p_in;
    P.ga_out = a.ga_out; P.gb_out = a.gb_out; P.p_out = a.p_out;
    P.ga_in = a.ga_in; P.gb_in = a.gb_in; P.gp_in = a.gp_in;

    // Enough tiles to give every CU two workgroups: one workgroup per tile
    // walks the whole sequence (no carries between workgroups).
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (l.ntiles >= 2 * static_cast<int64_t>(ncu)) {
        P.nblocks = (a.T + kBwdL * kBwdTileW - 1) / (kBwdL * kBwdTileW);
        P.npb = 1;
        // the LDS-staged loads move 16-byte chunks: whole chunks per row, aligned
        const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
        const bool staged = WKV_BWD_STAGE && a.C % (16 / static_cast<int64_t>(sizeof(TIn))) == 0 && a16(a.k) &&
                            a16(a.v) && a16(a.gy) && (P.r == nullptr || sizeof(TIn) != 2 || a16(P.r));
        const dim3 grid(static_cast<unsigned>(l.ntiles)), block(64 * kBwdTileW);
        if (st && staged)
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, false, true, true>), grid, block, 0, stream, P);
        else if (st)
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, false, false, true>), grid, block, 0, stream, P);
        else if (P.r != nullptr && staged)
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, true, true>), grid, block, 0, stream, P);
        else if (P.r != nullptr)
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, true, false>), grid, block, 0, stream, P);
        else if (staged)
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, false, true>), grid, block, 0, stream, P);
        else
            hipLaunchKernelGGL((bwd_tile_kernel<TIn, kBwdL, kBwdTileW, false, false>), grid, block, 0, stream, P);
        return hipGetLastError();
    }

    P.nblocks = l.nblocks;
    P.npb = l.nblocks;
    P.nstream = chain_streams(l.ntiles);
    P.carry = reinterpret_cast<float*>(ws + l.off_carry);
    P.carry_bytes = static_cast<uint32_t>(l.carry_bytes);
    if (st)
        hipLaunchKernelGGL((bwd_chunk_kernel<TIn, kBwdL, kBwdW, false, true>),
                           dim3(static_cast<unsigned>(l.ntiles * l.nblocks)), dim3(64 * kBwdW), 0, stream, P);
    else if (P.r != nullptr)
        hipLaunchKernelGGL((bwd_chunk_kernel<TIn, kBwdL, kBwdW, true>),
                           dim3(static_cast<unsigned>(l.ntiles * l.nblocks)), dim3(64 * kBwdW), 0, stream, P);
    else
        hipLaunchKernelGGL((bwd_chunk_kernel<TIn, kBwdL, kBwdW, false>),
                           dim3(static_cast<unsigned>(l.ntiles * l.nblocks)), dim3(64 * kBwdW), 0, stream, P);
    return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_bwd_chunk_t<uint16_t>(a, stream) : launch_bwd_chunk_t<float>(a, stream);
}

}  // namespace wkv
