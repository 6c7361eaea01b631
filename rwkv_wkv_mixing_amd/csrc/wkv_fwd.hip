// Chunked (time-split) WKV forward for gfx950.
//
// Work decomposition.  A workgroup owns one TILE of 64 channels of one batch
// row and one time BLOCK of W*L tokens; wave i of the workgroup owns the L
// tokens [i*L, (i+1)*L) of the block, one channel per lane, so every load and
// store of a wave is one contiguous 64-channel row segment (128 B for bf16,
// 256 B for fp32).  The inputs of a sub-chunk stay in registers, so HBM sees
// each input once and each output once.
//
//   local   every wave runs its L tokens from the empty state at one fixed
//           scale (that of its largest key), keeping for every token the
//           local numerator N_t = A_loc + e^{u+k} v and denominator
//           D_t = B_loc + e^{u+k}; the end state is the sub-chunk summary S_i
//   scan    through LDS every wave combines S_0..S_{i-1} into its prefix P_i;
//           the last wave also waits for the inclusive state E of the
//           previous time block of the same tile (each tile's blocks are
//           handed out by the tile's own atomic ticket in time order, so the
//           awaited block is already running) and publishes this block's
//           inclusive state, tagged with the tile's generation (wkv_scan.h)
//   output  with X = d^{iL} E + P_i the state before the sub-chunk,
//           y_t = (N_t + d^j X_A) / (D_t + d^j X_B)  for its j-th token,
//           and the saved block-start states for the backward.
//
// The fixed scale makes the local pass and the output branch-free straight
// line code.  It needs w >= 0, |u| <= kFastU, a local end state and output
// denominators no smaller than kTiny, and a carry-in that fits next to the
// local scale; a wave where any lane misses one of these runs the general path
// instead (a per-token lazy rescale, then a second recurrence from X), which
// also covers the current-token normalisation for any u.
//
// Chunkwise-parallel execution: "RWKV模型深度研究报告", section 1.4.1;
// prefix scan: "RWKV（Receptance Weighted Key Value）概念", section 3.4.
#include "wkv_launch.h"
#include "wkv_scan.h"

namespace wkv {

struct FwdChunk {
    int64_t B, T, C;
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    float* y;
    float* ckpt;
    int64_t nblk_ck;   // blocks of kCkptLen tokens (ckpt layout)
    int64_t nct;       // channel tiles per batch row
    int64_t ntiles;    // B * nct
    int64_t nblocks;   // time blocks per tile
    CallHdr* hdr;      // workspace header: error word, finished streams, generation (nblocks > 1)
    StreamCtr* sc;     // [kMaxStreams] ticket streams (nblocks > 1)
    int64_t nstream;   // streams in use; divides ntiles
    uint32_t spin;     // polls before a carry wait gives up
    float* carry;      // [ntiles][nblocks][64][4] inclusive block states + tag
    uint32_t carry_bytes;
    const void* r;      // receptance [B, T, C] (gated kernels only)
    const float* a_in;  // optional state before token 1, [B, C] each
    const float* b_in;
    const float* p_in;
    float* a_out;       // optional state after token T, [B, C] each
    float* b_out;
    float* p_out;
};

// The L tokens of one lane's sub-chunk, held in registers across both passes.
// bf16: k and v of a token share one 32-bit register (v in the high half).
template <typename TIn, int L>
struct SubChunk;

template <int L>
struct SubChunk<uint16_t, L> {
    uint32_t kv[L];
    __device__ __forceinline__ void load(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rk, voff, j * row, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rv, voff, j * row, 0);
            kv[j] = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ float k(int j) const { return __uint_as_float(kv[j] << 16); }
    __device__ __forceinline__ float v(int j) const { return __uint_as_float(kv[j] & 0xffff0000u); }
    // Hide the registers' contents from the optimiser (emits no code), so that
    // values unpacked in one pass are recomputed in the next instead of being
    // kept alive in extra registers.
    __device__ __forceinline__ void opaque() {
#pragma unroll
        for (int j = 0; j < L; ++j) asm volatile("" : "+v"(kv[j]));
    }
    // The same for one token: keeps its unpacking (and what follows from it)
    // after the previous token's stores instead of hoisted ahead of the loop.
    __device__ __forceinline__ void opaque(int j) { asm volatile("" : "+v"(kv[j])); }
};

template <int L>
struct SubChunk<float, L> {
    float kk[L], vv[L];
    __device__ __forceinline__ void load(Rsrc rk, Rsrc rv, uint32_t voff, uint32_t row) {
#pragma unroll
        for (int j = 0; j < L; ++j) {
            kk[j] = BufLd<float>::at(rk, voff, j * row);
            vv[j] = BufLd<float>::at(rv, voff, j * row);
        }
    }
    __device__ __forceinline__ float k(int j) const { return kk[j]; }
    __device__ __forceinline__ float v(int j) const { return vv[j]; }
    __device__ __forceinline__ void opaque() {}
    __device__ __forceinline__ void opaque(int j) { asm volatile("" : "+v"(kk[j]), "+v"(vv[j])); }
};

// General path over a sub-chunk: outputs from the carry-in state by a second
// recurrence with per-token rescales, and the state before every kCkptLen-th
// token into ckpt (when given).  Rare; reads one token at a time so that it
// adds no registers to the kernel.
template <bool Fast, bool Gated, typename TIn, int L>
__device__ __forceinline__ void general_outputs(St st, Rsrc rk, Rsrc rv, Rsrc rr, uint32_t vin, uint32_t row_in,
                                                int nvalid, const Chan& ch, float eu, Rsrc ry, uint32_t vout,
                                                uint32_t row_out, float* ckp, int64_t ckstride) {
#pragma unroll 1
    for (int j = 0; j < L; ++j) {
        if ((j % kCkptLen) == 0 && j < nvalid && ckp != nullptr) {
            float* cp = ckp + (j / kCkptLen) * 3 * ckstride;
            cp[0] = st.a;
            cp[ckstride] = st.b;
            cp[2 * ckstride] = static_cast<float>(st.s);
        }
        const Key kk = key_split(BufLd<TIn>::at(rk, vin, j * row_in));
        const float vj = BufLd<TIn>::at(rv, vin, j * row_in);
        const float e = key_weight(st, kk);
        float yj = Fast ? token_out_fast(st, e, vj, eu) : token_out(st, key_log2(st, kk), vj, ch).y;
        if (Gated) yj *= gate_of(BufLd<TIn>::at(rr, vin, j * row_in)).s;
        token_add(st, e, vj, ch);
        buf_store(yj, ry, vout, j * row_out);
    }
}

constexpr int kCarryAbove = 100;  // max log2 of the carry-in's b (and of a, + 20) above the local scale

// Local pass at the fixed scale sl (>= every key's n): returns the local end
// state, fills N and D, and keeps the local state before every kCkptLen-th token.
template <typename TIn, int L>
__device__ __forceinline__ St local_pass(const SubChunk<TIn, L>& sc, int sl, const Chan& ch, float eu,
                                         float (&N)[L], float (&D)[L], St (&mid)[L / kCkptLen]) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        if (j % kCkptLen == 0 && j > 0) mid[j / kCkptLen] = St{a, b, sl};
        // e = e^k / 2^sl from the key split: exact scaling, no rounding of
        // k log2 e - sl (an output before the sub-chunk's largest key sums only
        // keys far below sl, whose weights must not carry that rounding)
        const Key kk = key_split_bounded(sc.k(j));
        const float e = ldx(kk.em, kk.n - sl);
        const float v = sc.v(j);
        const float E = e * eu;
        N[j] = fmaf(E, v, a);
        D[j] = b + E;
        const float ev = e * v;
        a = fmaf(ch.dhi, a, fmaf(ch.dlo, a, ev));
        b = fmaf(ch.dhi, b, fmaf(ch.dlo, b, e));
    }
    return St{a, b, sl};
}

// Outputs from the local terms and the carry-in X brought to the local scale
// (times sigmoid(r) when gated); returns the smallest denominator used.
template <bool Gated, typename TIn, int L>
__device__ __forceinline__ float corrected_outputs(const St& X, int sl, const float (&N)[L], const float (&D)[L],
                                                   const Chunk1<TIn, L>& rch, const Chan& ch, Rsrc ry,
                                                   uint32_t vout, uint32_t row_out) {
    const float cA = ldx(X.a, X.s - sl), cB = ldx(X.b, X.s - sl);
    float dp = 1.f;  // d^j
    float dmin = INFINITY;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const float den = fmaf(dp, cB, D[j]);
        dmin = fminf(dmin, den);
        float yj = fmaf(dp, cA, N[j]) * rcp(den);
        if (Gated) yj *= gate_of(rch.at(j)).s;
        buf_store(yj, ry, vout, j * row_out);
        dp = fmaf(ch.dhi, dp, ch.dlo * dp);
    }
    return dmin;
}

// Where one wave's sub-chunk lives for one lane.  Tokens past T read as
// k = v = 0 (they follow every real token of the wave, so they change no real
// output) and their stores are dropped.
struct FwdGeo {
    Rsrc rk, rv, rr, ry;
    uint32_t vin, vout, row_in, row_out;
    int nvalid;  // real tokens in the sub-chunk
    float* ckp;  // saved states of the sub-chunk, or nullptr
};

template <typename TIn, int L, int W>
__device__ __forceinline__ FwdGeo fwd_geo(const FwdChunk& P, int64_t b, int64_t c, bool cok, int64_t blk, int wave) {
    constexpr int ES = BufLd<TIn>::kBytes;
    const int64_t tb0 = blk * (int64_t)(L * W);  // first token of the block
    const int64_t t0 = tb0 + (int64_t)wave * L;  // first token of this wave
    const int64_t rem = P.T - t0;
    const int64_t blk_tokens = (P.T - tb0) < (int64_t)(L * W) ? (P.T - tb0) : (int64_t)(L * W);
    const int64_t row0 = (b * P.T + tb0) * P.C;
    FwdGeo g;
    g.nvalid = rem <= 0 ? 0 : (rem >= L ? L : static_cast<int>(rem));
    g.rk = make_rsrc(static_cast<const TIn*>(P.k) + row0, (uint32_t)(blk_tokens * P.C * ES));
    g.rv = make_rsrc(static_cast<const TIn*>(P.v) + row0, (uint32_t)(blk_tokens * P.C * ES));
    g.rr = P.r != nullptr ? make_rsrc(static_cast<const TIn*>(P.r) + row0, (uint32_t)(blk_tokens * P.C * ES))
                          : make_rsrc(nullptr, 0);
    // y == nullptr (the backward's state-only run): a zero-size buffer drops every store
    g.ry = P.y != nullptr ? make_rsrc(P.y + row0, (uint32_t)(blk_tokens * P.C * 4)) : make_rsrc(nullptr, 0);
    const uint32_t lin = cok ? (uint32_t)((int64_t)wave * L * P.C + c) : kOffNone;  // element offset
    g.vin = cok ? lin * ES : kOffNone;
    g.vout = cok ? lin * 4 : kOffNone;
    g.row_in = (uint32_t)(P.C * ES);
    g.row_out = (uint32_t)(P.C * 4);
    g.ckp = (P.ckpt != nullptr && cok && g.nvalid > 0) ? P.ckpt + ((b * P.nblk_ck + t0 / kCkptLen) * 3) * P.C + c
                                                       : nullptr;
    return g;
}

// One wave's sub-chunk: the local pass (or general pass 1) and, once the
// carry-in is known, the outputs.
template <typename TIn, int L>
struct SubWork {
    float N[L], D[L];
    St mid[L / kCkptLen];
    St st;    // summary: the sub-chunk run from the empty state
    int sl;   // fixed local scale
    bool fast_local;

    __device__ __forceinline__ void local(SubChunk<TIn, L>& sc, const FwdGeo& g, const Chan& ch, float eu,
                                          float wc, float uc) {
        float kmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < L; ++j) kmax = fmaxf(kmax, sc.k(j));
        sc.opaque();
        sl = key_split(kmax).n;
        const bool keys_ok = kmax * kL2E < kNMax;
        fast_local = __all((wc >= 0.f) & (fabsf(uc) <= kFastU) & keys_ok);
        st = empty_state();
        if (fast_local) {
            st = local_pass(sc, sl, ch, eu, N, D, mid);
            fast_local = __all(st.b >= kTiny);
        }
        if (!fast_local) {  // general pass 1, reading one token at a time (rare: kept register-light)
            st = empty_state();
#pragma unroll 1
            for (int j = 0; j < L; ++j) {
                const float e = key_weight(st, key_split(BufLd<TIn>::at(g.rk, g.vin, j * g.row_in)));
                token_add(st, e, BufLd<TIn>::at(g.rv, g.vin, j * g.row_in), ch);
            }
        }
    }

    // Outputs (and saved states) from the carry-in X: the fixed-scale
    // correction, or the general second recurrence when the wave needs it.
    template <bool Gated>
    __device__ __forceinline__ void outputs(const St& X, const FwdGeo& g, const Chunk1<TIn, L>& rch, const Chan& ch,
                                            float eu, bool fast, bool want_y, int64_t C) const {
        // The carry enters token j as d^j X, with d^j a float32 running product.
        // Where d^j falls below float32's normal range its absolute error is
        // 2^-150, so the carry term X_B d^j (X_B < 2^lvl at the local scale)
        // is off by up to 2^(lvl - 150) against a denominator of at least
        // kTiny = 2^-100: the fast path then also needs lvl <= 24 (error below
        // 2^-26 of the denominator, and of |A/B| in the numerator); otherwise
        // the general path rescales per token.
        const int lvl = X.s - sl + __builtin_amdgcn_frexp_expf(X.b);
        const bool dp_normal = ipow<L - 1>(ch.dd) >= 0x1p-125;
        const bool carry_fits =
            !(X.b > 0.f) | ((lvl <= kCarryAbove) & (X.s - sl + __builtin_amdgcn_frexp_expf(X.a) <= kCarryAbove + 20) &
                            (dp_normal | (lvl <= 24)));
        bool fast_out = fast_local && __all(carry_fits);
        if (fast_out && want_y)
            fast_out = __all(corrected_outputs<Gated>(X, sl, N, D, rch, ch, g.ry, g.vout, g.row_out) >= kTiny);
        if (fast_out) {
            if (g.ckp != nullptr) {
                const double dck = ipow<kCkptLen>(ch.dd);
                double dq = 1.0;
#pragma unroll
                for (int q = 0; q < L / kCkptLen; ++q) {
                    if (q * kCkptLen < g.nvalid) {
                        const St x = q == 0 ? X : combine(X, mid[q], dq);
                        float* cp = g.ckp + q * 3 * C;
                        cp[0] = x.a;
                        cp[C] = x.b;
                        cp[2 * C] = static_cast<float>(x.s);
                    }
                    dq *= dck;
                }
            }
        } else if (fast) {  // general path: rewrites every output of the wave
            general_outputs<true, Gated, TIn, L>(X, g.rk, g.rv, g.rr, g.vin, g.row_in, g.nvalid, ch, eu, g.ry,
                                                 g.vout, g.row_out, g.ckp, C);
        } else {
            general_outputs<false, Gated, TIn, L>(X, g.rk, g.rv, g.rr, g.vin, g.row_in, g.nvalid, ch, eu, g.ry,
                                                  g.vout, g.row_out, g.ckp, C);
        }
    }
};

template <int W>
struct FwdShared {
    float a[W][64], b[W][64];
    int s[W][64];
    float ea[64], eb[64];  // block carry-in E
    int es[64];
    uint32_t ticket;
};

// Prefix of the summaries of waves 0..wave-1 of a block.
template <int W>
__device__ __forceinline__ St wave_prefix(const FwdShared<W>& sm, int wave, int lane, double dL) {
    St pref = empty_state();
    for (int i = 0; i < wave; ++i) pref = combine(pref, St{sm.a[i][lane], sm.b[i][lane], sm.s[i][lane]}, dL);
    return pref;
}

// Time-split forward: one workgroup per (tile, time block); blocks are
// chained in time through the coherent carry slots.
#ifndef WKV_FWD_OCC
#define WKV_FWD_OCC 1  // minimum waves per SIMD asked of the register allocator (ungated kernel)
#endif

template <typename TIn, int L, int W, bool Gated>
__global__ void __launch_bounds__(64 * W, Gated ? 1 : WKV_FWD_OCC) fwd_chunk_kernel(FwdChunk P) {
    __shared__ FwdShared<W> sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // stream j = blockIdx mod K hands out the time blocks of its tiles j, j + K, ..
    // in time order (wkv_scan.h), so the awaited block is already running
    const int64_t j = blockIdx.x % P.nstream;
    const int64_t per = P.ntiles / P.nstream;  // tiles per stream
    int64_t tile = blockIdx.x, blk = 0;
    uint32_t tag = 0, done_before = 0;
    if (P.nblocks > 1) {
        if (threadIdx.x == 0) {
            sm.ticket = stream_ticket(P.sc + j);
            if (sm.ticket >= per * P.nblocks) hdr_flag(P.hdr, kErrTicket);  // a workspace not zeroed before first use
        }
        __syncthreads();
        const int64_t k = sm.ticket;
        if (wave == W - 1) tag = stream_tag(P.sc + j);  // the carry wave's
        if (k >= per * P.nblocks) {  // uniform per workgroup: nothing to compute
            if (wave == W - 1)
                stream_finish(P.hdr, P.sc, j, stream_count(P.sc, j, lane), static_cast<uint32_t>(per * P.nblocks),
                              static_cast<uint32_t>(P.nstream), tag, lane);
            return;
        }
        blk = k / per;
        tile = j + P.nstream * (k - blk * per);
    }
    const int64_t b = tile / P.nct;
    const int64_t c = (tile - b * P.nct) * 64 + lane;
    const bool cok = c < P.C;
    const float wc = cok ? P.w[c] : 0.f;
    const float uc = cok ? P.u[c] : 0.f;
    const Chan ch = make_chan(wc, uc);
    const bool fast = __all((fabsf(uc) <= kFastU) & (wc >= 0.f));
    const float eu = ex2(ch.u2);
    const double dL = ipow<L>(ch.dd);

    // a given state before token 1 is block 0's carry-in: converted here, while
    // few registers are live, and parked in the LDS words the carry uses
    const bool state_in = blk == 0 && wave == W - 1 && P.a_in != nullptr;
    if (state_in) {
        const int64_t i = b * P.C + (cok ? c : 0);
        const St E0 = cok ? state_from_abp(P.a_in[i], P.b_in[i], P.p_in[i]) : empty_state();
        sm.ea[lane] = E0.a;
        sm.eb[lane] = E0.b;
        sm.es[lane] = E0.s;
    }

    const FwdGeo g = fwd_geo<TIn, L, W>(P, b, c, cok, blk, wave);
    SubChunk<TIn, L> sc;
    sc.load(g.rk, g.rv, g.vin, g.row_in);
    SubWork<TIn, L> sw;
    sw.local(sc, g, ch, eu, wc, uc);
    Chunk1<TIn, L> rch;  // the gate's inputs, loaded once the key/value registers are free
    if (Gated) rch.load(g.rr, g.vin, g.row_in);
    sm.a[wave][lane] = sw.st.a;
    sm.b[wave][lane] = sw.st.b;
    sm.s[wave][lane] = sw.st.s;
    __syncthreads();

    // every wave: prefix of the sub-chunks before it; the last wave also forms
    // the block aggregate and fetches / publishes the block carry
    const St pref = wave_prefix(sm, wave, lane, dL);
    if (wave == W - 1) {
        St E = empty_state();
        if (state_in) E = St{sm.ea[lane], sm.eb[lane], sm.es[lane]};  // written by this wave above
        if (P.nblocks > 1) {
            double dTB = 1.0;
#pragma unroll
            for (int i = 0; i < W; ++i) dTB *= dL;
            const Rsrc rc = make_rsrc(P.carry, P.carry_bytes);
            const uint32_t slot = (uint32_t)(((tile * P.nblocks + blk) * 64 + lane) * 16);
            if (blk > 0) E = wait_state(rc, slot - 64 * 16, tag, P.spin, P.hdr);  // block blk-1, same lane
            if (blk < P.nblocks - 1)  // then this block is full
                publish_state(rc, slot, combine(E, combine(pref, sw.st, dL), dTB), tag);
            done_before = stream_count(P.sc, j, lane);
        }
        sm.ea[lane] = E.a;
        sm.eb[lane] = E.b;
        sm.es[lane] = E.s;
    }
    __syncthreads();
    double dpow = 1.0;
    for (int i = 0; i < wave; ++i) dpow *= dL;
    const St s2 = combine(St{sm.ea[lane], sm.eb[lane], sm.es[lane]}, pref, dpow);
    sw.template outputs<Gated>(s2, g, rch, ch, eu, fast, P.y != nullptr, P.C);

    // the state after token T, from the wave that holds it: its carry-in
    // combined with its summary when the sub-chunk is full, else a re-run of
    // its real tokens from the carry-in (the padding past T must not enter it)
    if (P.a_out != nullptr && g.nvalid > 0 && blk * (int64_t)(L * W) + (int64_t)wave * L + g.nvalid == P.T) {
        St st = s2;
        if (g.nvalid == L) {
            st = combine(s2, sw.st, dL);
        } else {
#pragma unroll 1
            for (int j = 0; j < g.nvalid; ++j) {
                const float e = key_weight(st, key_split(BufLd<TIn>::at(g.rk, g.vin, j * g.row_in)));
                token_add(st, e, BufLd<TIn>::at(g.rv, g.vin, j * g.row_in), ch);
            }
        }
        if (cok) {
            const int64_t i = b * P.C + c;
            state_to_abp(st, P.a_out[i], P.b_out[i], P.p_out[i]);
        }
    }
    if (P.nblocks > 1 && wave == W - 1)  // the carry wave
        stream_finish(P.hdr, P.sc, j, done_before, static_cast<uint32_t>(per * P.nblocks),
                      static_cast<uint32_t>(P.nstream), tag, lane);
}


// Whole-tile forward (bf16 inputs): one workgroup per (batch row, 64-channel
// tile) walks the time blocks of its tile in order, so the carry between
// blocks stays in the workgroup: no carry slots, tickets or workspace.  Used
// when there are enough tiles to give every CU two workgroups.
//
// Per block of W L tokens (wave i owning tokens [iL, (i+1)L)):
//   stage   the next block's k and v stream into LDS by asynchronous buffer ->
//           LDS copies (16 bytes per lane, stage_rows) while this block is
//           computed; a wave reads its own rows of the staged block into
//           registers, waits for those LDS reads, then starts the copies of its
//           next rows into the same LDS rows.  The copies are not tracked by the
//           compiler: wait_staged() before the LDS reads, wait_lds_reads()
//           before the next copies.
//   local   every wave runs its L tokens from the empty state at the fixed
//           scale of its largest key, keeping the local numerator and
//           denominator of every token (as the time-split kernel);
//   scan    the last wave walks the block's W summaries in order from the
//           block's carry-in, X_{i+1} = d^L X_i + S_i (W combines per block,
//           in float64, so that a saved state is rounded to float32 once
//           however many combines carried it), and leaves every wave's
//           carry-in X_i in LDS; it keeps X_W, the next block's carry-in;
//   output  y = (N + d^j X_A) / (D + d^j X_B) as the time-split kernel.
// bf16 inputs carry 2^-8 relative rounding and their outputs a 2e-3 bound, so
// inside a sub-chunk the key weight is one exp2 of k log2 e - scale (two FMAs,
// log2 e in two words) and the decay one float32 product per token; the
// carries between sub-chunks keep the exact decay powers.  (The float32 path keeps the
// exact key split and the two-term decay of the time-split kernel.)
// Barriers fence LDS only (lds_sync_lgkm): the staged copies and the output
// stores stay in flight across them.
template <int L, int W>
struct FwdStage {
    uint16_t x[W][2][L][64];  // [wave][k, v][token][channel]
};

template <int W>
struct TileShared {
    float sa[W][64], sb[W][64];  // wave summaries
    int ss[W][64];
    float xa[W][64], xb[W][64];  // wave carry-ins
    int xs[W][64];
};

template <int L>
struct TileWork {
    float N[L], D[L];
    St st;   // summary of the sub-chunk from the empty state
    int sl;  // fixed local scale
    bool fast_local;

    // kv: k in the low, v in the high half of each word (bf16 bits)
    __device__ __forceinline__ void local(const uint32_t (&kv)[L], const FwdGeo& g, const Chan& ch, float eu,
                                          float d, bool lane_ok) {
        float kmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < L; ++j) kmax = fmaxf(kmax, __uint_as_float(kv[j] << 16));
        sl = key_split(kmax).n;
        fast_local = __all(lane_ok & (kmax * kL2E < kNMax));
        if (fast_local) {
            const float slf = static_cast<float>(sl);
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int j = 0; j < L; ++j) {
                const float kj = __uint_as_float(kv[j] << 16);
                const float vj = __uint_as_float(kv[j] & 0xffff0000u);
                const float e = ex2(fmaf(kj, kL2E_lo, fmaf(kj, kL2E, -slf)));
                const float E = e * eu;
                N[j] = fmaf(E, vj, a);
                D[j] = b + E;
                a = fmaf(d, a, e * vj);
                b = fmaf(d, b, e);
            }
            st = St{a, b, sl};
            fast_local = __all(b >= kTiny);
        }
        if (!fast_local) {  // general pass 1, reading one token at a time (rare: kept register-light)
            st = empty_state();
#pragma unroll 1
            for (int j = 0; j < L; ++j) {
                const float e = key_weight(st, key_split(BufLd<uint16_t>::at(g.rk, g.vin, j * g.row_in)));
                token_add(st, e, BufLd<uint16_t>::at(g.rv, g.vin, j * g.row_in), ch);
            }
        }
    }

    // Outputs (and the saved state at the sub-chunk's start) from the carry-in X.
    template <bool Gated>
    __device__ __forceinline__ void outputs(const St& X, const FwdGeo& g, const Chunk1<uint16_t, L>& rch,
                                            const Chan& ch, float eu, bool fast, bool want_y, int64_t C) const {
        static_assert(L == kCkptLen, "one saved state per sub-chunk");
        const int lvl = X.s - sl + __builtin_amdgcn_frexp_expf(X.b);
        const bool dp_normal = ipow<L - 1>(ch.dd) >= 0x1p-125;  // see SubWork::outputs
        const bool carry_fits =
            !(X.b > 0.f) | ((lvl <= kCarryAbove) & (X.s - sl + __builtin_amdgcn_frexp_expf(X.a) <= kCarryAbove + 20) &
                            (dp_normal | (lvl <= 24)));
        bool fast_out = fast_local && __all(carry_fits);
        if (fast_out && want_y)
            fast_out = __all(corrected_outputs<Gated>(X, sl, N, D, rch, ch, g.ry, g.vout, g.row_out) >= kTiny);
        if (fast_out) {
            if (g.ckp != nullptr) {
                g.ckp[0] = X.a;
                g.ckp[C] = X.b;
                g.ckp[2 * C] = static_cast<float>(X.s);
            }
        } else if (fast) {  // general path: rewrites every output of the wave
            general_outputs<true, Gated, uint16_t, L>(X, g.rk, g.rv, g.rr, g.vin, g.row_in, g.nvalid, ch, eu, g.ry,
                                                      g.vout, g.row_out, g.ckp, C);
        } else {
            general_outputs<false, Gated, uint16_t, L>(X, g.rk, g.rv, g.rr, g.vin, g.row_in, g.nvalid, ch, eu,
                                                       g.ry, g.vout, g.row_out, g.ckp, C);
        }
    }
};

// Last: no saved states are written, so no backward will read k, v again: they are staged
// non-temporal (kStageLast); a forward saving states for its backward keeps the default policy.
template <int L, int W, bool Gated, bool Last>
__global__ void __launch_bounds__(64 * W, 4) fwd_tile_kernel(FwdChunk P) {
    __shared__ TileShared<W> sm;
    __shared__ FwdStage<L, W> stage;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / P.nct;
    const int64_t c0 = (tile - b * P.nct) * 64;
    const int64_t c = c0 + lane;
    const bool cok = c < P.C;
    const float wc = cok ? P.w[c] : 0.f;
    const float uc = cok ? P.u[c] : 0.f;
    const Chan ch = make_chan(wc, uc);
    const bool lane_ok = (wc >= 0.f) & (fabsf(uc) <= kFastU);
    const bool fast = __all(lane_ok);
    const float eu = ex2(ch.u2);
    const float d = static_cast<float>(ch.dd);
    const double dL = ipow<L>(ch.dd);

    // the scanning wave's running carry, in float64: the state before the current block
    StD E = to_d(empty_state());
    if (wave == W - 1 && P.a_in != nullptr && cok) {
        const int64_t i = b * P.C + c;
        E = to_d(state_from_abp(P.a_in[i], P.b_in[i], P.p_in[i]));
    }

    {
        const FwdGeo g0 = fwd_geo<uint16_t, L, W>(P, b, c, cok, 0, wave);
        stage_rows<uint16_t, L, Last ? kStageLast : kStageKeep>(g0.rk, stage.x[wave][0], int64_t{wave} * L, c0, P.C, lane);
        stage_rows<uint16_t, L, Last ? kStageLast : kStageKeep>(g0.rv, stage.x[wave][1], int64_t{wave} * L, c0, P.C, lane);
    }
    for (int64_t blk = 0; blk < P.nblocks; ++blk) {
        const FwdGeo g = fwd_geo<uint16_t, L, W>(P, b, c, cok, blk, wave);
        uint32_t kv[L];
        // after the first block, every path issued at least the L output stores of the previous
        // block after this block's copies (outputs runs corrected_outputs whenever y is wanted)
        if (blk == 0 || P.y == nullptr)
            wait_staged();
        else
            wait_staged_before<L>();
#pragma unroll
        for (int j = 0; j < L; ++j)
            kv[j] = static_cast<uint32_t>(stage.x[wave][0][j][lane]) |
                    (static_cast<uint32_t>(stage.x[wave][1][j][lane]) << 16);
        wait_lds_reads();
        if (blk + 1 < P.nblocks) {
            const FwdGeo gn = fwd_geo<uint16_t, L, W>(P, b, c, cok, blk + 1, wave);
            stage_rows<uint16_t, L, Last ? kStageLast : kStageKeep>(gn.rk, stage.x[wave][0], int64_t{wave} * L, c0, P.C, lane);
            stage_rows<uint16_t, L, Last ? kStageLast : kStageKeep>(gn.rv, stage.x[wave][1], int64_t{wave} * L, c0, P.C, lane);
        }
        TileWork<L> tw;
        tw.local(kv, g, ch, eu, d, lane_ok);
        Chunk1<uint16_t, L> rch;  // the gate's inputs, read from global memory
        if (Gated) rch.load(g.rr, g.vin, g.row_in);
        sm.sa[wave][lane] = tw.st.a;
        sm.sb[wave][lane] = tw.st.b;
        sm.ss[wave][lane] = tw.st.s;
        lds_sync_lgkm();
        if (wave == W - 1) {
            StD X = E;
#pragma unroll 1
            for (int i = 0; i < W; ++i) {
                const St xf = to_f(X);
                sm.xa[i][lane] = xf.a;
                sm.xb[i][lane] = xf.b;
                sm.xs[i][lane] = xf.s;
                X = combine_d(X, St{sm.sa[i][lane], sm.sb[i][lane], sm.ss[i][lane]}, dL);
            }
            E = X;
        }
        lds_sync_lgkm();
        const St Xw{sm.xa[wave][lane], sm.xb[wave][lane], sm.xs[wave][lane]};
        tw.template outputs<Gated>(Xw, g, rch, ch, eu, fast, P.y != nullptr, P.C);
        if (P.a_out != nullptr && g.nvalid > 0 && blk * (int64_t)(L * W) + (int64_t)wave * L + g.nvalid == P.T) {
            St st = Xw;
            if (g.nvalid == L) {
                st = combine(Xw, tw.st, dL);
            } else {
#pragma unroll 1
                for (int j = 0; j < g.nvalid; ++j) {
                    const float e = key_weight(st, key_split(BufLd<uint16_t>::at(g.rk, g.vin, j * g.row_in)));
                    token_add(st, e, BufLd<uint16_t>::at(g.rv, g.vin, j * g.row_in), ch);
                }
            }
            if (cok) {
                const int64_t i = b * P.C + c;
                state_to_abp(st, P.a_out[i], P.b_out[i], P.p_out[i]);
            }
        }
    }
}

// T == 0: the state after the (empty) sequence is the state before it.
__global__ void state_passthrough_kernel(int64_t n, const float* a_in, const float* b_in, const float* p_in,
                                         float* a_out, float* b_out, float* p_out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float a = 0.f, b = 0.f, p = -1e38f;
    if (a_in != nullptr) {
        a = a_in[i];
        b = b_in[i];
        p = p_in[i];
    }
    a_out[i] = a;
    b_out[i] = b;
    p_out[i] = p;
}

namespace {
#ifndef WKV_FWD_L
#define WKV_FWD_L 32
#endif
#ifndef WKV_FWD_W
#define WKV_FWD_W 8
#endif
constexpr int kFwdL = WKV_FWD_L;  // tokens per wave (sub-chunk)
constexpr int kFwdW = WKV_FWD_W;  // waves per workgroup
#ifndef WKV_FWD_TILE_L
#define WKV_FWD_TILE_L 16
#endif
#ifndef WKV_FWD_TILE_W
#define WKV_FWD_TILE_W 4
#endif
#ifndef WKV_FWD_TILE_W_LAST
#define WKV_FWD_TILE_W_LAST 8
#endif
constexpr int kTileL = WKV_FWD_TILE_L;  // whole-tile kernel: tokens per wave
// whole-tile kernel: waves per workgroup, for a forward that saves the backward's states (a training
// step: 4-wave workgroups make the following backward 1.5 % faster at B=8 T=1024 C=4096, with the
// forward itself unchanged) and for one that saves none (8 waves: 4 % faster there)
constexpr int kTileW = WKV_FWD_TILE_W;
constexpr int kTileWLast = WKV_FWD_TILE_W_LAST;
static_assert(kFwdL % kCkptLen == 0 && kTileL % kCkptLen == 0, "sub-chunks must start on saved-state boundaries");

struct FwdLayout {
    int64_t nct, ntiles, nblocks;
    size_t off_carry, carry_bytes, bytes;
};

FwdLayout fwd_layout(int64_t B, int64_t T, int64_t C) {
    FwdLayout l{};
    l.nct = (C + 63) / 64;
    l.ntiles = B * l.nct;
    l.nblocks = (T + kFwdL * kFwdW - 1) / (kFwdL * kFwdW);
    if (l.nblocks <= 1) return l;  // no cross-workgroup carries, no workspace
    l.off_carry = kWsPrefix;  // after the counters (wkv_scan.h)
    l.carry_bytes = static_cast<size_t>(l.ntiles * l.nblocks * 64) * 16;
    l.bytes = l.off_carry + l.carry_bytes;
    if (l.carry_bytes > 0xffffffffull) l.bytes = SIZE_MAX;  // carries are addressed through a 32-bit buffer resource
    return l;
}
}  // namespace

size_t fwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t C) { return fwd_layout(B, T, C).bytes; }

#ifndef WKV_FWD_TILE
#define WKV_FWD_TILE 1  // whole-tile forward where there are enough tiles
#endif

template <typename TIn>
hipError_t launch_fwd_chunk_t(const FwdArgs& a, hipStream_t stream) {
    const FwdLayout l = fwd_layout(a.B, a.T, a.C);
    FwdChunk P{};
    P.B = a.B; P.T = a.T; P.C = a.C;
    P.w = a.w; P.u = a.u; P.k = a.k; P.v = a.v; P.y = a.y;
    P.ckpt = static_cast<float*>(a.ckpt);
    P.nblk_ck = a.nblk;
    P.nct = l.nct; P.ntiles = l.ntiles; P.nblocks = l.nblocks;
    P.nstream = 1;
    P.r = a.r;
    P.a_in = a.a_in; P.b_in = a.b_in; P.p_in = a.p_in;
    P.a_out = a.a_out; P.b_out = a.b_out; P.p_out = a.p_out;

    // Enough tiles to give every CU two workgroups, and rows of whole 16-byte
    // chunks for the LDS staging: one workgroup per tile walks the sequence.
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    (void)a16;
    if constexpr (sizeof(TIn) == 2) {
        if (WKV_FWD_TILE && l.ntiles >= 2 * static_cast<int64_t>(ncu) && a.C % 8 == 0 && a16(a.k) && a16(a.v)) {
            const bool last = P.ckpt == nullptr;
            const int tw = last ? kTileWLast : kTileW;
            P.nblocks = (a.T + kTileL * tw - 1) / (kTileL * tw);
            const dim3 grid(static_cast<unsigned>(l.ntiles)), block(64 * tw);
            if (P.r != nullptr && last)
                hipLaunchKernelGGL((fwd_tile_kernel<kTileL, kTileWLast, true, true>), grid, block, 0, stream, P);
            else if (P.r != nullptr)
                hipLaunchKernelGGL((fwd_tile_kernel<kTileL, kTileW, true, false>), grid, block, 0, stream, P);
            else if (last)
                hipLaunchKernelGGL((fwd_tile_kernel<kTileL, kTileWLast, false, true>), grid, block, 0, stream, P);
            else
                hipLaunchKernelGGL((fwd_tile_kernel<kTileL, kTileW, false, false>), grid, block, 0, stream, P);
            return hipGetLastError();
        }
    }

    if (l.nblocks > 1) {
        char* ws = static_cast<char*>(a.ws);
        P.hdr = reinterpret_cast<CallHdr*>(ws);
        P.sc = reinterpret_cast<StreamCtr*>(ws + kWsStreamOff);
        P.nstream = chain_streams(l.ntiles);
        P.spin = spin_limit();
        P.carry = reinterpret_cast<float*>(ws + l.off_carry);
        P.carry_bytes = static_cast<uint32_t>(l.carry_bytes);
    }
    const int64_t grid = l.ntiles * l.nblocks;
    if (P.r != nullptr)
        hipLaunchKernelGGL((fwd_chunk_kernel<TIn, kFwdL, kFwdW, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * kFwdW), 0, stream, P);
    else
        hipLaunchKernelGGL((fwd_chunk_kernel<TIn, kFwdL, kFwdW, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * kFwdW), 0, stream, P);
    return hipGetLastError();
}

hipError_t launch_state_passthrough(const FwdArgs& a, hipStream_t stream) {
    const int64_t n = a.B * a.C;
    if (n == 0 || a.a_out == nullptr) return hipSuccess;
    hipLaunchKernelGGL(state_passthrough_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       n, a.a_in, a.b_in, a.p_in, a.a_out, a.b_out, a.p_out);
    return hipGetLastError();
}

hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t stream) {
    return a.bf16 ? launch_fwd_chunk_t<uint16_t>(a, stream) : launch_fwd_chunk_t<float>(a, stream);
}

}  // namespace wkv
