// Multi-head matrix-state WKV on MFMA: RWKV-5's forward and backward, and RWKV-6's
// forward (the same state with a per-token decay, further below).
//
// Per head (N = 64 channels; "RWKV模型深度研究报告", sections 1.3.2 and 1.3.3:
// a matrix-valued state with per-channel decay, updated by a diagonal decay
// and a value-key outer product; the intelliparadigm.com post, section 2.1:
// channel groups with their own decay rates):
//     S_t = diag(e^{-w}) S_{t-1} + k_t^T v_t                  (S: key x value)
//     o_t = r_t (S_{t-1} + diag(u) k_t^T v_t)
// Chunkwise-parallel form ("RWKV模型深度研究报告", section 1.4.1): a chunk of
// 64 tokens t0 + tau, tau < 64, starting from the state S0, gives
//     o_tau = (r_tau . e^{-w tau}) S0                               (inter)
//           + sum_{sig < tau} (sum_i r_tau,i k_sig,i e^{-w_i (tau-1-sig)}) v_sig
//           + (sum_i r_tau,i u_i k_tau,i) v_tau                     (intra)
//     S_end = diag(e^{-w n}) S0 + sum_{sig < n} diag(e^{-w (n-1-sig)}) k_sig^T v_sig
// with n the chunk's token count.  Every product above is a 64 x 64 x 64 (or
// smaller) matrix product: bf16 operands on v_mfma_f32_16x16x16_bf16, float32
// accumulation.  The decay factors are split so that no operand exceeds its
// inputs: between 16-token blocks P > Q the factor e^{-w (tau-1-sig)} is
// e^{-w (tau-p0)} e^{-w (p0-1-sig)} with p0 the first token of block P (both
// <= 1); inside a diagonal block it is e^{-w (tau-c)} e^{w (sig+1-c)} about
// the block's middle c, with w capped at kWCap there so that neither factor
// exceeds e^{80} (a channel decaying by more than e^{-10} per token then keeps
// its older in-block terms at most e^{-10} of the token's own term too large).
//
// One workgroup of four waves per (batch row, head) walks the chunks in order.
// Wave w owns key rows 16w..16w+15 of the state (four 16 x 16 accumulator
// tiles, float32) and output tokens 16w..16w+15 of each chunk.  The next
// chunk's r, k, v stream into LDS by asynchronous buffer -> LDS copies while
// the current one is computed; the state crosses the waves through LDS as
// bf16, transposed, for the inter-chunk product.  Two barriers per chunk: one
// before the chunk's inputs and state are read, one before the state in LDS
// is overwritten.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_device.h"
#include "wkv_launch.h"
#include "wkv_scan.h"

namespace wkv {
namespace {

constexpr int kN = 64;       // head size
constexpr int kLc = 64;      // tokens per chunk
constexpr int kWaves5 = 4;   // 16 tokens / key rows per wave
constexpr float kWCap = 10.f;

typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// LDS rows are read one row per lane (16 lanes at a time), so rows that are a
// multiple of the bank span would put all 16 reads in the same banks.  The
// tables and the state are padded by 16 bytes a row; the staged inputs, whose
// rows the buffer -> LDS copies write back to back, are swizzled instead: the
// 16-byte chunk q of row t sits in slot q ^ (t & 7) (see sw()).
constexpr int kPadF = kN + 4;  // float rows
constexpr int kPadH = kN + 8;  // bf16 rows

struct Wkv5Shared {
    uint16_t in[2][3][kLc][kN];  // staged r, k, v of a chunk, [token][swizzled channel], two chunks
    uint16_t st[kN][kPadH];      // state before the chunk, bf16, [value][key]
    float pw[kLc + 1][kPadF];    // e^{-w n}, n = 0..64
    float pe[17][kPadF];         // e^{w' m}, m = -8..8, w' = min(w, kWCap)
    float uu[kN];
};

// position of channel c in swizzled row t of a staged input
__device__ __forceinline__ int sw(int t, int c) { return (((c >> 3) ^ (t & 7)) << 3) | (c & 7); }

__device__ __forceinline__ f4 mfma(s4 a, s4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }

__device__ __forceinline__ uint32_t pk2(float a, float b) {
    const f2 p = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf2));
}

typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ s4 pack4(float a, float b, float c, float d) {
    const u2 x = {pk2(a, b), pk2(c, d)};
    return __builtin_bit_cast(s4, x);
}

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

// four consecutive bf16 of an LDS row, widened
__device__ __forceinline__ f4 row4(const uint16_t* p) {
    const u16x4 x = *reinterpret_cast<const u16x4*>(p);
    return f4{bf(x[0]), bf(x[1]), bf(x[2]), bf(x[3])};
}

__device__ __forceinline__ f4 frow4(const float* p) { return *reinterpret_cast<const f4*>(p); }

__device__ __forceinline__ s4 mul_pack(f4 x, f4 f) { return pack4(x[0] * f[0], x[1] * f[1], x[2] * f[2], x[3] * f[3]); }

__device__ __forceinline__ s4 as_s4(uint16_t a, uint16_t b, uint16_t c, uint16_t d) {
    const u16x4 x = {a, b, c, d};
    return __builtin_bit_cast(s4, x);
}

// four consecutive bf16 of an LDS row as an MFMA operand, unchanged
__device__ __forceinline__ s4 raw4(const uint16_t* p) { return __builtin_bit_cast(s4, *reinterpret_cast<const u16x4*>(p)); }

// The 16 x 16 x 32 product (gfx950) for the backwards' products whose operands are both staged rows,
// unchanged: each lane gives eight consecutive bf16 (one 16-byte LDS read) of its row of A and of its
// column of B.  Which eight of the 32 contracted indices a lane holds is the same for A and B, so
// loading both from channels c8 .. c8 + 7, c8 = 32 J + 8 g, contracts over channels 32 J .. 32 J + 31
// whatever the instruction's order inside the slice; the 4 outputs per lane are laid out as in the
// 16 x 16 x 16 product.
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf8 raw8(const uint16_t* p) { return __builtin_bit_cast(bf8, *reinterpret_cast<const u16x8*>(p)); }
__device__ __forceinline__ f4 mfma32(bf8 a, bf8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// Tokens tb + 4 g + e (e = 0..3) of channel c0 + l16 of a staged 64 x 64 tile (a column) as a raw
// MFMA operand, by one transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// q reads four channels of one row and lane j receives element j % 4 of lane 4 e + j / 4's read,
// so lane (l16, g) names row tb + 4 g + l16 / 4, channels c0 + 4 (l16 % 4) .. + 3.
__device__ __forceinline__ s4 col_tr(const uint16_t (*X)[kN], int tb, int c0, int l16, int g) {
    const int t = tb + 4 * g + (l16 >> 2), c = c0 + 4 * (l16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)&X[t][sw(t, c)]);
}

// kOut = false: a state-only pass (no outputs, only the chunk-start states in P.ckpt
// and the final state), as the backward needs.  kLast: the call is its inputs' last reader (an
// output pass saving no chunk-start states: no backward follows to read r, k, v again), so they
// are staged non-temporal.
template <bool kOut, bool kLast = false>
__global__ void __launch_bounds__(64 * kWaves5, 2) wkv5_fwd_kernel(Wkv5Args P) {
    __shared__ Wkv5Shared sm;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g = lane >> 4;  // MFMA lane coordinates: row/column l16, k-group g
    // time split (P.nseg > 1): this workgroup runs segment seg of (batch row, head) bh
    const int64_t seg = blockIdx.x % P.nseg;
    const int64_t bh = blockIdx.x / P.nseg;
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int64_t nch = (P.T + kLc - 1) / kLc;

    // tables of the head's decay powers and bonus
    for (int q = threadIdx.x; q < (kLc + 1) * kN; q += 64 * kWaves5) {
        const int n = q / kN, i = q % kN;
        sm.pw[n][i] = ex2(-P.w[h * kN + i] * static_cast<float>(n) * kL2E);
    }
    for (int q = threadIdx.x; q < 17 * kN; q += 64 * kWaves5) {
        const int m = q / kN - 8, i = q % kN;
        sm.pe[m + 8][i] = ex2(fminf(P.w[h * kN + i], kWCap) * static_cast<float>(m) * kL2E);
    }
    if (threadIdx.x < kN) sm.uu[threadIdx.x] = P.u[h * kN + threadIdx.x];

    // the state: wave wv, tile J, lane (l16, g), element e holds S[16 wv + 4 g + e][16 J + l16]
    f4 S[4];
    const int64_t ch_lo = P.nseg > 1 ? seg * P.cps : 0;
    const int64_t ch_hi = P.nseg > 1 && ch_lo + P.cps < nch ? ch_lo + P.cps : nch;
    const int64_t sbase = (bh * P.nseg + seg) * kN * kN;  // this segment's start and end state
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[J][e] = P.s_in != nullptr ? P.s_in[sbase + (16 * wv + 4 * g + e) * kN + 16 * J + l16] : 0.f;

    // the rows of head h, batch row b, chunk ch as a buffer: [token][C] bf16, head offset h*64
    auto chunk_rsrc = [&](const uint16_t* base, int64_t ch) {
        const int64_t t0 = ch * kLc;
        const int64_t n = (P.T - t0) < kLc ? (P.T - t0) : kLc;
        return make_rsrc(base + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((n - 1) * C + kN) * 2));
    };
    auto stage = [&](int64_t ch, int buf) {  // wave wv copies rows 16 wv .. 16 wv + 15 of r, k, v
        const uint16_t* src[3] = {P.r, P.k, P.v};
#pragma unroll
        for (int a = kOut ? 0 : 1; a < 3; ++a) {  // a state-only pass needs no r
            const Rsrc rs = chunk_rsrc(src[a], ch);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 16 * wv + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);  // the global chunk that lands in slot lane % 8
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(row) * C) * 2 + q * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.in[buf][a][16 * wv + 8 * i][0], 16, voff, 0, 0, kLast ? kStageLast : kStageKeep);
            }
        }
    };
    auto put_state = [&]() {  // bf16, transposed: st[value][key]
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const uint32_t lo = pk2(S[J][0], S[J][1]), hi = pk2(S[J][2], S[J][3]);
            uint32_t* p = reinterpret_cast<uint32_t*>(&sm.st[16 * J + l16][16 * wv + 4 * g]);
            p[0] = lo;
            p[1] = hi;
        }
    };

    stage(ch_lo, 0);
    if constexpr (kOut) put_state();
    wait_staged();
    const int P0 = 16 * wv;  // first token of this wave's output block, chunk-relative

    // Each wave confirms its copy of chunk ch + 1 (issued at the start of chunk
    // ch) just before storing chunk ch's outputs, so the barrier that opens a
    // chunk needs no memory wait and the stores drain during the next chunk.
    for (int64_t ch = ch_lo; ch < ch_hi; ++ch) {
        const int buf = static_cast<int>((ch - ch_lo) & 1);
        const int64_t t0 = ch * kLc;
        const int nv = static_cast<int>((P.T - t0) < kLc ? (P.T - t0) : kLc);
        lds_sync();  // this chunk's inputs, the tables and the state are in LDS for every wave
        if (ch + 1 < ch_hi) stage(ch + 1, buf ^ 1);
        if (P.ckpt != nullptr) {  // the state before the chunk, bf16 [key][value], for the backward
            uint16_t* cp = P.ckpt + (bh * nch + ch) * kN * kN;
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t h2 = pk2(S[J][e], 0.f);
                    cp[(16 * wv + 4 * g + e) * kN + 16 * J + l16] = static_cast<uint16_t>(h2 & 0xffffu);
                }
        }

        const uint16_t(*R)[kN] = sm.in[buf][0];
        const uint16_t(*K)[kN] = sm.in[buf][1];
        const uint16_t(*V)[kN] = sm.in[buf][2];
        const int tau = P0 + l16;  // this lane's output token (as the m / n index of the products)

        // ---- inter-chunk: O[J] = sum_I (r . e^{-w tau}) S0 --------------------------
        f4 O[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) O[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = 0; I < 4 && kOut; ++I) {
            const int c4 = 16 * I + 4 * g;
            const s4 a = mul_pack(row4(&R[tau][sw(tau, c4)]), frow4(&sm.pw[tau][c4]));
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                O[J] = mfma(a, raw4(&sm.st[16 * J + l16][c4]), O[J]);
            }
        }

        // ---- values as B operands: Vb[Q][J] holds V[16 Q + 4 g + e][16 J + l16] -------
        s4 Vb[4][4];
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
#pragma unroll
            for (int J = 0; J < 4; ++J) Vb[Q][J] = col_tr(V, 16 * Q, 16 * J, l16, g);

        // ---- intra-chunk attention, transposed: At[sig][tau], lane holds
        //      A[tau = P0 + l16][sig = 16 Q + 4 g + e] (the A operand of A V) -----------
        s4 rof[4];  // r_tau e^{-w (tau - P0)}, the off-diagonal blocks' receptance operand
#pragma unroll
        for (int I = 0; I < 4 && kOut; ++I) {
            const int c4 = 16 * I + 4 * g;
            rof[I] = mul_pack(row4(&R[tau][sw(tau, c4)]), frow4(&sm.pw[tau - P0][c4]));
        }
#pragma unroll
        for (int Q = 0; Q < 4 && kOut; ++Q) {
            if (Q > wv) break;
            f4 At = {0.f, 0.f, 0.f, 0.f};
            const int sig = 16 * Q + l16;  // this lane's key token (m index of K~)
            if (Q < wv) {  // factors about p0 = P0: e^{-w (tau - p0)}, e^{-w (p0 - 1 - sig)}
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int c4 = 16 * I + 4 * g;
                    const s4 ka = mul_pack(row4(&K[sig][sw(sig, c4)]), frow4(&sm.pw[P0 - 1 - sig][c4]));
                    At = mfma(ka, rof[I], At);
                }
            } else {  // diagonal block: about c = P0 + 8, w capped; then the bonus on the diagonal
                f4 Bn = {0.f, 0.f, 0.f, 0.f};
                const int mid = P0 + 8;
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int c4 = 16 * I + 4 * g;
                    const f4 kr = row4(&K[sig][sw(sig, c4)]), rr = row4(&R[tau][sw(tau, c4)]);
                    const s4 ka = mul_pack(kr, frow4(&sm.pe[sig + 1 - mid + 8][c4]));
                    const s4 rb = mul_pack(rr, frow4(&sm.pe[mid - tau + 8][c4]));
                    At = mfma(ka, rb, At);
                    const s4 kp = raw4(&K[sig][sw(sig, c4)]);
                    const s4 ru = mul_pack(rr, frow4(&sm.uu[c4]));
                    Bn = mfma(kp, ru, Bn);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {  // lane holds (sig_local = 4 g + e, tau_local = l16)
                    const int sl = 4 * g + e;
                    At[e] = sl < l16 ? At[e] : (sl == l16 ? Bn[e] : 0.f);
                }
            }
            const s4 a = pack4(At[0], At[1], At[2], At[3]);
#pragma unroll
            for (int J = 0; J < 4; ++J) O[J] = mfma(a, Vb[Q][J], O[J]);
        }
        if constexpr (kOut) lds_sync();  // every wave has read the state before it is overwritten

        // ---- state update: S = diag(e^{-w nv}) S + sum_sig (k_sig e^{-w (nv-1-sig)})^T v_sig
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float dn = sm.pw[nv][16 * wv + 4 * g + e];
#pragma unroll
            for (int J = 0; J < 4; ++J) S[J][e] *= dn;
        }
        const int key = 16 * wv + l16;  // m index of K^T
#pragma unroll
        for (int Q = 0; Q < 4; ++Q) {
            float kk[4];
            const u16x4 kc = __builtin_bit_cast(u16x4, col_tr(K, 16 * Q, 16 * wv, l16, g));  // K[s][key]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * Q + 4 * g + e;
                const int n = nv - 1 - s;
                kk[e] = n >= 0 ? bf(kc[e]) * sm.pw[n >= 0 ? n : 0][key] : 0.f;  // past the chunk's end: 0
            }
            const s4 a = pack4(kk[0], kk[1], kk[2], kk[3]);
#pragma unroll
            for (int J = 0; J < 4; ++J) S[J] = mfma(a, Vb[Q][J], S[J]);
        }
        if constexpr (kOut) put_state();
        wait_staged();
        if constexpr (!kOut) continue;

        // ---- outputs: lane holds O[tau = P0 + 4 g + e][16 J + l16] ---------------------
        const Rsrc ro = make_rsrc(P.o + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = static_cast<uint32_t>(((P0 + 4 * g + e) * C + 16 * J + l16) * 4);
                buf_store(O[J][e], ro, off, 0);
            }
    }

    if (P.s_out != nullptr) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) P.s_out[sbase + (16 * wv + 4 * g + e) * kN + 16 * J + l16] = S[J][e];
    }
}

// Output rows are written 64 bytes of a 128-byte line at a time, the two halves by
// different tiles; plain write-back stores let L2 join them (non-temporal ones reached
// memory as up to 1.23x the bytes).
__device__ __forceinline__ void store_wb(float v, Rsrc r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, 0, 0);
}

// ---- RWKV-6: the same operator with a per-token decay --------------------------------------
// S_t = diag(e^{-w_t}) S_{t-1} + k_t^T v_t, o_t = r_t (S_{t-1} + diag(u) k_t^T v_t), w [B, T, C].
// Inside a chunk every decay between two points is e^{-(E[a] - E[b])} with the chunk-local
// cumulative rate E[t] = sum_{t' < t} w'_t' (t = 0..64) and w' = min(w, kWCap6).  The table holds
// log2(e) E[t], so that each factor is one exp2 of a difference of two entries; the factors are
// split exactly as for RWKV-5: about the later 16-token block's first token off the diagonal (both
// factors <= 1) and about the block's middle on it (each factor at most e^{8 kWCap6}).  A rate
// above kWCap6 acts as kWCap6 (the state then keeps at most e^{-10} of itself at that token
// instead of less).
constexpr float kWCap6 = 10.f;

struct Wkv6Shared {
    uint16_t in[2][3][kLc][kN];  // staged r, k, v of a chunk, [token][swizzled channel], two chunks
    uint16_t st[kN][kPadH];      // state before the chunk, bf16, [value][key]
    float E[kLc + 1][kN];        // E[t][i], float4 slot (i / 4) ^ (t & 15) of row t
    float uu[kN];
};

// position of channel c in row t of the cumulative-rate table
__device__ __forceinline__ int swE(int t, int c) { return (((c >> 2) ^ (t & 15)) << 2) | (c & 3); }

__device__ __forceinline__ f4 exp2_neg4(f4 x) {  // 2^{-x}, elementwise: e^{-x} for base-2 table entries
    return f4{ex2(-x[0]), ex2(-x[1]), ex2(-x[2]), ex2(-x[3])};
}

// kOut = false: a state-only pass (the chunk-start states into P.ckpt and the final state).
// kLast as for RWKV-5.
template <bool kOut, bool kLast = false>
__global__ void __launch_bounds__(64 * kWaves5, 2) wkv6_fwd_kernel(Wkv6Args P) {
    __shared__ Wkv6Shared sm;
    // lane coordinates; made opaque at the top of every chunk so that lane-dependent LDS
    // addresses are recomputed inside the chunk instead of being held in registers across it
    int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int l16 = lane & 15, g = lane >> 4;
    // time split (P.nseg > 1): this workgroup runs segment seg of (batch row, head) bh
    const int64_t seg = blockIdx.x % P.nseg;
    const int64_t bh = blockIdx.x / P.nseg;
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int64_t nch = (P.T + kLc - 1) / kLc;
    const int P0 = 16 * wv;

    if (threadIdx.x < kN) {
        sm.uu[threadIdx.x] = P.u[h * kN + threadIdx.x];
        sm.E[0][threadIdx.x] = 0.f;  // row 0 is never staged over
    }
    f4 S[4];  // S[J][e] = S[16 wv + 4 g + e][16 J + l16]
    const int64_t ch_lo = P.nseg > 1 ? seg * P.cps : 0;
    const int64_t ch_hi = P.nseg > 1 && ch_lo + P.cps < nch ? ch_lo + P.cps : nch;
    const int64_t sbase = (bh * P.nseg + seg) * kN * kN;  // this segment's start and end state
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[J][e] = P.s_in != nullptr ? P.s_in[sbase + (16 * wv + 4 * g + e) * kN + 16 * J + l16] : 0.f;

    auto chunk_rows = [&](int64_t ch) {
        const int64_t t0 = ch * kLc;
        return (P.T - t0) < kLc ? (P.T - t0) : kLc;
    };
    auto stage = [&](int64_t ch, int buf) {  // wave wv copies rows 16 wv .. 16 wv + 15 of r, k, v
        const uint16_t* src[3] = {P.r, P.k, P.v};
        const int64_t n = chunk_rows(ch);
#pragma unroll
        for (int a = kOut ? 0 : 1; a < 3; ++a) {  // a state-only pass needs no r
            const Rsrc rs = make_rsrc(src[a] + ((b * P.T + ch * kLc) * C + h * kN), static_cast<uint32_t>(((n - 1) * C + kN) * 2));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = 16 * wv + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(row) * C) * 2 + q * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.in[buf][a][16 * wv + 8 * i][0], 16, voff, 0, 0, kLast ? kStageLast : kStageKeep);
            }
        }
    };
    // the rates one lane scans, straight into registers a chunk ahead: lane (l16, g) of wave wv takes
    // channel 16 wv + l16 over tokens 16 g .. 16 g + 15 (zeros past the sequence, by the range check)
    auto load_w = [&](int64_t ch, float (&x)[16]) {
        const int64_t n = chunk_rows(ch);
        const Rsrc rs = make_rsrc(P.w + ((b * P.T + ch * kLc) * C + h * kN), static_cast<uint32_t>(((n - 1) * C + kN) * 4));
        const uint32_t v0 = static_cast<uint32_t>((static_cast<int64_t>(16 * g) * C + 16 * wv + l16) * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            x[i] = BufLd<float>::at(rs, v0 + static_cast<uint32_t>(i * C * 4), 0);
    };
    auto put_state = [&]() {  // bf16, transposed: st[value][key]
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const uint32_t lo = pk2(S[J][0], S[J][1]), hi = pk2(S[J][2], S[J][3]);
            uint32_t* p = reinterpret_cast<uint32_t*>(&sm.st[16 * J + l16][16 * wv + 4 * g]);
            p[0] = lo;
            p[1] = hi;
        }
    };
    auto e4 = [&](int t, int c4) { return frow4(&sm.E[t][swE(t, c4)]); };  // E[t][c4 .. c4 + 3]
    auto e1 = [&](int t, int c) { return sm.E[t][swE(t, c)]; };

    float wn[16];  // the rates of the chunk about to be scanned
    stage(ch_lo, 0);
    load_w(ch_lo, wn);
    if constexpr (kOut) put_state();
    wait_staged();

    float rsum = 0.f;  // wave 0, lane = channel: the segment's summed capped rates (log2 e units)
    for (int64_t ch = ch_lo; ch < ch_hi; ++ch) {
        asm volatile("" : "+v"(lane), "+v"(l16), "+v"(g));
        const int buf = static_cast<int>((ch - ch_lo) & 1);
        const int64_t t0 = ch * kLc;
        const int nv = static_cast<int>(chunk_rows(ch));
        lds_sync();  // this chunk's r, k, v and state are in LDS, and every wave is done with the last E
        {  // E[t + 1] = E[t] + min(w_t, cap), in base-2 units (zero rates past the chunk): wave wv takes
           // channels 16 wv .. 16 wv + 15, lane (c, seg) the tokens 16 seg .. 16 seg + 15 of channel c
           // (its rates already in registers); the segments' totals are scanned across the four lanes
           // of a channel
            const int c = 16 * wv + l16, t1 = 16 * g + 1;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = fminf(wn[i], kWCap6) * kL2E;
#pragma unroll
            for (int i = 1; i < 16; ++i) x[i] += x[i - 1];
            float off = 0.f;
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const float v = __shfl_up(x[15], 16 * k, 64);
                if (g >= k) off += v;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.E[t1 + i][swE(t1 + i, c)] = x[i] + off;
        }
        if (ch + 1 < ch_hi) load_w(ch + 1, wn);  // a whole chunk to arrive
        lds_sync();  // E ready
        if (P.seg_rates != nullptr && wv == 0) rsum += sm.E[nv][swE(nv, lane)];
        if (ch + 1 < ch_hi) stage(ch + 1, buf ^ 1);
        if (P.ckpt != nullptr) {  // the state before the chunk, bf16 [key][value], for the backward
            uint16_t* cp = P.ckpt + (bh * nch + ch) * kN * kN;
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    cp[(16 * wv + 4 * g + e) * kN + 16 * J + l16] = static_cast<uint16_t>(pk2(S[J][e], 0.f) & 0xffffu);
        }

        const uint16_t(*R)[kN] = sm.in[buf][0];
        const uint16_t(*K)[kN] = sm.in[buf][1];
        const uint16_t(*V)[kN] = sm.in[buf][2];
        const int tau = P0 + l16;  // this lane's output token (as the m / n index of the products)

        // ---- inter-chunk: O[J] = sum_I (r . e^{-E[tau]}) S0 ----------------------------------
        f4 O[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) O[J] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int I = 0; I < 4 && kOut; ++I) {
            const int c4 = 16 * I + 4 * g;
            const s4 a = mul_pack(row4(&R[tau][sw(tau, c4)]), exp2_neg4(e4(tau, c4)));
#pragma unroll
            for (int J = 0; J < 4; ++J) O[J] = mfma(a, raw4(&sm.st[16 * J + l16][c4]), O[J]);
        }

        // ---- values as B operands: Vb[Q][J] holds V[16 Q + 4 g + e][16 J + l16] -------------
        s4 Vb[4][4];
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
#pragma unroll
            for (int J = 0; J < 4; ++J) Vb[Q][J] = col_tr(V, 16 * Q, 16 * J, l16, g);

        // ---- intra-chunk attention, transposed (lane: A[tau = P0 + l16][sig = 16 Q + 4 g + e]) --
        s4 rof[4];  // r_tau e^{-(E[tau] - E[P0])}, the off-diagonal blocks' receptance operand
#pragma unroll
        for (int I = 0; I < 4 && kOut; ++I) {
            const int c4 = 16 * I + 4 * g;
            rof[I] = mul_pack(row4(&R[tau][sw(tau, c4)]), exp2_neg4(e4(tau, c4) - e4(P0, c4)));
        }
#pragma unroll
        for (int Q = 0; Q < 4 && kOut; ++Q) {
            if (Q > wv) break;
            f4 At = {0.f, 0.f, 0.f, 0.f};
            const int sig = 16 * Q + l16;  // this lane's key token (m index of K~)
            if (Q < wv) {  // e^{-(E[P0] - E[sig + 1])}
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int c4 = 16 * I + 4 * g;
                    const s4 ka = mul_pack(row4(&K[sig][sw(sig, c4)]), exp2_neg4(e4(P0, c4) - e4(sig + 1, c4)));
                    At = mfma(ka, rof[I], At);
                }
            } else {  // about mid = P0 + 8: e^{E[sig + 1] - E[mid]} and e^{-(E[tau] - E[mid])}; then the bonus
                f4 Bn = {0.f, 0.f, 0.f, 0.f};
                const int mid = P0 + 8;
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int c4 = 16 * I + 4 * g;
                    const f4 kr = row4(&K[sig][sw(sig, c4)]), rr = row4(&R[tau][sw(tau, c4)]);
                    const f4 em = e4(mid, c4);
                    const s4 ka = mul_pack(kr, exp2_neg4(em - e4(sig + 1, c4)));
                    const s4 rb = mul_pack(rr, exp2_neg4(e4(tau, c4) - em));
                    At = mfma(ka, rb, At);
                    Bn = mfma(raw4(&K[sig][sw(sig, c4)]), mul_pack(rr, frow4(&sm.uu[c4])), Bn);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {  // lane holds (sig_local = 4 g + e, tau_local = l16)
                    const int sl = 4 * g + e;
                    At[e] = sl < l16 ? At[e] : (sl == l16 ? Bn[e] : 0.f);
                }
            }
            const s4 a = pack4(At[0], At[1], At[2], At[3]);
#pragma unroll
            for (int J = 0; J < 4; ++J) O[J] = mfma(a, Vb[Q][J], O[J]);
        }

        // ---- state update operands, read from E before it is overwritten --------------------------
        //      S = diag(e^{-E[n]}) S + sum_sig (k_sig e^{-(E[n] - E[sig + 1])})^T v_sig
        float dn[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) dn[e] = ex2(-e1(nv, 16 * wv + 4 * g + e));
        s4 aS[4];
        {
            const int key = 16 * wv + l16;  // m index of K^T
            const float en = e1(nv, key);
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                float kk[4];
                const u16x4 kc = __builtin_bit_cast(u16x4, col_tr(K, 16 * Q, 16 * wv, l16, g));  // K[s][key]
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * Q + 4 * g + e;
                    kk[e] = s < nv ? bf(kc[e]) * ex2(e1(s + 1, key) - en) : 0.f;
                }
                aS[Q] = pack4(kk[0], kk[1], kk[2], kk[3]);
            }
        }
        lds_sync();  // every wave has read the state and E
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int J = 0; J < 4; ++J) S[J][e] *= dn[e];
#pragma unroll
        for (int Q = 0; Q < 4; ++Q)
#pragma unroll
            for (int J = 0; J < 4; ++J) S[J] = mfma(aS[Q], Vb[Q][J], S[J]);
        if constexpr (kOut) put_state();
        wait_staged();
        if constexpr (!kOut) continue;

        // ---- outputs: lane holds O[tau = P0 + 4 g + e][16 J + l16] --------------------------------
        const Rsrc ro = make_rsrc(P.o + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = static_cast<uint32_t>(((P0 + 4 * g + e) * C + 16 * J + l16) * 4);
                store_wb(O[J][e], ro, off);
            }
    }

    if (P.seg_rates != nullptr && wv == 0) P.seg_rates[(bh * P.nseg + seg) * kN + lane] = rsum;
    if (P.s_out != nullptr) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) P.s_out[sbase + (16 * wv + 4 * g + e) * kN + 16 * J + l16] = S[J][e];
    }
}

// ---- backward ---------------------------------------------------------------------
// For L = sum_t <go_t, o_t> + <dS_T, S_T>, with the adjoint state
// G_{t-1} = diag(d) G_t + r_t^T go_t (d = e^{-w}; G after the last token is dS_T), per chunk of n tokens with S0 the
// state before it and G1 the adjoint after it (local indices s, sig, tau < n):
//     dv_sig = (k_sig . d^{n-1-sig}) G1 + sum_{s >= sig} A[s][sig] go_s     (A: the forward's
//              attention, its diagonal the bonus sum_i r_s,i u_i k_s,i)
//     dk_sig = d^{n-1-sig} . (G1 v_sig^T) + sum_{s > sig} C[s][sig] r_s d^{s-1-sig}
//              + u . r_sig C[sig][sig]                                      (C = GO V^T)
//     dr_s   = d^s . (S0 go_s^T) + sum_{sig < s} C[s][sig] k_sig d^{s-1-sig} + u . k_s C[s][s]
//     du    += sum_s r_s . k_s C[s][s]
//     dw    -= n d^n . rowsum(G1 . S0) + sum_sig (n-1-sig) d^{n-1-sig} . k_sig . (G1 v_sig^T)
//              + sum_s s d^s . r_s . (S0 go_s^T)
//              + sum_{sig < s} (s-1-sig) d^{s-1-sig} . r_s . k_sig C[s][sig]
//     G0     = d^n . G1 + sum_s (r_s . d^s)^T go_s                (the adjoint before the chunk)
// (dw = -d . sum_t rowsum(G_t . S_{t-1}) expanded over the chunk and multiplied by d).
// The in-chunk sums are matrix products with the decay split about the later
// 16-token block's first token (off-diagonal blocks: both factors <= 1) or
// about the block's middle with w capped at kWCapB (diagonal blocks); lag d^lag
// splits the same way into (s - p) d^{s-p} d^{p-1-sig} + d^{s-p} (p-1-sig) d^{p-1-sig} off the
// diagonal, where both parts are >= 0; inside a diagonal block the two parts would have opposite
// signs and cancel, so that term is taken elementwise with the exact weight (s-1-sig) d^{s-1-sig}.
//
// One workgroup of four waves per (batch row, head) walks the chunks last to first.  Wave w owns
// token block w (its rows of dr, dk, dv) and key rows 16w..16w+15 of G, in registers.  Per
// chunk r, k, v, go and the forward's bf16 chunk-start state arrive by buffer -> LDS copies;
// G crosses the waves through LDS as bf16 for the next chunk's dv and dk.
constexpr float kWCapB = 8.f;  // keeps every in-block intermediate below e^64 times its inputs

struct Wkv5BwdFinal {         // the per-(batch row, head) sums of dw, du, after the chunk walk
    float dwa[kN][17];         // rowsum term: [key][lane l16]
    float dv[kWaves5][4][2][kN];  // [wave][k-group g][dw, du][channel]
    float dd[kWaves5][kN];     // diagonal blocks' lag-weighted term: [wave][channel]
};

struct Wkv5BwdShared {
    union {
        uint16_t in[4][kLc][kN];  // r, k, v, go of the chunk, [token][swizzled channel]
        Wkv5BwdFinal fin;
    };
    uint16_t gs[kN][kPadH];    // G1, bf16, [key][value]
    uint16_t ss[kN][kN];       // S0, bf16, [key][swizzled value], staged like the inputs
    float pw[kLc + 1][kPadF];  // e^{-w n}
    float pe[17][kPadF];       // e^{w' m}, m = -8..8, w' = min(w, kWCapB)
    float uu[kN];
    float cd[kLc];             // C[s][s] = go_s . v_s
    float cdg[kWaves5][16][16];  // each wave's diagonal block of C by lag: [s - 1 - sig][s], lag >= 1 (float32)
};

__global__ void __launch_bounds__(64 * kWaves5, 2) wkv5_bwd_kernel(Wkv5BwdArgs P) {
    __shared__ Wkv5BwdShared sm;
    // lane coordinates; made opaque at the top of every chunk so that the many lane-dependent
    // LDS addresses are recomputed inside the chunk instead of being held in registers across it
    int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int l16 = lane & 15, g = lane >> 4;
    const int64_t seg = blockIdx.x % P.nseg, bh = blockIdx.x / P.nseg;
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int64_t nch = (P.T + kLc - 1) / kLc;
    const int P0 = 16 * wv;
    // time split: this workgroup walks chunks ch_lo .. ch_hi - 1 of its segment from the adjoint after it
    const int64_t ch_lo = P.nseg > 1 ? seg * P.cps : 0;
    const int64_t ch_hi = P.nseg > 1 && ch_lo + P.cps < nch ? ch_lo + P.cps : nch;
    const float* g_end = P.nseg > 1 ? P.gstart + (bh * P.nseg + seg) * kN * kN
                                    : (P.ds_out != nullptr ? P.ds_out + bh * kN * kN : nullptr);

    for (int q = threadIdx.x; q < (kLc + 1) * kN; q += 64 * kWaves5) {
        const int n = q / kN, i = q % kN;
        sm.pw[n][i] = ex2(-P.w[h * kN + i] * static_cast<float>(n) * kL2E);
    }
    for (int q = threadIdx.x; q < 17 * kN; q += 64 * kWaves5) {
        const int m = q / kN - 8, i = q % kN;
        sm.pe[m + 8][i] = ex2(fminf(P.w[h * kN + i], kWCapB) * static_cast<float>(m) * kL2E);
    }
    if (threadIdx.x < kN) sm.uu[threadIdx.x] = P.u[h * kN + threadIdx.x];

    // G: wave wv, tile J, lane (l16, g), element e holds G[16 wv + 4 g + e][16 J + l16];
    // after the last token it is the final state's gradient (or zero)
    f4 G[4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = P0 + 4 * g + e, j = 16 * J + l16;
            G[J][e] = g_end != nullptr ? g_end[key * kN + j] : 0.f;
            sm.gs[key][j] = static_cast<uint16_t>(pk2(G[J][e], 0.f) & 0xffffu);
        }
    float dwv[4] = {0.f, 0.f, 0.f, 0.f}, duv[4] = {0.f, 0.f, 0.f, 0.f};  // channel 16 I + l16
    float dwk[4] = {0.f, 0.f, 0.f, 0.f};                                  // key P0 + 4 g + e (rowsum term)
    float dwd = 0.f;                                                      // channel lane (diagonal blocks)

    const uint16_t(*R)[kN] = sm.in[0];
    const uint16_t(*K)[kN] = sm.in[1];
    const uint16_t(*V)[kN] = sm.in[2];
    const uint16_t(*GO)[kN] = sm.in[3];
    auto rd = [](const uint16_t(*X)[kN], int t, int c) { return bf(X[t][sw(t, c)]); };
    auto row4s = [](const uint16_t(*X)[kN], int t, int c4) { return row4(&X[t][sw(t, c4)]); };
    auto raw4s = [](const uint16_t(*X)[kN], int t, int c4) { return raw4(&X[t][sw(t, c4)]); };
    auto raw8s = [](const uint16_t(*X)[kN], int t, int c8) { return raw8(&X[t][sw(t, c8)]); };
    // tokens t0 + 4 g + e (e = 0..3) of channel c0 + l16 of a staged input (a column), as a raw
    // operand, by one transposing LDS read: in each group of 16 lanes, lane q reads four
    // channels of one row and lane j receives element j % 4 of lane 4 e + j / 4's read, so lane
    // (l16, g) names row t0 + 4 g + l16 / 4, channels c0 + 4 (l16 % 4) .. + 3
    auto colT = [&](const uint16_t(*X)[kN], int tb, int c0) {
        const int t = tb + 4 * g + (l16 >> 2), c = c0 + 4 * (l16 & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)&X[t][sw(t, c)]);
    };
    auto colTp = [&](const uint16_t(*X)[kPadH], int tb, int c0) {  // the same for a padded, unswizzled tile
        const int t = tb + 4 * g + (l16 >> 2), c = c0 + 4 * (l16 & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)&X[t][c]);
    };
    auto colTf = [&](const uint16_t(*X)[kN], int tb, int c0) {
        const u16x4 x = __builtin_bit_cast(u16x4, colT(X, tb, c0));
        return f4{bf(x[0]), bf(x[1]), bf(x[2]), bf(x[3])};
    };

    for (int64_t ch = ch_hi - 1; ch >= ch_lo; --ch) {
        asm volatile("" : "+v"(lane), "+v"(l16), "+v"(g));
        const int64_t t0 = ch * kLc;
        const int nv = static_cast<int>((P.T - t0) < kLc ? (P.T - t0) : kLc);
        // ---- stage r, k, v, go (swizzled rows) and S0 ------------------------------------
        const uint16_t* src[4] = {P.r, P.k, P.v, P.go};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const Rsrc rs = make_rsrc(src[a] + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 2));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = P0 + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(row) * C) * 2 + q * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.in[a][P0 + 8 * i][0], 16, voff, 0, 0, kStageLast);
            }
        }
        {  // the state before the chunk, 8 KB of [key][value] bf16: rows P0 .. P0 + 15 by this wave
            const Rsrc rs = make_rsrc(P.ckpt + (bh * nch + ch) * kN * kN, kN * kN * 2);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = P0 + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&sm.ss[P0 + 8 * i][0],
                                                         16, static_cast<uint32_t>(row * kN * 2 + q * 16), 0, 0, kStageLast);
            }
        }
        wait_staged();
        lds_sync();

        // ---- C[s][s] of this wave's tokens, from the diagonal block of GO V^T ------------
        f4 Cpp = {0.f, 0.f, 0.f, 0.f};  // lane: C[s = P0 + 4 g + e][sig = P0 + l16]
#pragma unroll
        for (int J = 0; J < 2; ++J) {
            const int j8 = 32 * J + 8 * g;
            Cpp = mfma32(raw8s(GO, P0 + l16, j8), raw8s(V, P0 + l16, j8), Cpp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)  // read back only by this wave (in order)
            if (4 * g + e == l16) sm.cd[P0 + l16] = Cpp[e];

        // Each part below first builds its small A operands (8 registers a set), then walks
        // the output's 16-column tiles two at a time (a loop unrolled by two: the second tile's
        // LDS reads overlap the first's arithmetic, 4 % faster than one at a time and 2 % faster
        // than all four, at the same register count), one accumulator a tile, storing each
        // tile; the per-channel dw / du partials of tile I rotate into slot 0 for its iteration.
        const int sig = P0 + l16;  // this lane's key token as an m index
        const int mid = P0 + 8;    // the diagonal block's reference token
        auto rot = [](float (&x)[4]) {
            const float t = x[0];
            x[0] = x[1];
            x[1] = x[2];
            x[2] = x[3];
            x[3] = t;
        };
        // ---- dv: (k . d^{n-1-sig}) G1 + sum_{s >= sig} A[s][sig] go_s -------------------------
        {
            const int nk = nv - 1 - sig;
            s4 aK[4];  // [m = sig][k = i]: k_sig,i d_i^{n-1-sig} (zero past the chunk's end)
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int c4 = 16 * I + 4 * g;
                aK[I] = nk >= 0 ? mul_pack(row4s(K, sig, c4), frow4(&sm.pw[nk >= 0 ? nk : 0][c4])) : s4{0, 0, 0, 0};
            }
            s4 aA[4];  // aA[Q], Q >= wv: [m = sig][k = s]: A[s = 16 Q + 4 g + e][sig = P0 + l16]
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aA[Q] = s4{0, 0, 0, 0};
                if (Q < wv) continue;
                f4 At = {0.f, 0.f, 0.f, 0.f};  // lane: A[s = 16 Q + 4 g + e][sig = P0 + l16]
                const int s_m = 16 * Q + l16;  // the s of this lane's A-operand row
                if (Q > wv) {
                    const int p0 = 16 * Q;
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        const int c4 = 16 * I + 4 * g;
                        const s4 ra = mul_pack(row4s(R, s_m, c4), frow4(&sm.pw[s_m - p0][c4]));
                        const s4 kb = mul_pack(row4s(K, sig, c4), frow4(&sm.pw[p0 - 1 - sig][c4]));
                        At = mfma(ra, kb, At);
                    }
                } else {
                    f4 Bn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        const int c4 = 16 * I + 4 * g;
                        const f4 rr = row4s(R, s_m, c4), kk = row4s(K, sig, c4);
                        At = mfma(mul_pack(rr, frow4(&sm.pe[mid - s_m + 8][c4])),
                                  mul_pack(kk, frow4(&sm.pe[sig + 1 - mid + 8][c4])), At);
                        Bn = mfma(mul_pack(rr, frow4(&sm.uu[c4])), pack4(kk[0], kk[1], kk[2], kk[3]), Bn);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {  // (s_local = 4 g + e, sig_local = l16): keep s > sig, bonus on s == sig
                        const int sl = 4 * g + e;
                        At[e] = sl > l16 ? At[e] : (sl == l16 ? Bn[e] : 0.f);
                    }
                }
                aA[Q] = pack4(At[0], At[1], At[2], At[3]);
            }
            const Rsrc rv = make_rsrc(P.dv + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int J = 0; J < 4; ++J) {
                f4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int I = 0; I < 4; ++I) D = mfma(aK[I], colTp(sm.gs, 16 * I, 16 * J), D);
#pragma unroll
                for (int Q = 0; Q < 4; ++Q)
                    if (Q >= wv) D = mfma(aA[Q], colT(GO, 16 * Q, 16 * J), D);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    store_wb(D[e], rv, static_cast<uint32_t>(((P0 + 4 * g + e) * C + 16 * J + l16) * 4));
            }
        }

        // ---- dk: d^{n-1-sig} X + sum_{s > sig} C[s][sig] r_s d^{s-1-sig} + u r C[sig][sig] ---
        {
            s4 aC[4];  // aC[Q], Q >= wv: [m = sig][k = s]: C[s = 16 Q + 4 g + e][sig = P0 + l16], s > sig
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aC[Q] = s4{0, 0, 0, 0};
                if (Q < wv) continue;
                f4 Cq = {0.f, 0.f, 0.f, 0.f};
                if (Q == wv) {
                    Cq = Cpp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) Cq[e] = 4 * g + e > l16 ? Cq[e] : 0.f;
                } else {
#pragma unroll
                    for (int J = 0; J < 2; ++J) {
                        const int j8 = 32 * J + 8 * g;
                        Cq = mfma32(raw8s(GO, 16 * Q + l16, j8), raw8s(V, sig, j8), Cq);
                    }
                }
                aC[Q] = pack4(Cq[0], Cq[1], Cq[2], Cq[3]);
            }
            const Rsrc rk = make_rsrc(P.dk + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int I = 0; I < 4; ++I) {  // lane: dk[sig = P0 + 4 g + e][i = 16 I + l16]
                const int i = 16 * I + l16;
                f4 X = {0.f, 0.f, 0.f, 0.f};  // X = V G1^T
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    X = mfma32(raw8s(V, sig, j8), raw8(&sm.gs[i][j8]), X);
                }
                const f4 kc = colTf(K, P0, 16 * I);
                f4 D;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sg = P0 + 4 * g + e, nk = nv - 1 - sg;
                    const float pk = nk >= 0 ? sm.pw[nk][i] : 0.f;
                    dwv[0] -= static_cast<float>(nk) * pk * kc[e] * X[e];  // (n-1-sig) d^{n-1-sig} k X
                    D[e] = X[e] * pk;
                }
#pragma unroll
                for (int Q = 0; Q < 4; ++Q) {
                    if (Q < wv) continue;
                    const int p0 = 16 * Q;
                    const f4 rc = colTf(R, p0, 16 * I);
                    float rb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = p0 + 4 * g + e;
                        rb[e] = rc[e] * (Q > wv ? sm.pw[s - p0][i] : sm.pe[mid - s + 8][i]);
                    }
                    const f4 M = mfma(aC[Q], pack4(rb[0], rb[1], rb[2], rb[3]), f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sg = P0 + 4 * g + e;
                        D[e] += M[e] * (Q > wv ? sm.pw[p0 - 1 - sg][i] : sm.pe[sg + 1 - mid + 8][i]);
                    }
                }
                const f4 rcp = colTf(R, P0, 16 * I);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sg = P0 + 4 * g + e;
                    store_wb(D[e] + sm.uu[i] * rcp[e] * sm.cd[sg], rk, static_cast<uint32_t>((sg * C + i) * 4));
                }
                rot(dwv);
            }
        }

        // ---- dr, du: d^s Y + sum_{sig < s} C[s][sig] k_sig d^{s-1-sig} + u k C[s][s] ---------
        {
            const int s_n = P0 + l16;  // this lane's s as the m / n index
            s4 aR[4];  // aR[Q], Q <= wv: [m = s][k = sig]: C[s = P0 + l16][sig = 16 Q + 4 g + e], sig < s
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aR[Q] = s4{0, 0, 0, 0};
                if (Q > wv) continue;
                f4 Cq = {0.f, 0.f, 0.f, 0.f};  // from V_Q GO_P^T
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    Cq = mfma32(raw8s(V, 16 * Q + l16, j8), raw8s(GO, s_n, j8), Cq);
                }
                if (Q == wv) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        Cq[e] = 4 * g + e < l16 ? Cq[e] : 0.f;
                        const int lag = l16 - 1 - 4 * g - e;  // C[s = P0 + l16][sig = P0 + 4 g + e]
                        if (lag >= 1) sm.cdg[wv][lag][l16] = Cq[e];
                    }
                }
                aR[Q] = pack4(Cq[0], Cq[1], Cq[2], Cq[3]);
            }
            const Rsrc rr = make_rsrc(P.dr + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int I = 0; I < 4; ++I) {  // lane: dr[s = P0 + 4 g + e][i = 16 I + l16]
                const int i = 16 * I + l16;
                f4 Y = {0.f, 0.f, 0.f, 0.f};  // Y = GO S0^T
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    Y = mfma32(raw8s(GO, s_n, j8), raw8(&sm.ss[i][sw(i, j8)]), Y);
                }
                const f4 rc = colTf(R, P0, 16 * I);
                f4 D;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = P0 + 4 * g + e;
                    const float ps = sm.pw[s][i];
                    dwv[0] -= static_cast<float>(s) * ps * rc[e] * Y[e];  // s d^s r Y
                    D[e] = Y[e] * ps;
                }
#pragma unroll
                for (int Q = 0; Q < 4; ++Q) {
                    if (Q > wv) continue;
                    const f4 kc = colTf(K, 16 * Q, 16 * I);
                    float kb[4], kw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {  // k_sig d^{p-1-sig} and (p-1-sig) times it, p = P0 or mid
                        const int sg = 16 * Q + 4 * g + e;
                        const int lg = Q < wv ? P0 - 1 - sg : mid - 1 - sg;
                        const float f = Q < wv ? sm.pw[lg][i] : sm.pe[sg + 1 - mid + 8][i];
                        kb[e] = kc[e] * f;
                        kw[e] = kb[e] * static_cast<float>(lg);
                    }
                    const f4 M1 = mfma(aR[Q], pack4(kb[0], kb[1], kb[2], kb[3]), f4{0.f, 0.f, 0.f, 0.f});
                    if (Q == wv) {  // the diagonal block's lag-weighted dw term is taken elementwise below
#pragma unroll
                        for (int e = 0; e < 4; ++e) D[e] += M1[e] * sm.pe[mid - (P0 + 4 * g + e) + 8][i];
                        continue;
                    }
                    // off the diagonal both parts of the lag, s - P0 and P0 - 1 - sig, are >= 0
                    const f4 M2 = mfma(aR[Q], pack4(kw[0], kw[1], kw[2], kw[3]), f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ls = 4 * g + e;  // s - P0
                        const float f = sm.pw[ls][i];
                        D[e] += M1[e] * f;
                        dwv[0] -= rc[e] * f * (static_cast<float>(ls) * M1[e] + M2[e]);
                    }
                }
                const f4 kcol = colTf(K, P0, 16 * I);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = P0 + 4 * g + e;
                    const float kc = kcol[e] * sm.cd[s];
                    duv[0] += rc[e] * kc;
                    store_wb(D[e] + sm.uu[i] * kc, rr, static_cast<uint32_t>((s * C + i) * 4));
                }
                rot(dwv);
                rot(duv);
            }
        }

        // ---- the lag-weighted dw term inside this wave's block, elementwise with exact weights:
        //      dw_i -= sum_{sig < s} (s-1-sig) d_i^{s-1-sig} r_s,i k_sig,i C[s][sig]
        //            = sum_L L d_i^L Z_L,   Z_L = sum_s r_s,i k_{s-1-L},i C[s][s-1-L]
        //      (lane = channel i; lag 0 has weight 0; the C entries of lag L are row L of cdg)
        {
            const int i = lane;
            float rr[16], kr[14];
#pragma unroll
            for (int a = 0; a < 16; ++a) rr[a] = rd(R, P0 + a, i);
#pragma unroll
            for (int a = 0; a < 14; ++a) kr[a] = rd(K, P0 + a, i);
            float acc = 0.f;
#pragma unroll
            for (int L = 1; L < 15; ++L) {
                const f4* crow = reinterpret_cast<const f4*>(&sm.cdg[wv][L][0]);
                float z = 0.f;
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    if (4 * c4 + 3 < L + 1) continue;  // s >= L + 1 only
                    const f4 cv = crow[c4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sl = 4 * c4 + e;
                        if (sl >= L + 1) z = fmaf(rr[sl] * kr[sl - 1 - L], cv[e], z);
                    }
                }
                acc = fmaf(static_cast<float>(L) * sm.pw[L][i], z, acc);
                __builtin_amdgcn_sched_barrier(0);  // keep each lag's loads with it (register pressure)
            }
            dwd -= acc;
        }

        // ---- the rowsum term of dw, and G0 = d^n G1 + sum_s (r_s d^s)^T go_s ------------------
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = P0 + 4 * g + e;
            const float dn = sm.pw[nv][key];
            float acc = 0.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) acc += G[J][e] * bf(sm.ss[key][sw(key, 16 * J + l16)]);
            dwk[e] -= static_cast<float>(nv) * dn * acc;
#pragma unroll
            for (int J = 0; J < 4; ++J) G[J][e] *= dn;
        }
        const int key = P0 + l16;  // the m index of (R^)^T
#pragma unroll 2
        for (int Q = 0; Q < 4; ++Q) {
            float ra[4];
            const f4 rc = colTf(R, 16 * Q, P0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * Q + 4 * g + e;
                ra[e] = s < nv ? rc[e] * sm.pw[s][key] : 0.f;
            }
            const s4 a = pack4(ra[0], ra[1], ra[2], ra[3]);
#pragma unroll
            for (int J = 0; J < 4; ++J) G[J] = mfma(a, colT(GO, 16 * Q, 16 * J), G[J]);
        }
        lds_sync();  // every wave is done with this chunk's G1 and inputs
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.gs[P0 + 4 * g + e][16 * J + l16] = static_cast<uint16_t>(pk2(G[J][e], 0.f) & 0xffffu);
    }

    if (P.ds_in != nullptr && seg == 0) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) P.ds_in[bh * kN * kN + (P0 + 4 * g + e) * kN + 16 * J + l16] = G[J][e];
    }
    // ---- dw, du of this (batch row, head), summed in a fixed order (the inputs' LDS is free) ---
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.fin.dwa[P0 + 4 * g + e][l16] = dwk[e];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        sm.fin.dv[wv][g][0][16 * I + l16] = dwv[I];
        sm.fin.dv[wv][g][1][16 * I + l16] = duv[I];
    }
    sm.fin.dd[wv][lane] = dwd;
    lds_sync();
    if (threadIdx.x < kN) {
        const int i = threadIdx.x;
        float sw_ = 0.f, su = 0.f;
        for (int ww = 0; ww < kWaves5; ++ww) {
            for (int gg = 0; gg < 4; ++gg) {
                sw_ += sm.fin.dv[ww][gg][0][i];
                su += sm.fin.dv[ww][gg][1][i];
            }
            sw_ += sm.fin.dd[ww][i];
        }
        for (int c = 0; c < 16; ++c) sw_ += sm.fin.dwa[i][c];
        const int64_t row = seg * P.B * P.H + bh;
        P.part[(row * 2 + 0) * kN + i] = sw_;
        P.part[(row * 2 + 1) * kN + i] = su;
    }
}

// ---- RWKV-6 backward -----------------------------------------------------------------------
// The RWKV-5 backward with every decay between two points of a chunk e^{-(E[a] - E[b])} (E the
// chunk-local cumulative capped rates of the RWKV-6 forward), and the rate's gradient per token,
//     dw_tau = -e^{-w_tau} rowsum(G_tau . S_{tau-1})
//            = -[ e^{-E[n]} rowsum(G1 . S0)                                             (a)
//                 + sum_{sig < tau} q_sig,   q_sig = e^{-(E[n] - E[sig+1])} k_sig . (G1 v_sig^T)   (b)
//                 + sum_{s > tau} p_s,       p_s = e^{-E[s]} r_s . (S0 go_s^T)                     (c)
//                 + sum_{sig < tau < s} X[s][sig] ],
//       X[s][sig] = e^{-(E[s] - E[sig+1])} r_s . k_sig C[s][sig]                                   (d)
// for the operator with capped rates, as the forward computes it.  (b) and (c) are prefix and
// suffix sums of per-token terms the dk and dr products already form.  (d) splits by 16-token
// blocks: whole block pairs on either side of tau's block (F), pairs with one end in tau's block
// (prefix / suffix sums of the per-block dk and dr terms) and pairs inside it (elementwise).
// Every piece is a sum of products of the inputs with positive weights: no difference of large
// sums, which at bf16 precision would swamp the small dw of fast-decaying channels.
struct Wkv6BwdShared {
    union {
        uint16_t in[4][kLc][kN];    // r, k, v, go of the chunk, [token][swizzled channel]
        float fin[kWaves5][4][kN];  // du partials [wave][k-group][channel], after the chunk walk
    };
    uint16_t gs[kN][kPadH];         // G1, bf16, [key][value]
    uint16_t ss[kN][kN];            // S0, bf16, [key][swizzled value]
    union {
        float E[kLc + 1][kN];       // cumulative capped rates, float4 slot (i / 4) ^ (t & 15) of row t
        float dwt[kLc][kN];         // the chunk's dw partials, [token][channel], after its last barrier
    };
    float uu[kN];
    float cd[kLc];                  // C[s][s] = go_s . v_s
    float cdg[kWaves5][16][16];     // each block's diagonal block of C, [s][sig], sig < s
    float xa[kN];                   // (a) per channel
    float xq[kWaves5][kN];          // block totals of q
    float xp[kWaves5][kN];          // block totals of p
    float F[kWaves5][kWaves5][kN];  // F[A][B]: sum over sig in block A, s in block B > A of X[s][sig]
};

// float4 reads and writes of the tables need 16-byte aligned rows (the block's only shared object starts at 0)
static_assert(offsetof(Wkv6BwdShared, E) % 16 == 0 && offsetof(Wkv6BwdShared, cdg) % 16 == 0 &&
                  offsetof(Wkv6BwdShared, uu) % 16 == 0 && sizeof(Wkv6BwdShared) <= 80 * 1024,
              "RWKV-6 backward LDS layout");

// Over the 16 tokens 4 g + e of a wave's block (lanes l16, l16 + 16, l16 + 32, l16 + 48 hold
// tokens 4 g .. 4 g + 3 of column l16): exclusive prefix and suffix sums of v.
__device__ __forceinline__ void scan16(const f4& v, int g, f4& pre, f4& suf) {
    const float t = v[0] + v[1] + v[2] + v[3];
    float below = 0.f, above = 0.f;
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const float up = __shfl_up(t, 16 * k, 64), dn = __shfl_down(t, 16 * k, 64);
        if (g >= k) below += up;
        if (g + k < 4) above += dn;
    }
    pre[0] = below;
    pre[1] = below + v[0];
    pre[2] = pre[1] + v[1];
    pre[3] = pre[2] + v[2];
    suf[3] = above;
    suf[2] = above + v[3];
    suf[1] = suf[2] + v[2];
    suf[0] = suf[1] + v[1];
}

// the sum of x over the four k-groups of a column (tokens of a block), in a fixed order
__device__ __forceinline__ float sum_groups(float x) {
    const float a = x + __shfl_xor(x, 16, 64);
    return a + __shfl_xor(a, 32, 64);
}

__global__ void __launch_bounds__(64 * kWaves5, 2) wkv6_bwd_kernel(Wkv6BwdArgs P) {
    __shared__ Wkv6BwdShared sm;
    // lane coordinates; made opaque at the top of every chunk (as in the RWKV-5 backward)
    int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int l16 = lane & 15, g = lane >> 4;
    const int64_t seg = blockIdx.x % P.nseg, bh = blockIdx.x / P.nseg;
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int64_t nch = (P.T + kLc - 1) / kLc;
    const int P0 = 16 * wv;
    // time split: this workgroup walks chunks ch_lo .. ch_hi - 1 of its segment from the adjoint after it
    const int64_t ch_lo = P.nseg > 1 ? seg * P.cps : 0;
    const int64_t ch_hi = P.nseg > 1 && ch_lo + P.cps < nch ? ch_lo + P.cps : nch;
    const float* g_end = P.nseg > 1 ? P.gstart + (bh * P.nseg + seg) * kN * kN
                                    : (P.ds_out != nullptr ? P.ds_out + bh * kN * kN : nullptr);

    if (threadIdx.x < kN) {
        sm.uu[threadIdx.x] = P.u[h * kN + threadIdx.x];
    }
    // G: wave wv, tile J, lane (l16, g), element e holds G[16 wv + 4 g + e][16 J + l16]
    f4 G[4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = P0 + 4 * g + e, j = 16 * J + l16;
            G[J][e] = g_end != nullptr ? g_end[key * kN + j] : 0.f;
            sm.gs[key][j] = static_cast<uint16_t>(pk2(G[J][e], 0.f) & 0xffffu);
        }
    float duv[4] = {0.f, 0.f, 0.f, 0.f};  // channel 16 I + l16

    auto rd = [](const uint16_t(*X)[kN], int t, int c) { return bf(X[t][sw(t, c)]); };
    auto row4s = [](const uint16_t(*X)[kN], int t, int c4) { return row4(&X[t][sw(t, c4)]); };
    auto raw4s = [](const uint16_t(*X)[kN], int t, int c4) { return raw4(&X[t][sw(t, c4)]); };
    auto raw8s = [](const uint16_t(*X)[kN], int t, int c8) { return raw8(&X[t][sw(t, c8)]); };
    auto colTp = [&](const uint16_t(*X)[kPadH], int tb, int c0) {  // col_tr for the padded, unswizzled G tile
        const int t = tb + 4 * g + (l16 >> 2), c = c0 + 4 * (l16 & 3);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)&X[t][c]);
    };
    auto colTf = [&](const uint16_t(*X)[kN], int tb, int c0) {
        const u16x4 x = __builtin_bit_cast(u16x4, col_tr(X, tb, c0, l16, g));
        return f4{bf(x[0]), bf(x[1]), bf(x[2]), bf(x[3])};
    };
    auto e4 = [&](int t, int c4) { return frow4(&sm.E[t][swE(t, c4)]); };  // E[t][c4 .. c4 + 3]
    auto e1 = [&](int t, int c) { return sm.E[t][swE(t, c)]; };
    auto xe = [](float x) { return ex2(-x); };  // e^{-x} for x a difference of (base-2) table entries
    auto rot = [](float (&x)[4]) {
        const float t = x[0];
        x[0] = x[1];
        x[1] = x[2];
        x[2] = x[3];
        x[3] = t;
    };
    auto rot4 = [](f4 (&x)[4]) {
        const f4 t = x[0];
        x[0] = x[1];
        x[1] = x[2];
        x[2] = x[3];
        x[3] = t;
    };

    // chunk c's r, k, v, go (swizzled rows) and its start state S0, by buffer -> LDS copies; wave wv
    // copies rows 16 wv .. 16 wv + 15 of each
    auto stage_inputs = [&](int64_t c) {
        const int64_t t0 = c * kLc;
        const int nv = static_cast<int>((P.T - t0) < kLc ? (P.T - t0) : kLc);
        const uint16_t* src[4] = {P.r, P.k, P.v, P.go};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const Rsrc rs = make_rsrc(src[a] + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 2));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = P0 + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(row) * C) * 2 + q * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.in[a][P0 + 8 * i][0], 16, voff, 0, 0, kStageLast);
            }
        }
        {
            const Rsrc rs = make_rsrc(P.ckpt + (bh * nch + c) * kN * kN, kN * kN * 2);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = P0 + 8 * i + lane / 8;
                const int q = (lane % 8) ^ (row & 7);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)&sm.ss[P0 + 8 * i][0],
                                                         16, static_cast<uint32_t>(row * kN * 2 + q * 16), 0, 0, kStageLast);
            }
        }
    };

    stage_inputs(ch_hi - 1);
    for (int64_t ch = ch_hi - 1; ch >= ch_lo; --ch) {
        asm volatile("" : "+v"(lane), "+v"(l16), "+v"(g));
        const int64_t t0 = ch * kLc;
        const int nv = static_cast<int>((P.T - t0) < kLc ? (P.T - t0) : kLc);
        lds_sync();  // the previous chunk's dw assembly has left the rate table
        // ---- the rates into E rows 1 + token (this chunk's r, k, v, go and S0 are already on the way)
        if (threadIdx.x < kN) sm.E[0][threadIdx.x] = 0.f;  // the dw partials overwrote row 0
        {
            const Rsrc rs = make_rsrc(P.w + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = P0 + 4 * i + lane / 16;  // token; LDS row t + 1
                const int q = (lane % 16) ^ ((t + 1) & 15);
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(t) * C) * 4 + q * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.E[P0 + 4 * i + 1][0], 16, voff, 0, 0, kStageLast);
            }
        }
        wait_staged();
        lds_sync();
        {  // E[t + 1] = E[t] + min(w_t, cap) in base-2 units, as in the forward
            const int c = P0 + l16, t1 = 16 * g + 1;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = fminf(sm.E[t1 + i][swE(t1 + i, c)], kWCap6) * kL2E;
#pragma unroll
            for (int i = 1; i < 16; ++i) x[i] += x[i - 1];
            float off = 0.f;
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const float v = __shfl_up(x[15], 16 * k, 64);
                if (g >= k) off += v;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.E[t1 + i][swE(t1 + i, c)] = x[i] + off;
        }
        lds_sync();  // E ready

        const uint16_t(*R)[kN] = sm.in[0];
        const uint16_t(*K)[kN] = sm.in[1];
        const uint16_t(*V)[kN] = sm.in[2];
        const uint16_t(*GO)[kN] = sm.in[3];
        const uint16_t(*SS)[kN] = sm.ss;

        // ---- C[s][s] of this wave's tokens -------------------------------------------------------
        f4 Cpp = {0.f, 0.f, 0.f, 0.f};  // lane: C[s = P0 + 4 g + e][sig = P0 + l16]
#pragma unroll
        for (int J = 0; J < 2; ++J) {
            const int j8 = 32 * J + 8 * g;
            Cpp = mfma32(raw8s(GO, P0 + l16, j8), raw8s(V, P0 + l16, j8), Cpp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)  // read back only by this wave (in order)
            if (4 * g + e == l16) sm.cd[P0 + l16] = Cpp[e];

        const int sig = P0 + l16;  // this lane's key token as an m index
        const int mid = P0 + 8;    // the diagonal block's reference token
        f4 dwp[4];                 // dw partials, [tile I]: token P0 + 4 g + e, channel 16 I + l16
#pragma unroll
        for (int I = 0; I < 4; ++I) dwp[I] = f4{0.f, 0.f, 0.f, 0.f};

        // ---- dv: (k . e^{-(E[n]-E[sig+1])}) G1 + sum_{s >= sig} A[s][sig] go_s ----------------------
        {
            const int nk = nv - 1 - sig;
            s4 aK[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int c4 = 16 * I + 4 * g;
                aK[I] = nk >= 0 ? mul_pack(row4s(K, sig, c4), exp2_neg4(e4(nv, c4) - e4(sig + 1, c4))) : s4{0, 0, 0, 0};
            }
            s4 aA[4];  // aA[Q], Q >= wv: [m = sig][k = s]: A[s = 16 Q + 4 g + e][sig]
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aA[Q] = s4{0, 0, 0, 0};
                if (Q < wv) continue;
                f4 At = {0.f, 0.f, 0.f, 0.f};
                const int s_m = 16 * Q + l16;
                if (Q > wv) {
                    const int p0 = 16 * Q;
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        const int c4 = 16 * I + 4 * g;
                        const f4 ep = e4(p0, c4);
                        const s4 ra = mul_pack(row4s(R, s_m, c4), exp2_neg4(e4(s_m, c4) - ep));
                        const s4 kb = mul_pack(row4s(K, sig, c4), exp2_neg4(ep - e4(sig + 1, c4)));
                        At = mfma(ra, kb, At);
                    }
                } else {
                    f4 Bn = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        const int c4 = 16 * I + 4 * g;
                        const f4 rr = row4s(R, s_m, c4), kk = row4s(K, sig, c4), em = e4(mid, c4);
                        At = mfma(mul_pack(rr, exp2_neg4(e4(s_m, c4) - em)), mul_pack(kk, exp2_neg4(em - e4(sig + 1, c4))), At);
                        Bn = mfma(mul_pack(rr, frow4(&sm.uu[c4])), pack4(kk[0], kk[1], kk[2], kk[3]), Bn);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int sl = 4 * g + e;
                        At[e] = sl > l16 ? At[e] : (sl == l16 ? Bn[e] : 0.f);
                    }
                }
                aA[Q] = pack4(At[0], At[1], At[2], At[3]);
            }
            const Rsrc rv = make_rsrc(P.dv + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int J = 0; J < 4; ++J) {
                f4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int I = 0; I < 4; ++I) D = mfma(aK[I], colTp(sm.gs, 16 * I, 16 * J), D);
#pragma unroll
                for (int Q = 0; Q < 4; ++Q)
                    if (Q >= wv) D = mfma(aA[Q], col_tr(GO, 16 * Q, 16 * J, l16, g), D);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    store_wb(D[e], rv, static_cast<uint32_t>(((P0 + 4 * g + e) * C + 16 * J + l16) * 4));
            }
        }

        // ---- dk, with dw's (b) terms q and its column sums toward later blocks -------------------
        {
            s4 aC[4];  // aC[Q], Q >= wv: [m = sig][k = s]: C[s = 16 Q + 4 g + e][sig], s > sig
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aC[Q] = s4{0, 0, 0, 0};
                if (Q < wv) continue;
                f4 Cq = {0.f, 0.f, 0.f, 0.f};
                if (Q == wv) {
                    Cq = Cpp;
#pragma unroll
                    for (int e = 0; e < 4; ++e) Cq[e] = 4 * g + e > l16 ? Cq[e] : 0.f;
                } else {
#pragma unroll
                    for (int J = 0; J < 2; ++J) {
                        const int j8 = 32 * J + 8 * g;
                        Cq = mfma32(raw8s(GO, 16 * Q + l16, j8), raw8s(V, sig, j8), Cq);
                    }
                }
                aC[Q] = pack4(Cq[0], Cq[1], Cq[2], Cq[3]);
            }
            const Rsrc rk = make_rsrc(P.dk + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int I = 0; I < 4; ++I) {  // lane: dk[sig = P0 + 4 g + e][i = 16 I + l16]
                const int i = 16 * I + l16;
                f4 X = {0.f, 0.f, 0.f, 0.f};  // X = V G1^T
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    X = mfma32(raw8s(V, sig, j8), raw8(&sm.gs[i][j8]), X);
                }
                const f4 kc = colTf(K, P0, 16 * I);
                const float en = e1(nv, i);
                f4 D, q, cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sg = P0 + 4 * g + e;
                    const float pk = sg < nv ? xe(en - e1(sg + 1, i)) : 0.f;
                    D[e] = X[e] * pk;
                    q[e] = kc[e] * D[e];
                }
#pragma unroll
                for (int Q = 0; Q < 4; ++Q) {
                    if (Q < wv) continue;
                    const int p0 = 16 * Q;
                    const int ref = Q > wv ? p0 : mid;  // the split point
                    const float er = e1(ref, i);
                    const f4 rc = colTf(R, p0, 16 * I);
                    float rb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) rb[e] = rc[e] * xe(e1(p0 + 4 * g + e, i) - er);
                    const f4 M = mfma(aC[Q], pack4(rb[0], rb[1], rb[2], rb[3]), f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = M[e] * xe(er - e1(P0 + 4 * g + e + 1, i));
                        D[e] += t;
                        if (Q > wv) cs[e] += kc[e] * t;  // pairs reaching a later block
                    }
                }
                const f4 rcp = colTf(R, P0, 16 * I);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sg = P0 + 4 * g + e;
                    store_wb(D[e] + sm.uu[i] * rcp[e] * sm.cd[sg], rk, static_cast<uint32_t>((sg * C + i) * 4));
                }
                f4 pre, suf;
                scan16(q + cs, g, pre, suf);
                dwp[0] += pre;
                const float tq = sum_groups(q[0] + q[1] + q[2] + q[3]);
                if (g == 0) sm.xq[wv][i] = tq;
                rot4(dwp);
            }
        }

        // ---- dr, du, with dw's (c) terms p and its row sums from earlier blocks --------------------
        {
            const int s_n = P0 + l16;
            s4 aR[4];  // aR[Q], Q <= wv: [m = s][k = sig]: C[s = P0 + l16][sig = 16 Q + 4 g + e], sig < s
#pragma unroll
            for (int Q = 0; Q < 4; ++Q) {
                aR[Q] = s4{0, 0, 0, 0};
                if (Q > wv) continue;
                f4 Cq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    Cq = mfma32(raw8s(V, 16 * Q + l16, j8), raw8s(GO, s_n, j8), Cq);
                }
                if (Q == wv) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) Cq[e] = 4 * g + e < l16 ? Cq[e] : 0.f;
                    *reinterpret_cast<f4*>(&sm.cdg[wv][l16][4 * g]) = Cq;  // [s][sig]
                }
                aR[Q] = pack4(Cq[0], Cq[1], Cq[2], Cq[3]);
            }
            const Rsrc rr = make_rsrc(P.dr + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll 2
            for (int I = 0; I < 4; ++I) {  // lane: dr[s = P0 + 4 g + e][i = 16 I + l16]
                const int i = 16 * I + l16;
                f4 Y = {0.f, 0.f, 0.f, 0.f};  // Y = GO S0^T
#pragma unroll
                for (int J = 0; J < 2; ++J) {
                    const int j8 = 32 * J + 8 * g;
                    Y = mfma32(raw8s(GO, s_n, j8), raw8(&SS[i][sw(i, j8)]), Y);
                }
                const f4 rc = colTf(R, P0, 16 * I);
                f4 D, p, rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    D[e] = Y[e] * xe(e1(P0 + 4 * g + e, i));
                    p[e] = rc[e] * D[e];
                }
#pragma unroll
                for (int Q = 0; Q < 4; ++Q) {
                    if (Q > wv) continue;
                    const int ref = Q < wv ? P0 : mid;
                    const float er = e1(ref, i);
                    const f4 kc = colTf(K, 16 * Q, 16 * I);
                    float kb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) kb[e] = kc[e] * xe(er - e1(16 * Q + 4 * g + e + 1, i));
                    const f4 M1 = mfma(aR[Q], pack4(kb[0], kb[1], kb[2], kb[3]), f4{0.f, 0.f, 0.f, 0.f});
                    float fq = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = M1[e] * xe(e1(P0 + 4 * g + e, i) - er);
                        D[e] += t;
                        if (Q < wv) {  // pairs from an earlier block
                            const float x = rc[e] * t;
                            rs[e] += x;
                            fq += x;
                        }
                    }
                    if (Q < wv) {
                        const float tf = sum_groups(fq);
                        if (g == 0) sm.F[Q][wv][i] = tf;
                    }
                }
                const f4 kcol = colTf(K, P0, 16 * I);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = P0 + 4 * g + e;
                    const float kc = kcol[e] * sm.cd[s];
                    duv[0] += rc[e] * kc;
                    store_wb(D[e] + sm.uu[i] * kc, rr, static_cast<uint32_t>((s * C + i) * 4));
                }
                f4 pre, suf;
                scan16(p + rs, g, pre, suf);
                dwp[0] += suf;
                const float tp = sum_groups(p[0] + p[1] + p[2] + p[3]);
                if (g == 0) sm.xp[wv][i] = tp;
                rot4(dwp);
                rot(duv);
            }
        }

        // ---- (a): e^{-E[n]} rowsum(G1 . S0), and G0 = e^{-E[n]} . G1 + sum_s (r_s e^{-E[s]})^T go_s ---
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = P0 + 4 * g + e;
            const float dn = xe(e1(nv, key));
            float acc = 0.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) acc += G[J][e] * bf(SS[key][sw(key, 16 * J + l16)]);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            acc += __shfl_xor(acc, 4, 64);
            acc += __shfl_xor(acc, 8, 64);
            if (l16 == 0) sm.xa[key] = dn * acc;
#pragma unroll
            for (int J = 0; J < 4; ++J) G[J][e] *= dn;
        }
        {
            const int key = P0 + l16;  // the m index of (R^)^T
#pragma unroll 2
            for (int Q = 0; Q < 4; ++Q) {
                float ra[4];
                const f4 rc = colTf(R, 16 * Q, P0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 16 * Q + 4 * g + e;
                    ra[e] = s < nv ? rc[e] * xe(e1(s, key)) : 0.f;
                }
                const s4 a = pack4(ra[0], ra[1], ra[2], ra[3]);
#pragma unroll
                for (int J = 0; J < 4; ++J) G[J] = mfma(a, col_tr(GO, 16 * Q, 16 * J, l16, g), G[J]);
            }
        }

        // ---- (d) inside this block, lane = channel: Z[tau] = sum_{sig < tau < s} X[s][sig] ----------
        float Z[16];
        {
            const int i = lane;
            const float em = e1(mid, i);
            float rf[16], kg[16];
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                rf[a] = rd(R, P0 + a, i) * xe(e1(P0 + a, i) - em);
                kg[a] = rd(K, P0 + a, i) * xe(em - e1(P0 + a + 1, i));
                Z[a] = 0.f;
            }
#pragma unroll
            for (int s = 2; s < 16; ++s) {
                const f4* crow = reinterpret_cast<const f4*>(&sm.cdg[wv][s][0]);
                float pre = 0.f;
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    if (4 * c4 + 1 > s - 1) continue;  // sig = tau - 1 <= s - 2
                    const f4 cv = crow[c4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tau = 4 * c4 + e + 1;  // pairs sig < tau, taken up to sig = tau - 1
                        if (tau <= s - 1) {
                            pre = fmaf(rf[s] * kg[tau - 1], cv[e], pre);
                            Z[tau] += pre;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // keep each row's loads with it (register pressure)
            }
        }
        lds_sync();  // every wave is done with this chunk's G1, inputs, E and block totals are written
        if (ch > ch_lo) stage_inputs(ch - 1);  // the next chunk's inputs load during the dw assembly
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.gs[P0 + 4 * g + e][16 * J + l16] = static_cast<uint16_t>(pk2(G[J][e], 0.f) & 0xffffu);

        // ---- assemble dw for this block: the partials through LDS to one lane per channel --------
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.dwt[P0 + 4 * g + e][16 * I + l16] = dwp[I][e];
        {
            const int i = lane;
            float base = sm.xa[i];
            for (int A = 0; A < wv; ++A) base += sm.xq[A][i];
            for (int B = wv + 1; B < kWaves5; ++B) base += sm.xp[B][i];
            for (int A = 0; A < wv; ++A)
                for (int B = wv + 1; B < kWaves5; ++B) base += sm.F[A][B][i];
            const Rsrc rw = make_rsrc(P.dw + ((b * P.T + t0) * C + h * kN), static_cast<uint32_t>(((nv - 1) * C + kN) * 4));
#pragma unroll
            for (int a = 0; a < 16; ++a)
                store_wb(-(sm.dwt[P0 + a][i] + Z[a] + base), rw, static_cast<uint32_t>(((P0 + a) * C + i) * 4));
        }
    }

    if (P.ds_in != nullptr && seg == 0) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int e = 0; e < 4; ++e) P.ds_in[bh * kN * kN + (P0 + 4 * g + e) * kN + 16 * J + l16] = G[J][e];
    }
    // ---- du of this (batch row, head), summed in a fixed order ------------------------------------
    lds_sync();  // every wave is done with the last chunk's dw assembly
#pragma unroll
    for (int I = 0; I < 4; ++I) sm.fin[wv][g][16 * I + l16] = duv[I];
    lds_sync();
    if (threadIdx.x < kN) {
        const int i = threadIdx.x;
        float su = 0.f;
        for (int ww = 0; ww < kWaves5; ++ww)
            for (int gg = 0; gg < 4; ++gg) su += sm.fin[ww][gg][i];
        P.part[(seg * P.B * P.H + bh) * kN + i] = su;
    }
}

// du[h, i] = sum over batch rows (in order) of the per-(batch row, head) partials
__global__ void wkv6_du_reduce_kernel(const float* part, int64_t B, int64_t H, float* du) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (q >= H * kN) return;
    float c = 0.f;
    for (int64_t b = 0; b < B; ++b) c += part[b * H * kN + q];
    du[q] = c;
}

// dw[h, i], du[h, i] = sum over batch rows (in order) of the per-(batch row, head) partials
__global__ void wkv5_reduce_kernel(const float* part, int64_t B, int64_t H, float* dw, float* du) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (q >= H * kN) return;
    const int64_t h = q / kN, i = q % kN;
    float a = 0.f, c = 0.f;
    for (int64_t b = 0; b < B; ++b) {
        a += part[((b * H + h) * 2 + 0) * kN + i];
        c += part[((b * H + h) * 2 + 1) * kN + i];
    }
    dw[q] = a;
    du[q] = c;
}

// T == 0: the state after the sequence is the state before it (or zero).
__global__ void wkv5_state_copy_kernel(const float* s_in, float* s_out, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) s_out[i] = s_in != nullptr ? s_in[i] : 0.f;
}

}  // namespace

hipError_t launch_wkv5_state_copy(const float* s_in, float* s_out, int64_t n, hipStream_t stream) {
    if (n <= 0 || s_out == nullptr || s_in == s_out) return hipSuccess;
    hipLaunchKernelGGL(wkv5_state_copy_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       s_in, s_out, n);
    return hipGetLastError();
}

hipError_t launch_wkv5_bwd(const Wkv5BwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(wkv5_bwd_kernel, dim3(static_cast<unsigned>(a.B * a.H * a.nseg)), dim3(64 * kWaves5), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = a.H * kN;
    hipLaunchKernelGGL(wkv5_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, a.part,
                       a.B * a.nseg, a.H, a.dw, a.du);  // (segment, batch row) partials
    return hipGetLastError();
}

hipError_t launch_wkv6_bwd(const Wkv6BwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(wkv6_bwd_kernel, dim3(static_cast<unsigned>(a.B * a.H * a.nseg)), dim3(64 * kWaves5), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = a.H * kN;
    hipLaunchKernelGGL(wkv6_du_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                       a.part, a.B * a.nseg, a.H, a.du);
    return hipGetLastError();
}

// ---- a few tokens (decoding): the state in, updated token by token in registers, out ------------
// For short T the chunked kernels would run their 64-token machinery for a handful of tokens; a
// decode step is bound by reading and writing the 64 x 64 float32 state of each (batch row, head).
// Per (batch row, head) and token, in order:
//     o_j = sum_i r_i S_ij + (sum_i r_i u_i k_i) v_j,    S <- diag(e^{-w_i}) S + k^T v
// in float32 (RWKV-5: w [H, 64]; RWKV-6: the token's rates [B, 1, C], a rate above kWCap6 acting as
// kWCap6 as in the chunked kernel).  One wave per (batch row, head): lane (q, g) owns columns
// 4q .. 4q + 3 of rows g, g + 4, .., g + 60, so each 16-byte load and store of the row-major state is
// coalesced over four whole rows; a column's sum meets across its four lanes by shuffles in a fixed
// order.  Needs the state, o and the saved state 16-byte aligned (else the chunked kernel runs).
struct Wkv56StepArgs {
    int64_t B, T, H;
    const float* w;  // RWKV-5: [H, 64]; RWKV-6: [B, C]
    const float* u;
    const uint16_t* r;
    const uint16_t* k;
    const uint16_t* v;
    float* o;            // [B, C] or NULL (state only)
    const float* s_in;   // [B, H, 64, 64] or NULL (zero)
    float* s_out;        // or NULL; may be s_in
    uint16_t* ckpt;      // [B, H, 64, 64] bf16 copy of the state before the token, or NULL
};

template <bool kPerToken>
__global__ void __launch_bounds__(256) wkv56_step_kernel(Wkv56StepArgs P) {
    __shared__ float tab[4][3][kN];  // per wave: r, k, decay factor of each key channel (one token)
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = static_cast<int64_t>(blockIdx.x) * 4 + wv;
    if (bh >= P.B * P.H) return;  // a whole wave; the kernel has no barrier
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int q = lane & 15, g = lane >> 4;

    // every row is loaded before anything is stored: the loads issue together although s_out, ckpt
    // and s_in may alias as far as the compiler knows (and s_out may be s_in).  The state moves
    // non-temporal both ways: a decoding model touches every other layer's state (hundreds of MB at
    // serving batch sizes) before it needs this one again (32 layers x 256 streams x 64 heads:
    // 93.9 us per call against 102.9 us with the default policy, the same bits)
    const int64_t e0 = bh * kN * kN + g * kN + 4 * q;  // element (row g, column 4q) of the state
    f4 x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        x[m] = P.s_in != nullptr ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(P.s_in + e0 + 4 * m * kN))
                                 : f4{0.f, 0.f, 0.f, 0.f};
    if (P.ckpt != nullptr) {  // the state before the (only) chunk
#pragma unroll
        for (int m = 0; m < 16; ++m)
            *reinterpret_cast<uint2*>(P.ckpt + e0 + 4 * m * kN) = uint2{pk2(x[m][0], x[m][1]), pk2(x[m][2], x[m][3])};
    }
    const float ul = P.u[h * kN + lane];
#pragma unroll 1
    for (int64_t t = 0; t < P.T; ++t) {
        const int64_t xi = (b * P.T + t) * C + h * kN;  // this token of this (batch row, head)
        const float rl = bf(P.r[xi + lane]), kl = bf(P.k[xi + lane]);
        const float wl = kPerToken ? fminf(P.w[xi + lane], kWCap6) : P.w[h * kN + lane];
        tab[wv][0][lane] = rl;
        tab[wv][1][lane] = kl;
        tab[wv][2][lane] = ex2(-wl * kL2E);
        float bonus = rl * ul * kl;  // sum over the wave's 64 key channels, fixed order
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) bonus += __shfl_xor(bonus, m, 64);
        const u16x4 vq = *reinterpret_cast<const u16x4*>(P.v + xi + 4 * q);
        const float vj[4] = {bf(vq[0]), bf(vq[1]), bf(vq[2]), bf(vq[3])};
        f4 op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = g + 4 * m;
            const float ri = tab[wv][0][i], ki = tab[wv][1][i], di = tab[wv][2][i];
            op += ri * x[m];
#pragma unroll
            for (int c = 0; c < 4; ++c) x[m][c] = fmaf(di, x[m][c], ki * vj[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            op[c] += __shfl_xor(op[c], 16, 64);
            op[c] += __shfl_xor(op[c], 32, 64);
        }
        if (P.o != nullptr && g == 0) {
            f4 oo;
#pragma unroll
            for (int c = 0; c < 4; ++c) oo[c] = fmaf(bonus, vj[c], op[c]);
            *reinterpret_cast<f4*>(P.o + xi + 4 * q) = oo;
        }
    }
    if (P.s_out != nullptr) {
#pragma unroll
        for (int m = 0; m < 16; ++m) __builtin_nontemporal_store(x[m], reinterpret_cast<f4*>(P.s_out + e0 + 4 * m * kN));
    }
}

#ifndef WKV_STEP_MAX_T
#define WKV_STEP_MAX_T 16
#endif
// whether a call may take the token-by-token kernel: few enough tokens that the state's one trip
// through HBM outweighs the per-token arithmetic, and aligned state, outputs and saved state for
// its 16-byte accesses
bool step_ok(int64_t T, const void* o, const void* s_in, const void* s_out, const void* ckpt) {
    const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return T >= 1 && T <= WKV_STEP_MAX_T && a16(o) && a16(s_in) && a16(s_out) && a16(ckpt);
}

template <bool kPerToken, class A>
hipError_t launch_step(const A& a, hipStream_t stream) {
    const Wkv56StepArgs s{a.B, a.T, a.H, a.w, a.u, a.r, a.k, a.v, a.o, a.s_in, a.s_out, a.ckpt};
    hipLaunchKernelGGL(wkv56_step_kernel<kPerToken>, dim3(static_cast<unsigned>((a.B * a.H + 3) / 4)), dim3(256), 0,
                       stream, s);
    return hipGetLastError();
}

// ---- time split of the backwards: each segment's adjoint from a zero adjoint after it ------------
// The adjoint recurrence G_{t-1} = diag(d_t) G_t + r_t^T go_t is linear in G: over a segment the
// adjoint before it is D G_after + L, D the segment's total decay per key row and L what the segment
// alone gives from G_after = 0.  This kernel forms L per (batch row, head, segment), walking the
// segment's chunks last to first with the backwards' own chunk update
//     G0 = diag(e^{-E[n]}) G1 + sum_s (r_s . e^{-E[s]})^T go_s
// (E[s] the rates of the chunk's tokens before s: RWKV-5 w s; RWKV-6 summed, each capped at kWCap6
// as the forward caps it) on bf16 matrix-core products with float32 accumulation; for RWKV-6 it
// also writes the segment's summed rates (log2 e units) for the chain.  One 4-wave workgroup per
// (batch row, head, segment); wave w owns key rows 16 w .. 16 w + 15 of L, as in the backwards.
struct AdjLocalShared {
    uint16_t in[2][2][kLc][kN];  // [buffer][r, go] of a chunk, [token][swizzled channel]
    float f[kLc + 1][kPadF];     // e^{-E[t]}, t = 0 .. 64, per channel
    float blk[kWaves5][kN];      // RWKV-6: each wave's 16-token rate sums
};

template <bool kPerToken>
__global__ void __launch_bounds__(64 * kWaves5) wkv56_adj_local_kernel(AdjLocalArgs P) {
    __shared__ AdjLocalShared sm;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int64_t seg = blockIdx.x % P.nseg, bh = blockIdx.x / P.nseg;
    const int64_t b = bh / P.H, h = bh - b * P.H;
    const int64_t C = P.H * kN;
    const int64_t nch = (P.T + kLc - 1) / kLc;
    const int64_t ch_lo = seg * P.cps;
    const int64_t ch_hi = ch_lo + P.cps < nch ? ch_lo + P.cps : nch;
    const int P0 = 16 * wv;
    auto chunk_len = [&](int64_t c) { return static_cast<int>((P.T - c * kLc) < kLc ? (P.T - c * kLc) : kLc); };
    // chunk c's r and go into buffer q by buffer -> LDS copies (wave w: rows 16 w .. 16 w + 15; rows
    // past the sequence's end read as zero through the buffer range)
    auto stage = [&](int64_t c, int q) {
        const int nvc = chunk_len(c);
        const uint16_t* src[2] = {P.r, P.go};
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const Rsrc rs = make_rsrc(src[a] + ((b * P.T + c * kLc) * C + h * kN), static_cast<uint32_t>(((nvc - 1) * C + kN) * 2));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = P0 + 8 * i + lane / 8;
                const int sq = (lane % 8) ^ (row & 7);
                const uint32_t voff = static_cast<uint32_t>((static_cast<int64_t>(row) * C) * 2 + sq * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void*)&sm.in[q][a][P0 + 8 * i][0], 16, voff, 0, 0, kStageKeep);
            }
        }
    };
    // RWKV-6: chunk c's rates of tokens P0 .. P0 + 15, channel lane, into registers (0 past its end)
    auto load_w = [&](int64_t c, float (&x)[16]) {
        const int nvc = chunk_len(c);
        const float* wr = P.w + (b * P.T + c * kLc + P0) * C + h * kN + lane;
#pragma unroll
        for (int a = 0; a < 16; ++a) x[a] = P0 + a < nvc ? wr[a * C] : 0.f;
    };

    f4 G[4];  // G[J][e] = L[P0 + 4 g + e][16 J + l16]
#pragma unroll
    for (int J = 0; J < 4; ++J) G[J] = f4{0.f, 0.f, 0.f, 0.f};
    float rsum = 0.f;  // RWKV-6, last wave: channel lane's summed capped rates over the segment
    float xw[16];      // RWKV-6: the current chunk's rates
    stage(ch_hi - 1, 0);
    if (kPerToken) {
        load_w(ch_hi - 1, xw);
    } else {  // RWKV-5: the same table for every chunk
        const float wl = P.w[h * kN + lane] * kL2E;
#pragma unroll
        for (int a = 0; a < 16; ++a) sm.f[P0 + a + 1][lane] = ex2(-wl * static_cast<float>(P0 + a + 1));
    }
    if (wv == 0) sm.f[0][lane] = 1.f;

    for (int64_t ch = ch_hi - 1; ch >= ch_lo; --ch) {
        const int nv = chunk_len(ch);
        const int q = static_cast<int>((ch_hi - 1 - ch) & 1);
        if (kPerToken) {  // E[t + 1] = E[t] + min(w_t, cap) log2 e: 16-token prefix sums, then the offsets
            float x[16];
#pragma unroll
            for (int a = 0; a < 16; ++a) x[a] = fminf(xw[a], kWCap6) * kL2E;
#pragma unroll
            for (int a = 1; a < 16; ++a) x[a] += x[a - 1];
            sm.blk[wv][lane] = x[15];
            lds_sync();  // also: every wave is done with the previous chunk's table
            float off = 0.f;
            for (int A = 0; A < wv; ++A) off += sm.blk[A][lane];
#pragma unroll
            for (int a = 0; a < 16; ++a) sm.f[P0 + a + 1][lane] = ex2(-(x[a] + off));
            if (wv == kWaves5 - 1) rsum += x[15] + off;  // the chunk's total (tokens past nv add 0)
        }
        wait_staged();
        lds_sync();  // this chunk's inputs and table are in LDS; the other buffer is free
        if (ch > ch_lo) {  // the next chunk loads while this one is computed
            stage(ch - 1, q ^ 1);
            if (kPerToken) load_w(ch - 1, xw);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float dn = sm.f[nv][P0 + 4 * g + e];
#pragma unroll
            for (int J = 0; J < 4; ++J) G[J][e] *= dn;
        }
        const int key = P0 + l16;
#pragma unroll
        for (int Q = 0; Q < 4; ++Q) {
            const u16x4 rx = __builtin_bit_cast(u16x4, col_tr(sm.in[q][0], 16 * Q, P0, l16, g));  // r[16 Q + 4 g + e][key]
            float ra[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * Q + 4 * g + e;
                ra[e] = s < nv ? bf(rx[e]) * sm.f[s][key] : 0.f;
            }
            const s4 a = pack4(ra[0], ra[1], ra[2], ra[3]);
#pragma unroll
            for (int J = 0; J < 4; ++J) G[J] = mfma(a, col_tr(sm.in[q][1], 16 * Q, 16 * J, l16, g), G[J]);
        }
    }
    float* lo = P.loc + (bh * P.nseg + seg) * kN * kN;
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int e = 0; e < 4; ++e) lo[(P0 + 4 * g + e) * kN + 16 * J + l16] = G[J][e];
    if (kPerToken && wv == kWaves5 - 1) P.rates[(bh * P.nseg + seg) * kN + lane] = rsum;
}

hipError_t launch_adj_local(const AdjLocalArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * a.nseg));
    if (a.per_token)
        hipLaunchKernelGGL(wkv56_adj_local_kernel<true>, grid, dim3(64 * kWaves5), 0, stream, a);
    else
        hipLaunchKernelGGL(wkv56_adj_local_kernel<false>, grid, dim3(64 * kWaves5), 0, stream, a);
    return hipGetLastError();
}

// ---- time split: the segments' start states ---------------------------------------------------
// With few (batch row, head) pairs the forwards split each sequence into segments: a state-only
// pass runs every segment from the zero state (its local end state L_s, and for RWKV-6 its summed
// rates), this kernel chains them in order, start_0 = S0 and start_{s+1} = D_s start_s + L_s with
// D_s the segment's total decay per key row (the recurrence is linear in the state), and the
// output pass runs every segment from its start.  The backwards' adjoint obeys the same kind of
// recurrence backwards in time, G_before = D_s G_after + L_s (L_s from wkv56_adj_local_kernel), so
// with reverse set the chain runs last segment first from s_in = the final state's gradient and
// start receives the adjoint after each segment.  One thread per state element, float32.
__global__ void wkv56_seg_chain_kernel(SegChainArgs P) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= P.BH * kN * kN) return;
    const int64_t bh = idx / (kN * kN);
    const int e = static_cast<int>(idx - bh * kN * kN), i = e / kN;  // key row i
    const int64_t h = bh % P.H;
    float S = P.s_in != nullptr ? P.s_in[idx] : 0.f;
    for (int64_t n = 0; n < P.nseg; ++n) {
        const int64_t s = P.reverse ? P.nseg - 1 - n : n;
        const int64_t q = (bh * P.nseg + s) * kN * kN + e;
        P.start[q] = S;
        float dl;  // the segment's decay exponent in log2 units
        if (P.rates6 != nullptr) {
            dl = P.rates6[(bh * P.nseg + s) * kN + i];
        } else {
            const int64_t t0 = s * P.cps * kLc;
            const int64_t t1 = P.T < t0 + P.cps * kLc ? P.T : t0 + P.cps * kLc;
            dl = P.w5[h * kN + i] * kL2E * static_cast<float>(t1 - t0);
        }
        S = fmaf(ex2(-dl), S, P.loc[q]);
    }
    if (P.s_out != nullptr) P.s_out[idx] = S;
}

hipError_t launch_seg_chain(const SegChainArgs& a, hipStream_t stream) {
    const int64_t n = a.BH * kN * kN;
    hipLaunchKernelGGL(wkv56_seg_chain_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Segments per sequence: only for at most max_bh pairs, about 512 workgroups in all (two per CU
// fit at once), and at least two chunks per segment.  Measured: at 256 pairs two segments make the
// backwards 1.4x faster but not the forwards; at 384 pairs (768 workgroups) both get slower.
int64_t wkv56_segments(int64_t BH, int64_t T, int64_t* cps, int64_t max_bh) {
    const int64_t nch = (T + kLc - 1) / kLc;
    *cps = nch;
    if (BH <= 0 || BH > max_bh || nch < 4) return 1;
    int64_t want = (512 + BH - 1) / BH;
    if (want > nch / 2) want = nch / 2;
    if (want < 2) return 1;
    const int64_t c = (nch + want - 1) / want;
    *cps = c;
    return (nch + c - 1) / c;
}

hipError_t launch_wkv6_fwd(const Wkv6Args& a, hipStream_t stream) {
    if (a.nseg == 1 && step_ok(a.T, a.o, a.s_in, a.s_out, a.ckpt)) return launch_step<true>(a, stream);
    const dim3 grid(static_cast<unsigned>(a.B * a.H * a.nseg));
    if (a.o == nullptr) {
        hipLaunchKernelGGL(wkv6_fwd_kernel<false>, grid, dim3(64 * kWaves5), 0, stream, a);
        return hipGetLastError();
    }
    if (a.ckpt == nullptr)  // no backward will read the inputs again
        hipLaunchKernelGGL((wkv6_fwd_kernel<true, true>), grid, dim3(64 * kWaves5), 0, stream, a);
    else
        hipLaunchKernelGGL((wkv6_fwd_kernel<true, false>), grid, dim3(64 * kWaves5), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_wkv5_fwd(const Wkv5Args& a, hipStream_t stream) {
    if (a.nseg == 1 && step_ok(a.T, a.o, a.s_in, a.s_out, a.ckpt)) return launch_step<false>(a, stream);
    const dim3 grid(static_cast<unsigned>(a.B * a.H * a.nseg));
    if (a.o == nullptr) {
        hipLaunchKernelGGL(wkv5_fwd_kernel<false>, grid, dim3(64 * kWaves5), 0, stream, a);
        return hipGetLastError();
    }
    if (a.ckpt == nullptr)  // no backward will read the inputs again
        hipLaunchKernelGGL((wkv5_fwd_kernel<true, true>), grid, dim3(64 * kWaves5), 0, stream, a);
    else
        hipLaunchKernelGGL((wkv5_fwd_kernel<true, false>), grid, dim3(64 * kWaves5), 0, stream, a);
    return hipGetLastError();
}

}  // namespace wkv
