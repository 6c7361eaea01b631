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

#include <stddef.h>

#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkv {

// Combine a state X (at the start of an n-token interval) with the summary S
// of that interval; D = d^n in double.  D is split into its mantissa, applied
// as a float32 hi + lo product, and its binary exponent, which joins X's
// integer scale: a decay far below float32's normal range (fast channels over
// many tokens) keeps full precision instead of passing through a denormal.
// The result keeps that scale unless the summary would not fit (lazy
// rescale).  Scales are integers, so bringing both terms to the common scale
// is exact and the only roundings are the decay product and the final sums.
__device__ __forceinline__ St combine(const St& X, const St& S, double D) {
    const double Dm = __builtin_amdgcn_frexp_mant(D);  // D = Dm 2^De, Dm in [0.5, 1) (0 for D = 0)
    const int De = __builtin_amdgcn_frexp_exp(D);
    const float Dhi = static_cast<float>(Dm);
    const float Dlo = static_cast<float>(Dm - static_cast<double>(Dhi));
    const float xa = fmaf(Dhi, X.a, Dlo * X.a);
    const float xb = fmaf(Dhi, X.b, Dlo * X.b);
    const int xs = X.s + De;
    if (!(S.b > 0.f)) return St{xa, xb, xs};
    if (!(xb > 0.f)) return S;
    int sn = xs;
    const int ls = S.s + __builtin_amdgcn_frexp_expf(S.b);  // S.b 2^S.s < 2^ls
    if ((ls > xs + static_cast<int>(kBig)) | (xb < kLo) | (xb > kHi))
        sn = max(xs + __builtin_amdgcn_frexp_expf(xb), ls);
    return St{ldx(xa, xs - sn) + ldx(S.a, S.s - sn), ldx(xb, xs - sn) + ldx(S.b, S.s - sn), sn};
}

// A carried state in float64, (a, b) at the integer scale s, for a running
// carry that passes many combines: each combine in float32 rounds the carry
// twice, and along a slowly decaying channel those roundings compound into the
// saved states (a few 1e-7 relative after a few dozen combines), which the
// backward's gradient sums of many terms then pick up.  In float64 the carry
// is rounded to float32 once, where it is used.
struct StD {
    double a, b;
    int s;
};

__device__ __forceinline__ StD to_d(const St& x) { return StD{x.a, x.b, x.s}; }
__device__ __forceinline__ St to_f(const StD& x) {
    return St{static_cast<float>(x.a), static_cast<float>(x.b), x.s};
}

// X d^n + S with X in float64 (D = d^n); the result is renormalised to
// b in [0.5, 1) so that neither sum can leave float64's range.
__device__ __forceinline__ StD combine_d(const StD& X, const St& S, double D) {
    const double xa = X.a * D, xb = X.b * D;
    if (!(S.b > 0.f)) {
        if (!(xb > 0.0)) return StD{0.0, 0.0, kSEmpty};
        const int e = __builtin_amdgcn_frexp_exp(xb);
        return StD{ldexp(xa, -e), ldexp(xb, -e), X.s + e};
    }
    if (!(xb > 0.0)) {
        const int e = __builtin_amdgcn_frexp_expf(S.b);
        return StD{ldexp(static_cast<double>(S.a), -e), ldexp(static_cast<double>(S.b), -e), S.s + e};
    }
    const int sn = max(X.s + __builtin_amdgcn_frexp_exp(xb), S.s + __builtin_amdgcn_frexp_expf(S.b));
    const double a = ldexp(xa, X.s - sn) + ldexp(static_cast<double>(S.a), S.s - sn);
    const double b = ldexp(xb, X.s - sn) + ldexp(static_cast<double>(S.b), S.s - sn);
    return StD{a, b, sn};
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

// LDS barrier that waits only on this wave's LDS operations (lgkmcnt).  A
// workgroup fence on LDS also waits for every asynchronous buffer -> LDS copy
// in flight (vmcnt), since those write LDS too; in the staged kernels each
// wave copies rows that only it reads (after its own wait), so their barriers
// need not wait for the copies, which then stay in flight across them.  The
// memory clobbers keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---- carries between workgroups --------------------------------------------------
// A chained scan along time: the workgroup of time block j waits for the
// inclusive state of block j-1 of the same tile and publishes its own.  Each
// (tile, block, lane) slot is 16 bytes (a, b, s bits, tag) written with ONE
// 16-byte store and polled with 16-byte loads, both with the system-coherent
// cache policy (sc0 sc1), which bypasses the per-XCD L2s.  So no release or
// acquire fence is needed: such fences would write back or invalidate the
// whole L2 of the XCD on every exchange, which the bandwidth-bound stream of
// outputs from the other workgroups cannot afford.  Always taking block j-1's
// state (never a look-back over several aggregates) keeps the rounding, and
// therefore the result, independent of timing.
//
// Slots are not cleared between calls: a slot is valid when its tag equals
// the call's tag (the workspace's generation + 1), so what an earlier call
// left behind, of any shape, never matches.
//
// Every RWKV-4 workspace starts with the same fixed prefix (kWsPrefix bytes),
// used for counters only, whatever the shape:
//   [0, 256)        CallHdr: the sticky error word, a count of finished
//                   streams and the generation
//   [256, 4352)     64 stream lines (StreamCtr, 64 bytes each)
//   [4352, 8448)    64 lines of dw/du fold counts (backward)
// Ticket streams: the grid's workgroups are dealt to K streams (K divides the
// tile count, at most 64; workgroup i joins stream i mod K), and stream j
// owns the tiles j, j + K, j + 2K, ...  Each stream's atomic ticket hands out
// its tiles' time blocks in time order (all of its tiles' first blocks, then
// their second, ...), so the block a workgroup waits for was handed out
// earlier on the same stream and is already running: no deadlock, whatever
// order the hardware dispatches in.  Per-stream lines keep the atomics apart:
// one ticket and one finish counter for the whole grid serialised every
// workgroup on a single address, which more than doubled the time of a long
// single sequence (8,192 workgroups).  The last workgroup of a stream returns
// its counters to zero and counts the stream as finished; the last stream
// returns that count to zero and advances the generation, in the header and
// in every stream line's copy (each workgroup reads its stream's copy).  So a
// workspace has to hold zeros before its first call only, and its counters
// never share memory with the carries or partials, whose offsets depend on
// the shape.
constexpr int kCoherent = 1 | 16;  // sc0 | sc1
constexpr int kMaxStreams = 64;
constexpr int kFoldLines = 64;
constexpr size_t kWsStreamOff = 256;
constexpr size_t kWsFoldOff = kWsStreamOff + 64 * kMaxStreams;
constexpr size_t kWsPrefix = kWsFoldOff + 64 * kFoldLines;

struct CallHdr {
    uint32_t unused0;
    uint32_t error;         // sticky: bit 0 a carry wait gave up, bit 1 a ticket out of range
    uint32_t streams_done;  // streams of this call that have finished
    uint32_t gen;           // call generation; tag = gen + 1 (never 0)
};
static_assert(sizeof(CallHdr) == sizeof(CallHdrLayout) && offsetof(CallHdr, error) == offsetof(CallHdrLayout, error),
              "one header layout");

struct StreamCtr {
    uint32_t ticket;  // next ticket of this stream
    uint32_t done;    // workgroups of this stream that have finished
    uint32_t gen;     // copy of the header's generation
    uint32_t pad[13];
};
static_assert(sizeof(StreamCtr) == 64, "one line per stream");

constexpr uint32_t kErrWait = 1u;
constexpr uint32_t kErrTicket = 2u;

__device__ __forceinline__ uint32_t hdr_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void hdr_flag(CallHdr* h, uint32_t bits) {
    __hip_atomic_fetch_or(&h->error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ CallHdr* ws_hdr(void* ws) { return static_cast<CallHdr*>(ws); }
__device__ __forceinline__ StreamCtr* ws_streams(void* ws) {
    return reinterpret_cast<StreamCtr*>(static_cast<char*>(ws) + kWsStreamOff);
}

// One thread per workgroup, first: this workgroup's ticket on stream s.
__device__ __forceinline__ uint32_t stream_ticket(StreamCtr* s) {
    return __hip_atomic_fetch_add(&s->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The call's tag, by the wave that exchanges carries (after stream_ticket; the
// load's latency then hides behind the work before the first exchange).
__device__ __forceinline__ uint32_t stream_tag(StreamCtr* s) { return hdr_load(&s->gen) + 1u; }

// The wave that exchanges the workgroup's carries, right after the last of
// them: counts the workgroup as finished on stream j and returns the count
// before it (lane 0 issues the atomic; its result is waited for only in
// stream_finish, so the latency hides behind the rest of the workgroup's work).
__device__ __forceinline__ uint32_t stream_count(StreamCtr* lines, int64_t j, int lane) {
    uint32_t d = 0;
    if (lane == 0) d = __hip_atomic_fetch_add(&lines[j].done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return d;
}

// The same wave, last: if its count was the last of stream j's `groups`
// workgroups, reset the stream's counters and count the stream; the last of the
// `nstreams` streams resets that count and advances the generation (header and
// every stream line), so that the next call's tag differs from this one's.
__device__ __forceinline__ void stream_finish(CallHdr* h, StreamCtr* lines, int64_t j, uint32_t d, uint32_t groups,
                                              uint32_t nstreams, uint32_t tag, int lane) {
    d = __builtin_amdgcn_readfirstlane(d);
    if (d + 1u != groups) return;
    uint32_t f = 0;
    if (lane == 0) {
        __hip_atomic_store(&lines[j].ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&lines[j].done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f = __hip_atomic_fetch_add(&h->streams_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    f = __builtin_amdgcn_readfirstlane(f);
    if (f + 1u != nstreams) return;
    const uint32_t g = tag == 0xffffffffu ? 0u : tag;
    if (lane < kMaxStreams) __hip_atomic_store(&lines[lane].gen, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) {
        __hip_atomic_store(&h->streams_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&h->gen, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Streams for a grid of ntiles x nblocks chained workgroups: the largest
// divisor of ntiles not above kMaxStreams.
inline int64_t chain_streams(int64_t ntiles) {
    for (int64_t k = kMaxStreams; k > 1; --k)
        if (ntiles % k == 0) return k;
    return 1;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void publish_state(Rsrc r, uint32_t off, const St& st, uint32_t tag) {
    const f32x4 v = {st.a, st.b, __int_as_float(st.s), __uint_as_float(tag)};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}

// Wait for the state published at `off` with this call's tag; after `spin`
// polls give up, flag the header's error word and return the empty state
// (results are then invalid, but every wave terminates; the caller reads the
// word through wkv_workspace_status).
__device__ __forceinline__ St wait_state(Rsrc r, uint32_t off, uint32_t tag, uint32_t spin, CallHdr* h) {
    for (uint32_t it = 0; it < spin; ++it) {
        const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
        if (__float_as_uint(v.w) == tag) return St{v.x, v.y, __float_as_int(v.z)};
        __builtin_amdgcn_s_sleep(1);
    }
    hdr_flag(h, kErrWait);
    return empty_state();
}

}  // namespace wkv
