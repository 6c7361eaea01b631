// Host-side launch interface between the C ABI (wkv_api.hip) and the kernel
// translation units.  Internal to the library; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wkv {

constexpr int64_t kCkptLen = 16;  // = WKV_CKPT_LEN in include/wkv.h

// Polls a wait for a carry between workgroups makes before it gives up and
// flags the workspace's error word (wkv_debug_spin_limit sets it; default 2^22).
uint32_t spin_limit();

// Header at the start of a wkv_forward / wkv_backward workspace (the device
// code's CallHdr in wkv_scan.h has this layout).
struct CallHdrLayout {
    uint32_t unused0, error, streams_done, gen;
};

struct FwdArgs {
    int64_t B, T, C;
    bool bf16;
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    float* y;
    void* ckpt;     // nullable
    int64_t nblk;   // ceil(T / kCkptLen)
    void* ws;
    size_t ws_bytes;
    // optional receptance [B, T, C] (in dtype): y becomes sigmoid(r) y
    const void* r = nullptr;
    // optional state before token 1 and after token T, each [B, C] (a, b, p as
    // wkv_step): all three pointers NULL or all set
    const float* a_in = nullptr;
    const float* b_in = nullptr;
    const float* p_in = nullptr;
    float* a_out = nullptr;
    float* b_out = nullptr;
    float* p_out = nullptr;
};

struct BwdArgs {
    int64_t B, T, C;
    bool bf16;
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    const void* gy;
    float* dk;
    float* dv;
    float* dw;
    float* du;
    const void* ckpt;  // nullable
    int64_t nblk;
    void* ws;
    size_t ws_bytes;
    // optional receptance [B, T, C] (in dtype): gy is then the gradient of
    // sigmoid(r) y, and dr [B, T, C] float32 receives the gradient of r
    const void* r = nullptr;
    float* dr = nullptr;
    // optional, through carried state ([B, C] each; each triple all NULL or all set): the state before
    // token 1 (as FwdArgs), the gradient (ga, gb) of the state after token T at the p the forward
    // wrote, and the gradients (ga, gb, gp) of the state before token 1 (needs a_in)
    const float* a_in = nullptr;
    const float* b_in = nullptr;
    const float* p_in = nullptr;
    const float* ga_out = nullptr;
    const float* gb_out = nullptr;
    const float* p_out = nullptr;
    float* ga_in = nullptr;
    float* gb_in = nullptr;
    float* gp_in = nullptr;
};

struct StepArgs {
    int64_t L, B, C;
    bool bf16;
    bool vec4;
    const float* w;
    const float* u;
    const void* k;
    const void* v;
    float* y;
    float* a;
    float* b;
    float* p;
};

struct ShiftArgs {
    int64_t B, T, C, M;
    bool bf16;
    bool vec;              // 16-byte vectors: C a multiple of 16 / element size, pointers 16-byte aligned
    const float* mu;       // [M, C]
    const void* x;         // [B, T, C]
    const void* x_prev;    // [B, C] or NULL (zeros)
    void* out;             // forward: [M, B, T, C], dtype of x
    const void* g;         // backward: [M, B, T, C], dtype of x
    float* dx;             // backward: [B, T, C]
    float* dmu;            // backward: [M, C]
    float* dx_prev;        // backward: [B, C] or NULL
    float* ws;             // backward: shift_partial_rows(B, T) * M * C floats
};

struct Wkv5Args {
    int64_t B, T, H;     // head size 64; C = 64 H
    const float* w;      // [H, 64] decay rates
    const float* u;      // [H, 64] bonus
    const uint16_t* r;   // [B, T, C] bf16, 16-byte aligned
    const uint16_t* k;
    const uint16_t* v;
    float* o;            // [B, T, C]
    const float* s_in;   // [B, H, 64, 64] or NULL (zero state)
    float* s_out;        // [B, H, 64, 64] or NULL
    uint16_t* ckpt = nullptr;  // [B, H, nchunks, 64, 64] bf16 [key][value]: the state before each chunk, or NULL
    // time split: nseg > 1 runs segment s of (batch row, head) bh as workgroup bh * nseg + s over
    // chunks [s cps, (s + 1) cps), with s_in / s_out then [B * H, nseg, 64, 64] (the segments' own
    // start and end states); the saved states keep their global chunk index
    int64_t nseg = 1, cps = 0;
    float* seg_rates = nullptr;  // RWKV-6 only: [B * H, nseg, 64] each segment's summed capped rates (log2 e units)
};

// The segments' start states from their local end states (time split), and the final state.
struct SegChainArgs {
    int64_t BH, H, T, nseg, cps;
    const float* w5;         // RWKV-5: [H, 64] rates, or NULL
    const float* rates6;     // RWKV-6: [BH, nseg, 64] summed capped rates (log2 e units), or NULL
    const float* s_in;       // [BH, 64, 64] or NULL (zero)
    const float* loc;        // [BH, nseg, 64, 64] each segment's end state from the zero state
    float* start;            // [BH, nseg, 64, 64] each segment's start state
    float* s_out;            // [BH, 64, 64] or NULL
    int reverse = 0;         // 1: the backwards' adjoint chain, last segment first (start = the adjoint after it)
};

hipError_t launch_seg_chain(const SegChainArgs& a, hipStream_t stream);

// time split of the matrix-state backwards: every segment's adjoint before it from a zero adjoint
// after it (and, per token rates, the segment's summed capped rates in log2 e units)
struct AdjLocalArgs {
    int64_t B, T, H, nseg, cps;
    const float* w;          // RWKV-5: [H, 64]; RWKV-6: [B, T, C] per-token rates
    bool per_token;          // RWKV-6
    const uint16_t* r;
    const uint16_t* go;
    float* loc;              // [BH, nseg, 64, 64]
    float* rates;            // [BH, nseg, 64] (per_token only)
};

hipError_t launch_adj_local(const AdjLocalArgs& a, hipStream_t stream);
// segments for a time split of B * H (batch row, head) pairs over T tokens (1: no split); the
// forwards split below 256 pairs, the backwards up to 256
int64_t wkv56_segments(int64_t BH, int64_t T, int64_t* cps, int64_t max_bh = 255);

struct Wkv5BwdArgs {
    int64_t B, T, H;
    const float* w;
    const float* u;
    const uint16_t* r;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* go;     // [B, T, C] bf16 gradient of o
    const uint16_t* ckpt;   // as Wkv5Args::ckpt
    const float* ds_out;    // [B, H, 64, 64] gradient of the final state, or NULL (zero)
    float* dr;              // [B, T, C]
    float* dk;
    float* dv;
    float* part;            // [nseg, B, H, 2, 64]: dw, du of each (segment, batch row, head)
    float* dw;              // [H, 64], summed over batch rows
    float* du;
    float* ds_in;           // [B, H, 64, 64] gradient of the initial state, or NULL
    int64_t nseg = 1, cps = 0;      // time split: segments per sequence, chunks per segment
    const float* gstart = nullptr;  // nseg > 1: [B H, nseg, 64, 64] the adjoint after each segment
};

// chunked forward (wkv_fwd.hip)
hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t stream);
// T == 0 with a state: the output state is the input state (or the empty one)
hipError_t launch_state_passthrough(const FwdArgs& a, hipStream_t stream);
size_t fwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t C);

// chunked backward (wkv_bwd.hip)
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t stream);
size_t bwd_chunk_workspace_bytes(int64_t B, int64_t T, int64_t C);

// token-shift mix (wkv_shift.hip)
hipError_t launch_shift_fwd(const ShiftArgs& a, hipStream_t stream);
hipError_t launch_shift_bwd(const ShiftArgs& a, hipStream_t stream);
hipError_t launch_shift_zero(float* p, int64_t n, hipStream_t stream);
int64_t shift_partial_rows(int64_t B, int64_t T);
int shift_vector_width(bool bf16, bool bwd);

// RWKV-5 matrix-state forward (wkv5.hip)
hipError_t launch_wkv5_fwd(const Wkv5Args& a, hipStream_t stream);

struct Wkv6Args {
    int64_t B, T, H;     // head size 64; C = 64 H
    const float* w;      // [B, T, C] per-token decay rates (>= 0)
    const float* u;      // [H, 64] bonus
    const uint16_t* r;   // [B, T, C] bf16, 16-byte aligned
    const uint16_t* k;
    const uint16_t* v;
    float* o;            // [B, T, C]
    const float* s_in;   // [B, H, 64, 64] or NULL (zero state)
    float* s_out;        // [B, H, 64, 64] or NULL
    uint16_t* ckpt = nullptr;  // as Wkv5Args::ckpt
    int64_t nseg = 1, cps = 0;   // as Wkv5Args
    float* seg_rates = nullptr;
};

hipError_t launch_wkv6_fwd(const Wkv6Args& a, hipStream_t stream);

struct Wkv6BwdArgs {
    int64_t B, T, H;
    const float* w;         // [B, T, C] per-token rates
    const float* u;
    const uint16_t* r;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* go;     // [B, T, C] bf16 gradient of o
    const uint16_t* ckpt;   // as Wkv6Args::ckpt
    const float* ds_out;    // [B, H, 64, 64] gradient of the final state, or NULL (zero)
    float* dr;              // [B, T, C]
    float* dk;
    float* dv;
    float* dw;              // [B, T, C], per token
    float* part;            // [nseg, B, H, 64]: du of each (segment, batch row, head)
    float* du;              // [H, 64]
    float* ds_in;           // [B, H, 64, 64] or NULL
    int64_t nseg = 1, cps = 0;      // as Wkv5BwdArgs
    const float* gstart = nullptr;
};

hipError_t launch_wkv6_bwd(const Wkv6BwdArgs& a, hipStream_t stream);
hipError_t launch_wkv5_state_copy(const float* s_in, float* s_out, int64_t n, hipStream_t stream);
hipError_t launch_wkv5_bwd(const Wkv5BwdArgs& a, hipStream_t stream);

// decode step (wkv_step.hip)
hipError_t launch_step(const StepArgs& s, hipStream_t stream);

}  // namespace wkv
