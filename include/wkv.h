/*
 * wkv.h - C ABI of the RWKV-4 WKV time-mixing operator for AMD MI355X (gfx950),
 * with the receptance gate and the token-shift mix around it, and the
 * matrix-state WKV of RWKV-5 and RWKV-6 (per-token decay), forward and
 * backward.
 *
 * The operator, per channel c of each batch row b, tokens t = 1..T
 * ("RWKV（Receptance Weighted Key Value）概念", section 3.2; and
 *  "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", sections
 *  "一句话总结" and "关键设计 2：WKV 算子"):
 *
 *     y_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t})
 *     A_t = e^{-w} A_{t-1} + e^{k_t} v_t,    B_t = e^{-w} B_{t-1} + e^{k_t}
 *     A_0 = B_0 = 0 (empty history)
 *
 * w is the per-channel decay RATE (decay factor e^{-w}), u the per-channel
 * bonus of the current token.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP global memory) of the GPU
 *    that is current on the calling thread.  Tensors are dense, row-major,
 *    channel dimension fastest: sequences are [B, T, C], decode tensors
 *    [L, B, C], parameters [C] (or [L, C] for wkv_step).
 *  - Inputs k, v, gy have dtype WKV_F32 (float) or WKV_BF16 (bfloat16 bits,
 *    uint16).  w, u, all outputs and all states are float32.
 *  - Every call only enqueues work on `hip_stream` (a hipStream_t; NULL means
 *    the default stream) and returns without synchronising.  Errors from
 *    the kernels themselves surface at the caller's next synchronisation.
 *    No call allocates, synchronises or enqueues a memset or copy node, so
 *    the calls may be captured in a HIP graph and replayed (the scratch they
 *    clear is cleared by kernels).
 *  - The library allocates no device memory and keeps no global state
 *    (apart from the test hook wkv_debug_spin_limit): scratch memory is the
 *    caller's `workspace`, sized by wkv_workspace_bytes().  Calls on disjoint
 *    buffers are thread-safe.  Two calls that share a workspace must be
 *    ordered (same stream).
 *  - A wkv_forward / wkv_backward workspace must hold zeros before its FIRST
 *    call (hipMemset once after allocating it, or torch.zeros), and the
 *    caller must not write it between calls.  Every call leaves it ready for
 *    the next: its counters back at zero, its generation advanced (the
 *    carries between workgroups are tagged with the call's generation instead
 *    of being cleared on every call, which would take a kernel of its own).
 *    Forward and backward calls of any shape may share one buffer of the
 *    largest size they need: the counters sit at fixed offsets for every
 *    shape.  The first 16 bytes are a header; bytes 4..7 are an error word
 *    that the calls only ever set: read it with wkv_workspace_status().
 *  - Status codes: nothing aborts and no exception crosses the ABI.
 *    WKV_EINVAL    a dimension < 0, or a NULL pointer where data is needed;
 *    WKV_EDTYPE    unknown input dtype or op;
 *    WKV_ESIZE     an element or byte count overflows int64, or the lane
 *                  count (B*C, or L*B*C) reaches 2^39;
 *    WKV_EALIGN    a pointer not aligned to its element size;
 *    WKV_EWORKSPACE workspace NULL or smaller than wkv_workspace_bytes();
 *    WKV_EHIP      a HIP launch or query failed (wkv_last_hip_error() has
 *                  the HIP message of the last such failure on this thread).
 *    WKV_ETIMEOUT  returned by wkv_workspace_status() only: a wait between
 *                  workgroups gave up since the word was last cleared, so
 *                  the outputs of the call(s) since then are invalid.
 *    A call with B, T, C (or L) equal to 0 is a no-op returning WKV_OK,
 *    except that wkv_backward with C > 0 and B*T == 0 sets dw = du = 0.
 *  - Numerics: float32 arithmetic on states (a, b) with an integer log2
 *    scale s (A = a 2^s, B = b 2^s), so changes of scale are exact; k log2 e
 *    is formed with log2 e in two float32 words.  Carries between sub-chunks
 *    use float64 decay powers d^n, split into mantissa and binary exponent.
 *    With float32 inputs, and in the backward, each key weight is split once
 *    as e^k = em 2^n (n an integer) and the decay e^{-w} is applied per token
 *    as a two-term (hi + lo) product, so that no systematic rounding of the
 *    decay builds up over long sequences.  The bf16-input forward at shapes
 *    with two or more 64-channel tiles per CU (one workgroup per tile) weighs
 *    keys by one exp2 at its sub-chunk's scale, decays within a 16-token
 *    sub-chunk by a float32 product, and carries the state between sub-chunks
 *    in float64 (its saved states are rounded to float32 once).  The
 *    backward keeps its per-token reverse running sums in float32 (float64
 *    when the library is built with WKV_BWD_ACC_F64=1) and composes its span
 *    maps and the carries between workgroups in float64.  Results are
 *    finite for finite inputs with w >= 0, |u| <= 80, |v| < 2^60 and
 *    |k| < 2.9e6; outside that range the math is still defined but may
 *    overflow.  NaN/Inf inputs propagate.  For decay rates w below ~1e-5
 *    the per-token float32 rounding of the state itself changes by only a
 *    few ulps per token and no longer averages out; float32 state then
 *    limits the forward to roughly 1e-4 relative error on such channels.
 */
#ifndef WKV_MI355X_H
#define WKV_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int wkv_status_t;

enum {
    WKV_OK = 0,
    WKV_EINVAL = 1,
    WKV_EDTYPE = 2,
    WKV_ESIZE = 3,
    WKV_EALIGN = 4,
    WKV_EWORKSPACE = 5,
    WKV_EHIP = 6,
    WKV_ETIMEOUT = 7,
    WKV_ESCRATCH = 8
};

/* dtype of the INPUT sequences k, v, gy. */
enum { WKV_F32 = 0, WKV_BF16 = 1 };

/* op selector for wkv_workspace_bytes. */
enum { WKV_OP_FORWARD = 0, WKV_OP_BACKWARD = 1 };

/* Length, in tokens, of the blocks whose start states wkv_forward can save
 * for wkv_backward (see `ckpt`). */
#define WKV_CKPT_LEN 16

/* Bytes of scratch memory a call needs (0 is possible).  Returns 0 for
 * invalid arguments.  The value depends only on (op, B, T, C, in_dtype). */
size_t wkv_workspace_bytes(int op, int64_t B, int64_t T, int64_t C, int in_dtype);

/* Bytes of a forward-state checkpoint buffer for a [B, T, C] sequence:
 * 3 float32 per (b, block, c) with ceil(T / WKV_CKPT_LEN) blocks.  The
 * contents are opaque: only wkv_backward reads them. */
size_t wkv_ckpt_bytes(int64_t B, int64_t T, int64_t C);

/*
 * wkv_forward - the whole-sequence (time-parallel) forward.
 *
 * Defines: y_t above for every (b, t, c); the history starts empty.
 *   "RWKV（Receptance Weighted Key Value）概念" section 3.2 (weighted sum),
 *   equivalently the recurrence of "RWKV - 把 RNN 重新带回 Transformer 时代的
 *   线性大模型" section "关键设计 2"; section "关键设计 4" names this
 *   time-parallel mode for training.
 *
 * B, T, C   batch rows, tokens, channels (>= 0).
 * in_dtype  WKV_F32 or WKV_BF16: dtype of k and v.
 * w, u      [C] float32: decay rate and current-token bonus.
 * k, v      [B, T, C] keys and values (in_dtype).
 * y         [B, T, C] float32 output, fully overwritten; must not alias inputs.
 * ckpt      NULL, or a buffer of wkv_ckpt_bytes(B, T, C) bytes that receives
 *           the state at the start of each WKV_CKPT_LEN-token block, for a
 *           later wkv_backward on the same inputs.
 * workspace wkv_workspace_bytes(WKV_OP_FORWARD, ...) bytes (may be NULL if
 *           that is 0), 256-byte aligned, zero-filled before its first call
 *           (see the conventions above).
 */
wkv_status_t wkv_forward(int64_t B, int64_t T, int64_t C, int in_dtype,
                         const float* w, const float* u, const void* k, const void* v,
                         float* y, void* ckpt, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/*
 * wkv_forward_state - wkv_forward from a given state, also returning the state
 * after the last token.
 *
 * Defines: y_t above with A_0 = a_in e^{p_in}, B_0 = b_in e^{p_in} (the
 * history of an earlier segment) instead of the empty history, and
 * (a_out, b_out, p_out) with a_out e^{p_out} = A_T, b_out e^{p_out} = B_T.
 *   "RWKV模型深度研究报告" section 4.4.2 (encode a long input segment by
 *   segment, carrying the state), and "RWKV - 把 RNN 重新带回 Transformer 时代
 *   的线性大模型" section "关键设计 4" (the recurrent mode keeps a constant
 *   per-layer state): a prefill hands its state to wkv_step.
 *
 * a_in, b_in, p_in   [B, C] float32, all NULL (empty history) or all set; the
 *                    representation of wkv_step (any b <= 0 means empty).
 * a_out, b_out, p_out [B, C] float32, all NULL or all set; written with
 *                    the state after token T (for T == 0, the input state).
 *                    They may alias a_in, b_in, p_in (in-place update).
 * Other arguments as wkv_forward.  A ckpt written here holds states that
 * include the given history; wkv_backward then returns the gradients of the
 * T tokens' inputs with that history held fixed (dw omits the decay of the
 * history itself).
 */
wkv_status_t wkv_forward_state(int64_t B, int64_t T, int64_t C, int in_dtype,
                               const float* w, const float* u, const void* k, const void* v, float* y,
                               const float* a_in, const float* b_in, const float* p_in,
                               float* a_out, float* b_out, float* p_out,
                               void* ckpt, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * wkv_forward_state_noalloc - wkv_forward_state for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * The same kernels and results, bit for bit, as wkv_forward_state with a
 * zero-filled workspace of its own; the workspace is instead a static device
 * array inside the library, one per GPU it runs on, of WKV_STATIC_SCRATCH_BYTES
 * bytes, held until the process ends.  The call allocates nothing and makes no
 * allocating call; its first call on a device looks up that device's copy of
 * the array (a symbol lookup, no allocation).
 *
 * Arguments, layouts and ownership as wkv_forward_state, without workspace and
 * workspace_bytes.  Errors as wkv_forward_state, and WKV_ESCRATCH (nothing is
 * launched) when wkv_workspace_bytes(WKV_OP_FORWARD, B, T, C, in_dtype) exceeds
 * WKV_STATIC_SCRATCH_BYTES (B*T*C must stay below 2^29: 2 x 32768 x 4096
 * fits, 4 x 32768 x 4096 does not).
 *
 * Every call on one GPU shares that GPU's array, whose header and carries the
 * last call leaves ready for the next: calls on one GPU must not overlap in
 * time (issue them on one stream, or order the streams); overlapping calls
 * race, and their outputs are then invalid.  A wait between workgroups that
 * gives up (see wkv_debug_spin_limit) flags the array's own error word, which
 * no call reports: wkv_workspace_status needs a workspace of the caller's.
 */
#define WKV_STATIC_SCRATCH_BYTES (32u << 20)
wkv_status_t wkv_forward_state_noalloc(int64_t B, int64_t T, int64_t C, int in_dtype,
                                       const float* w, const float* u, const void* k, const void* v,
                                       float* y, const float* a_in, const float* b_in, const float* p_in,
                                       float* a_out, float* b_out, float* p_out, void* ckpt, void* hip_stream);

/*
 * wkv_backward - gradients of L = sum_{b,t,c} gy * y through the forward.
 *
 * Defines (derived by differentiating the section-3.2 weighted sum of
 * "RWKV（Receptance Weighted Key Value）概念"; the pages print no backward):
 *   dk = dL/dk, dv = dL/dv   [B, T, C] float32, fully overwritten;
 *   dw = dL/dw, du = dL/du   [C] float32, summed over b and t, overwritten
 *                            (not accumulated into).
 * The forward is recomputed on chip from k, v (no saved activations), which
 * is the fused forward+backward design named on "rwkv-cuda linear attention
 * gpu" (ainews.cool).  If `ckpt` is non-NULL it must hold what wkv_forward
 * wrote for exactly these B, T, C, in_dtype, w, u, k, v; the backward then
 * skips recomputing the block start states.  gy has dtype in_dtype.
 * dw and du are reduced in a fixed order: results are bitwise reproducible
 * from run to run on the same GPU.
 */
wkv_status_t wkv_backward(int64_t B, int64_t T, int64_t C, int in_dtype,
                          const float* w, const float* u, const void* k, const void* v,
                          const void* gy, float* dk, float* dv, float* dw, float* du,
                          const void* ckpt, void* workspace, size_t workspace_bytes,
                          void* hip_stream);

/*
 * wkv_backward_state - gradients through a segment that starts from a given
 * state and hands its state on: the backward of wkv_forward_state.
 *
 * Defines (derived; the pages print no backward): with the history A_0, B_0
 * of (a_in, b_in, p_in) and the handed-on sums A_T, B_T, the gradients of
 *     L = sum_{b,t,c} gy * y + sum_{b,c} (gA A_T + gB B_T),
 * where gA = ga_out e^{-p_out}, gB = gb_out e^{-p_out} are the gradient of L
 * with respect to (a_out, b_out) as wkv_forward_state wrote them, carried to
 * the plain sums they stand for.  Carrying the state from segment to segment is
 * "RWKV模型深度研究报告" section 4.4.2; run backwards, the gradients the later
 * segment returns for its given state are this segment's (ga_out, gb_out).
 *   dk, dv [B, T, C] and dw, du [C] as wkv_backward; dw includes the decay of
 *   the given history itself (e^{-w t} A_0 before every token t).
 *   ga_in, gb_in, gp_in [B, C]: the gradient of L with respect to a_in, b_in,
 *   p_in (A_0 = a_in e^{p_in}, B_0 = b_in e^{p_in}): e^{p_in} dL/dA_0,
 *   e^{p_in} dL/dB_0 and a_in ga_in + b_in gb_in.  An empty given state
 *   (b_in <= 0) is a constant: zeros.
 * No gradient of p_out is taken: for a loss that depends on the handed-on
 * state only through the sums it stands for it is a_out ga_out + b_out gb_out.
 *
 * a_in, b_in, p_in     the state wkv_forward_state was given, or all NULL
 *                      (the empty history).
 * ga_out, gb_out, p_out [B, C] float32, all NULL (no gradient on the handed-on
 *                      state) or all set; p_out is the p_out that
 *                      wkv_forward_state wrote.
 * ga_in, gb_in, gp_in  [B, C] float32, all NULL or all set (then a_in is
 *                      required); fully overwritten.  They must not alias
 *                      other arguments.
 * ckpt                 NULL, or what wkv_forward_state wrote for these inputs
 *                      and this given state.
 * Other arguments, workspace (wkv_workspace_bytes(WKV_OP_BACKWARD, ...)) and
 * errors as wkv_backward.  With every state argument NULL this is
 * wkv_backward.  With T == 0: dw = du = 0 and the handed-on state's gradient
 * passes back to the given state.
 */
wkv_status_t wkv_backward_state(int64_t B, int64_t T, int64_t C, int in_dtype,
                                const float* w, const float* u, const void* k, const void* v,
                                const void* gy, const float* a_in, const float* b_in, const float* p_in,
                                const float* ga_out, const float* gb_out, const float* p_out,
                                float* dk, float* dv, float* dw, float* du,
                                float* ga_in, float* gb_in, float* gp_in,
                                const void* ckpt, void* workspace, size_t workspace_bytes,
                                void* hip_stream);

/*
 * wkv_forward_gated / wkv_backward_gated - the operator with the receptance
 * gate of the time-mixing output fused in.
 *
 * Defines ("RWKV（Receptance Weighted Key Value）概念", section 3.2: the
 * time-mixing output is sigmoid(receptance) times wkv, elementwise):
 *     out_t = sigmoid(r_t) * y_t            (y_t as wkv_forward)
 * and, for L = sum gout * out, the WKV gradients for gy = gout sigmoid(r)
 * together with dr = gout * y * sigmoid(r) * (1 - sigmoid(r)).
 *
 * r, gout   [B, T, C] in_dtype (r is read by both calls).
 * out       [B, T, C] float32, fully overwritten.
 * dk, dv, dr [B, T, C] float32, fully overwritten; dw, du [C] as wkv_backward.
 * ckpt      as wkv_forward / wkv_backward; the saved states do not depend on
 *           r, so a ckpt of wkv_forward serves wkv_backward_gated and back.
 * Other arguments, sizes and errors as wkv_forward / wkv_backward (the same
 * workspace sizes).  Saves the round trip of y and gy through memory that a
 * separate gate would cost.
 */
wkv_status_t wkv_forward_gated(int64_t B, int64_t T, int64_t C, int in_dtype,
                               const float* w, const float* u, const void* k, const void* v, const void* r,
                               float* out, void* ckpt, void* workspace, size_t workspace_bytes,
                               void* hip_stream);

wkv_status_t wkv_backward_gated(int64_t B, int64_t T, int64_t C, int in_dtype,
                                const float* w, const float* u, const void* k, const void* v, const void* r,
                                const void* gout, float* dk, float* dv, float* dr, float* dw, float* du,
                                const void* ckpt, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * wkv5_forward - the multi-head, matrix-state WKV of RWKV-5, forward.
 *
 * Defines ("RWKV模型深度研究报告（截至2026年初）", sections 1.3.2 and 1.3.3:
 * version 5 carries a matrix-valued state per head whose update is a diagonal
 * decay of the previous state plus a value-key outer product; the
 * intelliparadigm.com post, section "2.1 WKV的数学表达与实现": channel groups
 * with their own decay rates; the readout with receptance and the current
 * token's bonus u follows RWKV-4, "RWKV（Receptance Weighted Key Value）概念",
 * section 3.2), for each head h of size N = 64 (C = 64 H channels, head h
 * owning channels 64h .. 64h + 63) and each batch row:
 *     S_t = diag(e^{-w_h}) S_{t-1} + k_t^T v_t         (S: 64 x 64, key x value)
 *     o_t = r_t (S_{t-1} + diag(u_h) k_t^T v_t)
 * computed chunkwise (64 tokens per chunk) with bf16 matrix-core products and
 * float32 accumulation and state.  Channels decaying faster than e^{-10} per
 * token keep terms older than one token inside a 16-token block as if their
 * rate were 10 (an error below e^{-10} of the token's own term).  Up to 16
 * tokens (decoding with the state carried from call to call, short
 * continuations) are computed token by token in float32 with the state held
 * in registers, when s_in, s_out, o and ckpt are 16-byte aligned (NULL counts
 * as aligned): the state makes one trip through memory.
 *
 * B, T, H   batch, tokens, heads (>= 0).  N  head size: must be 64.
 * in_dtype  WKV_BF16 only (WKV_EDTYPE otherwise).
 * w, u      [H, 64] float32: decay rates (decay factor e^{-w}) and bonus.
 * r, k, v   [B, T, 64 H] bf16, 16-byte aligned.
 * o         [B, T, 64 H] float32, fully overwritten.
 * s_in      [B, H, 64, 64] float32 state before token 1 (key-major), or NULL
 *           for the zero state.
 * s_out     [B, H, 64, 64] float32 state after token T, or NULL; may be s_in
 *           (updated in place).  With T == 0 it receives s_in (or zeros).
 * ckpt      NULL, or wkv5_ckpt_bytes() bytes (16-byte aligned) that receive
 *           the state before every 64-token chunk, for a later wkv5_backward
 *           on the same inputs (2 bytes per channel and token written).
 * workspace NULL (no time split), or wkv5_forward_workspace_bytes() bytes,
 *           256-byte aligned (WKV_EWORKSPACE otherwise); clobbered.
 * Errors as the other entry points (WKV_EINVAL also for N != 64).
 */
wkv_status_t wkv5_forward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype,
                          const float* w, const float* u, const void* r, const void* k, const void* v,
                          float* o, const float* s_in, float* s_out, void* ckpt, void* workspace,
                          size_t workspace_bytes, void* hip_stream);

/* Bytes of the optional scratch of wkv5_forward / wkv6_forward: nonzero only when
 * there are fewer than 256 (batch row, head) pairs and at least 4 chunks, where
 * the calls split each sequence into segments run in parallel (a state-only
 * pass per segment, the segments' start states chained in float32, then the
 * outputs of every segment from its start; r, k, v are read twice).  0 for
 * invalid arguments or when no split would be made. */
size_t wkv5_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N);
size_t wkv6_forward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N);

/*
 * wkv6_forward - the matrix-state WKV with a per-token (data-dependent) decay,
 * RWKV-6.
 *
 * Defines ("RWKV模型深度研究报告（截至2026年初）", section 1.3.2: RWKV-5 and
 * RWKV-6 share the matrix-valued state; "RWKV（Receptance Weighted Key Value）
 * 概念", section 13, and "RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型",
 * the lineage figure: the sixth generation makes the decay data dependent),
 * per head of 64 channels and batch row, with w_t a per-token rate:
 *     S_t = diag(e^{-w_t}) S_{t-1} + k_t^T v_t          (S: 64 x 64, key x value)
 *     o_t = r_t (S_{t-1} + diag(u_h) k_t^T v_t)
 * The rates come from whatever projection the model uses (the pages' low-rank
 * mix); this call takes them as an input.  Computed chunkwise like
 * wkv5_forward (bf16 matrix-core products, float32 accumulation and state),
 * from chunk-local cumulative rates in float32; up to 16 tokens as in
 * wkv5_forward (float32, when aligned).  A rate above 10 acts as 10: a term's
 * decay across such a token is then at most e^{-10} instead of less.
 *
 * B, T, H, N, in_dtype, u, r, k, v, o, s_in, s_out, ckpt, workspace  as wkv5_forward
 *           (ckpt: wkv5_ckpt_bytes() bytes, for a later wkv6_backward).
 * w         [B, T, 64 H] float32 rates, >= 0 and finite, 16-byte aligned.
 * Errors as wkv5_forward.
 */
wkv_status_t wkv6_forward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype,
                          const float* w, const float* u, const void* r, const void* k, const void* v,
                          float* o, const float* s_in, float* s_out, void* ckpt, void* workspace,
                          size_t workspace_bytes, void* hip_stream);

/* Bytes of wkv5_forward's chunk-start states for (B, T, H, N): bf16
 * [B, H, ceil(T/64), 64, 64] (key-major), rounded up to 256.  Opaque to the
 * caller: only wkv5_backward reads them.  0 for invalid arguments. */
size_t wkv5_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t N);

/* Bytes of scratch memory wkv5_backward needs: 2 x 64 float32 per (batch
 * row, head), plus wkv5_ckpt_bytes() when it is called without a ckpt and
 * recomputes the chunk-start states itself.  With at most 256 (batch row,
 * head) pairs and at least 4 chunks the backward splits each sequence into
 * segments run in parallel (the forward's time split, applied to the adjoint
 * state), which needs per segment another 2 x 64 float32 per pair plus
 * (2 x 64 x 64 + 64) float32 per pair.  flags: WKV_WS_HAVE_CKPT when a ckpt
 * will be passed; WKV_WS_NO_SPLIT for the smaller size that runs unsplit.
 * 0 for invalid arguments or B*T == 0. */
#define WKV_WS_HAVE_CKPT 1
#define WKV_WS_NO_SPLIT 2
size_t wkv5_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N, int flags);

/*
 * wkv5_backward - gradients of wkv5_forward.
 *
 * The pages give no backward; this is the derivative of the recurrence that
 * wkv5_forward defines, for the loss L = sum_t <go_t, o_t> + <ds_out, S_T>.
 * With the adjoint state G_T = ds_out (0 when NULL),
 * G_{t-1} = diag(e^{-w}) G_t + r_t^T go_t:
 *     dr_t = S_{t-1} go_t^T + u . k_t (v_t . go_t)
 *     dk_t = G_t v_t^T + u . r_t (v_t . go_t)
 *     dv_t = k_t G_t + (sum_i r_t,i u_i k_t,i) go_t
 *     du   = sum_{b,t} r_t . k_t (v_t . go_t)
 *     dw   = -e^{-w} . sum_{b,t} rowsum(G_t . S_{t-1})
 *     dS0  = G_0 (before the first token)
 * The call reads the state before every chunk from ckpt or, when ckpt is NULL,
 * first recomputes it (a forward pass without outputs, into the workspace),
 * then walks the chunks backwards with
 * the same bf16 matrix-core products and float32 accumulation as the forward;
 * dw and du are summed over the batch in a fixed order (bitwise
 * reproducible).  Inside a 16-token block, channels with w above 8 use 8 for
 * terms more than one token apart (as the forward does above 10).
 *
 * B, T, H, N, in_dtype, w, u, r, k, v, s_in  as wkv5_forward.
 * go        [B, T, 64 H] bf16, 16-byte aligned: the gradient of o.
 * ds_out    [B, H, 64, 64] float32 gradient of the final state, or NULL (zero):
 *           the ds_in of the next segment when a sequence is split.
 * dr, dk, dv [B, T, 64 H] float32, fully overwritten.
 * dw, du    [H, 64] float32, overwritten (zeros when B*T == 0).
 * ds_in     [B, H, 64, 64] float32 gradient of s_in (key-major), or NULL;
 *           with B*T == 0 it receives ds_out (or zeros).  It may be the
 *           ds_out buffer (each workgroup reads its part of ds_out before
 *           writing the same part of ds_in).
 * ckpt      the ckpt a wkv5_forward call on the same w, u, r, k, v and s_in
 *           wrote, or NULL (then s_in is read to recompute it).  The
 *           recompute splits time exactly where wkv5_forward given its
 *           workspace does (below 256 pairs), so with the full workspace its
 *           states are the bits such a forward saves and both gradients agree
 *           bit for bit; with the WKV_WS_NO_SPLIT size it matches a forward
 *           run without a workspace.
 * workspace wkv5_backward_workspace_bytes(..., flags) bytes, 256-byte
 *           aligned; clobbered.  Not needed when B*T == 0.  At least the
 *           size without WKV_WS_NO_SPLIT: the time split (when the shape
 *           asks for one); else at least the WKV_WS_NO_SPLIT size: unsplit.
 *           The two orders of summation agree to rounding, not bitwise.
 * Errors as the other entry points (WKV_EINVAL also for N != 64; nothing
 * is written on an error).
 */
wkv_status_t wkv5_backward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype,
                           const float* w, const float* u, const void* r, const void* k, const void* v,
                           const void* go, const float* s_in, const float* ds_out, float* dr, float* dk,
                           float* dv, float* dw, float* du, float* ds_in, const void* ckpt, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/* Sizes for the RWKV-6 calls: the same layouts as wkv5_ckpt_bytes() and
 * wkv5_backward_workspace_bytes() (the backward's scratch is only the du
 * partials and, without a ckpt, the recomputed chunk-start states). */
size_t wkv6_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t N);
size_t wkv6_backward_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t N, int flags);

/*
 * wkv6_backward - gradients of wkv6_forward.
 *
 * The pages give no backward; this is the derivative of the recurrence that
 * wkv6_forward defines, for L = sum_t <go_t, o_t> + <ds_out, S_T>.  With the
 * adjoint state G_T = ds_out (0 when NULL),
 * G_{t-1} = diag(e^{-w_t}) G_t + r_t^T go_t, dr, dk, dv, du and dS0 are as for
 * wkv5_backward, and each token's rate has its own gradient
 *     dw_t = -e^{-w_t} . rowsum(G_t . S_{t-1})          ([B, T, 64 H], not summed)
 * Computed chunkwise with the same bf16 matrix-core products and float32
 * accumulation as the forward; dw_t is assembled from prefix and suffix sums
 * of non-negative-weight terms inside the chunk (no difference of large sums).
 * Rates above 10 act as 10, as in the forward: such a token's dw is that of
 * the operator with the rate 10 (e^{-10} times the adjoint-state product),
 * not 0, so the cap does not cut the gradient off.
 *
 * B, T, H, N, in_dtype, w, u, r, k, v, s_in  as wkv6_forward.
 * go, ds_out, dr, dk, dv, du, ds_in, workspace  as wkv5_backward
 *           (workspace: wkv6_backward_workspace_bytes(..., flags), time split
 *           as there).
 * dw        [B, T, 64 H] float32, fully overwritten.
 * ckpt      the ckpt a wkv6_forward call on the same w, u, r, k, v and s_in
 *           wrote, or NULL (then s_in is read to recompute it).
 * du is summed over the batch in a fixed order (bitwise reproducible).
 * Errors as wkv5_backward (nothing is written on an error).
 */
wkv_status_t wkv6_backward(int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype,
                           const float* w, const float* u, const void* r, const void* k, const void* v,
                           const void* go, const float* s_in, const float* ds_out, float* dr, float* dk,
                           float* dv, float* dw, float* du, float* ds_in, const void* ckpt, void* workspace,
                           size_t workspace_bytes, void* hip_stream);

/*
 * wkv_token_shift / wkv_token_shift_backward - the token-shift mix that
 * produces the inputs of the time-mixing projections.
 *
 * Defines ("RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section
 * "关键设计 1：Token Shift - 给并行投影注入前一时刻", where r, k and v each
 * project their own mix; "RWKV（Receptance Weighted Key Value）概念", section
 * 3.3, the same mix before channel mixing), for M mixing vectors mu_j:
 *     out_j[b, t, c] = mu_j[c] x[b, t, c] + (1 - mu_j[c]) x[b, t-1, c]
 * where x[b, -1, c] is x_prev[b, c] (the previous input that the state tuple
 * of section "整体架构" carries from an earlier segment or decode step), or 0
 * when x_prev is NULL.  Only the elementwise mix: the projections are
 * ordinary matrix products outside this library.  Evaluated in float32 as
 * xs + mu (x - xs) with one fused multiply-add.
 *
 * B, T, C   batch, tokens, channels (>= 0).  M  number of mixes, 1..4 (3 for
 *           the time-mixing r, k, v; 2 for channel mixing); else WKV_EINVAL.
 * in_dtype  dtype of x, x_prev, out and gout.
 * mu        [M, C] float32 mixing vectors.
 * x         [B, T, C] input.  x_prev  [B, C] or NULL.  The x_prev of the next
 *           segment is x[:, T-1, :] of this one (a view; nothing is stored).
 * out       [M, B, T, C] in_dtype, fully overwritten (bf16: float32 result
 *           rounded to nearest even).  Must not overlap x or x_prev.
 *
 * Backward, for L = sum_j <gout_j, out_j>:
 *     dx[b, t]    = sum_j mu_j gout_j[b, t] + (1 - mu_j) gout_j[b, t+1]
 *                   (no t+1 term at t = T-1)
 *     dmu[j]      = sum_{b,t} gout_j[b, t] (x[b, t] - x[b, t-1])
 *     dx_prev[b]  = sum_j (1 - mu_j) gout_j[b, 0]
 * gout      [M, B, T, C] in_dtype.
 * dx        [B, T, C] float32, fully overwritten; must not overlap an input.
 * dmu       [M, C] float32, overwritten (summed over b and t, in a fixed
 *           order: bitwise reproducible).  Set to 0 when B*T == 0.
 * dx_prev   [B, C] float32 or NULL; overwritten when given (0 when T == 0).
 * workspace at least wkv_token_shift_workspace_bytes(B, T, C, M) bytes,
 *           256-byte aligned (partial sums of dmu).
 * Errors as the other entry points.  Full speed needs C a multiple of 8
 * (bf16) or 4 (float32) and 16-byte aligned tensors; other shapes take a
 * one-element-per-thread path with the same results.
 */
size_t wkv_token_shift_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t M);

wkv_status_t wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, int in_dtype,
                             const float* mu, const void* x, const void* x_prev, void* out,
                             void* hip_stream);

wkv_status_t wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M, int in_dtype,
                                      const float* mu, const void* x, const void* x_prev,
                                      const void* gout, float* dx, float* dmu, float* dx_prev,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * wkv_step - one recurrent-mode (decode) token for L x B independent states.
 *
 * Defines ("RWKV - 把 RNN 重新带回 Transformer 时代的线性大模型", section
 * "关键设计 4：双执行模式"; state tuple in section "整体架构"): with the
 * state carried as (a, b, p), A = a e^p and B = b e^p,
 *     y  = (A + e^{u+k} v) / (B + e^{u+k})        (from the previous state)
 *     A' = e^{-w} A + e^{k} v,  B' = e^{-w} B + e^{k}
 * The exponent p is the stability exponent of that section: it is moved to
 * the running max max(k, p + ln b) whenever a new key exceeds it by more than
 * e^22 or b leaves [2^-32, 2^32], so that no exponential overflows; between
 * such moves the decay is applied to (a, b).  Callers must therefore compare
 * states through a/b and ln(b) + p, never the raw triples.
 *
 * L, B, C   layers, streams, channels (>= 0).  One call advances all L*B
 *           states by one token.
 * in_dtype  dtype of k and v.
 * w, u      [L, C] float32 per-layer parameters.
 * k, v      [L, B, C] current-token inputs.
 * y         [L, B, C] float32 output.
 * a, b, p   [L, B, C] float32 state, read and overwritten in place.  The
 *           empty state is a = b = 0, p = -1e38 (any p <= -1e30).  Any
 *           (a e^s, b e^s, p - s) represents the same state.
 */
wkv_status_t wkv_step(int64_t L, int64_t B, int64_t C, int in_dtype,
                      const float* w, const float* u, const void* k, const void* v,
                      float* y, float* a, float* b, float* p, void* hip_stream);

/*
 * wkv_workspace_status - the error word of a wkv_forward / wkv_backward
 * (or the gated calls') workspace.
 *
 * Where a call splits a sequence over workgroups chained in time (few 64-channel
 * tiles: B*C small next to the GPU, or float32 inputs), each workgroup waits for
 * its predecessor's carry.  A wait is bounded: after wkv_debug_spin_limit()
 * polls (default 2^22, about a second) it gives up so that every kernel ends,
 * and sets the error word in the workspace header.  A workspace that was not
 * zero-filled before its first call sets it too.  The word is sticky.
 *
 * Synchronises hip_stream, then reads the word (a 4-byte device-to-host copy;
 * not for use inside HIP graph capture).  Returns WKV_OK if it is clear,
 * WKV_ETIMEOUT if it is set (the outputs written since it was last cleared
 * are invalid), and clears it when `clear` is nonzero.  WKV_EINVAL for a NULL
 * workspace, WKV_EWORKSPACE for fewer than 8 bytes or a workspace not
 * 256-byte aligned, WKV_EHIP if the copy fails.
 */
wkv_status_t wkv_workspace_status(const void* workspace, size_t workspace_bytes, int clear, void* hip_stream);

/*
 * wkv_debug_spin_limit - test hook: sets the number of polls after which a
 * wait between workgroups gives up (process-wide; applies to calls launched
 * afterwards) and returns the previous value.  0 makes every such wait give up
 * at once, so a test can check that the error word is set and reported while
 * every kernel still runs to its end.  Not for production use.
 */
uint32_t wkv_debug_spin_limit(uint32_t polls);

/* Static description of a status code. */
const char* wkv_status_str(wkv_status_t s);

/* HIP error string of the last WKV_EHIP on this thread ("" if none). */
const char* wkv_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* wkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV_MI355X_H */
