/*
 * gdn2.h - C ABI of libgdn2, the MI355X (gfx950) Gated DeltaNet-2 token mixer.
 *
 * The operation (snilld.dk, "Gated DeltaNet-2 fra NVIDIA ...", section "Hvad
 * Gated DeltaNet-2 ændrer", compact update equation), per sequence and head:
 *
 *     S_t = (I - k_t (b_t * k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t
 *
 * with state S in R^{dk x dv} (rows are key channels), channel-wise decay
 * alpha_t = exp(log_alpha_t) in (0, 1]^{dk} applied before the edit, erase
 * gate b_t in [0, 1]^{dk} and write gate w_t in [0, 1]^{dv} (both already
 * passed through their sigmoid), and readout after the update (aifetchly-
 * blog.pages.dev, "Gated DeltaNet-2 Guide", layer workflow step 4). No query
 * scale is applied. A missing initial state means zeros, and the final state
 * is returned, as in that guide's "End-to-End PyTorch Implementation".
 *
 * Conventions for every entry point:
 *  - All pointers are DEVICE pointers except where stated. The caller owns
 *    every buffer; the library allocates no device memory and keeps no pointer
 *    after a call returns.
 *  - Layouts are dense row-major. Token tensors are [tokens, H, d], where
 *    tokens = B*T (equal-length rows back to back) or the packed total.
 *  - Work is enqueued on the calling thread's stream (gdn2_set_stream) and the
 *    call returns without synchronising. Device-side faults surface at the
 *    caller's next synchronisation, like any other stream work.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    non-OK status nothing has been launched. GDN2_ERR_HIP reports a launch
 *    error from the HIP runtime.
 *  - Preconditions that are not checked on the host: contiguity; finite
 *    log_alpha <= 0; cu_seqlens starting at 0, non-decreasing and ending at T.
 *  - Device pointers must be 16-byte aligned.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN2_OK = 0,
    GDN2_ERR_INVALID = 1,     /* null/misaligned pointer, bad size or dims    */
    GDN2_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dims, dtype) */
    GDN2_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
    GDN2_ERR_HIP = 4          /* the HIP runtime reported an error            */
} gdn2_status;

/* Values of the in_dtype / out_dtype arguments. Those arguments are plain
 * ints, so that any value a caller passes is well defined on the library's
 * side; a value that is not one of these gives GDN2_ERR_INVALID. */
typedef enum {
    GDN2_F32 = 0,
    GDN2_BF16 = 1
} gdn2_dtype;

/*
 * Gate layouts for the *_gates entry points. A set bit means that gate holds
 * one value per token and head ([tokens, H], or [N, H] for a decode step)
 * instead of one per channel; the value applies to every channel. Kimi Delta
 * Attention is the erase and write gates collapsed to one scalar beta per
 * token-head (pass GDN2_GATE_B_PER_HEAD | GDN2_GATE_W_PER_HEAD with b == w),
 * and Gated DeltaNet additionally has a scalar decay (also set
 * GDN2_GATE_ALPHA_PER_HEAD): the special cases that Gated DeltaNet-2 reduces
 * to (snilld.dk, section "Hvad Gated DeltaNet-2 ændrer").
 */
typedef enum {
    GDN2_GATES_PER_CHANNEL = 0,
    GDN2_GATE_B_PER_HEAD = 1,
    GDN2_GATE_W_PER_HEAD = 2,
    GDN2_GATE_ALPHA_PER_HEAD = 4
} gdn2_gate_layout;

/* Set the HIP stream (a hipStream_t) used by this thread's later calls.
 * NULL selects the default stream. Always returns GDN2_OK. */
int gdn2_set_stream(void *hip_stream);

/* The stream set by this thread (NULL = default stream). */
void *gdn2_get_stream(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char *gdn2_status_string(int status);

/*
 * Bytes of device workspace that gdn2_chunk_fwd needs for these sizes, or 0
 * if the arguments are invalid or unsupported. `varlen` is 1 when the call
 * will pass cu_seqlens (then B must be 1 and T is the total token count).
 */
size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv,
                                      int in_dtype, int varlen);

/*
 * Prefill forward over a batch, chunkwise (64-token chunks, WY form: the
 * chunk's rank-one erase factors with the cumulative decay folded in are
 * applied as one block per chunk, snilld.dk, section "Hvad betyder det for
 * træning og inferens").
 *
 *   q, k, b    [tokens, H, dk]  in_dtype (GDN2_BF16 or GDN2_F32)
 *   v, w       [tokens, H, dv]  in_dtype
 *   log_alpha  [tokens, H, dk]  float, finite, <= 0
 *   S0         [N, H, dk, dv]   float, or NULL for zeros
 *   o          [tokens, H, dv]  out_dtype (GDN2_F32 only)
 *   ST         [N, H, dk, dv]   float, or NULL; may alias S0
 *   cu_seqlens [N + 1]          int32 device array, or NULL
 *
 * Without cu_seqlens the batch is B sequences of T tokens each and N must
 * equal B. With cu_seqlens, B must be 1, T is the total token count and
 * sequence i is tokens [cu_seqlens[i], cu_seqlens[i+1]); sequences may be
 * empty (then ST[i] = S0[i]). Outputs must not alias the token inputs.
 * Supported head dims: dk in {32, 64, 128} for bf16 inputs and
 * {16, 32, 64, 128} for f32 inputs; dv in {16, 32, 64, 128}.
 * workspace: device memory of at least gdn2_chunk_fwd_workspace_bytes(...).
 *
 * Value range (bf16 inputs, whose products run on f16 matrix cores): q_t
 * and k_t must have at most unit L2 norm per token and head, as the layer's
 * L2 normalisation gives them (bf16 rounding aside; "Gated DeltaNet-2 Guide",
 * section "2. Normalization and Short Convolutions"). v, w, S0 and the state
 * have no bound: every value column of the state, of w * v and of the
 * corrected writes is carried through the f16 products with its own power of
 * two scale, chosen each chunk, so large states stay finite and small ones
 * keep full precision. fp32 inputs run on fp32 matrix cores.
 */
int gdn2_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const void *b, const void *w, const float *S0, void *o, float *ST,
                   const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                   int in_dtype, int out_dtype, void *workspace,
                   size_t workspace_bytes);

/*
 * gdn2_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, which instead lives in a fixed
 * device array of GDN2_NOALLOC_WORKSPACE_MAX bytes inside the library, one
 * per device, held until the process ends. Nothing is allocated or freed
 * during the call. Sizes whose workspace (gdn2_chunk_fwd_workspace_bytes)
 * exceeds GDN2_NOALLOC_WORKSPACE_MAX give GDN2_ERR_WORKSPACE, with nothing
 * launched; e.g. 4 x 4096 tokens x 16 heads at d = 128 fit (254 MB). Every
 * call on one device shares that device's array: calls that can overlap on
 * one device (other streams, other host threads) race and must be
 * serialised by the caller. Results are those of gdn2_chunk_fwd.
 */
#define GDN2_NOALLOC_WORKSPACE_MAX (256u << 20)
int gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                           const void *b, const void *w, const float *S0, void *o, float *ST,
                           const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                           int in_dtype, int out_dtype);

/*
 * gdn2_chunk_fwd with the gate layouts given by `gates` (gdn2_gate_layout
 * bits): b is [tokens, H] when GDN2_GATE_B_PER_HEAD is set, w is [tokens, H]
 * with GDN2_GATE_W_PER_HEAD and log_alpha is [tokens, H] with
 * GDN2_GATE_ALPHA_PER_HEAD; the other arguments, the workspace size and the
 * errors are those of gdn2_chunk_fwd. Unknown bits give GDN2_ERR_INVALID.
 * gdn2_chunk_fwd is this call with gates = GDN2_GATES_PER_CHANNEL.
 */
int gdn2_chunk_fwd_gates(const void *q, const void *k, const void *v, const float *log_alpha,
                         const void *b, const void *w, int gates, const float *S0, void *o, float *ST,
                         const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                         int in_dtype, int out_dtype, void *workspace,
                         size_t workspace_bytes);

/*
 * Chunk-size variants of the prefill forward: gdn2_chunk_fwd with chunks of
 * `chunk` tokens, 32, 64 or 128 (snilld.dk, section "POC-matrix der dækker
 * de hårde hjørner": latency, throughput and peak memory at C = 32 and 128
 * besides the C = 64 of the implementation). The result is the same
 * recurrence; a longer chunk halves the serial chain over chunks and
 * doubles the triangular work per token. chunk = 64 is gdn2_chunk_fwd.
 *
 * Arguments, layouts, ownership and errors as gdn2_chunk_fwd (per-channel
 * gates), with the workspace size from gdn2_chunk_fwd_sized_workspace_bytes
 * for the same chunk. A chunk other than 32, 64 or 128 gives
 * GDN2_ERR_INVALID; f32 inputs with dk = 128 and chunk = 128 give
 * GDN2_ERR_UNSUPPORTED (the preparation kernel's tiles would not fit one
 * compute unit's 160 KB of LDS).
 */
size_t gdn2_chunk_fwd_sized_workspace_bytes(int B, int T, int N, int H, int dk, int dv,
                                            int in_dtype, int varlen, int chunk);
int gdn2_chunk_fwd_sized(const void *q, const void *k, const void *v, const float *log_alpha,
                         const void *b, const void *w, const float *S0, void *o, float *ST,
                         const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                         int in_dtype, int out_dtype, int chunk, void *workspace,
                         size_t workspace_bytes);

/*
 * One recurrent decode step for N independent sequences (the same update
 * and readout for a single token; constant-size state, aifetchly, "Gated
 * DeltaNet-2 Guide", section "3. Chunkwise Parallel Algorithm ...": O(1)
 * memory during token generation).
 *
 *   q, k, b    [N, H, dk]       in_dtype
 *   v, w       [N, H, dv]       in_dtype
 *   log_alpha  [N, H, dk]       float, finite, <= 0
 *   S          [N, H, dk, dv]   float, read and updated in place
 *   o          [N, H, dv]       out_dtype (GDN2_F32 only)
 *
 * dk, dv in {16, 32, 64, 128}. S is read once and written once. Successive
 * calls from one thread on the same S visit the (sequence, head) chains in
 * alternating order (the chains written last, still in the last-level cache,
 * are read first); the results do not depend on the order.
 */
int gdn2_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                     const void *b, const void *w, float *S, void *o, int N, int H, int dk,
                     int dv, int in_dtype, int out_dtype);

/*
 * gdn2_decode_step with the gate layouts given by `gates`: b, w and
 * log_alpha are [N, H] where their bit is set. Unknown bits give
 * GDN2_ERR_INVALID.
 */
int gdn2_decode_step_gates(const void *q, const void *k, const void *v, const float *log_alpha,
                           const void *b, const void *w, int gates, float *S, void *o, int N, int H, int dk,
                           int dv, int in_dtype, int out_dtype);

/*
 * Fused input prologue. The layer computes the mixer's inputs from its
 * projections as q = L2Norm(ShortConv(q_raw)), k = L2Norm(ShortConv(k_raw)),
 * v = ShortConv(v_raw), b = sigmoid(b_logit), w = sigmoid(w_logit)
 * (aifetchly-blog.pages.dev, "Gated DeltaNet-2 Guide", the "Architectural
 * Workflow" diagram, steps 1 and 2, and section "2. Normalization and Short
 * Convolutions"). The *_prologue entry points take the raw tensors and do
 * these steps inside the mixer's own kernels, so q, k, v, b and w never
 * travel through memory.
 *
 * ShortConv is a causal depthwise convolution of kernel 4 along the tokens
 * of each sequence: for channel c of head h (row h*d + c of the weights),
 *     y_t = bias[c] + sum_{j=0..3} weight[c][j] * x_{t-3+j}
 * so weight[c][3] multiplies the current token; no activation follows (the
 * construction in that guide's "End-to-End PyTorch Implementation"). L2Norm
 * divides by max(||y||_2, 1e-12) over the head's channels.
 *
 * All pointers in the struct are device pointers; the struct itself is
 * read on the host during the call.
 *   weight_q, weight_k  [H*dk, 4] float   required
 *   weight_v            [H*dv, 4] float   required
 *   bias_q, bias_k      [H*dk] float, or NULL for no bias
 *   bias_v              [H*dv] float, or NULL
 *   state_in_q/k/v      [N, H, 3, d] in_dtype: the three raw inputs before
 *                       each sequence's first token, oldest first; all three
 *                       NULL means zeros (sequences that start here)
 *   state_out_q/k/v     [N, H, 3, d] in_dtype: receives the last three raw
 *                       inputs of each sequence (reaching back into
 *                       state_in when a sequence is shorter than three
 *                       tokens), or all three NULL; may alias state_in
 * Only all-or-none of the three state_in (and of the three state_out)
 * pointers may be NULL, else GDN2_ERR_INVALID.
 */
typedef struct gdn2_short_conv {
    const float *weight_q, *weight_k, *weight_v;
    const float *bias_q, *bias_k, *bias_v;
    const void *state_in_q, *state_in_k, *state_in_v;
    void *state_out_q, *state_out_k, *state_out_v;
} gdn2_short_conv;

/*
 * gdn2_chunk_fwd on the raw tensors, with the prologue above fused in.
 *   q_raw, k_raw, b_logit  [tokens, H, dk]  in_dtype
 *   v_raw, w_logit         [tokens, H, dv]  in_dtype
 *   conv                   host pointer to the convolution parameters
 * log_alpha, S0, o, ST, cu_seqlens, sizes, dtypes, workspace (the size from
 * gdn2_chunk_fwd_workspace_bytes) and errors are those of gdn2_chunk_fwd.
 * Gates are per channel. The state_out tensors are written after every
 * read of state_in, so the two may alias.
 */
int gdn2_chunk_fwd_prologue(const void *q_raw, const void *k_raw, const void *v_raw, const float *log_alpha,
                            const void *b_logit, const void *w_logit, const gdn2_short_conv *conv,
                            const float *S0, void *o, float *ST, const int32_t *cu_seqlens, int B, int T,
                            int N, int H, int dk, int dv, int in_dtype, int out_dtype,
                            void *workspace, size_t workspace_bytes);

/*
 * gdn2_decode_step on the raw inputs of one token per sequence
 * (q_raw, k_raw, b_logit [N, H, dk]; v_raw, w_logit [N, H, dv]), with the
 * prologue fused in. conv->state_in_* is the convolution history (NULL:
 * zeros, the sequence's first token); conv->state_out_* receives the history
 * shifted by this token and may alias state_in_* (the usual in-place cache).
 */
int gdn2_decode_step_prologue(const void *q_raw, const void *k_raw, const void *v_raw, const float *log_alpha,
                              const void *b_logit, const void *w_logit, const gdn2_short_conv *conv, float *S,
                              void *o, int N, int H, int dk, int dv, int in_dtype, int out_dtype);

/*
 * Backward of gdn2_chunk_fwd: the gradients of a scalar loss L with respect
 * to every input, given dL/do and dL/dS_T. The chunkwise form runs the
 * forward again (keeping each chunk's start state and corrected writes),
 * passes the state gradient from the last chunk to the first, then forms
 * the per-chunk gradients in parallel (the pages name a fused chunkwise WY
 * backward for training: snilld.dk, section "Hvad betyder det for træning og
 * inferens"; aifetchly, "Gated DeltaNet-2 Guide", section "3. Chunkwise
 * Parallel Algorithm for GPU Training").
 *
 *   q, k, v, log_alpha, b, w, S0, cu_seqlens, B, T, N, H, dk, dv, in_dtype
 *                    as in gdn2_chunk_fwd (gates per channel)
 *   dO               [tokens, H, dv] float: dL/do
 *   dST              [N, H, dk, dv] float, or NULL for zero
 *   dq, dk_, db, dlog_alpha   [tokens, H, dk] float (written)
 *   dv_, dw          [tokens, H, dv] float (written)
 *   dS0              [N, H, dk, dv] float, or NULL (not written)
 *   workspace        device memory of at least
 *                    gdn2_chunk_bwd_workspace_bytes(...) bytes
 * Gradient outputs must not alias any input. Errors as in gdn2_chunk_fwd.
 * Any log_alpha <= 0 is handled (16-token blocks whose decay is too wide for
 * the factored form take exact pairwise exponents). Value range: with bf16
 * inputs the chunk start states, corrected writes and end-state gradients
 * that the backward keeps between its kernels are f16 without scales, so
 * their entries must stay below 65504 in magnitude (the forward alone has no
 * such bound).
 */
size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv,
                                      int in_dtype, int varlen);

int gdn2_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                   const void *b, const void *w, const float *S0, const float *dO, const float *dST,
                   const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                   int in_dtype, float *dq, float *dk_, float *dv_, float *dlog_alpha,
                   float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes);

/*
 * The training pair: gdn2_chunk_fwd_keep is gdn2_chunk_fwd (per-channel
 * gates) that also leaves in `workspace` what the backward would otherwise
 * recompute (each chunk's operand block, start state S_c and corrected
 * writes), and gdn2_chunk_bwd_kept is gdn2_chunk_bwd without its own run of
 * the forward, starting from what a gdn2_chunk_fwd_keep left there. A
 * training step thus runs the forward once (the chunkwise form for GPU
 * training: aifetchly, "Gated DeltaNet-2 Guide", section "3. Chunkwise
 * Parallel Algorithm for GPU Training"; snilld.dk, section "Hvad betyder det
 * for træning og inferens").
 *
 * gdn2_chunk_fwd_keep: arguments as gdn2_chunk_fwd, except that `workspace`
 *   holds at least gdn2_chunk_bwd_workspace_bytes(...) bytes. o and S_T are
 *   those gdn2_chunk_fwd returns for the same inputs, bit for bit.
 * gdn2_chunk_bwd_kept: arguments as gdn2_chunk_bwd. The workspace, q, k, v,
 *   log_alpha, b, w, S0, cu_seqlens and sizes must be those of the last
 *   gdn2_chunk_fwd_keep on this workspace, with the workspace untouched since
 *   (on the same stream, or ordered after it); then the gradients equal those
 *   of gdn2_chunk_bwd bit for bit. Nothing checks this pairing on the device:
 *   a workspace that another call overwrote gives meaningless gradients.
 * Errors as in gdn2_chunk_fwd / gdn2_chunk_bwd; nothing is launched on an
 * error.
 */
int gdn2_chunk_fwd_keep(const void *q, const void *k, const void *v, const float *log_alpha,
                        const void *b, const void *w, const float *S0, void *o, float *ST,
                        const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                        int in_dtype, int out_dtype, void *workspace, size_t workspace_bytes);

int gdn2_chunk_bwd_kept(const void *q, const void *k, const void *v, const float *log_alpha,
                        const void *b, const void *w, const float *S0, const float *dO, const float *dST,
                        const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                        int in_dtype, float *dq, float *dk_, float *dv_, float *dlog_alpha,
                        float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes);

/*
 * Per-kernel timing, for measurement tools (not needed for computing).
 * gdn2_profile_begin(max_calls) makes this thread's next gdn2_chunk_fwd /
 * gdn2_decode_step calls (up to max_calls of them, 1..4096) record a HIP
 * event before and after each kernel they launch, on the call's stream.
 * Events are created here, on the current device. gdn2_profile_end() stops
 * recording and returns the number of calls recorded (or a negative status).
 * gdn2_profile_kernel(idx, ...) then reports, for the idx-th distinct kernel
 * name in launch order, its launch count and summed duration in ms; it waits
 * for the recorded events and returns GDN2_ERR_INVALID when idx is past the
 * last kernel. `name` points to static storage.
 */
int gdn2_profile_begin(int max_calls);
int gdn2_profile_end(void);
int gdn2_profile_kernel(int idx, const char **name, int *launches, double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
