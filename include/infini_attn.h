/*
 * infini_attn.h -- C-ABI of the Infini-attention layer forward for AMD MI355X (gfx950).
 *
 * The method: "Leave No Context Behind: Efficient Infinite Context Transformers with
 * Infini-attention" (arXiv 2404.07143), as stated in the architecture summary on
 * paper-graph-ui.vercel.app, section 3.4 "Detailed, Sentence-Based Technical Breakdown".
 * For each segment of N tokens, per (batch element, head):
 *
 *   A_dot = softmax(scale * Q K^T, causal inside the segment) V          (Eq. 6)
 *   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)                  (Eq. 7)
 *   A     = sigmoid(beta_h) A_mem + (1 - sigmoid(beta_h)) A_dot           (Eq. 10)
 *   linear: M_s = M_{s-1} + sigma(K)^T V                                  (Eq. 8)
 *   delta:  M_s = M_{s-1} + sigma(K)^T (V - sigma(K) M_{s-1} / (sigma(K) z_{s-1} + eps))  (Eq. 9)
 *   z_s = z_{s-1} + sum_t sigma(K_t)                                      (Eq. 8, both rules)
 *
 * with sigma = ELU + 1 (alpha = 1).  The state (M, z) is carried from segment to segment
 * and from call to call (Eq. 4, "The Recurrent Formulation of Infini-Attention").
 *
 * Boundary.  The core calls sit after the Q/K/V projections (Eq. 5) and before the
 * output projection W_O (Eq. 11): callers pass per-head Q, K, V and receive the per-head
 * gated context A.  The layer calls at the end of this header add the two projections
 * (project_qkv, project_out, and forward_layer for the whole of Eq. 5 -> Eq. 11).
 *
 * Layout.  Q, K, V and out are dense [B, H, T, d] arrays (d fastest), T = tokens of the
 * call, element type io_dtype.  Segments start at the first token of every call; a last
 * segment shorter than N is processed with its own length.  M is [B, H, d_key, d_value]
 * float32 row-major (M[i][j] binds key feature i to value feature j), z is [B, H, d_key]
 * float32.
 *
 * Ownership.  The caller owns Q, K, V and out (device pointers).  The library owns M, z,
 * the gate values and its workspace, all on the device of the create call.  out must not
 * overlap any input.  A handle is not thread-safe.
 *
 * Execution.  Compute calls are enqueued on the HIP stream passed in (NULL = the null
 * stream) and return without waiting for the device.  Consecutive calls on one handle
 * must be ordered on one stream (or synchronised by the caller).
 *
 * Errors.  Every entry point returns INFINI_OK (0) or a negative status.  Argument
 * errors are found before anything is enqueued and leave the state untouched.  HIP
 * errors from launches are reported as INFINI_ERR_HIP.  Numerics are not checked: NaN
 * in the inputs propagates as the equations dictate.
 */
#ifndef INFINI_ATTN_H
#define INFINI_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define INFINI_OK 0
#define INFINI_ERR_INVALID_ARG (-1)
#define INFINI_ERR_UNSUPPORTED (-2)
#define INFINI_ERR_HIP (-3)
#define INFINI_ERR_OOM (-4)
#define INFINI_ERR_SCRATCH (-5) /* forward_stream_noalloc: one segment's workspace exceeds its
                                   static scratch array */

typedef struct infini_attn* infini_attn_t;

/* Memory update rule: Eq. 8 (linear) or Eq. 9 (delta). */
typedef enum { INFINI_UPDATE_LINEAR = 0, INFINI_UPDATE_DELTA = 1 } infini_update_t;

/* Element type of Q, K, V and out.  bf16 runs the bf16 matrix-core path; f32 runs an
 * all-float32 path meant for small shapes and checks. */
typedef enum { INFINI_DTYPE_BF16 = 0, INFINI_DTYPE_F32 = 1 } infini_dtype_t;

typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t heads;          /* H >= 1; each head has its own M, z and beta ("Multi-Head Infini-Attention") */
  int32_t head_dim;       /* d = d_key = d_value; 64 or 128 */
  int32_t segment_len;    /* 1 <= N <= 2^22 (one segment's d-wide rows stay within a 32-bit
                             byte range); larger: INFINI_ERR_UNSUPPORTED */
  int32_t update;         /* infini_update_t */
  int32_t io_dtype;       /* infini_dtype_t */
  float eps;              /* >= 0; added to the retrieval denominator in Eq. 7 and Eq. 9.  With
                             eps = 0 the first segment (zero memory) yields 0/0 = NaN. */
  float softmax_scale;    /* > 0, or <= 0 for 1/sqrt(head_dim) */
  int32_t max_window_segments; /* segments processed per internal window of forward_stream;
                                  bounds the workspace; <= 0 picks a default */
} infini_attn_config_t;

/* Create a layer (architecture summary, section "Multi-Head Infini-Attention": every head
 * keeps its own compressive memory, a d_key x d_value matrix M and a d_key vector z, and
 * its own gate scalar beta; Eq. 10 mixes the two arms with sigmoid(beta)).
 * beta_host: H gate logits (host memory, copied; +-inf allowed: sigmoid(beta) and
 * 1 - sigmoid(beta) are formed in double as exact complements, so +-inf selects one arm).
 * Allocates M = 0, z = 0 (the empty memory before the first segment, Eq. 4), the gate
 * values and the workspace on the current device.  hip_stream orders the zero fill.
 * *out receives the handle.  Errors: INVALID_ARG for a bad config or NULL pointers,
 * UNSUPPORTED for head_dim other than 64 / 128 or segment_len > 2^22, OOM, HIP. */
int infini_attn_create(const infini_attn_config_t* cfg, const float* beta_host,
                       void* hip_stream, infini_attn_t* out);

/* One segment (Eq. 4): 1 <= n_tokens <= N tokens of Q/K/V [B,H,n_tokens,d] -> out.
 * Reads the state, writes out, advances the state by this segment.  This is the
 * streaming call (the summary page's section 1: a stream processed segment by segment
 * with bounded memory).  Since the segment's output depends only on the state carried in
 * (Eq. 7 reads M_{s-1}, z_{s-1}), a bf16 handle runs the memory update (Eq. 8 / 9) on a
 * second stream of its own while the attention runs on hip_stream: once the call's work
 * on hip_stream has completed, q, k, v and out may be reused; the new state itself may
 * still be in the making, and every later call on the handle (on any stream) waits for it
 * before it touches the state.  With few (batch, head) pairs the attention splits each
 * query tile's keys over several workgroups (results do not vary from run to run).  The
 * same applies to forward_stream calls of one segment without a_mem / a_dot.
 * Device memory for this (the split partials, two bf16 copies of M^T and of z) is
 * allocated by create and counted by device_bytes. */
int infini_attn_forward_segment(infini_attn_t h, const void* q, const void* k, const void* v,
                                void* out, int32_t n_tokens, void* hip_stream);

/* A stream of n_tokens >= 1 tokens, cut into ceil(n_tokens / N) segments processed in
 * order (section "Training Infrastructure for Recurrent Attention", segment chunking).
 * Same result as calling forward_segment once per segment. */
int infini_attn_forward_stream(infini_attn_t h, const void* q, const void* k, const void* v,
                               void* out, int64_t n_tokens, void* hip_stream);

/* forward_stream that also writes the two gated terms for checks: a_mem (Eq. 7) and
 * a_dot (Eq. 6), float32 [B,H,n_tokens,d] each; either may be NULL. */
int infini_attn_forward_stream_ex(infini_attn_t h, const void* q, const void* k, const void* v,
                                  void* out, float* a_mem, float* a_dot, int64_t n_tokens,
                                  void* hip_stream);

/* forward_stream with separate Q and K for the local softmax attention (Eq. 6), e.g.
 * position-embedded ones: the summary page's training notes apply position embeddings to
 * the local arm's Q and K only, after the memory has been read and updated ("Compressive
 * Memory" and "Training Infrastructure for Recurrent Attention" subsections).  q and k
 * (PE-free) feed the retrieval (Eq. 7) and the memory update (Eq. 8-9); q_local and k_local
 * feed Eq. 6.  Same layout, element type and alignment as q; NULL means "same as q / k".
 * They must not overlap out.  Everything else as forward_stream. */
int infini_attn_forward_stream_local(infini_attn_t h, const void* q, const void* k, const void* v,
                                     const void* q_local, const void* k_local, void* out,
                                     int64_t n_tokens, void* hip_stream);

/* forward_stream for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * arguments, with the window workspace (chunk partials of the state pass, the recorded
 * M^T_{s-1} and z_{s-1} of every segment) taken from a static device array of 32 MiB that
 * the library holds on each device from its first use there until the process ends,
 * instead of the handle's workspace.  The call allocates nothing; the handle (state, gate
 * values) comes from infini_attn_create as usual.  Windows are as long as the handle's
 * window and the array allow; with a window as long as forward_stream's the results are
 * bit-identical to it.  If the workspace of one segment (about 97 KB per (batch, head)
 * at d = 128, linear rule; 225 KB delta) exceeds the array, returns INFINI_ERR_SCRATCH
 * before enqueuing anything.  Every call on a device shares that device's array: calls
 * that may overlap on one device (other streams, other threads, other handles) race and
 * must be serialised by the caller.  Nothing in the array needs to start at zero: each
 * window writes every part of it it reads. */
int infini_attn_forward_stream_noalloc(infini_attn_t h, const void* q, const void* k, const void* v,
                                       void* out, int64_t n_tokens, void* hip_stream);

/* M = 0, z = 0: the memory before the first segment of a new stream (Eq. 4 with an
 * empty history).  Takes effect for every later call on the handle; enqueues no device
 * work (the next forward reads the state as zero; get_state / set_state write the zeros
 * out first on their stream).  hip_stream is accepted for symmetry and not used. */
int infini_attn_reset_state(infini_attn_t h, void* hip_stream);

/* Copy the state out / in.  M: [B,H,d,d] float32, z: [B,H,d] float32, device or host
 * pointers (hipMemcpyDefault).  get_state waits for the copy to finish. */
int infini_attn_get_state(infini_attn_t h, float* M, float* z, void* hip_stream);
int infini_attn_set_state(infini_attn_t h, const float* M, const float* z, void* hip_stream);

/* Replace the H gate logits beta of Eq. 10 (host memory; one per head, section "The Gating
 * Mechanism").  Waits for the device to be idle first, so no call in flight sees a mix. */
int infini_attn_set_beta(infini_attn_t h, const float* beta_host);

/* Device bytes the handle holds: state + gate values + workspace, plus the layer scratch
 * once forward_layer has run (at most one window's worth) and the decode cache once
 * decode_step has run (one segment, plus the split-key partial slots with few pairs).  Independent of how many tokens have been processed:
 * the bounded-memory property of the compressive memory (summary page, "Multi-Head
 * Infini-Attention", memory footprint per layer: H (d_key d_value + d_key) numbers of
 * state, here in fp32, 66,048 bytes per head at d = 128). */
int64_t infini_attn_device_bytes(infini_attn_t h);

/* Tokens per internal window of forward_stream (window segments * N). */
int64_t infini_attn_window_tokens(infini_attn_t h);

/* ---- The layer around the heads (Eq. 5 and Eq. 11; bf16 io_dtype only) ----------------
 *
 * X and O are [B, T, d_model] (d_model fastest), T = n_tokens.  Weights are bf16 in the
 * "out x in" layout (row j holds the d_model, resp. H*d, input weights of output feature
 * j), i.e. the transposes of the pages' W_Q, W_K, W_V (d_model x d each per head) and
 * W_O (H*d x d_model):
 *   w_qkv: [3*H*d, d_model]; row h*d + j is column j of head h's W_Q, row H*d + h*d + j
 *          of its W_K, row 2*H*d + h*d + j of its W_V;
 *   w_o:   [d_model, H*d]; column h*d + j multiplies feature j of head h's output A_h,
 *          so O = [A_1; ...; A_H] W_O with the heads concatenated in order (Eq. 11).
 * Products accumulate in float32 and are rounded once to bf16 where they are stored:
 * Q, K, V and A are bf16 between the steps, as in the per-head calls.
 * Requirements: d_model a multiple of 32; X, weights 16-byte aligned; outputs 8-byte
 * aligned; outputs must not overlap inputs.  Errors: INFINI_ERR_UNSUPPORTED for an f32
 * handle, INFINI_ERR_INVALID_ARG otherwise, before anything is enqueued. */

/* Q, K, V [B, H, n_tokens, d] (the per-head layout above) from X (Eq. 5). */
int infini_attn_project_qkv(infini_attn_t h, const void* x, const void* w_qkv, void* q, void* k,
                            void* v, int64_t n_tokens, int32_t d_model, void* hip_stream);

/* O [B, n_tokens, d_model] = [A_1; ...; A_H] W_O from the per-head A [B, H, n_tokens, d]
 * (Eq. 11). */
int infini_attn_project_out(infini_attn_t h, const void* a, const void* w_o, void* out,
                            int64_t n_tokens, int32_t d_model, void* hip_stream);

/* The whole layer on a stream of n_tokens tokens: project_qkv, forward_stream,
 * project_out, one internal window (window_tokens tokens) at a time, with Q, K, V and A
 * in library-owned device memory (allocated on first use and grown when a call needs more;
 * released by destroy; 4 * B * H * d * 2 bytes per window token).  Same result as the
 * three calls on the whole stream; the state advances as in forward_stream. */
int infini_attn_forward_layer(infini_attn_t h, const void* x, const void* w_qkv, const void* w_o,
                              void* out, int64_t n_tokens, int32_t d_model, void* hip_stream);

/* ---- Incremental decoding (one token per sequence per call) ------------------------------
 *
 * Streaming generation inside a segment (the summary's "fast streaming inference", with
 * the segment-wise recurrence of Eq. 4): the handle keeps the open segment's keys and
 * values (a cache of at most N tokens per (b, h), library-owned, allocated on the first
 * decode_step: 2 * B * H * N * d elements of io_dtype) next to M, z.  For each token the
 * output is, per (b, h), row p of the segment computation: the local softmax attention
 * (Eq. 6) over the segment's tokens 0 .. p (the cached ones and this one), the memory read
 * (Eq. 7) from the state before the segment, gated by Eq. 10.  When the N-th token of the
 * segment has been processed the segment is written to the memory (Eq. 8 / 9) and the next
 * call starts a new segment.  Feeding a stream token by token therefore gives the outputs
 * of forward_stream on the same stream, and, once the last segment is complete or
 * flushed, the same state.
 *
 * decode_step: q, k, v, out are [B, H, d] (this token of every sequence), io_dtype; q, k,
 *   v 16-byte aligned; out must not overlap them.  With fewer than 128 (batch, head) pairs
 *   the keys of a long open segment are split over several workgroups per pair, whose
 *   partial results the handle keeps in a library-owned buffer (B * H * 17 * (d + 2) floats
 *   and B * H counters, allocated on the first step that splits; INFINI_ERR_OOM if that
 *   fails).
 * decode_flush: writes an open partial segment to the memory (as forward_stream does with a
 *   short last segment); no-op when none is open.
 * decode_position: tokens of the open segment (0 .. N-1).
 * While a segment is open, forward_segment / forward_stream* / forward_layer return
 * INFINI_ERR_INVALID_ARG (flush first); reset_state drops the open segment; get_state
 * returns the state before it; set_state replaces the state its remaining tokens read. */
int infini_attn_decode_step(infini_attn_t h, const void* q, const void* k, const void* v, void* out,
                            void* hip_stream);
int infini_attn_decode_flush(infini_attn_t h, void* hip_stream);
int64_t infini_attn_decode_position(infini_attn_t h);

/* ---- Backward (training): gradients through the whole stream -----------------------------
 *
 * For a call's stream (n_tokens tokens from the initial state (m0, z0); NULL for both means
 * zero), the gradients of  loss = <d_out, O> + <dm_final, M_final> + <dz_final, z_final>
 * with respect to Q, K, V, the gate logits beta and the initial state, back through the
 * M / z recurrence over all the call's segments (backpropagation through time,
 * "Training Infrastructure for Recurrent Attention"; the forward is recomputed segment by
 * segment first).  Same readings as the forward (eps in both retrieval denominators, one
 * beta per head, the delta rule's retrieved value from the state before the segment).
 *   q, k, v, d_out: [B, H, n_tokens, d] io_dtype (16-byte aligned for bf16);
 *   m0 [B, H, d, d], z0 [B, H, d], dm_final, dz_final: float32 device pointers or NULL;
 *   dq, dk, dv: float32 [B, H, n_tokens, d]; dbeta: float32 [H];
 *   dm0 [B, H, d, d], dz0 [B, H, d]: float32 or NULL (not wanted).
 * The handle's own state is neither read nor changed.  A call longer than one internal
 * window (window_tokens) runs the memory recurrence forward once to record the state at
 * every window start (B*H*(d*d + d)*4 bytes per window), then the windows in reverse, each
 * recomputing its forward from its recorded start state and passing the gradient of that
 * state to the window before it: the gradients are those of the whole call.  Device memory
 * for the recomputed forward and the gradient scratch (per-token terms for the whole call,
 * per-segment terms for one window) is library-owned and kept for reuse. */
int infini_attn_backward(infini_attn_t h, const void* q, const void* k, const void* v, const void* d_out,
                         const float* m0, const float* z0, const float* dm_final, const float* dz_final,
                         float* dq, float* dk, float* dv, float* dbeta, float* dm0, float* dz0,
                         int64_t n_tokens, void* hip_stream);

/* Per-kernel timing with HIP events, for measurement.  While enabled, every kernel the
 * handle launches is bracketed by two events on the stream it runs on (the call's stream,
 * or the handle's second stream for the memory update of a one-segment call).  profile_read waits
 * for the recorded events, reports the summed durations per kernel kind, and clears the
 * record.  Kernel kinds: 0 = key sums (delta rule only), 1 = state pass (per-segment
 * sigma(K)^T V, key sums, delta Gram term), 2 = memory chain (Eq. 8/9
 * recurrence), 3 = fused local attention + retrieval + gate (Eq. 6, 7, 10),
 * 4 = Q/K/V projection (Eq. 5), 5 = output projection (Eq. 11), 6 = decoding step,
 * 7 = backward (all gradient kernels of one call; the recomputed forward counts as 0-3). */
#define INFINI_KERNEL_KINDS 8
typedef struct {
  double total_ms[INFINI_KERNEL_KINDS];
  int64_t launches[INFINI_KERNEL_KINDS];
} infini_attn_profile_t;
int infini_attn_profile_enable(infini_attn_t h, int enable);
int infini_attn_profile_read(infini_attn_t h, infini_attn_profile_t* out);

/* Waits for pending work on the handle's device, then frees everything.  NULL is a no-op. */
int infini_attn_destroy(infini_attn_t h);

/* Static text for a status code. */
const char* infini_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* INFINI_ATTN_H */
