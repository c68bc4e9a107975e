/*
 * kda.h -- C ABI of libkda, the Kimi Delta Attention (KDA) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [Walkthrough]   "Kimi K3的线性注意力：从源码看懂KDA如何更新记忆"
 *   [Replication-1] "KIMIK3轻量化复刻解析，KDA机制如何实现通道级可控遗忘"
 *   [Replication-2] "KimiK3轻量化复刻实现KDA并行解析，Chunkwise并行与状态压缩机制详解"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every tensor pointer is DEVICE memory owned by the caller, dense,
 *           row-major and contiguous, aligned to at least 16 bytes.  The library
 *           allocates nothing, keeps no global mutable state and never
 *           synchronises the host with the device.
 * Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *           and is asynchronous: outputs are valid once that stream has reached
 *           the enqueued work.
 * Packing.  Variable-length batches are packed along the token axis; cu_seqlens
 *           is an int32 DEVICE array of num_seqs+1 non-decreasing offsets with
 *           cu_seqlens[0] = 0 and cu_seqlens[num_seqs] = total_tokens.  NULL means
 *           one sequence of total_tokens tokens (num_seqs must then be 1).  Its
 *           contents cannot be checked on the host without a sync; offsets
 *           outside [0, total_tokens] are clamped by the kernels, so a malformed
 *           array yields unspecified values but no out-of-bounds access.
 * Dtypes.   `dtype` names the activation dtype (q, k, v, conv input/output,
 *           conv weights and conv state); `out_dtype` the read-out o of the
 *           recurrence (fp32, or bf16 with bf16 inputs).  Gates (g, beta) and
 *           recurrent states are always fp32.  bf16 results are rounded to
 *           nearest even.
 * Empty.    With zero tokens (batch 0 for decode) the activation pointers may be
 *           NULL; states are still copied/produced as documented.
 * Errors.   Every call returns a kda_status_t.  Argument checks run on the host
 *           before anything is enqueued; a failed check enqueues nothing and
 *           leaves every output untouched.  KDA_ERR_HIP reports a launch failure
 *           (kda_last_error() gives the HIP message).  Nothing throws across the
 *           ABI.  The calls are thread-safe and re-entrant across streams.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KDA_API
#define KDA_API __attribute__((visibility("default")))
#endif

/* Status codes and dtypes are plain 32-bit integers with named values (not C
   enum types), so that any value a caller passes or receives is well defined on
   both sides of the ABI; out-of-range values are rejected, never undefined. */
typedef int32_t kda_status_t;
enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* NULL required pointer, negative size, inconsistent sizes */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not implemented shape / dtype / gate bound */
    KDA_ERR_HIP = 3,         /* the HIP runtime rejected a launch */
    KDA_ERR_WORKSPACE = 4    /* workspace NULL or smaller than the call needs */
};

typedef int32_t kda_dtype_t;
enum {
    KDA_DTYPE_F32 = 0,
    KDA_DTYPE_BF16 = 1
};

/*
 * kda_short_conv -- causal depthwise convolution + SiLU, optionally followed by
 * a per-head L2 normalisation (the q/k/v prologue of the KDA layer).
 *
 * Defined by [Walkthrough] 第二站 (each of q, k, v passes a width-4 causal conv
 * that mixes the current position with up to three earlier ones, SiLU lives in
 * the conv module, a conv cache carries the history between calls, packed
 * sequences are passed by cu_seqlens; q and k are then L2-normalised inside the
 * KDA operator) and [Replication-2] (per-channel width-4 causal Conv1D).
 *
 * For sequence n and channel c (C = num_heads * head_dim channels), with history
 * h_0..h_{W-2} (oldest first) = conv_state_in[n, :, c] or zeros, the j-th token
 * of the sequence gets
 *     y = bias[c] + sum_{i=0}^{W-1} weight[c, i] * xe[j + i],
 *     xe = [h_0, .., h_{W-2}, x_bos, .., x_{eos-1}]
 * (weight[c, W-1] multiplies the current token), then y <- y * sigmoid(y) if
 * apply_silu, then, if l2_normalize, every group of head_dim channels of a
 * token is scaled by 1 / sqrt(sum y^2 + l2_eps).  The history restarts at every
 * sequence start.  With bf16 the whole chain is evaluated in fp64 and rounded
 * once, so every output is the correctly rounded (nearest-even) bf16 value;
 * with fp32 the arithmetic is fp32.
 *
 *   x              [total_tokens, num_heads * head_dim]   dtype
 *   weight         [num_heads * head_dim, width]           dtype
 *   bias           [num_heads * head_dim] dtype, or NULL
 *   conv_state_in  [num_seqs, width-1, num_heads*head_dim] dtype, or NULL (zeros)
 *   conv_state_out same shape, or NULL; receives the last width-1 inputs of each
 *                  sequence (history included when the sequence is shorter).
 *                  May alias conv_state_in.
 *   y              [total_tokens, num_heads, head_dim]     dtype; must not alias x.
 * Supported: width in 1..4; head_dim a multiple of 4 (a lane of the kernel
 * owns 4 channels); with l2_normalize, head_dim / 4 must be a power of two
 * <= 64 (head_dim <= 256); total_tokens >= 0 (0 enqueues only the state copy).
 */
KDA_API kda_status_t kda_short_conv(const void *x, const void *weight, const void *bias,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t num_heads, int32_t head_dim, int32_t width,
                            const void *conv_state_in, void *conv_state_out,
                            int32_t apply_silu, int32_t l2_normalize, float l2_eps,
                            kda_dtype_t dtype, void *y, void *stream);

/*
 * kda_chunk_fwd -- chunkwise-parallel KDA prefill over packed sequences.
 *
 * Computes exactly the token-by-token recurrence of [Walkthrough] 第三站-第五站:
 * for each (sequence n, head h), S <- initial_state[n,h] (or zeros) and per token
 *     S <- diag(exp(g_t)) S;  e = v_t - S^T k_t;  S <- S + beta_t k_t e^T;
 *     o_t = scale * S^T q_t,
 * and final_state[n,h] = S after the sequence.  The work is organised in chunks
 * of chunk_size tokens that pass the state from chunk to chunk while the work
 * inside a chunk runs as matrix products ([Walkthrough] 彩蛋; [Replication-2]
 * 图1); chunks restart at every sequence start and the last one may be partial.
 * The result does not depend on chunk_size beyond rounding.
 *
 *   q, k           [total_tokens, num_heads, dk]   dtype (q, k usually unit length)
 *   v              [total_tokens, num_heads, dv]   dtype
 *   g              [total_tokens, num_heads, dk]   fp32 log-decay, gate_lower_bound <= g <= 0
 *   beta           [total_tokens, num_heads]       fp32
 *   initial_state  [num_seqs, num_heads, dk, dv]   fp32 (key index first), or NULL = zeros
 *   final_state    [num_seqs, num_heads, dk, dv]   fp32, or NULL = not written;
 *                  may alias initial_state.
 *   o              [total_tokens, num_heads, dv]   out_dtype; must not alias any input.
 *   workspace      device scratch of at least kda_chunk_fwd_workspace_size() bytes,
 *                  16-byte aligned, owned by the caller, not aliasing any argument;
 *                  its contents on entry do not matter and are undefined on exit
 *                  (NULL is allowed with zero tokens).  It holds, for every token
 *                  and head, the token's row of Tb = (I + diag(beta) A)^{-1} diag(beta)
 *                  and of scale * P within its chunk (see below); calls that share
 *                  a workspace must be ordered on one stream.
 * scale is the read-out scale (the pages leave the query scale to the caller;
 * dk^-1/2 is the usual choice).  gate_lower_bound is the floor of g promised by
 * the caller ([Walkthrough] 彩蛋: the bounded gate keeps sub-chunk decay products
 * inside the floating-point range); it must be in [-9, 0].  g below the
 * promised floor gives unspecified accuracy but no out-of-bounds access.
 * Supported: dk, dv in {16, 32, 64, 128}; chunk_size in {16, 32, 64};
 * |q|, |k| entries below 1e3.
 * Chunking.  chunk_size is the caller's chunk; the kernels always walk 16-token
 * chunks, whatever chunk_size is (16 tokens keep every in-chunk decay factor
 * inside fp32 for gates down to -9, and a 16-token step is the shortest serial
 * step on this GPU).  The result does not depend on the chunking beyond
 * rounding.  Two kernels run on `stream`: the first computes, for every 16-token
 * chunk and head at once, the chunk's Tb and the decayed, scaled in-chunk
 * products scale * P_ti = scale * sum_c q_tc k_ic e^{G_tc - G_ic} (i <= t, G the
 * in-chunk cumulative g), which depend on q, k, g, beta only, into the workspace;
 * the second walks the chunks of every sequence with the state on chip, the
 * sequences of a packed batch (up to 1024 of them) longest first.  The
 * fp32 dtype computes in fp32 throughout; the bf16 dtype runs its products on
 * bf16 matrix cores with fp32 accumulation, keeps the recurrent state in fp32 and
 * gives every product split operands (x = hi + lo, both bf16; three-term
 * products), which keeps the products near fp32 accuracy.
 * Errors: KDA_ERR_WORKSPACE when workspace is NULL (with tokens) or
 * workspace_bytes is below kda_chunk_fwd_workspace_size().
 */
KDA_API kda_status_t kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const int32_t *cu_seqlens, int32_t num_seqs,
                           int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                           int32_t chunk_size, float scale, float gate_lower_bound,
                           const float *initial_state, float *final_state, void *o,
                           void *workspace, size_t workspace_bytes, kda_dtype_t dtype,
                           kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_phases -- kda_chunk_fwd in two separately enqueued parts, so that
 * the first can overlap independent work on another stream (for instance the
 * convolution of v, which it does not read).
 *
 *   phases = KDA_PHASE_PREP: the prep only -- a packed batch's walking order and,
 *            for every chunk and head, Tb and scale * P -- into the workspace.  It
 *            reads q, k, g, beta and cu_seqlens; it does not touch v,
 *            initial_state, final_state or o.
 *   phases = KDA_PHASE_WALK: the walk over the chunks only.  It reads the workspace
 *            as left by a PREP call with the same arguments, which the caller must
 *            order before it (same stream, or an event between streams), and
 *            writes o and final_state.
 *   phases = KDA_PHASE_ALL:  both, exactly kda_chunk_fwd.
 * PREP then WALK gives results bit-identical to kda_chunk_fwd.  Every other
 * argument, the workspace size, the supported shapes and the errors are those of
 * kda_chunk_fwd (both parts check all of them, v and o included); a phases
 * value other than these three is KDA_ERR_INVALID_ARG.
 */
enum {
    KDA_PHASE_PREP = 1,
    KDA_PHASE_WALK = 2,
    KDA_PHASE_ALL = 3
};
KDA_API kda_status_t kda_chunk_fwd_phases(const void *q, const void *k, const void *v,
                                          const float *g, const float *beta,
                                          const int32_t *cu_seqlens, int32_t num_seqs,
                                          int64_t total_tokens, int32_t num_heads, int32_t dk,
                                          int32_t dv, int32_t chunk_size, float scale,
                                          float gate_lower_bound, const float *initial_state,
                                          float *final_state, void *o, void *workspace,
                                          size_t workspace_bytes, kda_dtype_t dtype,
                                          kda_dtype_t out_dtype, int32_t phases, void *stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and arguments without the workspace.
 * The Tb / P rows go to a static device array of the library (64 MiB per GPU,
 * held from the library's load until the process ends), so the call itself
 * allocates nothing.  Limit: total_tokens * num_heads <= 524288 (4096 tokens x
 * 128 heads; the prefill workload's 4096 x 96 fits); a larger call returns
 * KDA_ERR_UNSUPPORTED and enqueues nothing.  The scratch of a GPU is shared by
 * every call on it: two such calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and give undefined results; calls
 * ordered on one stream are safe.  The device used is the calling thread's
 * current HIP device, which must be the device of `stream`.  Its address is
 * looked up once per device (hipGetSymbolAddress) on the first call there.
 * Every other argument, the supported shapes and the errors are those of
 * kda_chunk_fwd.
 */
KDA_API kda_status_t kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                           const float *g, const float *beta,
                                           const int32_t *cu_seqlens, int32_t num_seqs,
                                           int64_t total_tokens, int32_t num_heads, int32_t dk,
                                           int32_t dv, int32_t chunk_size, float scale,
                                           float gate_lower_bound, const float *initial_state,
                                           float *final_state, void *o, kda_dtype_t dtype,
                                           kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_gated -- kda_chunk_fwd with the bounded forget gate fused in.
 *
 * Instead of the log-decay g the caller passes the gate's pre-activation z and
 * its parameters; the kernels form, as they read each value,
 *     g[t, h, c] = lower_bound * sigmoid(exp(a_log[h]) * (z[t, h, c] + dt_bias[h, c]))
 * ([Walkthrough] 彩蛋: the gate function with a lower bound; K3 uses -5), in
 * fp32 (hardware exp2 and reciprocal, a few ulps), so lower_bound <= g <= 0 by
 * construction and g never goes through memory.  With bf16 activations z is
 * bf16: half the bytes of g.
 *
 *   z        [total_tokens, num_heads, dk]  dtype
 *   a_log    [num_heads] fp32, or NULL (0: no scaling)
 *   dt_bias  [num_heads, dk] fp32, or NULL (0)
 *   lower_bound  in [-9, 0]; it is also the chunk algorithm's gate floor.
 * Every other argument, the workspace (kda_chunk_fwd_workspace_size), the
 * supported shapes and the errors are those of kda_chunk_fwd; o must not alias
 * z, a_log or dt_bias either.
 */
KDA_API kda_status_t kda_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                         const void *z, const float *a_log, const float *dt_bias,
                                         float lower_bound, const float *beta,
                                         const int32_t *cu_seqlens, int32_t num_seqs,
                                         int64_t total_tokens, int32_t num_heads, int32_t dk,
                                         int32_t dv, int32_t chunk_size, float scale,
                                         const float *initial_state, float *final_state, void *o,
                                         void *workspace, size_t workspace_bytes,
                                         kda_dtype_t dtype, kda_dtype_t out_dtype, void *stream);

/*
 * kda_chunk_fwd_workspace_size -- bytes of device workspace kda_chunk_fwd needs
 * for these sizes (written to *bytes): 2 * total_tokens * num_heads * 16 * 4 + 4096
 * (one row of Tb and one of scale * P per token and head, 16 fp32 each, and the
 * order in which a packed batch of up to 1024 sequences is walked: longest
 * first), or 0 without tokens.
 * Returns the same status kda_chunk_fwd would return for an unsupported shape.
 */
KDA_API kda_status_t kda_chunk_fwd_workspace_size(int64_t total_tokens, int32_t num_heads,
                                                  int32_t dk, int32_t dv, int32_t chunk_size,
                                                  kda_dtype_t dtype, kda_dtype_t out_dtype,
                                                  size_t *bytes);

/*
 * kda_decode_step -- one recurrent KDA step for a batch of sequences, updating
 * the fp32 states in place (token-by-token execution for generation,
 * [Walkthrough] 彩蛋; update order of 第三站-第五站).
 *
 * For each (b, h): S <- diag(exp(g)) S; e = v - S^T k; S <- S + beta k e^T;
 * o = scale * S^T q.  Inputs are already conv-processed and q, k normalised;
 * the step does no convolution and no normalisation.
 *
 *   q, k   [batch, num_heads, dk]        dtype
 *   v      [batch, num_heads, dv]        dtype
 *   g      [batch, num_heads, dk]        fp32 log-decay
 *   beta   [batch, num_heads]            fp32
 *   state  [batch, num_heads, dk, dv]    fp32, read and written IN PLACE
 *   o      [batch, num_heads, dv]        out_dtype; must not alias any input.
 * Supported: dk, dv in {16, 32, 64, 128}.
 */
KDA_API kda_status_t kda_decode_step(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *state, int32_t batch, int32_t num_heads,
                             int32_t dk, int32_t dv, float scale, void *o, kda_dtype_t dtype,
                             kda_dtype_t out_dtype, void *stream);

/*
 * kda_gdn_chunk_fwd, kda_gdn_decode_step -- the same computations with one
 * decay per (token, head) instead of one per key channel: the head-wise forget
 * gate of Gated DeltaNet (GDN), which the pages set against KDA's channel-wise
 * one ([Replication-1]: GDN scales a head's whole state by one scalar).  The
 * recurrence is KDA's with g[t, h, c] = g[t, h] for every key channel c.
 *
 *   g   [total_tokens, num_heads] fp32 (chunk) / [batch, num_heads] fp32 (decode),
 *       gate_lower_bound <= g <= 0 for the chunk call.
 * Every other argument, the workspace, the supported shapes and the errors are
 * those of kda_chunk_fwd and kda_decode_step.
 */
KDA_API kda_status_t kda_gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                                       const float *beta, const int32_t *cu_seqlens,
                                       int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                       int32_t dk, int32_t dv, int32_t chunk_size, float scale,
                                       float gate_lower_bound, const float *initial_state,
                                       float *final_state, void *o, void *workspace,
                                       size_t workspace_bytes, kda_dtype_t dtype,
                                       kda_dtype_t out_dtype, void *stream);
KDA_API kda_status_t kda_gdn_decode_step(const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, float *state,
                                         int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                         float scale, void *o, kda_dtype_t dtype,
                                         kda_dtype_t out_dtype, void *stream);

/*
 * kda_decode_step_conv -- one generation step from this token's raw q/k/v
 * projections: the prologue of kda_short_conv (width-4 causal conv over the
 * conv cache, SiLU, q and k scaled to unit length; [Walkthrough] 第二站) and
 * kda_decode_step's recurrent step, fused in one launch; q, k and v stay on
 * chip in fp32 (they are not rounded to the activation dtype in between).
 *
 *   q_raw, k_raw  [batch, num_heads * dk]   dtype: this token's projections
 *   v_raw         [batch, num_heads * dv]   dtype
 *   w_q, w_k      [num_heads * dk, 4]       dtype (w[:, 3] multiplies the current token)
 *   w_v           [num_heads * dv, 4]       dtype
 *   conv_q, conv_k [batch, 3, num_heads * dk], conv_v [batch, 3, num_heads * dv]
 *                 dtype: the last three raw inputs of every sequence (oldest
 *                 first; the layout of kda_short_conv's conv_state), read and
 *                 updated IN PLACE to end with this token; three distinct buffers.
 *   l2_eps        the q / k normalisation's epsilon: u / sqrt(sum u^2 + l2_eps)
 *   g, beta, state, scale, o: as kda_decode_step.
 * No conv bias.  Supported: dk, dv in {16, 32, 64, 128}.  Cloning a sequence
 * for branching is a device copy of its state and conv caches.
 */
KDA_API kda_status_t kda_decode_step_conv(const void *q_raw, const void *k_raw, const void *v_raw,
                                          const void *w_q, const void *w_k, const void *w_v,
                                          void *conv_q, void *conv_k, void *conv_v, float l2_eps,
                                          const float *g, const float *beta, float *state,
                                          int32_t batch, int32_t num_heads, int32_t dk, int32_t dv,
                                          float scale, void *o, kda_dtype_t dtype,
                                          kda_dtype_t out_dtype, void *stream);

/*
 * kda_output_norm_gate -- the read-out's exit path before the output projection
 * ([Walkthrough] 第六站: a per-head RMSNorm, then the output gate scales each
 * channel).  For every row r (a (token, head) pair) of dv channels:
 *     y[r, c] = o[r, c] / sqrt(mean_c' o[r, c']^2 + eps) * weight[c] * sigmoid(gate[r, c])
 * in fp32, rounded once to the dtype of y.  The sigmoid is the reading taken
 * for the gate's nonlinearity (the pages name none); the gate's projection of
 * the layer input and the output projection are outside this library.
 *
 *   o       [rows, dv]  o_dtype (the read-out of kda_chunk_fwd or kda_decode_step)
 *   gate    [rows, dv]  dtype: the output gate's pre-activation
 *   weight  [dv] fp32 (the norm's per-channel weight, shared by the heads), or NULL (1)
 *   y       [rows, dv]  dtype; may be the same buffer as gate, or as o when o_dtype
 *           equals dtype; no other overlap with an input is allowed.
 * rows = tokens * heads (for o of shape [T, H, dv]).  Supported: dv in
 * {16, 32, 64, 128}; eps >= 0; a bf16 o needs dtype bf16.
 */
KDA_API kda_status_t kda_output_norm_gate(const void *o, const void *gate, const float *weight,
                                          float eps, int64_t rows, int32_t dv,
                                          kda_dtype_t o_dtype, kda_dtype_t dtype, void *y,
                                          void *stream);

/* Static description of a status code (never NULL). */
KDA_API const char *kda_status_string(kda_status_t status);

/* Detail of the last failed call on the calling thread ("" if none). */
KDA_API const char *kda_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
KDA_API int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
