/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet token mixer for AMD MI355X (gfx950).
 *
 * The mixer is the linear-attention layer of the Qwen3.5 / Qwen3-Next hybrid
 * models (three of every four decoder blocks: HF transformers Qwen3.5 docs
 * page, introduction).  Between its input projections and its output
 * projection it computes
 *
 *   conv     y = silu(causal depthwise conv1d, width 4, no bias) over the packed
 *            q|k|v channels (llm-arch-viz Qwen3.5-9B page, module tree:
 *            conv1d 8192x1x4);
 *   core     q, k L2-normalised per head, key heads repeated to the value-head
 *            count, gates g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b),
 *            and the gated delta rule on a dk x dv fp32 state per value head
 *              S_t = e^{g_t} S_{t-1} + beta_t k_t (v_t - (e^{g_t} S_{t-1})^T k_t)^T
 *              o_t = S_t^T q_t * scale
 *            (KerasFormers Qwen page, "Architecture notes": conv1d + delta rule;
 *            chunked and recurrent forms are algebraically identical, "Verified
 *            parity"); prefill uses a chunked form, decode one recurrent step
 *            (HF Qwen3.5 docs page, "Usage tips": chunked-prefill core, the
 *            single-token recurrence is memory-bandwidth-bound);
 *   norm     y = w * o / sqrt(mean(o^2) + eps) * silu(z) per value head, weight
 *            shared by all heads (llm-arch-viz Qwen3.5-9B page:
 *            Qwen3_5RMSNormGated, 128; eps 1e-6 from the KerasFormers Qwen3.5
 *            page, "API" table).
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps device memory between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).  No
 *     call synchronises the host.
 *   - Activations use the io dtype (GDN_F32 or GDN_BF16).  Parameters (conv
 *     weight, A_log, dt_bias, norm weight), the optional precomputed gates and
 *     every recurrent state are always fp32.
 *   - Packed sequences: `cu_seqlens` is a device int32 array [Ns + 1] of prefix
 *     offsets (cu[0] = 0, non-decreasing, cu[Ns] = N); NULL means a single
 *     sequence of N tokens (then Ns must be 1).  Offsets are trusted: they are
 *     read only on the device.
 *   - Nullable state pointers: an input state of NULL means zeros, an output
 *     state of NULL means "not written".  An input and its output may alias (the
 *     reads of every element happen before its write).
 *   - Layouts are row-major with the last index contiguous.
 *   - Errors: every call returns a gdn_status_t.  Argument errors are detected
 *     on the host before anything is enqueued.  gdn_last_error() returns a
 *     message for the calling thread's last failure.  There is no fallback path:
 *     a device that is not gfx950 gives GDN_ERR_UNSUPPORTED.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* bad shape, size or required NULL pointer          */
  GDN_ERR_UNSUPPORTED = 2, /* device is not gfx950, or head width / conv width   */
  GDN_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed          */
} gdn_status_t;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

/* Largest row stride, in elements, that gdn_chunk_prefill accepts for q, k, v
 * (the kernels address a chunk's rows with 24-bit row offsets). */
#define GDN_MAX_ROW_STRIDE (1LL << 20)

/* Message for the calling thread's most recent failed call ("" if none). */
const char* gdn_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* gdn_version(void);

/*
 * gdn_conv1d_fwd -- causal depthwise conv1d (width K = 4, no bias) + SiLU.
 *
 *   y[t, c] = silu( sum_{j=0..K-1} w[c, j] * xpad[t + j, c] ),
 *   xpad = [conv_state_in[s] (K-1 rows, oldest first) or zeros ; x rows of s]
 * so w[c, K-1] multiplies the current token.  Sequences never see each other's
 * rows.  conv_state_out[s] receives the last K-1 rows of xpad (the raw inputs,
 * so a sequence shorter than K-1 keeps part of its old state).
 * (llm-arch-viz Qwen3.5-9B page, module tree: conv1d 8192x1x4 -- depthwise,
 * no bias; KerasFormers Qwen page, "Generation": per-layer conv state.)
 *
 *   x               [N, Cq]       io      input rows (mixed q|k|v channels)
 *   w               [Cq, K]       fp32    taps
 *   y               [N, Cq]       io      output (may not alias x)
 *   cu_seqlens      [Ns + 1]      int32   or NULL (one sequence)
 *   conv_state_in   [Ns, K-1, Cq] io      or NULL (zeros)
 *   conv_state_out  [Ns, K-1, Cq] io      or NULL; may alias conv_state_in
 * Errors: K != 4 -> UNSUPPORTED; N < 0, Ns < 1, Cq < 1 or Cq % 8 != 0, NULL
 * x/w/y with N > 0 -> INVALID_ARG.  N = 0 is valid (only the state copy runs).
 */
gdn_status_t gdn_conv1d_fwd(const void* x, const float* w, void* y, const int32_t* cu_seqlens,
                            int Ns, int64_t N, int Cq, int K, const void* conv_state_in,
                            void* conv_state_out, gdn_dtype_t io, void* stream);

/*
 * gdn_chunk_prefill_workspace_size -- bytes of device workspace that
 * gdn_chunk_prefill (and gdn_conv_chunk_prefill) needs for N packed tokens in Ns
 * sequences with Hk key heads, Hv value heads, head width d (128) and io dtype io.
 * The workspace holds the chunk map of the packed sequences; for at most
 * ceil(N/64) + Ns 64-token chunks, per (chunk, value head) a 38912-byte record (the
 * chunk's 64 x 64 T' and P matrices as bf16 hi/lo parts plus per-token factors; bf16 io
 * lays them out as MFMA operand fragments in the first 34816 bytes, or 18432 without
 * P, for the sweep shapes that form P themselves) and,
 * for fp32 io only, per (chunk, key head) the bf16 hi/lo K and Q rows (69632 bytes);
 * and, where the intra-sequence scan may run, 7 segment-transition pairs of 128 KB per
 * (sequence, value head) pair: fp32 io with at most 64 pairs, bf16 io with at most 16
 * pairs and sequences of at least 256 chunks on average (ceil(N/64) / Ns >= 256).
 * Returns 0 for invalid sizes: those gdn_chunk_prefill rejects (Hv not a multiple of
 * Hk, more than 2^31 - 1 chunks or too many (sequence, head) pairs), and any whose byte
 * count could pass 2^62.
 * (The io argument is one more than the five of the plain form (N, Ns, Hk, Hv, d): the
 * fp32 io records are larger, so the size depends on it.)
 */
size_t gdn_chunk_prefill_workspace_size(int64_t N, int Ns, int Hk, int Hv, int d, gdn_dtype_t io);

/*
 * gdn_chunk_prefill -- gated delta rule over packed sequences, chunked form.
 *
 * For each sequence s and value head h (key/query head h / (Hv/Hk)):
 *   q^_t = q_t / sqrt(|q_t|^2 + 1e-6), likewise k^_t (if use_qk_l2norm),
 *   g_t = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h]), beta_t = sigmoid(b[t,h])
 *         (or g_opt / beta_opt when both are given),
 *   S_0 = state_in[s, h] or 0, then token by token
 *   S_t = e^{g_t} S_{t-1} + beta_t k^_t (v_t - e^{g_t} S_{t-1}^T k^_t)^T,
 *   o[t, h, :] = scale * S_t^T q^_t,     state_out[s, h] = S_last.
 * The kernels evaluate the exact chunked (WY/UT) rewriting of this recurrence
 * with 64-token chunks that restart at every sequence start (KerasFormers
 * Qwen page, "Verified parity": chunked and recurrent forms are
 * algebraically identical; HF Qwen3.5 docs page, "Usage tips": chunked-prefill
 * core).  Products run on bf16 MFMA with fp32 accumulation; the state is fp32.
 *
 *   q, k            row t at q + t*stride_q (resp. k, stride_k): Hk*dk values,
 *                   head-major (head kh at offset kh*dk)                  io
 *   v               row t at v + t*stride_v: Hv*dv values, head-major      io
 *                   (q, k, v are normally views into gdn_conv1d_fwd's y with
 *                   stride Cq; strides are in elements, >= the row width,
 *                   multiples of 8 and at most GDN_MAX_ROW_STRIDE)
 *   a, b            [N, Hv]                io   (ignored when g_opt, beta_opt given)
 *   A_log, dt_bias  [Hv]                   fp32 (ignored when g_opt, beta_opt given)
 *   g_opt, beta_opt [N, Hv]                fp32 log-decay and write strength, or NULL
 *   state_in        [Ns, Hv, dk, dv]       fp32 or NULL (zeros)
 *   state_out       [Ns, Hv, dk, dv]       fp32 or NULL; may alias state_in
 *   o               [N, Hv, dv]            io   (must not alias the inputs)
 *   cu_seqlens      [Ns + 1]               int32 or NULL
 *   scale           <= 0 selects 1/sqrt(dk)
 *   workspace       device buffer (256-byte aligned) of at least
 *                   gdn_chunk_prefill_workspace_size() bytes, owned by the caller;
 *                   its contents need no initialisation and are scratch
 * Errors: dk != 128 or dv != 128 -> UNSUPPORTED; Hk < 1, Hv % Hk != 0, Ns < 1,
 * N < 0, a stride below its row width, above GDN_MAX_ROW_STRIDE or not a
 * multiple of 8, NULL required
 * pointers, a missing, unaligned or too small workspace -> INVALID_ARG.
 */
gdn_status_t gdn_chunk_prefill(const void* q, const void* k, const void* v, int64_t stride_q,
                               int64_t stride_k, int64_t stride_v, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const float* g_opt,
                               const float* beta_opt, const float* state_in, float* state_out,
                               void* o, const int32_t* cu_seqlens, int Ns, int64_t N, int Hk,
                               int Hv, int dk, int dv, float scale, int use_qk_l2norm,
                               void* workspace, size_t ws_bytes, gdn_dtype_t io, void* stream);

/*
 * gdn_chunk_prefill_noalloc -- gdn_chunk_prefill without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The workspace is a fixed
 * GDN_NOALLOC_SCRATCH_BYTES array in device memory that the library holds on each device
 * it runs on until the process ends; the call allocates nothing.  Every call on one
 * device shares that array, so calls that overlap on one device (concurrent streams or
 * host threads) race and must be serialised by the caller.  Results are those of
 * gdn_chunk_prefill (the same kernels run).
 *
 * Arguments and errors as for gdn_chunk_prefill, and INVALID_ARG when the workspace
 * the sizes need (gdn_chunk_prefill_workspace_size) exceeds GDN_NOALLOC_SCRATCH_BYTES
 * (about 6,700 tokens of one sequence at 16 key / 32 value heads, bf16 io).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status_t gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                                       int64_t stride_q, int64_t stride_k, int64_t stride_v,
                                       const void* a, const void* b, const float* A_log,
                                       const float* dt_bias, const float* g_opt,
                                       const float* beta_opt, const float* state_in,
                                       float* state_out, void* o, const int32_t* cu_seqlens,
                                       int Ns, int64_t N, int Hk, int Hv, int dk, int dv,
                                       float scale, int use_qk_l2norm, gdn_dtype_t io,
                                       void* stream);

/*
 * gdn_conv_chunk_prefill -- gdn_conv1d_fwd and gdn_chunk_prefill in one call: the conv
 * window + SiLU of the raw projection rows x is written to y and the chunked delta rule
 * runs on q, k, v read from y (q = y[:, 0 : Hk*dk], k = y[:, Hk*dk : 2*Hk*dk],
 * v = y[:, 2*Hk*dk :], row stride Cq = 2*Hk*dk + Hv*dv).  The results are those of the two
 * calls (y, conv_state_out, o and state_out bit for bit as gdn_conv1d_fwd would write y).
 * For bf16 io the conv is formed by the chunk kernels themselves, per chunk and key
 * head, so its memory traffic overlaps their arithmetic; for fp32 io the two calls run in
 * sequence.  (The conv and the chunked core are the steps of one linear-attention layer:
 * llm-arch-viz Qwen3.5-9B page, module tree of Qwen3_5GatedDeltaNet; HF Qwen3.5 docs
 * page, "Usage tips": prefill runs the chunked core.)
 *
 *   x                [N, Cq]          io      raw projection rows (q|k|v channels)
 *   conv_w           [Cq, K]          fp32
 *   conv_state_in    [Ns, K-1, Cq]    io      or NULL (zeros)
 *   conv_state_out   [Ns, K-1, Cq]    io      or NULL; may alias conv_state_in
 *   y                [N, Cq]          io      conv output, written (may not alias x)
 * All other arguments, the workspace (gdn_chunk_prefill_workspace_size) and the errors
 * as for gdn_chunk_prefill and gdn_conv1d_fwd.
 */
gdn_status_t gdn_conv_chunk_prefill(const void* x, const float* conv_w, const void* conv_state_in,
                                    void* conv_state_out, void* y, const void* a, const void* b,
                                    const float* A_log, const float* dt_bias, const float* g_opt,
                                    const float* beta_opt, const float* state_in,
                                    float* state_out, void* o, const int32_t* cu_seqlens, int Ns,
                                    int64_t N, int Hk, int Hv, int dk, int dv, int K, float scale,
                                    int use_qk_l2norm, void* workspace, size_t ws_bytes,
                                    gdn_dtype_t io, void* stream);

/*
 * gdn_prefill_layer -- the whole prefill layer in one call: gdn_conv1d_fwd, the chunked
 * delta rule and gdn_gated_rmsnorm, i.e. gdn_conv_chunk_prefill followed by
 *   y[t, h, :] = norm_w * o[t, h, :] / sqrt(mean(o[t, h, :]^2) + eps) * silu(z[t, h, :])
 * on the core output o as stored (rounded to io): the norm kernel runs after the core on the
 * same stream, so y equals the result of the separate calls bit for bit.  (The
 * conv, the delta rule and the z-gated norm are the steps of one linear-attention layer:
 * llm-arch-viz Qwen3.5-9B page, module tree of Qwen3_5GatedDeltaNet, with
 * Qwen3_5RMSNormGated 128.)
 *
 *   z                [N, Hv*dv]       io      gate input
 *   norm_w           [dv]             fp32    norm weight (applied directly)
 *   eps              >= 0 (the family's 1e-6)
 *   y                [N, Hv, dv]      io      norm output (may alias o)
 *   o                [N, Hv, dv]      io      core output, written
 * All other arguments, the workspace (gdn_chunk_prefill_workspace_size) and the errors as
 * for gdn_conv_chunk_prefill; also INVALID_ARG for NULL y, z or norm_w with N > 0, eps < 0,
 * or z, norm_w, y not 16-byte aligned.
 */
gdn_status_t gdn_prefill_layer(const void* x, const float* conv_w, const void* conv_state_in,
                               void* conv_state_out, void* y_conv, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const float* g_opt,
                               const float* beta_opt, const float* state_in, float* state_out,
                               void* o, const void* z, const float* norm_w, float eps, void* y,
                               const int32_t* cu_seqlens, int Ns, int64_t N, int Hk, int Hv,
                               int dk, int dv, int K, float scale, int use_qk_l2norm,
                               void* workspace, size_t ws_bytes, gdn_dtype_t io, void* stream);

/*
 * gdn_recurrent_step -- one decode token for each of B independent sequences,
 * updating the conv state and the recurrent state IN PLACE.
 * (KerasFormers Qwen page, "Generation": decode carries the per-layer conv
 * state and delta-rule recurrent state; HF Qwen3.5 docs page: the single-token
 * recurrence is memory-bandwidth-bound.)
 *
 * Per sequence: window = [conv_state (K-1 rows, oldest first); x],
 * y = silu(sum_j w[:, j] * window[j]), conv_state <- last K-1 rows of window,
 * then q, k, v = split(y) rounded to io, and for every value head one step of
 * the recurrence defined for gdn_chunk_prefill, o = scale * S^T q^.
 *
 *   x               [B, Cq]             io
 *   w               [Cq, K]             fp32
 *   conv_state      [B, K-1, Cq]        io    read and rewritten in place
 *   a, b            [B, Hv]             io    (ignored when g_opt, beta_opt given)
 *   A_log, dt_bias  [Hv]                fp32
 *   g_opt, beta_opt [B, Hv]             fp32 or NULL
 *   state           [B, Hv, dk, dv]     fp32  read and rewritten in place
 *   o               [B, Hv, dv]         io
 * with Cq = 2*Hk*dk + Hv*dv.
 * Errors: K != 4, dk != 128 or dv != 128 -> UNSUPPORTED; B < 0, Hk < 1,
 * Hv % Hk != 0, NULL required pointers -> INVALID_ARG.
 */
gdn_status_t gdn_recurrent_step(const void* x, const float* w, void* conv_state, const void* a,
                                const void* b, const float* A_log, const float* dt_bias,
                                const float* g_opt, const float* beta_opt, float* state, void* o,
                                int B, int Hk, int Hv, int dk, int dv, int K, float scale,
                                int use_qk_l2norm, gdn_dtype_t io, void* stream);

/*
 * gdn_recurrent_step_bf16_state -- gdn_recurrent_step with the recurrent state
 * stored as bf16 (llm-architectures-explained, Qwen3.5 397B-A17B page, "Modelled
 * costs": its cost model keeps the linear-attention state in BF16), which halves the
 * state traffic that bounds decode.  Each step reads the bf16 state, computes the step
 * in fp32 exactly as gdn_recurrent_step does (o from the updated fp32 state), and
 * writes the updated state back rounded to bf16 (round-to-nearest-even).
 *
 *   state           [B, Hv, dk, dv]     bf16  read and rewritten in place
 * All other arguments, layouts and errors as for gdn_recurrent_step.
 */
gdn_status_t gdn_recurrent_step_bf16_state(const void* x, const float* w, void* conv_state,
                                           const void* a, const void* b, const float* A_log,
                                           const float* dt_bias, const float* g_opt,
                                           const float* beta_opt, void* state, void* o, int B,
                                           int Hk, int Hv, int dk, int dv, int K, float scale,
                                           int use_qk_l2norm, gdn_dtype_t io, void* stream);

/*
 * gdn_recurrent_step_slots -- gdn_recurrent_step for a batch whose states live in
 * pools of n_slots entries: row b of x, a, b, g_opt, beta_opt and o belongs to the
 * sequence whose conv state and recurrent state are entry slots[b] of the pools.
 * (KerasFormers Qwen page, "Generation": each sequence carries its own per-layer conv
 * and recurrent state from step to step; a serving batch picks those states out of a
 * pool by index rather than copying them into a dense batch.)
 *
 *   conv_state_pool [n_slots, K-1, Cq]      io           entries slots[b] rewritten in place
 *   state_pool      [n_slots, Hv, dk, dv]   state_dtype  entries slots[b] rewritten in place
 *   state_dtype     GDN_F32, or GDN_BF16 (stored bf16, as gdn_recurrent_step_bf16_state)
 *   slots           [B] int32, device memory
 *   n_slots         >= 1
 * A row whose slot is negative or >= n_slots is padding: no pool entry is read or
 * written and its o row is set to zero.  Two rows with the same valid slot race on it
 * (the result is undefined, but no memory outside the pools and o is touched).
 * All other arguments, layouts and errors as for gdn_recurrent_step; also
 * INVALID_ARG for n_slots < 1, NULL slots with B > 0, or an unknown state_dtype.
 */
gdn_status_t gdn_recurrent_step_slots(const void* x, const float* w, void* conv_state_pool,
                                      const void* a, const void* b, const float* A_log,
                                      const float* dt_bias, const float* g_opt,
                                      const float* beta_opt, void* state_pool,
                                      gdn_dtype_t state_dtype, const int32_t* slots, int n_slots,
                                      void* o, int B, int Hk, int Hv, int dk, int dv, int K,
                                      float scale, int use_qk_l2norm, gdn_dtype_t io,
                                      void* stream);

/*
 * gdn_recurrent_step_norm -- the decode step and the z-gated RMSNorm of its output in one
 * launch: the same results as gdn_recurrent_step (or its bf16-state form) followed by
 * gdn_gated_rmsnorm on o (llm-arch-viz Qwen3.5-9B page, module tree: the linear-attention
 * block holds the gated norm, of width 128, next to its output projection; HF Qwen3.5 docs
 * page, "Usage tips": the single-token recurrence is bandwidth-bound, so o need not make a
 * round trip through memory).  o is normalised as the unfused call stores it (rounded
 * to io); the row sums of squares are accumulated in another order, so y may differ from
 * the two-call result by a rounding.
 *
 *   state_dtype     GDN_F32 (as gdn_recurrent_step) or GDN_BF16 (as
 *                   gdn_recurrent_step_bf16_state)
 *   z               [B, Hv, dv]   io
 *   norm_w          [dv]          fp32
 *   o_opt           [B, Hv, dv]   io, or NULL: o is then not written
 *   y               [B, Hv, dv]   io
 * Errors as for gdn_recurrent_step and gdn_gated_rmsnorm; also INVALID_ARG for NULL y, z
 * or norm_w, eps < 0 or an unknown state_dtype.
 */
gdn_status_t gdn_recurrent_step_norm(const void* x, const float* w, void* conv_state,
                                     const void* a, const void* b, const float* A_log,
                                     const float* dt_bias, const float* g_opt,
                                     const float* beta_opt, void* state, gdn_dtype_t state_dtype,
                                     const void* z, const float* norm_w, float eps, void* o_opt,
                                     void* y, int B, int Hk, int Hv, int dk, int dv, int K,
                                     float scale, int use_qk_l2norm, gdn_dtype_t io,
                                     void* stream);

/*
 * gdn_gated_rmsnorm -- z-gated RMSNorm over rows of D values:
 *   y[r, :] = w * o[r, :] / sqrt(mean(o[r, :]^2) + eps) * silu(z[r, :])
 * (llm-arch-viz Qwen3.5-9B page: Qwen3_5RMSNormGated with a [128] weight shared
 * by all value heads; KerasFormers Qwen3.5 page: norm_eps 1e-6.  The weight
 * multiplies directly and the gate is applied after normalisation.)
 *
 *   o   [rows, D]   io  (rows = tokens * Hv, D = dv; the core output [N, Hv, dv])
 *   z   [rows, D]   io  (the z projection [N, Hv*dv] viewed per head)
 *   w   [D]         fp32
 *   y   [rows, D]   io  (may alias o)
 * Errors: D != 128 -> UNSUPPORTED; rows < 0, NULL pointers with rows > 0,
 * eps < 0 -> INVALID_ARG.
 */
gdn_status_t gdn_gated_rmsnorm(const void* o, const void* z, const float* w, void* y,
                               int64_t rows, int D, float eps, gdn_dtype_t io, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
