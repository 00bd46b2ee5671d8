/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The operation (page "Notations mathematiques", table "Attention et KDA"):
 * per sequence and head, a state S in R^{d_k x d_v} evolves token by token as
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     alpha_t = exp(g_t)           (per-key-channel retention, row "alpha_t"),
 *     o_t     = S_t^T q_t          (raw output before the output gate, row "o~_t").
 * q_t and k_t are expected L2-normalised (rows q_t, k_t), g_t in [g_min, 0] with
 * g_min = -5 (rows g_t, g_min) and beta_t in [0, 1] (row beta_t).
 *
 * kda_chunk_fwd evaluates this recurrence for prefill with the chunkwise form
 * ("Glossaire", entry "Chunkwise": serial across blocks, parallel inside a
 * block, exact), block size C from table "Dimensions du modele", row C (64 or
 * 128).  kda_step_decode advances every request by one token ("Glossaire",
 * entry "Decode").
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major (last index fastest), token-major and
 *     packed: q, k, g are [total_tokens][H][d_k]; v, o are [total_tokens][H][d_v];
 *     beta is [total_tokens][H]; states are [num_seqs][H][d_k][d_v].
 *   - q, k, v and o share one element type (kda_dtype): fp32 or bf16.  g, beta
 *     and every state are always fp32.
 *   - Every pointer except the host-side sizes is a DEVICE pointer and must be
 *     16-byte aligned.
 *   - Supported sizes: d_k == d_v in {32, 64, 128}; chunk_size in {64, 128}
 *     (fp32 prefill with chunk_size 128 stops at d = 64: its 128 x 128 fp32
 *     tiles do not fit in the 160 KB of LDS a workgroup may use).
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises: work is enqueued on `stream` and the call returns at once.
 *     Buffers must stay alive until the stream has passed the work.
 *   - Arguments are validated on the host before any HIP call; an invalid call
 *     returns a status and enqueues nothing.  A launch failure returns
 *     KDA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation.  Input value ranges (normalised keys, g and beta ranges,
 *     monotone cu_seqlens) are preconditions and are not checked on the device.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

/* element type of q, k, v and o */
typedef int32_t kda_dtype;
#define KDA_F32 0
#define KDA_BF16 1

/* status codes */
typedef int32_t kda_status;
#define KDA_OK 0
#define KDA_ERR_NULL 1        /* a required pointer is NULL                     */
#define KDA_ERR_SHAPE 2       /* negative or inconsistent sizes                 */
#define KDA_ERR_UNSUPPORTED 3 /* head size, chunk size or dtype not supported   */
#define KDA_ERR_ALIGN 4       /* a pointer is not 16-byte aligned               */
#define KDA_ERR_WORKSPACE 5   /* workspace smaller than the size asked for      */
#define KDA_ERR_HIP 6         /* the HIP runtime reported an error at launch    */
#define KDA_ERR_TOO_LARGE 7   /* sizes exceed the static scratch of the
                                 no-allocation call                              */

/*
 * Prefill algorithms (both evaluate the same chunkwise form, "Glossaire",
 * entries "Chunkwise" and "UT"; they differ in where the intra-chunk work runs):
 *   KDA_ALGO_FUSED     one persistent kernel per (sequence, head, value slice)
 *                      forms every intra-chunk quantity on chip, one chunk
 *                      ahead of the state pass, in 64-token chunks; no
 *                      workspace.  C = 64 only (bf16 at every head size, fp32
 *                      up to d = 64).
 *   KDA_ALGO_TWO_PASS  a chunk-parallel intra pass writes, for every (chunk,
 *                      head), the operands of the state pass (K o e^G, Q o e^G,
 *                      (K o e^{G_n - G})^T, (I + A)^-1 Diag(beta), the masked
 *                      intra attention and the chunk decay) to the workspace;
 *                      a persistent state pass then walks the chunks in
 *                      order.  C = 64 or 128 (the chunk the state advances by).
 *   KDA_ALGO_AUTO      KDA_ALGO_FUSED where it applies, else KDA_ALGO_TWO_PASS.
 */
typedef int32_t kda_algo;
#define KDA_ALGO_AUTO 0
#define KDA_ALGO_FUSED 1
#define KDA_ALGO_TWO_PASS 2

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes (0 means the
 * workspace pointer may be NULL).  Pure host function; 0 for unsupported
 * arguments.  kda_chunk_fwd_algo_workspace_size is the same for a given
 * algorithm: 0 for KDA_ALGO_FUSED, and for KDA_ALGO_TWO_PASS
 *     (ceil(total_tokens / C) + num_seqs) * H * P bytes,
 * P the size of one (chunk, head) packet: 3 C d + m * 256 * (C/16) (C/16 + 1) / 2
 * elements of the input type (m = 3 for bf16, 2 for fp32) plus 4 d bytes,
 * rounded up to 256 bytes (bf16, d = 128: 65,024 B at C = 64, 154,112 B at
 * C = 128).
 */
size_t kda_chunk_fwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H,
                                    int32_t d_k, int32_t d_v, int32_t chunk_size,
                                    kda_dtype dtype);
size_t kda_chunk_fwd_algo_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H,
                                         int32_t d_k, int32_t d_v, int32_t chunk_size,
                                         kda_dtype dtype, kda_algo algo);

/*
 * Chunkwise prefill over packed variable-length sequences.
 *
 *   q, k          [total_tokens][H][d_k]  dtype         queries, keys (L2-normalised)
 *   v             [total_tokens][H][d_v]  dtype         values
 *   g             [total_tokens][H][d_k]  fp32          log-decay, alpha = exp(g)
 *   beta          [total_tokens][H]       fp32          write strength
 *   initial_state [num_seqs][H][d_k][d_v] fp32 or NULL  state entering each
 *                                                       sequence (NULL = zeros,
 *                                                       the S~ convention of the
 *                                                       notation table)
 *   cu_seqlens    [num_seqs + 1] int32 (device) or NULL.  Sequence n covers
 *                 tokens [cu[n], cu[n+1]); cu[0] = 0, non-decreasing,
 *                 cu[num_seqs] = total_tokens; zero-length sequences are allowed
 *                 (their final state is their initial state).  NULL means
 *                 num_seqs sequences of equal length total_tokens / num_seqs
 *                 (total_tokens must then be a multiple of num_seqs).
 *                 The host never reads cu_seqlens.
 *   chunk_size    64 or 128 (table "Dimensions du modele", row C): the block the
 *                 state advances by.  The chunkwise form is exact for any block
 *                 size, so results differ between the two only by rounding.
 *                 kda_chunk_fwd runs KDA_ALGO_AUTO (see kda_chunk_fwd_algo).
 *   o             [total_tokens][H][d_v]  dtype         o_t = S_t^T q_t; must not
 *                                                       alias an input.  May be
 *                                                       NULL when final_state is
 *                                                       not: only the states are
 *                                                       computed and q is not read
 *                                                       (it may then be NULL too)
 *   final_state   [num_seqs][H][d_k][d_v] fp32 or NULL  state after each sequence;
 *                                                       may alias initial_state
 *   v may be NULL, standing for zero values: with initial_state = I (d_v = d_k)
 *   and o = NULL the final state is then the transition product of each
 *   sequence ("Glossaire", entry "KCP": the segment summary M).
 *   workspace     device scratch of at least kda_chunk_fwd_workspace_size(...)
 *                 bytes (may be NULL when that size is 0), else
 *                 KDA_ERR_WORKSPACE.  Its contents on entry do not matter; it
 *                 is overwritten.
 * Limits: H * d_k * 4 < 2^24 (one token's fp32 g row below 16 MiB), else
 * KDA_ERR_SHAPE.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                         kda_dtype dtype, void *o, float *final_state, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd with the element type of o given apart: o_dtype is dtype or
 * KDA_F32.  With bf16 inputs and o_dtype = KDA_F32, o = S_t^T q_t is written
 * in fp32 without the final rounding to bf16: the attention output is kept in
 * FP32 during training (page "Vecteurs, embeddings, espaces de
 * representation", section "La precision numerique : FP32, BF16, FP8, FP4":
 * the format table and the box "Limite importante").  The products inside
 * still take bf16 operands with fp32 accumulation.  Any other o_dtype:
 * KDA_ERR_UNSUPPORTED.  kda_chunk_fwd(...) is kda_chunk_fwd_ex(..., dtype,
 * dtype, ...); every other argument is as there.
 */
kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                            kda_dtype dtype, kda_dtype o_dtype, void *o, float *final_state,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_fwd_ex with the algorithm chosen by the caller (kda_algo above).
 * The workspace must hold kda_chunk_fwd_algo_workspace_size(..., algo) bytes.
 * An algorithm that does not take these sizes, types or chunk size returns
 * KDA_ERR_UNSUPPORTED.  kda_chunk_fwd_ex(...) is kda_chunk_fwd_algo(...,
 * KDA_ALGO_AUTO, ...).  The two-pass path enqueues two kernels on `stream`.
 */
kda_status kda_chunk_fwd_algo(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *initial_state,
                              const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                              kda_dtype dtype, kda_dtype o_dtype, kda_algo algo, void *o,
                              float *final_state, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * The two-pass prefill (KDA_ALGO_TWO_PASS) for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Instead of a caller workspace it uses a static device
 * buffer of kda_chunk_fwd_static_scratch_bytes() bytes (256 MiB) inside the
 * library; it calls no hipMalloc, hipFree or allocating library routine.
 *   - Sizes whose kda_chunk_fwd_algo_workspace_size(..., KDA_ALGO_TWO_PASS)
 *     exceeds that buffer return KDA_ERR_TOO_LARGE before any HIP call (at
 *     H = 96, d = 128, bf16, C = 64: about 2,600 tokens of one sequence).
 *   - Each GPU the library runs on holds one such buffer until the process
 *     ends.  Every call on a GPU shares it: calls that overlap on one GPU (two
 *     streams, or two host threads) race and must be serialised by the caller.
 *     The buffer needs no clearing between calls.
 *   - Everything else (arguments, layouts, results, errors, o_dtype) is as in
 *     kda_chunk_fwd_algo with KDA_ALGO_TWO_PASS; results equal that call's
 *     bit for bit.
 */
kda_status kda_chunk_fwd_two_pass_static(const void *q, const void *k, const void *v,
                                         const float *g, const float *beta,
                                         const float *initial_state, const int32_t *cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens, int32_t H,
                                         int32_t d_k, int32_t d_v, int32_t chunk_size,
                                         kda_dtype dtype, kda_dtype o_dtype, void *o,
                                         float *final_state, hipStream_t stream);
size_t kda_chunk_fwd_static_scratch_bytes(void);

/*
 * One decode step: each of N requests appends one token and advances its own
 * state in place ("Glossaire", entry "Decode": bandwidth bound).
 *
 *   q, k   [N][H][d_k] dtype;  v [N][H][d_v] dtype;  g [N][H][d_k] fp32;
 *   beta   [N][H] fp32;
 *   state  [N][H][d_k][d_v] fp32, read and overwritten with S_t;
 *   o      [N][H][d_v] dtype, o_t = S_t^T q_t; must not alias any input.
 */
kda_status kda_step_decode(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype dtype, hipStream_t stream);

/*
 * kda_step_decode with the layer's output epilogue fused in: the step as in
 * kda_step_decode, then, per (request, head), over the d_v columns of o
 *     out = o / sqrt(mean(o^2) + eps) * weight * sigma(gate)
 * (page "Notations mathematiques": row o~_t "raw output, before the gate" and
 * the function table's RMSNorm; "Kimi K3" model tables: epsilon 1e-5 and the
 * full-rank sigmoid output gate) -- the same epilogue as kda_output_gate, on
 * the fp32 o before any rounding, with no separate pass over o.
 *   gate    [N][H][d_v] dtype   gate logits
 *   weight  [d_v] fp32          RMSNorm weight shared by the heads
 *   eps     >= 0
 *   out     [N][H][d_v] dtype   gated output; must not alias any input
 *   o_raw   [N][H][d_v] dtype or NULL: the raw o as well, when given
 * Every other argument, layout and error is as in kda_step_decode.
 */
kda_status kda_step_decode_gated(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, float *state, const void *gate,
                                 const float *weight, float eps, void *out, void *o_raw,
                                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 hipStream_t stream);

/*
 * Chunkwise prefill with the layer's front end fused in: the same operation as
 * kda_chunk_fwd, on inputs taken one step earlier in the KDA layer.
 *   - q = L2Norm(q_raw), k = L2Norm(k_raw) per (token, head) over d_k (page
 *     "Notations mathematiques": rows q_t, k_t "L2-normalised" and the
 *     function table's L2Norm(x) = x / ||x||_2; a zero row stays zero);
 *   - g = g_min sigma(e^{A_h} (z + b_alpha^h)), g_min = -5 ("Glossaire", entry
 *     "Decroissance bornee"; notation table rows A_h, b_alpha^h, z_t).  The bias
 *     is added to the logit before the per-head scale e^{A_h}.
 *
 *   q_raw, k_raw  [total_tokens][H][d_k]  dtype   unnormalised queries, keys
 *   z             [total_tokens][H][d_k]  dtype   decay logits (replace g)
 *   A_log         [H]        fp32                  per-head log scale A_h
 *   b_alpha       [H][d_k]   fp32                  per-head decay bias
 * All other arguments, the layouts, sizes, ownership, aliasing and errors are
 * those of kda_chunk_fwd; this call runs KDA_ALGO_FUSED, so chunk_size must
 * be 64.  The g stream shrinks from 4 to 2 bytes per element (bf16 logits),
 * and no separate normalisation pass is needed.
 */
kda_status kda_chunk_fwd_fused(const void *q_raw, const void *k_raw, const void *v, const void *z,
                               const float *A_log, const float *b_alpha, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                               int32_t d_v, int32_t chunk_size, kda_dtype dtype, void *o,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Steps of the front end done inside the prefill (kda_chunk_fwd_fused_ex). */
#define KDA_FUSE_GATE 1   /* z, A_log, b_alpha replace g (the bounded gate) */
#define KDA_FUSE_L2NORM 2 /* q, k arrive unnormalised (L2Norm in the kernel) */

/*
 * kda_chunk_fwd_fused with a choice of the front-end steps done in the
 * kernel: fuse = KDA_FUSE_GATE | KDA_FUSE_L2NORM is kda_chunk_fwd_fused;
 * fuse = KDA_FUSE_GATE takes q and k already L2-normalised (for instance by
 * kda_front_end with g = NULL) and fuses only the bounded gate.  Any other
 * value: KDA_ERR_UNSUPPORTED.  The row norms are reductions across the
 * channels that the kernel's elementwise layout spreads over four waves; in
 * the kernel they cost more than the separate normalisation pass, while the
 * gate, elementwise per channel, costs less in the kernel than its fp32 g
 * stream does outside.  Arguments, layouts and errors as kda_chunk_fwd_fused.
 */
kda_status kda_chunk_fwd_fused_ex(const void *q, const void *k, const void *v, const void *z,
                                  const float *A_log, const float *b_alpha, const float *beta,
                                  const float *initial_state, const int32_t *cu_seqlens,
                                  int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                                  int32_t d_v, int32_t chunk_size, kda_dtype dtype, int32_t fuse,
                                  void *o, float *final_state, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * The layer's front end as a pass of its own (the unfused alternative to
 * kda_chunk_fwd_fused): per (token, head) row of d elements
 *     q = L2Norm(q_raw), k = L2Norm(k_raw)   (a zero row stays zero)
 *     g = g_min sigma(e^{A_h} (z + b_alpha^h)), g_min = -5    when g != NULL
 * (page "Notations mathematiques", function table "L2Norm" and rows q_t, k_t;
 * "Glossaire", entry "Decroissance bornee"; notation table rows A_h,
 * b_alpha^h, z_t).  Bound by HBM bandwidth.
 *   q_raw, k_raw, z  [total_tokens][H][d] dtype     (z may be NULL if g is)
 *   A_log [H], b_alpha [H][d] fp32                   (NULL if g is)
 *   q, k  [total_tokens][H][d] dtype out; g [total_tokens][H][d] fp32 out or NULL
 * d in {32, 64, 128}.  Outputs must not alias inputs.  One launch on `stream`.
 */
kda_status kda_front_end(const void *q_raw, const void *k_raw, const void *z, const float *A_log,
                         const float *b_alpha, int64_t total_tokens, int32_t H, int32_t d,
                         kda_dtype dtype, void *q, void *k, float *g, hipStream_t stream);

/*
 * Output epilogue of the KDA layer: out = RMSNorm(o~) (.) sigma(gate), per row
 * (token, head) over d_v, RMSNorm(x) = x / sqrt(mean(x^2) + eps) (.) weight
 * (page "Notations mathematiques": row o~_t "raw output, before the gate" and
 * the function table's RMSNorm; "Kimi K3" model tables: epsilon 1e-5 and a
 * full-rank KDA output gate, i.e. one gate logit per output channel).
 *
 *   o_raw  [rows][d_v] dtype   the raw output (the o of kda_chunk_fwd or
 *                              kda_step_decode, rows = tokens * H)
 *   gate   [rows][d_v] dtype   gate logits
 *   weight [d_v] fp32          RMSNorm weight, shared by the heads
 *   eps    >= 0                RMSNorm epsilon
 *   out    [rows][d_v] dtype   may alias o_raw (each element is read before
 *                              it is written by the same thread)
 * d_v in {32, 64, 128}.  Device pointers, 16-byte aligned; host validation as
 * for the other calls.
 */
kda_status kda_output_gate(const void *o_raw, const void *gate, const float *weight, float eps,
                           void *out, int64_t rows, int32_t d_v, kda_dtype dtype,
                           hipStream_t stream);

/*
 * kda_output_gate with the element types of o_raw and out given apart, each
 * dtype or KDA_F32 (the gate logits are dtype): the epilogue of an fp32
 * attention output (kda_chunk_fwd_ex with o_dtype = KDA_F32), with a bf16 or
 * fp32 result.  out may alias o_raw only when o_dtype == out_dtype
 * (KDA_ERR_UNSUPPORTED for out == o_raw otherwise).  kda_output_gate(...) is
 * kda_output_gate_ex(o_raw, dtype, gate, weight, eps, out, dtype, rows, d_v,
 * dtype, stream).
 */
kda_status kda_output_gate_ex(const void *o_raw, kda_dtype o_dtype, const void *gate,
                              const float *weight, float eps, void *out, kda_dtype out_dtype,
                              int64_t rows, int32_t d_v, kda_dtype dtype, hipStream_t stream);

/*
 * ShortConv: causal depthwise convolution with 4 taps over each packed
 * sequence ("Notations mathematiques", function table "ShortConv"; "Glossaire",
 * entry "ShortConv"; "Kimi K3" model table: kernel 4).  No activation.
 *     y_t[c] = sum_{i=0..3} weight[c][i] * x_{t-3+i}[c],
 * where inputs before the sequence start come from conv_state or are zero.
 *
 *   x           [total_tokens][channels] dtype
 *   weight      [channels][4] fp32     tap 3 multiplies the current token
 *   cu_seqlens  as in kda_chunk_fwd (device, or NULL for equal lengths)
 *   conv_state  [num_seqs][3][channels] fp32 or NULL.  In: the three inputs
 *               before each sequence, oldest first.  Out: the last three
 *               inputs of each sequence (the entering ones kept in front when
 *               a sequence is shorter than three tokens).  NULL: zero history,
 *               nothing written.  A decode step is a call with num_seqs
 *               sequences of one token each.
 *   y           [total_tokens][channels] dtype; must not alias x.
 * channels must be a multiple of 4; total_tokens <= 65535 * 64 and
 * channels * 76 < 2^32 (else KDA_ERR_SHAPE).  Two launches on `stream` (the
 * output, then the state update).
 */
kda_status kda_short_conv(const void *x, const float *weight, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t channels,
                          float *conv_state, void *y, kda_dtype dtype, hipStream_t stream);

/*
 * kda_short_conv, then, with l2norm_d > 0, each output row of l2norm_d
 * channels (one head) L2-normalised (function table "L2Norm"; a zero row stays
 * zero; page "Notations mathematiques": q_t and k_t are the L2-normalised
 * outputs of the ShortConv of their projections): the layer's q and k in one
 * pass over the projections, with no separate normalisation pass.  The
 * streaming state holds the convolution's inputs as in kda_short_conv.
 * l2norm_d in {0, 32, 64, 128}, a divisor of channels (else
 * KDA_ERR_UNSUPPORTED).  Everything else as kda_short_conv.
 */
kda_status kda_short_conv_ex(const void *x, const float *weight, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t channels,
                             float *conv_state, void *y, kda_dtype dtype, int32_t l2norm_d,
                             hipStream_t stream);

/*
 * Composition of context-parallel segment summaries ("Glossaire", entry
 * "KCP"; notation table rows M_t and S~): for b < count,
 *     S_out[b] = M[b] S_in[b] + S_tilde[b]      (fp32 throughout).
 * M[b] is the product of a segment's transitions, obtained with kda_chunk_fwd
 * by running the segment from initial_state = I with v = 0 (so d_v = d_k);
 * S_tilde[b] is the segment's final state from S = 0.
 *
 *   M        [count][d_k][d_k]     S_in, S_tilde, S_out   [count][d_k][d_v]
 * d_k == d_v in {32, 64, 128}.  S_out may alias S_in or S_tilde, not M.
 * It runs as one step of kda_segment_scan (P = 1, the batch as its heads).
 */
kda_status kda_state_compose(const float *M, const float *S_in, const float *S_tilde,
                             float *S_out, int64_t count, int32_t d_k, int32_t d_v,
                             hipStream_t stream);

/*
 * Both summaries of each of num_segments packed segments, for all heads, in
 * one launch ("Glossaire", entry "KCP"; notation table rows M_t and S~):
 *     M[s]       = the product of segment s's transitions, M_T ... M_1 with
 *                  M_t = (I - beta_t k_t k_t^T) Diag(alpha_t): the final state
 *                  of the segment run from S = I with zero values;
 *     S_tilde[s] = the segment's final state from S = 0 with its values.
 * A workgroup runs one 64-column slice of one of the two: the slices of M and
 * of S~ of a head read the same k, g, beta, which the two runs share through
 * the cache instead of two launches reading them.
 *   k, v, g, beta, cu_seqlens   as in kda_chunk_fwd, the segments as sequences
 *   M, S_tilde  [num_segments][H][d][d] fp32 out
 * d in {32, 64, 128} for bf16, {32, 64} for fp32 (else KDA_ERR_UNSUPPORTED;
 * two state-only kda_chunk_fwd calls give the summaries there); chunk_size
 * 64.  Other errors as kda_chunk_fwd.  One launch on `stream`.
 */
kda_status kda_kcp_summaries(const void *k, const void *v, const float *g, const float *beta,
                             const int32_t *cu_seqlens, int32_t num_segments,
                             int64_t total_tokens, int32_t H, int32_t d, int32_t chunk_size,
                             kda_dtype dtype, float *M, float *S_tilde, hipStream_t stream);

/*
 * The whole scan over the summaries of P consecutive segments of each head,
 * in one launch ("Glossaire", entry "KCP": the summaries compose
 * associatively; notation table rows M_t and S~):
 *     S_in[0] = S0,  S_in[r + 1] = M[r] S_in[r] + S_tilde[r],  S_final = S_in[P]
 * in fp32.  (M[r], S_tilde[r]) are segment r's summaries as described for
 * kda_state_compose, for all heads at once.
 *   M, S_tilde  [P][H][d][d] fp32 (may be NULL when P == 0)
 *   S0          [H][d][d] fp32, or NULL for a zero initial state
 *   S_in        [P][H][d][d] fp32 out, the state entering each segment, or
 *               NULL when not wanted
 *   S_final     [H][d][d] fp32 out; may alias S0, must not alias the others
 * d in {32, 64, 128} (d_k == d_v).  One workgroup per (head, 32 columns) runs
 * the P steps in order; one launch on `stream`.
 */
kda_status kda_segment_scan(const float *M, const float *S_tilde, const float *S0, float *S_in,
                            float *S_final, int32_t P, int32_t H, int32_t d, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char *kda_status_string(kda_status status);

/* KDA_ABI_VERSION of the built library. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
