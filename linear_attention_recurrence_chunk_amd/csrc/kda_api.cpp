// C ABI of libkda.so: argument validation (host only, before any HIP call),
// dispatch to the gfx950 kernels, and launch-error mapping.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {
hipError_t launch_prefill(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int H, int d, int chunk, bool is_bf16, void *o,
                          bool o_f32, float *sf, hipStream_t stream);
hipError_t launch_chunked(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int64_t total_tokens, int H, int d, int chunk,
                          bool is_bf16, void *o, bool o_f32, float *sf, void *ws,
                          hipStream_t stream);
size_t chunked_packet_bytes(int d, int chunk, bool is_bf16);
size_t static_scratch_bytes();
hipError_t static_scratch_ptr(void **ptr);
hipError_t launch_prefill_fused(const void *q_raw, const void *k_raw, const void *v,
                                const void *z, const float *A_log, const float *b_alpha,
                                const float *beta, const float *s0, const int32_t *cu,
                                int num_seqs, int64_t seq_len, int H, int d, int chunk,
                                bool is_bf16, bool norm, void *o, float *sf, hipStream_t stream);
hipError_t launch_front_end(const void *q_raw, const void *k_raw, const void *z, const float *A_log,
                            const float *b_alpha, void *q, void *k, float *g, int64_t rows, int H,
                            int d, bool is_bf16, hipStream_t stream);
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int64_t NH, int d,
                         bool is_bf16, const void *gate, const float *gw, float eps, void *out,
                         hipStream_t stream);
hipError_t launch_output_gate(const void *o_raw, const void *gate, const float *w, float eps,
                              void *out, int64_t rows, int dv, bool is_bf16, bool in_f32,
                              bool out_f32, hipStream_t stream);
hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             int64_t ntok, int C, float *state, void *y, bool is_bf16, int normd,
                             hipStream_t stream);
hipError_t launch_scan(const float *M, const float *St, const float *S0, float *S_in,
                       float *S_fin, int P, int H, int d, hipStream_t stream);
hipError_t launch_kcp_summaries(const void *k, const void *v, const float *g, const float *beta,
                                const int32_t *cu, int num_seqs, int64_t seq_len, int H, int d,
                                bool is_bf16, float *M, float *St, hipStream_t stream);
}  // namespace kda

namespace {

bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool head_size_ok(int32_t d) { return d == 32 || d == 64 || d == 128; }

bool chunk_ok(int32_t c) { return c == 64 || c == 128; }

// Which prefill algorithm runs (KDA_ALGO_AUTO resolved), or -1 when the
// combination is not supported.  The fused kernel advances the state every
// 64 tokens and keeps everything on chip; it takes bf16 at every head size and
// fp32 up to d = 64.  The two-pass path takes both block sizes of the notation
// table; its fp32 tiles of 128 x 128 do not fit in LDS, so fp32 with C = 128
// stops at d = 64.
int resolve_algo(kda_algo algo, int32_t d, int32_t chunk, kda_dtype dt)
{
    const bool fused_ok = chunk == 64 && (dt == KDA_BF16 || d <= 64);
    const bool two_ok = dt == KDA_BF16 || chunk == 64 || d <= 64;
    switch (algo) {
        case KDA_ALGO_AUTO: return fused_ok ? KDA_ALGO_FUSED : (two_ok ? KDA_ALGO_TWO_PASS : -1);
        case KDA_ALGO_FUSED: return fused_ok ? KDA_ALGO_FUSED : -1;
        case KDA_ALGO_TWO_PASS: return two_ok ? KDA_ALGO_TWO_PASS : -1;
        default: return -1;
    }
}

size_t workspace_bytes_for(int alg, int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d,
                           int32_t chunk, kda_dtype dt)
{
    if (alg != KDA_ALGO_TWO_PASS || num_seqs <= 0 || H <= 0) return 0;
    // one packet per (chunk slot, head); slots stay below ceil(total / C) + num_seqs
    const int64_t slots = (total_tokens + chunk - 1) / chunk + num_seqs;
    return (size_t)slots * (size_t)H * kda::chunked_packet_bytes(d, chunk, dt == KDA_BF16);
}

kda_status prefill_check(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *s0, const int32_t *cu,
                         int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                         int32_t d_v, int32_t chunk, kda_dtype dt, kda_algo algo, const void *o,
                         const float *sf, const void *ws, size_t ws_bytes, bool optional_io,
                         bool check_ws = true)
{
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || !head_size_ok(d_k)) return KDA_ERR_UNSUPPORTED;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int alg = resolve_algo(algo, d_k, chunk, dt);
    if (alg < 0) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_SHAPE;
    if (!cu && num_seqs > 0 && total_tokens % num_seqs != 0) return KDA_ERR_SHAPE;
    // grid of the state pass: up to 8 value slices per (sequence, head)
    if ((int64_t)num_seqs * H * 8 > INT32_MAX) return KDA_ERR_SHAPE;
    // the kernel forms row offsets as 24-bit products: one token's fp32 g row
    // (H d_k 4 bytes) must stay below 2^24 bytes
    if ((int64_t)H * d_k * 4 >= ((int64_t)1 << 24)) return KDA_ERR_SHAPE;
    if (total_tokens > 0) {
        if (!k || !g || !beta) return KDA_ERR_NULL;
        if (optional_io) {
            // o may be NULL when the final state is wanted (q is then unused); v
            // may be NULL for zero values
            if (o ? !q : !sf) return KDA_ERR_NULL;
        } else if (!q || !v || !o) {
            return KDA_ERR_NULL;
        }
    }
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(beta) ||
        misaligned(s0) || misaligned(cu) || misaligned(o) || misaligned(sf) || misaligned(ws))
        return KDA_ERR_ALIGN;
    const size_t need = workspace_bytes_for(alg, num_seqs, total_tokens, H, d_k, chunk, dt);
    if (check_ws && (ws_bytes < need || (need > 0 && !ws))) return KDA_ERR_WORKSPACE;
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_chunk_fwd_algo_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H,
                                         int32_t d_k, int32_t d_v, int32_t chunk_size,
                                         kda_dtype dtype, kda_algo algo)
{
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || d_k != d_v || !head_size_ok(d_k) ||
        !chunk_ok(chunk_size) || (dtype != KDA_F32 && dtype != KDA_BF16))
        return 0;
    const int alg = resolve_algo(algo, d_k, chunk_size, dtype);
    return alg < 0 ? 0 : workspace_bytes_for(alg, num_seqs, total_tokens, H, d_k, chunk_size, dtype);
}

size_t kda_chunk_fwd_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t H,
                                    int32_t d_k, int32_t d_v, int32_t chunk_size, kda_dtype dtype)
{
    return kda_chunk_fwd_algo_workspace_size(num_seqs, total_tokens, H, d_k, d_v, chunk_size,
                                             dtype, KDA_ALGO_AUTO);
}

kda_status kda_chunk_fwd_algo(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *initial_state,
                              const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                              kda_dtype dtype, kda_dtype o_dtype, kda_algo algo, void *o,
                              float *final_state, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    const kda_status st =
        prefill_check(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, H,
                      d_k, d_v, chunk_size, dtype, algo, o, final_state, workspace,
                      workspace_bytes, true);
    if (st != KDA_OK) return st;
    if (o_dtype != dtype && o_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return KDA_OK;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    const int alg = resolve_algo(algo, d_k, chunk_size, dtype);
    const hipError_t e =
        alg == KDA_ALGO_FUSED
            ? kda::launch_prefill(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, seq_len,
                                  H, d_k, 64, dtype == KDA_BF16, o, o_dtype == KDA_F32,
                                  final_state, stream)
            : kda::launch_chunked(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, seq_len,
                                  total_tokens, H, d_k, chunk_size, dtype == KDA_BF16, o,
                                  o_dtype == KDA_F32, final_state, workspace, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd_two_pass_static(const void *q, const void *k, const void *v,
                                         const float *g, const float *beta,
                                         const float *initial_state, const int32_t *cu_seqlens,
                                         int32_t num_seqs, int64_t total_tokens, int32_t H,
                                         int32_t d_k, int32_t d_v, int32_t chunk_size,
                                         kda_dtype dtype, kda_dtype o_dtype, void *o,
                                         float *final_state, hipStream_t stream)
{
    // host checks first (workspace checked against the static scratch below)
    const kda_status st =
        prefill_check(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, H,
                      d_k, d_v, chunk_size, dtype, KDA_ALGO_TWO_PASS, o, final_state, nullptr, 0,
                      true, false);
    if (st != KDA_OK) return st;
    if (o_dtype != dtype && o_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    const size_t need = workspace_bytes_for(KDA_ALGO_TWO_PASS, num_seqs, total_tokens, H, d_k,
                                            chunk_size, dtype);
    if (need > kda::static_scratch_bytes()) return KDA_ERR_TOO_LARGE;
    if (num_seqs == 0) return KDA_OK;
    void *ws = nullptr;
    if (kda::static_scratch_ptr(&ws) != hipSuccess) return KDA_ERR_HIP;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    const hipError_t e = kda::launch_chunked(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs,
                                             seq_len, total_tokens, H, d_k, chunk_size,
                                             dtype == KDA_BF16, o, o_dtype == KDA_F32, final_state,
                                             ws, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_chunk_fwd_static_scratch_bytes(void) { return kda::static_scratch_bytes(); }

kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                            kda_dtype dtype, kda_dtype o_dtype, void *o, float *final_state,
                            void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return kda_chunk_fwd_algo(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens,
                              H, d_k, d_v, chunk_size, dtype, o_dtype, KDA_ALGO_AUTO, o,
                              final_state, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state,
                         const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                         kda_dtype dtype, void *o, float *final_state, void *workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    return kda_chunk_fwd_ex(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens,
                            H, d_k, d_v, chunk_size, dtype, dtype, o, final_state, workspace,
                            workspace_bytes, stream);
}

kda_status kda_chunk_fwd_fused_ex(const void *q, const void *k, const void *v, const void *z,
                                  const float *A_log, const float *b_alpha, const float *beta,
                                  const float *initial_state, const int32_t *cu_seqlens,
                                  int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                                  int32_t d_v, int32_t chunk_size, kda_dtype dtype, int32_t fuse,
                                  void *o, float *final_state, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream)
{
    if (fuse != (KDA_FUSE_GATE | KDA_FUSE_L2NORM) && fuse != KDA_FUSE_GATE)
        return KDA_ERR_UNSUPPORTED;
    // z stands in for g in the common checks (same shape and alignment rule)
    const kda_status st =
        prefill_check(q, k, v, reinterpret_cast<const float *>(z), beta, initial_state,
                      cu_seqlens, num_seqs, total_tokens, H, d_k, d_v, chunk_size, dtype,
                      KDA_ALGO_FUSED, o, final_state, workspace, workspace_bytes, false);
    if (st != KDA_OK) return st;
    if (total_tokens > 0 && (!A_log || !b_alpha)) return KDA_ERR_NULL;
    if (misaligned(A_log) || misaligned(b_alpha)) return KDA_ERR_ALIGN;
    if (num_seqs == 0) return KDA_OK;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    const hipError_t e = kda::launch_prefill_fused(q, k, v, z, A_log, b_alpha, beta, initial_state,
                                                   cu_seqlens, num_seqs, seq_len, H, d_k, 64,
                                                   dtype == KDA_BF16, (fuse & KDA_FUSE_L2NORM) != 0,
                                                   o, final_state, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd_fused(const void *q_raw, const void *k_raw, const void *v, const void *z,
                               const float *A_log, const float *b_alpha, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                               int32_t d_v, int32_t chunk_size, kda_dtype dtype, void *o,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    return kda_chunk_fwd_fused_ex(q_raw, k_raw, v, z, A_log, b_alpha, beta, initial_state,
                                  cu_seqlens, num_seqs, total_tokens, H, d_k, d_v, chunk_size,
                                  dtype, KDA_FUSE_GATE | KDA_FUSE_L2NORM, o, final_state,
                                  workspace, workspace_bytes, stream);
}

kda_status kda_front_end(const void *q_raw, const void *k_raw, const void *z, const float *A_log,
                         const float *b_alpha, int64_t total_tokens, int32_t H, int32_t d,
                         kda_dtype dtype, void *q, void *k, float *g, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (total_tokens < 0 || H < 1 || d < 1) return KDA_ERR_SHAPE;
    if (!head_size_ok(d)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens == 0) return KDA_OK;
    if (!q_raw || !k_raw || !q || !k) return KDA_ERR_NULL;
    if (g && (!z || !A_log || !b_alpha)) return KDA_ERR_NULL;
    if (misaligned(q_raw) || misaligned(k_raw) || misaligned(z) || misaligned(A_log) ||
        misaligned(b_alpha) || misaligned(q) || misaligned(k) || misaligned(g))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_front_end(q_raw, k_raw, z, A_log, b_alpha, q, k, g,
                                               total_tokens * H, H, d, dtype == KDA_BF16, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_gate_ex(const void *o_raw, kda_dtype o_dtype, const void *gate,
                              const float *weight, float eps, void *out, kda_dtype out_dtype,
                              int64_t rows, int32_t d_v, kda_dtype dtype, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((o_dtype != dtype && o_dtype != KDA_F32) || (out_dtype != dtype && out_dtype != KDA_F32))
        return KDA_ERR_UNSUPPORTED;
    // in place only with equal element sizes
    if (out == o_raw && o_raw && o_dtype != out_dtype) return KDA_ERR_UNSUPPORTED;
    if (rows < 0 || d_v < 1 || !(eps >= 0.f)) return KDA_ERR_SHAPE;
    if (d_v != 32 && d_v != 64 && d_v != 128) return KDA_ERR_UNSUPPORTED;
    if (rows == 0) return KDA_OK;
    if (!o_raw || !gate || !weight || !out) return KDA_ERR_NULL;
    if (misaligned(o_raw) || misaligned(gate) || misaligned(weight) || misaligned(out))
        return KDA_ERR_ALIGN;
    const hipError_t e =
        kda::launch_output_gate(o_raw, gate, weight, eps, out, rows, d_v, dtype == KDA_BF16,
                                o_dtype == KDA_F32, out_dtype == KDA_F32, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_gate(const void *o_raw, const void *gate, const float *weight, float eps,
                           void *out, int64_t rows, int32_t d_v, kda_dtype dtype,
                           hipStream_t stream)
{
    return kda_output_gate_ex(o_raw, dtype, gate, weight, eps, out, dtype, rows, d_v, dtype, stream);
}

kda_status kda_short_conv_ex(const void *x, const float *weight, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_tokens, int32_t channels,
                             float *conv_state, void *y, kda_dtype dtype, int32_t l2norm_d,
                             hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || total_tokens < 0 || channels < 1) return KDA_ERR_SHAPE;
    if (channels % 4 != 0) return KDA_ERR_UNSUPPORTED;
    if (l2norm_d != 0 && (!head_size_ok(l2norm_d) || channels % l2norm_d != 0))
        return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_SHAPE;
    if (!cu_seqlens && num_seqs > 0 && total_tokens % num_seqs != 0) return KDA_ERR_SHAPE;
    // grid limit (65535 blocks of 64 tokens) and the 32-bit offsets of 19 rows
    if (total_tokens > (int64_t)65535 * 64 || (int64_t)channels * 19 * 4 >= ((int64_t)1 << 32))
        return KDA_ERR_SHAPE;
    if (num_seqs == 0) return KDA_OK;
    if (!weight || (total_tokens > 0 && (!x || !y))) return KDA_ERR_NULL;
    if (misaligned(x) || misaligned(weight) || misaligned(cu_seqlens) || misaligned(conv_state) ||
        misaligned(y))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_short_conv(x, weight, cu_seqlens, num_seqs, total_tokens,
                                                channels, conv_state, y, dtype == KDA_BF16,
                                                l2norm_d, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_short_conv(const void *x, const float *weight, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t channels,
                          float *conv_state, void *y, kda_dtype dtype, hipStream_t stream)
{
    return kda_short_conv_ex(x, weight, cu_seqlens, num_seqs, total_tokens, channels, conv_state,
                             y, dtype, 0, stream);
}

kda_status kda_state_compose(const float *M, const float *S_in, const float *S_tilde,
                             float *S_out, int64_t count, int32_t d_k, int32_t d_v,
                             hipStream_t stream)
{
    if (count < 0 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
    if (count == 0) return KDA_OK;
    if (!M || !S_in || !S_tilde || !S_out) return KDA_ERR_NULL;
    if (misaligned(M) || misaligned(S_in) || misaligned(S_tilde) || misaligned(S_out))
        return KDA_ERR_ALIGN;
    // one step of the segment scan (P = 1, the batch as heads): each workgroup
    // reads its blocks of S_in and S~ before it writes that block of S_out
    if (count * (d_k / 32) > INT32_MAX) return KDA_ERR_SHAPE;
    const hipError_t e = kda::launch_scan(M, S_tilde, S_in, nullptr, S_out, 1, (int)count, d_k,
                                          stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_kcp_summaries(const void *k, const void *v, const float *g, const float *beta,
                             const int32_t *cu_seqlens, int32_t num_segments,
                             int64_t total_tokens, int32_t H, int32_t d, int32_t chunk_size,
                             kda_dtype dtype, float *M, float *S_tilde, hipStream_t stream)
{
    // the same inputs as a state-only prefill of the segments (q unused)
    const kda_status st =
        prefill_check(nullptr, k, v, g, beta, nullptr, cu_seqlens, num_segments, total_tokens, H,
                      d, d, chunk_size, dtype, KDA_ALGO_FUSED, nullptr, S_tilde, nullptr, 0, true);
    if (st != KDA_OK) return st;
    if (chunk_size != 64) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)num_segments * H * 16 > INT32_MAX) return KDA_ERR_SHAPE;
    if (num_segments == 0) return KDA_OK;
    if (!M || !S_tilde || (total_tokens > 0 && !v)) return KDA_ERR_NULL;
    if (misaligned(M)) return KDA_ERR_ALIGN;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_segments;
    const hipError_t e = kda::launch_kcp_summaries(k, v, g, beta, cu_seqlens, num_segments, seq_len,
                                                   H, d, dtype == KDA_BF16, M, S_tilde, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_segment_scan(const float *M, const float *S_tilde, const float *S0, float *S_in,
                            float *S_final, int32_t P, int32_t H, int32_t d, hipStream_t stream)
{
    if (P < 0 || H < 1 || d < 1) return KDA_ERR_SHAPE;
    if (d != 32 && d != 64 && d != 128) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)H * (d / 32) > INT32_MAX) return KDA_ERR_SHAPE;
    if (!S_final || (P > 0 && (!M || !S_tilde))) return KDA_ERR_NULL;
    if (misaligned(M) || misaligned(S_tilde) || misaligned(S0) || misaligned(S_in) ||
        misaligned(S_final))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_scan(M, S_tilde, S0, S_in, S_final, P, H, d, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_step_decode(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype dtype, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || !head_size_ok(d_k)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(beta) ||
        misaligned(state) || misaligned(o))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_decode(q, k, v, g, beta, state, o, (int64_t)N * H, d_k,
                                            dtype == KDA_BF16, nullptr, nullptr, 0.f, nullptr,
                                            stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_step_decode_gated(const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, float *state, const void *gate,
                                 const float *weight, float eps, void *out, void *o_raw,
                                 int32_t N, int32_t H, int32_t d_k, int32_t d_v, kda_dtype dtype,
                                 hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H < 1 || d_k < 1 || d_v < 1 || !(eps >= 0.f)) return KDA_ERR_SHAPE;
    if (d_k != d_v || !head_size_ok(d_k)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !gate || !weight || !out) return KDA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(beta) ||
        misaligned(state) || misaligned(gate) || misaligned(weight) || misaligned(out) ||
        misaligned(o_raw))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_decode(q, k, v, g, beta, state, o_raw, (int64_t)N * H, d_k,
                                            dtype == KDA_BF16, gate, weight, eps, out, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char *kda_status_string(kda_status s)
{
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "negative or inconsistent sizes";
        case KDA_ERR_UNSUPPORTED: return "head size, chunk size or dtype not supported";
        case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace smaller than kda_chunk_fwd_workspace_size";
        case KDA_ERR_HIP: return "HIP launch error";
        case KDA_ERR_TOO_LARGE: return "sizes need more than the static scratch of the no-allocation call";
        default: return "unknown status";
    }
}

int32_t kda_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
