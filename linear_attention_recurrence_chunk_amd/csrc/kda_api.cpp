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
hipError_t launch_prefill_fused(const void *q_raw, const void *k_raw, const void *v,
                                const void *z, const float *A_log, const float *b_alpha,
                                const float *beta, const float *s0, const int32_t *cu,
                                int num_seqs, int64_t seq_len, int H, int d, int chunk,
                                bool is_bf16, void *o, float *sf, hipStream_t stream);
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int64_t NH, int d,
                         bool is_bf16, hipStream_t stream);
hipError_t launch_output_gate(const void *o_raw, const void *gate, const float *w, float eps,
                              void *out, int64_t rows, int dv, bool is_bf16, bool in_f32,
                              bool out_f32, hipStream_t stream);
hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             int64_t ntok, int C, float *state, void *y, bool is_bf16,
                             hipStream_t stream);
hipError_t launch_compose(const float *M, const float *S_in, const float *S_tilde, float *S_out,
                          int64_t count, int d, hipStream_t stream);
}  // namespace kda

namespace {

bool misaligned(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool head_size_ok(int32_t d, kda_dtype dt, bool prefill)
{
    if (dt == KDA_BF16) return d == 32 || d == 64 || d == 128;
    if (dt == KDA_F32) return prefill ? (d == 32 || d == 64) : (d == 32 || d == 64 || d == 128);
    return false;
}

// Both block sizes of the notation table are accepted.  The kernel advances
// the state every 64 tokens for either value: the chunkwise form is exact for
// any block size, so the result is the same up to rounding, and on this
// design a 128-token intra-chunk block only adds work per token.
bool chunk_ok(int32_t c) { return c == 64 || c == 128; }

kda_status prefill_check(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *s0, const int32_t *cu,
                         int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                         int32_t d_v, int32_t chunk, kda_dtype dt, const void *o,
                         const float *sf, const void *ws, size_t ws_bytes, bool optional_io)
{
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || !head_size_ok(d_k, dt, true)) return KDA_ERR_UNSUPPORTED;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_SHAPE;
    if (!cu && num_seqs > 0 && total_tokens % num_seqs != 0) return KDA_ERR_SHAPE;
    if ((int64_t)num_seqs * H * 2 > INT32_MAX) return KDA_ERR_SHAPE;
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
    const size_t need =
        kda_chunk_fwd_workspace_size(num_seqs, total_tokens, H, d_k, d_v, chunk, dt);
    if (ws_bytes < need || (need > 0 && !ws)) return KDA_ERR_WORKSPACE;
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_chunk_fwd_workspace_size(int32_t, int64_t, int32_t, int32_t, int32_t, int32_t,
                                    kda_dtype)
{
    return 0;  // the fused kernel keeps every intermediate on chip
}

kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state,
                            const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t H, int32_t d_k, int32_t d_v, int32_t chunk_size,
                            kda_dtype dtype, kda_dtype o_dtype, void *o, float *final_state,
                            void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const kda_status st =
        prefill_check(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, H,
                      d_k, d_v, chunk_size, dtype, o, final_state, workspace, workspace_bytes, true);
    if (st != KDA_OK) return st;
    if (o_dtype != dtype && o_dtype != KDA_F32) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return KDA_OK;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    const hipError_t e = kda::launch_prefill(q, k, v, g, beta, initial_state, cu_seqlens,
                                             num_seqs, seq_len, H, d_k, 64, dtype == KDA_BF16, o,
                                             o_dtype == KDA_F32, final_state, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
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

kda_status kda_chunk_fwd_fused(const void *q_raw, const void *k_raw, const void *v, const void *z,
                               const float *A_log, const float *b_alpha, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_tokens, int32_t H, int32_t d_k,
                               int32_t d_v, int32_t chunk_size, kda_dtype dtype, void *o,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    // z stands in for g in the common checks (same shape and alignment rule)
    const kda_status st =
        prefill_check(q_raw, k_raw, v, reinterpret_cast<const float *>(z), beta, initial_state,
                      cu_seqlens, num_seqs, total_tokens, H, d_k, d_v, chunk_size, dtype, o,
                      final_state, workspace, workspace_bytes, false);
    if (st != KDA_OK) return st;
    if (total_tokens > 0 && (!A_log || !b_alpha)) return KDA_ERR_NULL;
    if (misaligned(A_log) || misaligned(b_alpha)) return KDA_ERR_ALIGN;
    if (num_seqs == 0) return KDA_OK;
    const int64_t seq_len = cu_seqlens ? 0 : total_tokens / num_seqs;
    const hipError_t e = kda::launch_prefill_fused(q_raw, k_raw, v, z, A_log, b_alpha, beta,
                                                   initial_state, cu_seqlens, num_seqs, seq_len,
                                                   H, d_k, 64, dtype == KDA_BF16, o, final_state,
                                                   stream);
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

kda_status kda_short_conv(const void *x, const float *weight, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_tokens, int32_t channels,
                          float *conv_state, void *y, kda_dtype dtype, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (num_seqs < 0 || total_tokens < 0 || channels < 1) return KDA_ERR_SHAPE;
    if (channels % 4 != 0) return KDA_ERR_UNSUPPORTED;
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
                                                channels, conv_state, y, dtype == KDA_BF16, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
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
    const hipError_t e = kda::launch_compose(M, S_in, S_tilde, S_out, count, d_k, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_step_decode(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype dtype, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    if (d_k != d_v || !head_size_ok(d_k, dtype, false)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(g) || misaligned(beta) ||
        misaligned(state) || misaligned(o))
        return KDA_ERR_ALIGN;
    const hipError_t e = kda::launch_decode(q, k, v, g, beta, state, o, (int64_t)N * H, d_k,
                                            dtype == KDA_BF16, stream);
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
        default: return "unknown status";
    }
}

int32_t kda_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
