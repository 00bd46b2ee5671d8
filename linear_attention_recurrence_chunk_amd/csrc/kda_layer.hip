// Kernels for the steps around the KDA recurrence in a KDA layer, on gfx950:
//   - output epilogue: RMSNorm of the raw recurrent output times a sigmoid
//     output gate (page "Notations mathematiques": row o~_t "raw output,
//     before the gate", function table RMSNorm; "Kimi K3" model tables: RMSNorm
//     epsilon 1e-5, full-rank KDA gate);
//   - ShortConv: causal depthwise convolution with 4 taps and a streaming state
//     (function table "ShortConv", "Glossaire" entry "ShortConv", model table
//     "ShortConv kernel (KDA) 4");
//   - state composition for context-parallel segments: S_out = M S_in + S~
//     ("Glossaire", entry "KCP"; notation table rows M_t and S~).
// The first two are elementwise and bound by HBM bandwidth: coalesced accesses
// (16-byte lanes for the gate, 8-byte for ShortConv), fp32 arithmetic.  The
// composition is a batch of dense fp32 products on the matrix cores
// (v_mfma_f32_16x16x4_f32).
#include "kda_common.hpp"

namespace kda {

// ---------------------------------------------------------------------------
// Output epilogue.  One row = one (token, head): out = o~ / sqrt(mean(o~^2) +
// eps) * w * sigma(gate).  TI, TG, TO: the types of o~, the gate logits and
// out (an fp32 o~ and out are the fp32-output option for bf16 data).  A lane
// holds 16 bytes of the widest of them (8 bf16 or 4 fp32 elements); the LPR
// lanes of a row reduce the sum of squares with xor shuffles.
template <typename TI, typename TG, typename TO, int DV>
__global__ __launch_bounds__(256) void output_gate_kernel(const TI *__restrict__ o_raw,
                                                          const TG *__restrict__ gate,
                                                          const float *__restrict__ w, float eps,
                                                          TO *__restrict__ out, int64_t rows)
{
    constexpr int WMAX = sizeof(TI) > sizeof(TG) ? (sizeof(TI) > sizeof(TO) ? sizeof(TI) : sizeof(TO))
                                                 : (sizeof(TG) > sizeof(TO) ? sizeof(TG) : sizeof(TO));
    constexpr int EPL = 16 / WMAX;               // elements per lane
    constexpr int LPR = DV / EPL;                // lanes per row
    constexpr int RPB = 256 / LPR;               // rows per block and step
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row mapping");
    typedef TI vin __attribute__((ext_vector_type(EPL)));
    typedef TG vgt __attribute__((ext_vector_type(EPL)));
    typedef TO vec __attribute__((ext_vector_type(EPL)));
    const int t = threadIdx.x, lr = t % LPR, c0 = lr * EPL;
    float wv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) wv[e] = w[c0 + e];
    for (int64_t row = (int64_t)blockIdx.x * RPB + t / LPR; row < rows;
         row += (int64_t)gridDim.x * RPB) {
        const vin x = __builtin_nontemporal_load(reinterpret_cast<const vin *>(o_raw + row * DV + c0));
        const vgt gl = __builtin_nontemporal_load(reinterpret_cast<const vgt *>(gate + row * DV + c0));
        float xf[EPL], ss = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            xf[e] = to_f32(x[e]);
            ss += xf[e] * xf[e];
        }
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m);
        const float r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
        vec y;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-to_f32(gl[e])));
            y[e] = from_f32<TO>(xf[e] * r * wv[e] * sg);
        }
        // a plain store: measured faster than a non-temporal one here
        *reinterpret_cast<vec *>(out + row * DV + c0) = y;
    }
}

template <typename TI, typename TG, typename TO, int DV>
static hipError_t launch_output_gate_t(const void *o_raw, const void *gate, const float *w,
                                       float eps, void *out, int64_t rows, hipStream_t stream)
{
    constexpr int WMAX = sizeof(TI) > sizeof(TG) ? (sizeof(TI) > sizeof(TO) ? sizeof(TI) : sizeof(TO))
                                                 : (sizeof(TG) > sizeof(TO) ? sizeof(TG) : sizeof(TO));
    constexpr int RPB = 256 / (DV / (16 / WMAX));
    const int64_t need = (rows + RPB - 1) / RPB;
    // four workgroups per CU stepping through the rows: with the plain stores,
    // 6.5 TB/s on 786432 rows of 128 bf16, against 6.3 with 8192 workgroups
    const int64_t blocks = need < 1024 ? need : 1024;
    hipLaunchKernelGGL((output_gate_kernel<TI, TG, TO, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const TI *)o_raw, (const TG *)gate, w, eps, (TO *)out, rows);
    return hipGetLastError();
}

template <typename TI, typename TG, typename TO>
static hipError_t launch_output_gate_d(const void *o_raw, const void *gate, const float *w,
                                       float eps, void *out, int64_t rows, int dv,
                                       hipStream_t stream)
{
    switch (dv) {
        case 32: return launch_output_gate_t<TI, TG, TO, 32>(o_raw, gate, w, eps, out, rows, stream);
        case 64: return launch_output_gate_t<TI, TG, TO, 64>(o_raw, gate, w, eps, out, rows, stream);
        case 128: return launch_output_gate_t<TI, TG, TO, 128>(o_raw, gate, w, eps, out, rows, stream);
    }
    return hipErrorInvalidValue;
}

// is_bf16: the gate logits (and o~, out unless fp32 is asked for) are bf16.
hipError_t launch_output_gate(const void *o_raw, const void *gate, const float *w, float eps,
                              void *out, int64_t rows, int dv, bool is_bf16, bool in_f32,
                              bool out_f32, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
#define KDA_OG_ARGS o_raw, gate, w, eps, out, rows, dv, stream
    if (!is_bf16) return launch_output_gate_d<float, float, float>(KDA_OG_ARGS);
    if (in_f32)
        return out_f32 ? launch_output_gate_d<float, bf16, float>(KDA_OG_ARGS)
                       : launch_output_gate_d<float, bf16, bf16>(KDA_OG_ARGS);
    return out_f32 ? launch_output_gate_d<bf16, bf16, float>(KDA_OG_ARGS)
                   : launch_output_gate_d<bf16, bf16, bf16>(KDA_OG_ARGS);
#undef KDA_OG_ARGS
}

// ---------------------------------------------------------------------------
// ShortConv.  y_t[c] = sum_{i<4} w[c][i] x_{t-3+i}[c] inside each sequence;
// the inputs before a sequence start come from the streaming state
// [N][3][C] (oldest first, fp32) or are zero.  The sequence of a token is
// found by a binary search of cu_seqlens (or by division for equal lengths).
__device__ __forceinline__ int seq_of(int64_t tok, const int32_t *__restrict__ cu, int nseq,
                                      int64_t seq_len)
{
    if (!cu) return (int)(tok / seq_len);
    int lo = 0, hi = nseq - 1;           // last n with cu[n] <= tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= tok) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// A thread owns VEC = 4 consecutive channels and a run of RUN consecutive
// tokens; a wave covers 64 channel groups of the same tokens.  (Four channels
// rather than a 16-byte vector of bf16: the smaller register footprint lets
// twice as many waves stream, 6.5 TB/s against 5.8.)  When the run and the three inputs before it lie in one
// sequence (the common case), the thread loads those RUN + 3 rows at once and
// then writes its RUN outputs, so that every load is in flight together.
// Otherwise it slides a three-input window along the run, restarting it at
// each sequence start from the streaming state or from zeros.  Either way
// every input is read once per run, plus the three-row halo.
template <typename T, int VEC, int RUN>
__global__ __launch_bounds__(256) void short_conv_kernel(const T *__restrict__ x,
                                                         const float *__restrict__ w,
                                                         const int32_t *__restrict__ cu,
                                                         int nseq, int64_t seq_len,
                                                         int64_t ntok, int C,
                                                         const float *__restrict__ state,
                                                         T *__restrict__ y)
{
    typedef T vecT __attribute__((ext_vector_type(VEC)));
    typedef float vecF __attribute__((ext_vector_type(VEC)));
    const int ng = C / VEC;
    const int grp = blockIdx.x * 64 + (threadIdx.x & 63);
    if (grp >= ng) return;
    const int c0 = grp * VEC;
    const int64_t t0 = ((int64_t)blockIdx.y * 4 + (threadIdx.x >> 6)) * RUN;   // wave-uniform
    if (t0 >= ntok) return;
    const int64_t t1 = t0 + RUN < ntok ? t0 + RUN : ntok;
    float wt[VEC][4];                                // wt[e][i]: channel c0 + e, tap i
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const f32x4 ww = *reinterpret_cast<const f32x4 *>(w + (c0 + e) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) wt[e][i] = ww[i];
    }
    int n = seq_of(t0, cu, nseq, seq_len);
    int64_t bos = cu ? (int64_t)cu[n] : (int64_t)n * seq_len;
    int64_t eos = cu ? (int64_t)cu[n + 1] : bos + seq_len;

    if (t0 - 3 >= bos && t1 == t0 + RUN && t1 <= eos) {
        // rows t0 - 3 .. t1 - 1 from a wave-uniform base, 32-bit lane offsets
        const char *xb = reinterpret_cast<const char *>(x + (t0 - 3) * C);
        char *yb = reinterpret_cast<char *>(y + t0 * C);
        const uint32_t rowb = (uint32_t)C * (uint32_t)sizeof(T), cb = (uint32_t)c0 * (uint32_t)sizeof(T);
        vecT xs[RUN + 3];
#pragma unroll
        for (int j = 0; j < RUN + 3; ++j)
            xs[j] = *reinterpret_cast<const vecT *>(xb + (uint32_t)j * rowb + cb);
#pragma unroll
        for (int t = 0; t < RUN; ++t) {
            vecT out;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                out[e] = from_f32<T>(wt[e][0] * to_f32(xs[t][e]) + wt[e][1] * to_f32(xs[t + 1][e]) +
                                     wt[e][2] * to_f32(xs[t + 2][e]) + wt[e][3] * to_f32(xs[t + 3][e]));
            __builtin_nontemporal_store(out, reinterpret_cast<vecT *>(yb + (uint32_t)t * rowb + cb));
        }
        return;
    }

    // window[j]: input x_{t-3+j} for the next token t, j = 0..2
    vecF win[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t src = t0 - 3 + j;
        if (src >= bos) {
            const vecT xx = *reinterpret_cast<const vecT *>(x + src * C + c0);
#pragma unroll
            for (int e = 0; e < VEC; ++e) win[j][e] = to_f32(xx[e]);
        } else if (state) {
            win[j] = *reinterpret_cast<const vecF *>(state + ((int64_t)n * 3 + j + (t0 - bos)) * C + c0);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) win[j][e] = 0.f;
        }
    }
    for (int64_t t = t0; t < t1; ++t) {
        while (t >= eos) {                           // next sequence: restart the window
            ++n;
            bos = eos;
            eos = cu ? (int64_t)cu[n + 1] : bos + seq_len;
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                if (state) {
                    win[j] = *reinterpret_cast<const vecF *>(state + ((int64_t)n * 3 + j) * C + c0);
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) win[j][e] = 0.f;
                }
            }
        }
        const vecT xx = *reinterpret_cast<const vecT *>(x + t * C + c0);
        vecF cur;
#pragma unroll
        for (int e = 0; e < VEC; ++e) cur[e] = to_f32(xx[e]);
        vecT out;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            out[e] = from_f32<T>(wt[e][0] * win[0][e] + wt[e][1] * win[1][e] +
                                 wt[e][2] * win[2][e] + wt[e][3] * cur[e]);
        *reinterpret_cast<vecT *>(y + t * C + c0) = out;
        win[0] = win[1];
        win[1] = win[2];
        win[2] = cur;
    }
}

// The state after each sequence: its last three inputs, with the entering
// state in front when the sequence is shorter than three tokens.  One thread
// per (sequence, four channels) rewrites the three rows in increasing order,
// each reading only rows it has not yet written.
template <typename T>
__global__ __launch_bounds__(256) void short_conv_state_kernel(const T *__restrict__ x,
                                                               const int32_t *__restrict__ cu,
                                                               int nseq, int64_t seq_len, int C,
                                                               float *__restrict__ state)
{
    typedef T vec4 __attribute__((ext_vector_type(4)));
    const int cq = C / 4;
    for (int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x; item < (int64_t)nseq * cq;
         item += (int64_t)gridDim.x * 256) {
        const int n = (int)(item / cq);
        const int c0 = (int)(item % cq) * 4;
        const int64_t bos = cu ? (int64_t)cu[n] : (int64_t)n * seq_len;
        const int64_t eos = cu ? (int64_t)cu[n + 1] : bos + seq_len;
        const int64_t len = eos - bos;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            f32x4 v;
            const int64_t src = eos - 3 + j;
            if (src >= bos) {
                const vec4 xx = *reinterpret_cast<const vec4 *>(x + src * C + c0);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = to_f32(xx[e]);
            } else {
                v = *reinterpret_cast<const f32x4 *>(state + ((int64_t)n * 3 + j + len) * C + c0);
            }
            *reinterpret_cast<f32x4 *>(state + ((int64_t)n * 3 + j) * C + c0) = v;
        }
    }
}

template <typename T>
static hipError_t launch_short_conv_t(const void *x, const float *w, const int32_t *cu, int nseq,
                                      int64_t ntok, int C, float *state, void *y,
                                      hipStream_t stream)
{
    constexpr int RUN = 16, VEC = 4;     // channels must be a multiple of 4
    const int64_t seq_len = cu ? 0 : ntok / nseq;
    if (ntok > 0) {
        const int64_t gy = (ntok + 4 * RUN - 1) / (4 * RUN);
        if (gy > 65535) return hipErrorInvalidValue;   // grid y limit: 4.19 M tokens per call
        // the fast path's 32-bit offsets: RUN + 3 rows of C elements
        if ((int64_t)(RUN + 3) * C * (int64_t)sizeof(T) >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((C / VEC + 63) / 64), (unsigned)gy);
        hipLaunchKernelGGL((short_conv_kernel<T, VEC, RUN>), grid, dim3(256), 0, stream,
                           (const T *)x, w, cu, nseq, seq_len, ntok, C, state, (T *)y);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (state) {
        const int64_t sitems = (int64_t)nseq * (C / 4);
        const int64_t need = (sitems + 255) / 256;
        const int64_t blocks = need < 4096 ? need : 4096;
        hipLaunchKernelGGL((short_conv_state_kernel<T>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const T *)x, cu, nseq, seq_len, C, state);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             int64_t ntok, int C, float *state, void *y, bool is_bf16,
                             hipStream_t stream)
{
    if (nseq == 0) return hipSuccess;
    return is_bf16 ? launch_short_conv_t<bf16>(x, w, cu, nseq, ntok, C, state, y, stream)
                   : launch_short_conv_t<float>(x, w, cu, nseq, ntok, C, state, y, stream);
}

// ---------------------------------------------------------------------------
// State composition S_out[b] = M[b] S_in[b] + S~[b], fp32.  A wave computes a
// 16-row strip by 64 columns (four 16 x 16 tiles) of one product, K = DK in
// steps of 4: lane (n16, grp) supplies M[row n16][k + grp] and
// S_in[k + grp][column n16] to v_mfma_f32_16x16x4_f32 and ends with
// D[4 grp + i][n16].
template <int DK, int DV>
__global__ __launch_bounds__(256) void compose_kernel(const float *__restrict__ M,
                                                      const float *__restrict__ S_in,
                                                      const float *S_tilde, float *S_out,
                                                      int64_t count)
{
    constexpr int NRS = DK / 16;                    // row strips
    constexpr int NCB = (DV + 63) / 64;             // 64-column blocks
    constexpr int NCT = (DV < 64 ? DV : 64) / 16;   // 16-column tiles per block
    const int lane = threadIdx.x & 63, n16 = lane & 15, grp = lane >> 4;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t b = wave / (NRS * NCB);
    if (b >= count) return;
    const int rs = (int)((wave / NCB) % NRS), cb = (int)(wave % NCB);
    const float *Mb = M + b * DK * DK;
    const float *Sb = S_in + b * DK * DV;
    f32x4 acc[NCT];
#pragma unroll
    for (int j = 0; j < NCT; ++j) acc[j] = zero4();
#pragma unroll 4
    for (int k = 0; k < DK; k += 4) {
        const float a = Mb[(16 * rs + n16) * DK + k + grp];
#pragma unroll
        for (int j = 0; j < NCT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                a, Sb[(k + grp) * DV + 64 * cb + 16 * j + n16], acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = b * DK * DV + (int64_t)(16 * rs + 4 * grp + i) * DV + 64 * cb + 16 * j + n16;
            S_out[off] = acc[j][i] + S_tilde[off];
        }
}

template <int D>
static hipError_t launch_compose_t(const float *M, const float *S_in, const float *S_tilde,
                                   float *S_out, int64_t count, hipStream_t stream)
{
    constexpr int NRS = D / 16, NCB = (D + 63) / 64;
    const int64_t waves = count * NRS * NCB;
    hipLaunchKernelGGL((compose_kernel<D, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, M, S_in, S_tilde, S_out, count);
    return hipGetLastError();
}

hipError_t launch_compose(const float *M, const float *S_in, const float *S_tilde, float *S_out,
                          int64_t count, int d, hipStream_t stream)
{
    if (count == 0) return hipSuccess;
    switch (d) {
        case 32: return launch_compose_t<32>(M, S_in, S_tilde, S_out, count, stream);
        case 64: return launch_compose_t<64>(M, S_in, S_tilde, S_out, count, stream);
        case 128: return launch_compose_t<128>(M, S_in, S_tilde, S_out, count, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
