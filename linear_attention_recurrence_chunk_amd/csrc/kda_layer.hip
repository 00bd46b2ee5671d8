// Kernels for the steps around the KDA recurrence in a KDA layer, on gfx950:
//   - output epilogue: RMSNorm of the raw recurrent output times a sigmoid
//     output gate (page "Notations mathematiques": row o~_t "raw output,
//     before the gate", function table RMSNorm; "Kimi K3" model tables: RMSNorm
//     epsilon 1e-5, full-rank KDA gate);
//   - ShortConv: causal depthwise convolution with 4 taps and a streaming state
//     (function table "ShortConv", "Glossaire" entry "ShortConv", model table
//     "ShortConv kernel (KDA) 4");
//   - the front end, unfused: L2Norm of q and k and the bounded gate
//     ("Glossaire", entry "Decroissance bornee"; function table "L2Norm");
//   - state composition for context-parallel segments: S_out = M S_in + S~
//     ("Glossaire", entry "KCP"; notation table rows M_t and S~), the whole
//     scan over P segments in one launch (one step over a batch is P = 1).
// The first three are elementwise and bound by HBM bandwidth: coalesced
// accesses (16-byte lanes for the gate and the front end, 8-byte for
// ShortConv), fp32 arithmetic.  The
// composition is a chain of dense fp32 products on the matrix cores
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
// Front end of the recurrence, unfused: L2Norm of the q and k rows (function
// table "L2Norm"; a zero row maps to zero) and, when asked for, the bounded
// gate's log-decay g = g_min sigma(e^{A_h} (z + b_alpha^h)) ("Glossaire",
// entry "Decroissance bornee", with the per-head bias of the notation table),
// g_min = -5.  One row = one (token, head); a lane holds 16 bytes of q and of
// k, the LPR lanes of a row reduce the sums of squares with xor shuffles.
template <typename T, int D, bool GATE>
__global__ __launch_bounds__(256) void front_end_kernel(const T *__restrict__ q_raw,
                                                        const T *__restrict__ k_raw,
                                                        const T *__restrict__ z,
                                                        const float *__restrict__ A_log,
                                                        const float *__restrict__ b_alpha,
                                                        T *__restrict__ q, T *__restrict__ k,
                                                        float *__restrict__ g, int64_t rows, int H)
{
    constexpr int EPL = 16 / (int)sizeof(T);     // elements per lane
    constexpr int LPR = D / EPL;                 // lanes per row
    constexpr int RPB = 256 / LPR;               // rows per block and step
    constexpr int U = 1;                         // rows per thread and step (2 measured slower)
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row mapping");
    typedef T vec __attribute__((ext_vector_type(EPL)));
    const int t = threadIdx.x, c0 = (t % LPR) * EPL;
    const int64_t step = (int64_t)gridDim.x * RPB;          // between a thread's rows
    int64_t row = (int64_t)blockIdx.x * RPB + t / LPR;
    // the head of a row, advanced without a 64-bit division per row
    int h = (int)(row % H);
    const int hstep = (int)(step % H);
    const auto adv = [&](int x) { x += hstep; return x >= H ? x - H : x; };
    for (; row < rows; row += U * step) {
        vec xq[U], xk[U], xz[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row + u * step;
            if (r < rows) {
                xq[u] = __builtin_nontemporal_load(reinterpret_cast<const vec *>(q_raw + r * D + c0));
                xk[u] = __builtin_nontemporal_load(reinterpret_cast<const vec *>(k_raw + r * D + c0));
                if (GATE) xz[u] = __builtin_nontemporal_load(reinterpret_cast<const vec *>(z + r * D + c0));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row + u * step;
            const int hu = h;
            h = adv(h);
            if (r >= rows) continue;
            float fq[EPL], fk[EPL], sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                fq[e] = to_f32(xq[u][e]);
                fk[e] = to_f32(xk[u][e]);
                sq += fq[e] * fq[e];
                sk += fk[e] * fk[e];
            }
#pragma unroll
            for (int m = 1; m < LPR; m <<= 1) {
                sq += __shfl_xor(sq, m);
                sk += __shfl_xor(sk, m);
            }
            const float iq = sq > 0.f ? __builtin_amdgcn_rsqf(sq) : 0.f;
            const float ik = sk > 0.f ? __builtin_amdgcn_rsqf(sk) : 0.f;
            vec yq, yk;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                yq[e] = from_f32<T>(fq[e] * iq);
                yk[e] = from_f32<T>(fk[e] * ik);
            }
            *reinterpret_cast<vec *>(q + r * D + c0) = yq;
            *reinterpret_cast<vec *>(k + r * D + c0) = yk;
            if (GATE) {
                const float eA = __expf(A_log[hu]);
                const float *bb = b_alpha + (int64_t)hu * D + c0;
#pragma unroll
                for (int e4 = 0; e4 < EPL; e4 += 4) {
                    f32x4 y;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = eA * (to_f32(xz[u][e4 + i]) + bb[e4 + i]);
                        y[i] = -5.f * __builtin_amdgcn_rcpf(1.f + __expf(-x));
                    }
                    *reinterpret_cast<f32x4 *>(g + r * D + c0 + e4) = y;
                }
            }
        }
    }
}

template <typename T, int D>
static hipError_t launch_front_end_t(const void *q_raw, const void *k_raw, const void *z,
                                     const float *A_log, const float *b_alpha, void *q, void *k,
                                     float *g, int64_t rows, int H, hipStream_t stream)
{
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    const int64_t need = (rows + RPB - 1) / RPB;
    const int64_t blocks = need < 1024 ? need : 1024;
    if (g)
        hipLaunchKernelGGL((front_end_kernel<T, D, true>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const T *)q_raw, (const T *)k_raw, (const T *)z, A_log, b_alpha,
                           (T *)q, (T *)k, g, rows, H);
    else
        hipLaunchKernelGGL((front_end_kernel<T, D, false>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, (const T *)q_raw, (const T *)k_raw, (const T *)nullptr,
                           (const float *)nullptr, (const float *)nullptr, (T *)q, (T *)k,
                           (float *)nullptr, rows, H);
    return hipGetLastError();
}

// rows = tokens x H; g == NULL: L2Norm only.
hipError_t launch_front_end(const void *q_raw, const void *k_raw, const void *z, const float *A_log,
                            const float *b_alpha, void *q, void *k, float *g, int64_t rows, int H,
                            int d, bool is_bf16, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
#define KDA_FE_ARGS q_raw, k_raw, z, A_log, b_alpha, q, k, g, rows, H, stream
    if (is_bf16) {
        switch (d) {
            case 32: return launch_front_end_t<bf16, 32>(KDA_FE_ARGS);
            case 64: return launch_front_end_t<bf16, 64>(KDA_FE_ARGS);
            case 128: return launch_front_end_t<bf16, 128>(KDA_FE_ARGS);
        }
    } else {
        switch (d) {
            case 32: return launch_front_end_t<float, 32>(KDA_FE_ARGS);
            case 64: return launch_front_end_t<float, 64>(KDA_FE_ARGS);
            case 128: return launch_front_end_t<float, 128>(KDA_FE_ARGS);
        }
    }
#undef KDA_FE_ARGS
    return hipErrorInvalidValue;
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
// NORMD > 0: each row of NORMD channels (one head) of the output is then
// L2-normalised (function table "L2Norm"; a zero row stays zero), so that the
// layer's q = L2Norm(ShortConv(.)) needs no pass of its own.  The NORMD / VEC
// lanes of a head are consecutive lanes of one wave, which all run the same
// tokens, and reduce the sum of squares with xor shuffles.
template <typename T, int VEC, int RUN, int NORMD>
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
    constexpr int LPH = NORMD / VEC;                 // lanes of a head (NORMD > 0)
    static_assert(NORMD == 0 || (LPH >= 1 && LPH <= 64 && (LPH & (LPH - 1)) == 0), "head lanes");
    // the output row of one token: L2-normalised over the head's lanes
    const auto finish = [&](float (&o)[VEC]) __attribute__((always_inline)) {
        if (NORMD > 0) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) ss += o[e] * o[e];
            if (LPH >= 16) {
                // within a row of 16 lanes with DPP moves, then across rows
                ss = row16_sum(ss);
                if (LPH == 32) ss += __shfl_xor(ss, 16);
            } else {
#pragma unroll
                for (int m = 1; m < LPH; m <<= 1) ss += __shfl_xor(ss, m);
            }
            const float r = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] *= r;
        }
    };
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
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                o[e] = wt[e][0] * to_f32(xs[t][e]) + wt[e][1] * to_f32(xs[t + 1][e]) +
                       wt[e][2] * to_f32(xs[t + 2][e]) + wt[e][3] * to_f32(xs[t + 3][e]);
            finish(o);
            vecT out;
#pragma unroll
            for (int e = 0; e < VEC; ++e) out[e] = from_f32<T>(o[e]);
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
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            o[e] = wt[e][0] * win[0][e] + wt[e][1] * win[1][e] + wt[e][2] * win[2][e] +
                   wt[e][3] * cur[e];
        finish(o);
        vecT out;
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[e] = from_f32<T>(o[e]);
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

template <typename T, int NORMD>
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
        hipLaunchKernelGGL((short_conv_kernel<T, VEC, RUN, NORMD>), grid, dim3(256), 0, stream,
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

// normd: 0, or the head size over which each output row is L2-normalised.
template <typename T>
static hipError_t launch_short_conv_n(const void *x, const float *w, const int32_t *cu, int nseq,
                                      int64_t ntok, int C, float *state, void *y, int normd,
                                      hipStream_t stream)
{
#define KDA_SC_ARGS x, w, cu, nseq, ntok, C, state, y, stream
    switch (normd) {
        case 0: return launch_short_conv_t<T, 0>(KDA_SC_ARGS);
        case 32: return launch_short_conv_t<T, 32>(KDA_SC_ARGS);
        case 64: return launch_short_conv_t<T, 64>(KDA_SC_ARGS);
        case 128: return launch_short_conv_t<T, 128>(KDA_SC_ARGS);
    }
#undef KDA_SC_ARGS
    return hipErrorInvalidValue;
}

hipError_t launch_short_conv(const void *x, const float *w, const int32_t *cu, int nseq,
                             int64_t ntok, int C, float *state, void *y, bool is_bf16, int normd,
                             hipStream_t stream)
{
    if (nseq == 0) return hipSuccess;
    return is_bf16 ? launch_short_conv_n<bf16>(x, w, cu, nseq, ntok, C, state, y, normd, stream)
                   : launch_short_conv_n<float>(x, w, cu, nseq, ntok, C, state, y, normd, stream);
}

// ---------------------------------------------------------------------------
// Scan over P segment summaries in one launch: for each head,
//     S_in[0] = S0,  S_in[r + 1] = M[r] S_in[r] + S~[r],  S_final = S_in[P].
// The columns of S evolve independently, so one workgroup owns one head's
// 32-column block for the whole scan and keeps it in LDS (d x 32 fp32, rows
// padded to 36 floats so that the four K rows of a fragment read fall in
// different banks; two copies, read and written by alternate steps).  Each step, wave w computes TPW 16 x 16 tiles of
// M[r] S + S~[r] on v_mfma_f32_16x16x4_f32; within a 16-wide K block, lane
// group grp supplies K index kb + 4 grp + s at sub-step s to both operands, so
// that its four M values are one 16-byte read.  M[r] and S~[r] are read once
// per column block (from L2 after the first), S_in[r] is written once.
template <int D>
__global__ __launch_bounds__(256) void scan_kernel(const float *__restrict__ M,
                                                   const float *__restrict__ St,
                                                   const float *S0, float *__restrict__ S_in,
                                                   float *S_fin, int P, int H)
{
    constexpr int CB = 32, NCB = D / CB, NCT = CB / 16, LDW = CB + 4;
    constexpr int TILES = (D / 16) * NCT, TPW = TILES / 4;
    static_assert(TPW >= 1 && TILES % 4 == 0, "shape");
    __shared__ float sS[2][D][LDW];    // the state entering step r is in sS[r & 1]

    const int lane = threadIdx.x & 63, n16 = lane & 15, grp = lane >> 4;
    const int w = threadIdx.x >> 6;
    // block b runs on XCD b mod 8: when H divides by 8, the NCB column blocks of
    // a head are given blocks of one XCD, so that M[r] comes from HBM once and
    // from that XCD's L2 for the other column blocks
    int item = blockIdx.x;
    if (H % 8 == 0) {
        const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
        item = (x * (H / 8) + slot / NCB) * NCB + slot % NCB;
    }
    const int h = item / NCB, c0 = (item % NCB) * CB;
    const int64_t DD = (int64_t)D * D;
    // block copies: thread t moves 4 consecutive columns of rows t / 8 + 32 j
    const int cr = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 4;

#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        f32x4 x = zero4();
        if (S0)
            x = *reinterpret_cast<const f32x4 *>(S0 + h * DD + (int64_t)(cr + 32 * j) * D + c0 + cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) sS[0][cr + 32 * j][cc + i] = x[i];
    }

    // one barrier a step: step r reads sS[r & 1] and writes sS[(r + 1) & 1],
    // which step r - 1 finished reading before this step's barrier
    for (int r = 0; r < P; ++r) {
        __syncthreads();   // S complete in sS[r & 1]
        const float(*cur)[LDW] = sS[r & 1];
        float(*nxt)[LDW] = sS[(r + 1) & 1];
        const int64_t base = ((int64_t)r * H + h) * DD;
        if (S_in) {
#pragma unroll
            for (int j = 0; j < D / 32; ++j) {
                const int row = cr + 32 * j;
                *reinterpret_cast<f32x4 *>(S_in + base + (int64_t)row * D + c0 + cc) =
                    f32x4{cur[row][cc], cur[row][cc + 1], cur[row][cc + 2], cur[row][cc + 3]};
            }
        }
        f32x4 acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = w * TPW + t, rs = tile / NCT, ct = tile % NCT;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = St[base + (int64_t)(16 * rs + 4 * grp + i) * D + c0 + 16 * ct + n16];
        }
        const float *Mr = M + base;
#pragma unroll 2
        for (int kb = 0; kb < D; kb += 16) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int tile = w * TPW + t, rs = tile / NCT, ct = tile % NCT;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(
                    Mr + (int64_t)(16 * rs + n16) * D + kb + 4 * grp);
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        a[sub], cur[kb + 4 * grp + sub][16 * ct + n16], acc[t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = w * TPW + t, rs = tile / NCT, ct = tile % NCT;
#pragma unroll
            for (int i = 0; i < 4; ++i) nxt[16 * rs + 4 * grp + i][16 * ct + n16] = acc[t][i];
        }
    }
    __syncthreads();
    const float(*fin)[LDW] = sS[P & 1];
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        const int row = cr + 32 * j;
        *reinterpret_cast<f32x4 *>(S_fin + h * DD + (int64_t)row * D + c0 + cc) =
            f32x4{fin[row][cc], fin[row][cc + 1], fin[row][cc + 2], fin[row][cc + 3]};
    }
}

template <int D>
static hipError_t launch_scan_t(const float *M, const float *St, const float *S0, float *S_in,
                                float *S_fin, int P, int H, hipStream_t stream)
{
    hipLaunchKernelGGL((scan_kernel<D>), dim3((unsigned)(H * (D / 32))), dim3(256), 0, stream, M,
                       St, S0, S_in, S_fin, P, H);
    return hipGetLastError();
}

hipError_t launch_scan(const float *M, const float *St, const float *S0, float *S_in,
                       float *S_fin, int P, int H, int d, hipStream_t stream)
{
    switch (d) {
        case 32: return launch_scan_t<32>(M, St, S0, S_in, S_fin, P, H, stream);
        case 64: return launch_scan_t<64>(M, St, S0, S_in, S_fin, P, H, stream);
        case 128: return launch_scan_t<128>(M, St, S0, S_in, S_fin, P, H, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
