// One-token KDA decode step on gfx950.
//
// Per (request, head) the state S (d_k x d_v fp32) advances by one token
// (page "Notations mathematiques", table "Attention et KDA", rows M_t, S_t):
//     S' = (I - beta k k^T) Diag(alpha) S + beta k v^T,  alpha = exp(g),
//     o  = S'^T q.
// Every column of S evolves on its own, so with a = alpha:
//     y_j = sum_c k_c a_c S_cj,   z_j = sum_c q_c a_c S_cj,
//     u_j = beta (v_j - y_j),     S'_cj = a_c S_cj + k_c u_j,
//     o_j = sum_c q_c S'_cj = z_j + (q . k) u_j.
// The state is read once and written once: the step is bound by HBM bandwidth
// ("Glossaire", entry "Decode"), 8 d_k d_v bytes per (request, head).
//
// Mapping: workgroups of NT threads (1024 at d = 128, 256 below) step through
// the (request, head) items with a grid stride.  Thread t owns four
// consecutive columns (one 16-byte vector) of rows r0, r0 + RPP, ...; a wave
// therefore reads whole rows, fully coalesced, and keeps its share of S in
// registers between the read and the write.  The next item's state is loaded
// while the current one is finished, so that every wave always has a state
// read in flight.  The shared arrays come in two sets used by alternate items,
// so that an item needs three barriers.  At d = 128 the wide workgroup keeps each thread's share of
// the current and next state at 4 + 4 vectors (under 100 VGPRs instead of 204
// with 256 threads), which lets more waves per SIMD stream: 6.1 TB/s against
// 5.4.  The per-row partial sums of y and z are first added across the lanes
// of a wave (a wave holds 64 / (d_v / 4) rows), so that the row threads add
// one partial per wave instead of one per row: 3 % off the step at d = 128.
//
// GATED: the layer's output epilogue is applied in the same kernel (page
// "Notations mathematiques": row o~_t and the function table's RMSNorm; "Kimi
// K3" model tables: epsilon and the full-rank sigmoid output gate):
//     out_j = o_j / sqrt(mean_j o_j^2 + eps) * w_j * sigma(gate_j),
// over the d_v columns of one (request, head), which the workgroup holds; the
// raw o is stored only when asked for.  The row threads' operands (v, beta,
// gate logits, norm weights) are read at the start of the item.
#include "kda_common.hpp"

namespace kda {

template <typename T, int DK, int DV, int NT, bool GATED>
__global__ __launch_bounds__(NT) void decode_kernel(const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ state,
                                                     T *__restrict__ o, int64_t NH,
                                                     const T *__restrict__ gate,
                                                     const float *__restrict__ gw, float eps,
                                                     T *__restrict__ out)
{
    constexpr int TPR = DV / 4;        // threads per state row
    constexpr int RPP = NT / TPR;      // rows covered per pass
    constexpr int NPASS = DK / RPP;    // passes over the rows
    static_assert(DK % RPP == 0 && NPASS >= 1, "shape");

    const int t = threadIdx.x;
    const int col = (t % TPR) * 4;
    const int r0 = t / TPR;

    // Shared arrays, two sets used by alternate items: a wave may start writing
    // item i + 1's set while others still read item i's, and item i + 1's first
    // barrier comes only after every wave has finished item i - 1, the last
    // user of that set, so an item needs three barriers, not four.
    constexpr int NW = NT / 64;        // waves
    __shared__ float sq[2][DK], sk[2][DK], sa[2][DK];
    __shared__ f32x4 ry[2][NW][TPR], rz[2][NW][TPR];
    __shared__ float su[2][DV];
    __shared__ float sqk[2];
    int pb = 0;

    int64_t nh = blockIdx.x;           // request * H + head
    f32x4 s[NPASS];
    if (nh < NH) {
        const float *S = state + nh * (int64_t)(DK * DV);
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
            s[p] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(S + (int64_t)(r0 + p * RPP) * DV + col));
    }
    for (; nh < NH; nh += gridDim.x) {
        float *S = state + nh * (int64_t)(DK * DV);
        const int64_t nx = nh + gridDim.x;
        f32x4 sn[NPASS];
        if (nx < NH) {
            const float *Sn = state + nx * (int64_t)(DK * DV);
#pragma unroll
            for (int p = 0; p < NPASS; ++p)
                sn[p] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(Sn + (int64_t)(r0 + p * RPP) * DV + col));
        }
        // the row threads' operands are read now, to arrive by the time the
        // column sums are reduced
        float vb = 0.f, vv[4] = {}, gl[4] = {}, wl[4] = {};
        if (t < TPR) {
            vb = beta[nh];
#pragma unroll
            for (int i = 0; i < 4; ++i) vv[i] = to_f32(v[nh * DV + col + i]);
            if (GATED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    gl[i] = to_f32(gate[nh * DV + col + i]);
                    wl[i] = gw[col + i];
                }
            }
        }

        for (int c = t; c < DK; c += NT) {
            sq[pb][c] = to_f32(q[nh * DK + c]);
            sk[pb][c] = to_f32(k[nh * DK + c]);
            sa[pb][c] = __expf(g[nh * DK + c]);
        }
        __syncthreads();

        if (t < 64) {  // q . k on wave 0
            float acc = 0.f;
            for (int c = t; c < DK; c += 64) acc += sq[pb][c] * sk[pb][c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
            if (t == 0) sqk[pb] = acc;
        }

        f32x4 y = zero4(), z = zero4();
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = r0 + p * RPP;
            const float a = sa[pb][c];
            const float ka = sk[pb][c] * a, qa = sq[pb][c] * a;
            y += ka * s[p];
            z += qa * s[p];
        }
        // a wave holds 64 / TPR rows: sum them across lanes first, so that the
        // row threads add NW partial sums instead of RPP
#pragma unroll
        for (int m = TPR; m < 64; m <<= 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[i] += __shfl_xor(y[i], m);
                z[i] += __shfl_xor(z[i], m);
            }
        }
        if ((t & 63) < TPR) {
            ry[pb][t / 64][t & 63] = y;
            rz[pb][t / 64][t & 63] = z;
        }
        __syncthreads();

        if (t < TPR) {
            f32x4 yy = zero4(), zz = zero4();
#pragma unroll
            for (int r = 0; r < NW; ++r) { yy += ry[pb][r][t]; zz += rz[pb][r][t]; }
            const float b = vb;
            const float qk = sqk[pb];
            float ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = b * (vv[i] - yy[i]);
                su[pb][col + i] = u;
                ov[i] = zz[i] + qk * u;
            }
            if (!GATED || o) {
                T *orow = o + nh * DV + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) orow[i] = from_f32<T>(ov[i]);
            }
            if (GATED) {
                // the TPR lanes of the row are lanes 0 .. TPR - 1 of wave 0
                float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
                for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m);
                const float r = __builtin_amdgcn_rsqf(ss * (1.f / DV) + eps);
                T *yrow = out + nh * DV + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-gl[i]));
                    yrow[i] = from_f32<T>(ov[i] * r * wl[i] * sg);
                }
            }
        }
        __syncthreads();

        const f32x4 u4 = f32x4{su[pb][col], su[pb][col + 1], su[pb][col + 2], su[pb][col + 3]};
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = r0 + p * RPP;
            const f32x4 ns = sa[pb][c] * s[p] + sk[pb][c] * u4;
            __builtin_nontemporal_store(
                ns, reinterpret_cast<f32x4 *>(S + (int64_t)(r0 + p * RPP) * DV + col));
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) s[p] = sn[p];
        pb ^= 1;
    }
}

// Enough workgroups to fill the chip several times over (256 CUs), few
// enough that each steps through several items and overlaps their reads.
constexpr int64_t kDecodeMaxBlocks = 4096;

template <typename T, int D>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int64_t NH,
                                  const void *gate, const float *gw, float eps, void *out,
                                  hipStream_t stream)
{
    const int64_t blocks = NH < kDecodeMaxBlocks ? NH : kDecodeMaxBlocks;
    constexpr int NT = D == 128 ? 1024 : 256;
    if (gate)
        hipLaunchKernelGGL((decode_kernel<T, D, D, NT, true>), dim3((unsigned)blocks), dim3(NT), 0,
                           stream, (const T *)q, (const T *)k, (const T *)v, g, beta, state,
                           (T *)o, NH, (const T *)gate, gw, eps, (T *)out);
    else
        hipLaunchKernelGGL((decode_kernel<T, D, D, NT, false>), dim3((unsigned)blocks), dim3(NT), 0,
                           stream, (const T *)q, (const T *)k, (const T *)v, g, beta, state,
                           (T *)o, NH, (const T *)nullptr, (const float *)nullptr, 0.f,
                           (T *)nullptr);
    return hipGetLastError();
}

// gate == NULL: the plain step (o written).  Otherwise the gated output goes
// to out and o (may be NULL) gets the raw output.
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int64_t NH, int d,
                         bool is_bf16, const void *gate, const float *gw, float eps, void *out,
                         hipStream_t stream)
{
#define KDA_DEC_ARGS q, k, v, g, beta, state, o, NH, gate, gw, eps, out, stream
    if (is_bf16) {
        switch (d) {
            case 32: return launch_decode_t<bf16, 32>(KDA_DEC_ARGS);
            case 64: return launch_decode_t<bf16, 64>(KDA_DEC_ARGS);
            case 128: return launch_decode_t<bf16, 128>(KDA_DEC_ARGS);
        }
    } else {
        switch (d) {
            case 32: return launch_decode_t<float, 32>(KDA_DEC_ARGS);
            case 64: return launch_decode_t<float, 64>(KDA_DEC_ARGS);
            case 128: return launch_decode_t<float, 128>(KDA_DEC_ARGS);
        }
    }
#undef KDA_DEC_ARGS
    return hipErrorInvalidValue;
}

}  // namespace kda
