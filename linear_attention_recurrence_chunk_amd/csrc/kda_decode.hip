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
// read in flight.  At d = 128 the wide workgroup keeps each thread's share of
// the current and next state at 8 + 8 vectors (86 VGPRs instead of 204 with
// 256 threads), which lets more waves per SIMD stream: 6.1 TB/s against 5.4.
#include "kda_common.hpp"

namespace kda {

template <typename T, int DK, int DV, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(const T *__restrict__ q,
                                                     const T *__restrict__ k,
                                                     const T *__restrict__ v,
                                                     const float *__restrict__ g,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ state,
                                                     T *__restrict__ o, int64_t NH)
{
    constexpr int TPR = DV / 4;        // threads per state row
    constexpr int RPP = NT / TPR;      // rows covered per pass
    constexpr int NPASS = DK / RPP;    // passes over the rows
    static_assert(DK % RPP == 0 && NPASS >= 1, "shape");

    const int t = threadIdx.x;
    const int col = (t % TPR) * 4;
    const int r0 = t / TPR;

    __shared__ float sq[DK], sk[DK], sa[DK];
    __shared__ f32x4 ry[RPP][TPR], rz[RPP][TPR];
    __shared__ float su[DV];
    __shared__ float sqk;

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

        for (int c = t; c < DK; c += NT) {
            sq[c] = to_f32(q[nh * DK + c]);
            sk[c] = to_f32(k[nh * DK + c]);
            sa[c] = __expf(g[nh * DK + c]);
        }
        __syncthreads();

        if (t < 64) {  // q . k on wave 0
            float acc = 0.f;
            for (int c = t; c < DK; c += 64) acc += sq[c] * sk[c];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
            if (t == 0) sqk = acc;
        }

        f32x4 y = zero4(), z = zero4();
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = r0 + p * RPP;
            const float a = sa[c];
            const float ka = sk[c] * a, qa = sq[c] * a;
            y += ka * s[p];
            z += qa * s[p];
        }
        ry[r0][t % TPR] = y;
        rz[r0][t % TPR] = z;
        __syncthreads();

        if (t < TPR) {
            f32x4 yy = zero4(), zz = zero4();
            for (int r = 0; r < RPP; ++r) { yy += ry[r][t]; zz += rz[r][t]; }
            const float b = beta[nh];
            const float qk = sqk;
            const T *vr = v + nh * DV + col;
            float ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = b * (to_f32(vr[i]) - yy[i]);
                su[col + i] = u;
                ov[i] = zz[i] + qk * u;
            }
            T *orow = o + nh * DV + col;
#pragma unroll
            for (int i = 0; i < 4; ++i) orow[i] = from_f32<T>(ov[i]);
        }
        __syncthreads();

        const f32x4 u4 = f32x4{su[col], su[col + 1], su[col + 2], su[col + 3]};
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int c = r0 + p * RPP;
            const f32x4 ns = sa[c] * s[p] + sk[c] * u4;
            __builtin_nontemporal_store(
                ns, reinterpret_cast<f32x4 *>(S + (int64_t)(r0 + p * RPP) * DV + col));
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p) s[p] = sn[p];
        __syncthreads();   // the shared arrays are reused by the next item
    }
}

// Enough workgroups to fill the chip several times over (256 CUs), few
// enough that each steps through several items and overlaps their reads.
constexpr int64_t kDecodeMaxBlocks = 4096;

template <typename T, int D>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int64_t NH,
                                  hipStream_t stream)
{
    const int64_t blocks = NH < kDecodeMaxBlocks ? NH : kDecodeMaxBlocks;
    constexpr int NT = D == 128 ? 1024 : 256;
    hipLaunchKernelGGL((decode_kernel<T, D, D, NT>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, g, beta, state, (T *)o, NH);
    return hipGetLastError();
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int64_t NH, int d,
                         bool is_bf16, hipStream_t stream)
{
    if (is_bf16) {
        switch (d) {
            case 32: return launch_decode_t<bf16, 32>(q, k, v, g, beta, state, o, NH, stream);
            case 64: return launch_decode_t<bf16, 64>(q, k, v, g, beta, state, o, NH, stream);
            case 128: return launch_decode_t<bf16, 128>(q, k, v, g, beta, state, o, NH, stream);
        }
    } else {
        switch (d) {
            case 32: return launch_decode_t<float, 32>(q, k, v, g, beta, state, o, NH, stream);
            case 64: return launch_decode_t<float, 64>(q, k, v, g, beta, state, o, NH, stream);
            case 128: return launch_decode_t<float, 128>(q, k, v, g, beta, state, o, NH, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
