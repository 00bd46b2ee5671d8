// Fused chunkwise KDA prefill on gfx950 (CDNA4).
//
// What is computed (page "Notations mathematiques", table "Attention et KDA"):
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     alpha_t = exp(g_t),  o_t = S_t^T q_t,
// evaluated block by block: serial across chunks of C tokens, parallel inside
// a chunk ("Glossaire", entry "Chunkwise"; it is an exact rewrite).  Inside a
// chunk of n <= C tokens entering with state S, with G the in-chunk inclusive
// cumulative sum of g (exp(G_r) is the cumulative decay gamma^{1->r} of the
// notation table) and B = Diag(beta):
//     A  = StrictTril( B (K o e^G)(K o e^-G)^T )        strictly lower, n x n
//     U  = (I + A)^-1 B (V - (K o e^G) S)               the UT transform of the
//                                                       "Glossaire" entry "UT"
//     O  = (Q o e^G) S + Tril((Q o e^G)(K o e^-G)^T) U  (Tril keeps the diagonal)
//     S' = Diag(e^{G_n}) S + (K o e^{G_n - G})^T U
// Every operator acts on S from the left, so each column of S evolves on its
// own: a workgroup owns one (sequence, head, slice of BV value columns).
//
// (I + A) is solved blockwise on 16-token sub-blocks: each diagonal block's
// inverse comes from the identity (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8)
// (N strictly lower 16 x 16, so N^16 = 0), evaluated with four matrix-core
// products, and U follows by block forward substitution
//     U_I = (I + A_II)^-1 (R_I - sum_{J<I} A_IJ U_J),   R = B (V - (K o e^G) S).
//
// Decay factors never leave the float range.  With L the sub-block-local
// inclusive cumulative sum of g and B_J the total log decay of sub-block J:
//   rows of sub-block I:        e^{L_r}                          in [e^-80, 1]
//   diagonal-block columns:     e^{B_I - L_j} * e^{-B_I}         in [1, e^80]
//   columns of J < I:           e^{B_J - L_j} * prod_{J<m<I} e^{B_m}   <= 1
// e^80 is the bound the "Glossaire" entry "Decroissance bornee" gives for
// g_min = -5 (16 tokens times 5; see also the box "Limite importante" of page
// "Vecteurs, embeddings, espaces de representation").  A factor that
// underflows is a product of true decays below 1e-38: no significant term is
// lost.  Products are taken in an order in which no intermediate overflows.
//
// Work split (8 waves).  Waves 0-3 ("state waves") hold the fp32 state slice
// in registers, invert the diagonal blocks and update the state; waves 4-7
// ("row waves") own the 16-token row block I = wave - 4 for the state
// read-out, the forward substitution (by value-column tile) and the output.
// Contractions run on the matrix cores (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x16_bf16, or v_mfma_f32_16x16x4_f32 for fp32 inputs) with
// fp32 accumulation; operands are rounded to the input type.
#include "kda_common.hpp"

namespace kda {

template <typename T, int DK, int BV>
struct Cfg64 {
    static constexpr int C = 64;
    static constexpr int NB = 4;                      // 16-token sub-blocks
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;
    static constexpr int PAD = 16 / (int)sizeof(T);   // 16-byte row padding
    static constexpr int LDK = DK + PAD;              // [token][channel] tiles
    static constexpr int LDC = C + PAD;               // [.][token] tiles
    static constexpr int LDV = BV + PAD;              // [token][value] tiles
    static constexpr int LDA = C + 4;                 // fp32 A rows
    static constexpr int NITEM = NB * DK;             // (sub-block, channel) items
    static constexpr int VPR = BV * (int)sizeof(T) / 16;   // 16-byte vectors per V row
    static constexpr int NVV = (C * VPR + NT - 1) / NT;
    static constexpr int NCT = DK / 16;               // state row tiles
    static constexpr int NVT = BV / 16;               // state column tiles
    static constexpr int SWPC = (NCT >= 4) ? 1 : 4 / NCT;   // state waves per row tile
    static constexpr int SCT = (NCT >= 4) ? NCT / 4 : 1;    // row tiles per state wave
    static constexpr int SVT = NVT / SWPC;                   // column tiles per state wave
    static_assert(NITEM <= NT, "elementwise mapping");
    static_assert(SVT >= 1 && NVT % SWPC == 0, "state tiling");
    static_assert(DK % Path<T>::KS == 0 && C % Path<T>::KS == 0, "k steps");
};

template <typename T, int DK, int BV>
struct Smem64 {
    typedef Cfg64<T, DK, BV> Cf;
    T Kr[Cf::C][Cf::LDK];      // K o e^{L}        row operand (and K e^G after e^{E_I})
    T Qr[Cf::C][Cf::LDK];      // Q o e^{L}
    T Kc[Cf::C][Cf::LDK];      // K o e^{B - L}    column operand, and K e^{G_n - G} after e^{...}
    T Tm[Cf::C][Cf::LDC];      // diagonal blocks of (I + A)^-1
    T P[Cf::C][Cf::LDC];       // Tril((Q o e^G)(K o e^-G)^T)
    T V[Cf::C][Cf::LDV];       // value slice
    T ST[BV][Cf::LDK];         // state slice, transposed operand copy
    T RT[BV][Cf::LDC];         // R^T, overwritten in place by U^T
    float A[Cf::C][Cf::LDA];   // A (beta applied, strictly lower)
    float scr[4][2][16][20];   // per-wave N^2, N^4 for the diagonal inverses
    float eB[Cf::NB][DK];      // e^{B_J}
    float rB[Cf::NB][DK];      // e^{-B_J}
    float beta[Cf::C];
};

// Raw inputs of one chunk, one item (sub-block, channel) per thread, held in
// registers one chunk ahead.
template <typename T, int DK, int BV>
struct ChunkRegs {
    typedef Cfg64<T, DK, BV> Cf;
    float g[16];
    T k[16], q[16];
    f32x4 v[Cf::NVV];
    float beta;
};

struct SeqView {
    int64_t bos, eos;   // token range of the sequence
    int head, H;
    int v0;             // first value column of the slice
};

template <typename T, int DK, int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, DK, BV> &R, const SeqView &sv,
                                           int64_t t0, const T *__restrict__ q,
                                           const T *__restrict__ k, const T *__restrict__ v,
                                           const float *__restrict__ g,
                                           const float *__restrict__ beta, int DV)
{
    typedef Cfg64<T, DK, BV> Cf;
    const int t = threadIdx.x;
    if (t < Cf::NITEM) {
        const int I = t / DK, c = t % DK;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t tok = t0 + 16 * I + r;
            const bool in = tok < sv.eos;
            const int64_t off = ((in ? tok : sv.bos) * sv.H + sv.head) * DK + c;
            R.g[r] = in ? g[off] : 0.f;
            R.k[r] = in ? k[off] : from_f32<T>(0.f);
            R.q[r] = in ? q[off] : from_f32<T>(0.f);
        }
    }
#pragma unroll
    for (int m = 0; m < Cf::NVV; ++m) {
        const int vi = t + Cf::NT * m;
        const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
        const int64_t tok = t0 + row;
        R.v[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < Cf::C && tok < sv.eos)
            R.v[m] = *reinterpret_cast<const f32x4 *>(
                v + (tok * sv.H + sv.head) * DV + sv.v0 + cv * (16 / (int)sizeof(T)));
    }
    R.beta = 0.f;
    if (t < Cf::C && t0 + t < sv.eos) R.beta = beta[(t0 + t) * sv.H + sv.head];
}

// Make this wave's LDS writes visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int N> __device__ __forceinline__ void load_f32(float *dst, const float *src)
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(src + i);
            dst[i] = x[0]; dst[i + 1] = x[1]; dst[i + 2] = x[2]; dst[i + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}

template <typename T, int DK, int BV, int DV>
__global__ __launch_bounds__(512, 1) void prefill64_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ s0, const int32_t *__restrict__ cu_seqlens, int num_seqs,
    int64_t seq_len, int H, T *__restrict__ o, float *__restrict__ sfinal)
{
    typedef Cfg64<T, DK, BV> Cf;
    typedef Path<T> PT;
    typedef Smem64<T, DK, BV> Sm;
    constexpr int C = Cf::C, NB = Cf::NB, NT = Cf::NT, KS = PT::KS, KPL = PT::KPL;
    constexpr int NSLICE = DV / BV;
    __shared__ __align__(16) unsigned char smem_raw[sizeof(Sm)];
    Sm &sm = *reinterpret_cast<Sm *>(smem_raw);

    // ---- work item: (sequence, head, value slice); slices of one head adjacent
    // and, when the count allows, on one XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so that they share q, k, g through that XCD's L2.
    const int64_t nwork = (int64_t)num_seqs * H * NSLICE;
    const int64_t b = blockIdx.x;
    const int64_t w = (nwork % 8 == 0) ? (b % 8) * (nwork / 8) + b / 8 : b;
    const int seq = (int)(w / ((int64_t)H * NSLICE));
    const int head = (int)((w / NSLICE) % H);
    const int slice = (int)(w % NSLICE);
    SeqView sv;
    if (cu_seqlens) {
        sv.bos = cu_seqlens[seq];
        sv.eos = cu_seqlens[seq + 1];
    } else {
        sv.bos = (int64_t)seq * seq_len;
        sv.eos = sv.bos + seq_len;
    }
    sv.head = head;
    sv.H = H;
    sv.v0 = slice * BV;

    const int t = threadIdx.x;
    const int lane = lane_id(), wv = wave_id();
    const int n16 = lane & 15, grp = lane >> 4;
    const bool state_wave = wv < 4;
    const int I_row = wv - 4;                        // row block of a row wave

    // ---- state slice in the registers of the state waves, D layout:
    // tile (ct, vt) holds S[16 ct + 4 grp + i][16 vt + n16]
    const int sw = state_wave ? wv : 0;
    const int ct0 = (sw / Cf::SWPC) * Cf::SCT;
    const int vt0 = (sw % Cf::SWPC) * Cf::SVT;
    f32x4 S[Cf::SCT][Cf::SVT];
    const int64_t sbase = ((int64_t)seq * H + head) * (int64_t)(DK * DV) + sv.v0;
#pragma unroll
    for (int a = 0; a < Cf::SCT; ++a)
#pragma unroll
        for (int bq = 0; bq < Cf::SVT; ++bq) {
            S[a][bq] = zero4();
            if (state_wave && s0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[a][bq][i] = s0[sbase + (int64_t)(16 * (ct0 + a) + 4 * grp + i) * DV +
                                     16 * (vt0 + bq) + n16];
            }
        }
    if (state_wave) {
#pragma unroll
        for (int a = 0; a < Cf::SCT; ++a)
#pragma unroll
            for (int bq = 0; bq < Cf::SVT; ++bq)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.ST[16 * (vt0 + bq) + n16][16 * (ct0 + a) + 4 * grp + i] =
                        from_f32<T>(S[a][bq][i]);
    }
    // constant zero blocks above the diagonal of P
    for (int e = t; e < C * C; e += NT) {
        const int r = e / C, j = e % C;
        if ((j >> 4) > (r >> 4)) sm.P[r][j] = from_f32<T>(0.f);
    }

    const int64_t nchunks = (sv.eos - sv.bos + C - 1) / C;
    ChunkRegs<T, DK, BV> R;
    if (nchunks > 0) load_chunk(R, sv, sv.bos, q, k, v, g, beta, DV);

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = sv.bos + ch * C;

        // ================= E: sub-block-local decays and operand tiles
        if (t < Cf::NITEM) {
            const int I = t / DK, c = t % DK;
            float a[16], eL[16], sfx[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = __expf(R.g[r]);
            eL[0] = a[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) eL[r] = eL[r - 1] * a[r];
            sfx[15] = 1.f;
#pragma unroll
            for (int r = 14; r >= 0; --r) sfx[r] = sfx[r + 1] * a[r + 1];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float kk = to_f32(R.k[r]), qq = to_f32(R.q[r]);
                sm.Kr[16 * I + r][c] = from_f32<T>(kk * eL[r]);
                sm.Qr[16 * I + r][c] = from_f32<T>(qq * eL[r]);
                sm.Kc[16 * I + r][c] = from_f32<T>(kk * sfx[r]);
            }
            sm.eB[I][c] = eL[15];
            sm.rB[I][c] = __builtin_amdgcn_rcpf(eL[15]);   // <= e^80
        }
        if (t < C) sm.beta[t] = R.beta;
#pragma unroll
        for (int m = 0; m < Cf::NVV; ++m) {
            const int vi = t + NT * m;
            const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
            if (row < C)
                *reinterpret_cast<f32x4 *>(&sm.V[row][cv * (16 / (int)sizeof(T))]) = R.v[m];
        }
        __syncthreads();   // ---------------------------------------------- B1
        if (ch + 1 < nchunks) load_chunk(R, sv, t0 + C, q, k, v, g, beta, DV);

        // ================= AP: 16x16 blocks (I, J <= I) of A and P
        for (int p = wv; p < NB * (NB + 1) / 2; p += Cf::NW) {
            int I = 0, rem = p;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / KS; ++ks) {
                const int kc = ks * KS + grp * KPL;
                const typename PT::frag ak = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
                const typename PT::frag aq = load_frag<T>(&sm.Qr[16 * I + n16][kc]);
                float xb[KPL], f[KPL];
                PT::unpack(load_frag<T>(&sm.Kc[16 * J + n16][kc]), xb);
                if (I == J) {
                    load_f32<KPL>(f, &sm.rB[I][kc]);              // -> K o e^{-L}
                } else {
#pragma unroll
                    for (int e = 0; e < KPL; ++e) f[e] = 1.f;
#pragma unroll
                    for (int m = 1; m < NB - 1; ++m)
                        if (m > J && m < I) {
                            float fm[KPL];
                            load_f32<KPL>(fm, &sm.eB[m][kc]);
#pragma unroll
                            for (int e = 0; e < KPL; ++e) f[e] *= fm[e];
                        }
                }
#pragma unroll
                for (int e = 0; e < KPL; ++e) xb[e] *= f[e];
                const typename PT::frag bk = PT::pack(xb);
                accA = PT::mma(ak, bk, accA);
                accP = PT::mma(aq, bk, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 4 * grp + i, jl = n16;
                float va = accA[i], vp = accP[i];
                if (I == J) {
                    if (jl >= rl) va = 0.f;
                    if (jl > rl) vp = 0.f;
                }
                sm.A[16 * I + rl][16 * J + jl] = va * sm.beta[16 * I + rl];
                sm.P[16 * I + rl][16 * J + jl] = from_f32<T>(vp);
            }
        }
        __syncthreads();   // ---------------------------------------------- B2

        constexpr int NVT = Cf::NVT;
        f32x4 accZ[NVT];
        if (state_wave) {
            // ============= diagonal-block inverses (I + N)^-1, N = A_II
            const int I = wv;
            float dN[4], aN[4], aN2[4], aN4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dN[i] = sm.A[16 * I + 4 * grp + i][16 * I + n16];
                aN[i] = sm.A[16 * I + n16][16 * I + 4 * grp + i];
            }
            const f32x4 N2 = PT::mma16(aN, dN, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.scr[I][0][4 * grp + i][n16] = N2[i];
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) aN2[i] = sm.scr[I][0][n16][4 * grp + i];
            float bN2[4] = {N2[0], N2[1], N2[2], N2[3]};
            const f32x4 N4 = PT::mma16(aN2, bN2, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.scr[I][1][4 * grp + i][n16] = N4[i];
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) aN4[i] = sm.scr[I][1][n16][4 * grp + i];
            float bN4[4] = {N4[0], N4[1], N4[2], N4[3]};
            f32x4 X = PT::mma16(aN4, bN4, zero4());            // N^8
#pragma unroll
            for (int i = 0; i < 4; ++i) X[i] += (4 * grp + i == n16) ? 1.f : 0.f;   // I + N^8
            float bX[4] = {X[0], X[1], X[2], X[3]};
            X = PT::mma16(aN4, bX, X);                           // (I + N^4)(I + N^8)
            float bY[4] = {X[0], X[1], X[2], X[3]};
            X = PT::mma16(aN2, bY, X);                           // (I + N^2)(...)
            float bZ[4] = {X[0], X[1], X[2], X[3]}, maN[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) maN[i] = -aN[i];
            X = PT::mma16(maN, bZ, X);                           // (I - N)(...)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.Tm[16 * I + 4 * grp + i][16 * I + n16] = from_f32<T>(X[i]);
        } else {
            // ============= state read-out for row block I: Y = K e^G S, Z = Q e^G S
            const int I = I_row;
            f32x4 accY[NVT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) { accY[vt] = zero4(); accZ[vt] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < DK / KS; ++ks) {
                const int kc = ks * KS + grp * KPL;
                float xk[KPL], xq[KPL], f[KPL];
                PT::unpack(load_frag<T>(&sm.Kr[16 * I + n16][kc]), xk);
                PT::unpack(load_frag<T>(&sm.Qr[16 * I + n16][kc]), xq);
#pragma unroll
                for (int e = 0; e < KPL; ++e) f[e] = 1.f;
#pragma unroll
                for (int m = 0; m < NB - 1; ++m)                 // e^{E_I} = prod_{m<I} e^{B_m}
                    if (m < I) {
                        float fm[KPL];
                        load_f32<KPL>(fm, &sm.eB[m][kc]);
#pragma unroll
                        for (int e = 0; e < KPL; ++e) f[e] *= fm[e];
                    }
#pragma unroll
                for (int e = 0; e < KPL; ++e) { xk[e] *= f[e]; xq[e] *= f[e]; }
                const typename PT::frag ak = PT::pack(xk), aq = PT::pack(xq);
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    const typename PT::frag bs = load_frag<T>(&sm.ST[16 * vt + n16][kc]);
                    accY[vt] = PT::mma(ak, bs, accY[vt]);
                    accZ[vt] = PT::mma(aq, bs, accZ[vt]);
                }
            }
            // R = B (V - Y), stored transposed
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * grp + i;
                    sm.RT[16 * vt + n16][r] =
                        from_f32<T>(sm.beta[r] * (to_f32(sm.V[r][16 * vt + n16]) - accY[vt][i]));
                }
        }
        __syncthreads();   // ---------------------------------------------- B3

        // state waves: column operand of the state update, (K o e^{G_n - G})^T
        typename PT::frag kb[Cf::SCT][C / KS];
        float gam[Cf::SCT][4];
        if (state_wave) {
#pragma unroll
            for (int a = 0; a < Cf::SCT; ++a) {
                const int c = 16 * (ct0 + a) + n16;
                float eb[NB];
#pragma unroll
                for (int m = 0; m < NB; ++m) eb[m] = sm.eB[m][c];
#pragma unroll
                for (int ks = 0; ks < C / KS; ++ks) {
                    const int kj = ks * KS + grp * KPL;
                    const int J = kj >> 4;
                    float f = 1.f;
#pragma unroll
                    for (int m = 1; m < NB; ++m)
                        if (m > J) f *= eb[m];
                    float x[KPL];
#pragma unroll
                    for (int e = 0; e < KPL; ++e) x[e] = to_f32(sm.Kc[kj + e][c]) * f;
                    kb[a][ks] = PT::pack(x);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cr = 16 * (ct0 + a) + 4 * grp + i;
                    float gm = 1.f;
#pragma unroll
                    for (int m = 0; m < NB; ++m) gm *= sm.eB[m][cr];
                    gam[a][i] = gm;
                }
            }
        } else {
            // ============= forward substitution U_I = T_II (R_I - sum_{J<I} A_IJ U_J),
            // one value-column tile at a time; U^T overwrites R^T in place
            for (int vt = I_row; vt < NVT; vt += 4) {
                f32x4 Ub[NB];
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    f32x4 X;
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[i] = to_f32(sm.RT[16 * vt + n16][16 * I + 4 * grp + i]);
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        float aA[4], bU[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            aA[i] = -sm.A[16 * I + n16][16 * J + 4 * grp + i];
                            bU[i] = Ub[J][i];
                        }
                        X = PT::mma16(aA, bU, X);
                    }
                    float aT[4], bX[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        aT[i] = to_f32(sm.Tm[16 * I + n16][16 * I + 4 * grp + i]);
                        bX[i] = X[i];
                    }
                    Ub[I] = PT::mma16(aT, bX, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sm.RT[16 * vt + n16][16 * I + 4 * grp + i] = from_f32<T>(Ub[I][i]);
                }
            }
        }
        __syncthreads();   // ---------------------------------------------- B4

        if (state_wave) {
            // ============= S' = Diag(gamma) S + (K o e^{G_n - G})^T U
#pragma unroll
            for (int a = 0; a < Cf::SCT; ++a)
#pragma unroll
                for (int bq = 0; bq < Cf::SVT; ++bq) {
                    f32x4 acc = S[a][bq];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] *= gam[a][i];
#pragma unroll
                    for (int ks = 0; ks < C / KS; ++ks) {
                        const int kj = ks * KS + grp * KPL;
                        acc = PT::mma(kb[a][ks],
                                      load_frag<T>(&sm.RT[16 * (vt0 + bq) + n16][kj]), acc);
                    }
                    S[a][bq] = acc;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sm.ST[16 * (vt0 + bq) + n16][16 * (ct0 + a) + 4 * grp + i] =
                            from_f32<T>(acc[i]);
                }
        } else {
            // ============= O = Z + P U for row block I, written straight to o
            const int I = I_row;
            const int nks = (16 * (I + 1) + KS - 1) / KS;
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = accZ[vt];
                for (int ks = 0; ks < nks; ++ks) {
                    const int kj = ks * KS + grp * KPL;
                    acc = PT::mma(load_frag<T>(&sm.P[16 * I + n16][kj]),
                                  load_frag<T>(&sm.RT[16 * vt + n16][kj]), acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t tok = t0 + 16 * I + 4 * grp + i;
                    if (tok < sv.eos)
                        o[(tok * H + head) * DV + sv.v0 + 16 * vt + n16] = from_f32<T>(acc[i]);
                }
            }
        }
        __syncthreads();   // ---------------------------------------------- B5
    }

    if (sfinal && state_wave) {
#pragma unroll
        for (int a = 0; a < Cf::SCT; ++a)
#pragma unroll
            for (int bq = 0; bq < Cf::SVT; ++bq)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sfinal[sbase + (int64_t)(16 * (ct0 + a) + 4 * grp + i) * DV +
                           16 * (vt0 + bq) + n16] = S[a][bq][i];
    }
}

template <typename T, int D, int BV>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int H, void *o, float *sf,
                                   hipStream_t stream)
{
    const int64_t nwork = (int64_t)num_seqs * H * (D / BV);
    if (nwork == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill64_kernel<T, D, BV, D>), dim3((unsigned)nwork), dim3(512), 0,
                       stream, (const T *)q, (const T *)k, (const T *)v, g, beta, s0, cu,
                       num_seqs, seq_len, H, (T *)o, sf);
    return hipGetLastError();
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int H, int d, int chunk, bool is_bf16, void *o,
                          float *sf, hipStream_t stream)
{
    if (chunk != 64) return hipErrorInvalidValue;
    if (is_bf16) {
        switch (d) {
            case 32:
                return launch_prefill_t<bf16, 32, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                      seq_len, H, o, sf, stream);
            case 64:
                return launch_prefill_t<bf16, 64, 64>(q, k, v, g, beta, s0, cu, num_seqs,
                                                      seq_len, H, o, sf, stream);
            case 128:
                return launch_prefill_t<bf16, 128, 64>(q, k, v, g, beta, s0, cu, num_seqs,
                                                       seq_len, H, o, sf, stream);
        }
    } else {
        switch (d) {
            case 32:
                return launch_prefill_t<float, 32, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                       seq_len, H, o, sf, stream);
            case 64:
                return launch_prefill_t<float, 64, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                       seq_len, H, o, sf, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
