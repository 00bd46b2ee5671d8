// Fused chunkwise KDA prefill on gfx950 (CDNA4).
//
// What is computed (page "Notations mathematiques", table "Attention et KDA"):
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     alpha_t = exp(g_t),  o_t = S_t^T q_t,
// evaluated block by block: serial across chunks of C tokens, parallel inside
// a chunk ("Glossaire", entry "Chunkwise"; it is an exact rewrite).  Inside a
// chunk of n <= C tokens entering with state S, with G the in-chunk inclusive
// cumulative sum of g (so exp(G_r) is the cumulative decay gamma^{1->r} of the
// notation table) and B = Diag(beta):
//     A  = StrictTril( B (K o e^G)(K o e^-G)^T )      strictly lower, n x n
//     T  = (I + A)^-1                                 the UT transform of the
//                                                     "Glossaire" entry "UT"
//     U  = T B (V - (K o e^G) S)                      delta-corrected values
//     O  = (Q o e^G) S + Tril((Q o e^G)(K o e^-G)^T) U  (Tril keeps the diagonal)
//     S' = Diag(e^{G_n}) S + (K o e^{G_n - G})^T U
// Every operator acts on S from the left, so each column of S evolves on its
// own: a workgroup owns one (sequence, head, slice of BV value columns).
//
// Decay factors never leave the float range.  Tokens are grouped in 16-token
// sub-blocks; with L the sub-block-local inclusive cumulative sum of g, every
// factor is written relative to a point inside or at the edge of a sub-block:
//   rows of sub-block I:        e^{L_r}            in [e^{-80}, 1]
//   diagonal columns:           e^{-L_j}           in [1, e^{80}]
//   off-diagonal columns J < I: e^{B_J - L_j} * prod_{J<m<I} e^{B_m}   <= 1
// where B_J is the total log decay of sub-block J.  The e^{80} bound is the
// one the "Glossaire" entry "Decroissance bornee" gives for g_min = -5 (and
// the box "Limite importante" of page "Vecteurs, embeddings, espaces de
// representation"): 16 tokens times 5.  A factor that underflows is a product
// of true decays that is itself below 1e-38, so no significant term is lost.
//
// Contractions run on the matrix cores (v_mfma_f32_16x16x32_bf16, or
// v_mfma_f32_16x16x4_f32 for fp32 inputs) with fp32 accumulation; the state is
// kept in fp32 registers for the whole sequence and rounded to the operand type
// only as a matrix-core operand.
#include "kda_common.hpp"

namespace kda {

template <typename T, int C, int DK, int BV>
struct PrefillCfg {
    static constexpr int NB = C / 16;                 // 16-token sub-blocks per chunk
    static constexpr int NW = NB;                     // one wave per sub-block
    static constexpr int NT = 64 * NW;
    static constexpr int PAD = 16 / (int)sizeof(T);   // 16-byte row padding
    static constexpr int LDK = DK + PAD;              // stride of [token][channel] tiles
    static constexpr int LDC = C + PAD;               // stride of [.][token] tiles
    static constexpr int LDV = BV + PAD;              // stride of [token][value] tiles
    static constexpr int LDA = C + 4;                 // fp32 A rows
    static constexpr int CPT = (NB * DK >= NT) ? (NB * DK / NT) : 1;  // channels per thread
    static constexpr int NITEM = NB * DK / CPT;       // (sub-block, channel group) items
    static constexpr int VPR = BV * (int)sizeof(T) / 16;              // 16-byte vectors per V row
    static constexpr int NVV = (C * VPR + NT - 1) / NT;               // V vectors per thread
    static constexpr int NCT = DK / 16;               // 16-row tiles of the state
    static constexpr int NVT = BV / 16;               // 16-column tiles of the state slice
    static constexpr int WPC = (NW > NCT) ? NW / NCT : 1;            // waves per state row-tile
    static constexpr int CTW = (NCT > NW) ? NCT / NW : 1;            // row-tiles per wave
    static constexpr int VTW = NVT / WPC;                            // column-tiles per wave
    static_assert(C == 64, "chunk size");
    static_assert(NITEM <= NT, "elementwise mapping");
    static_assert(CPT == 1 || CPT == 2 || CPT == 4, "channels per thread");
    static_assert(VTW >= 1 && NVT % WPC == 0, "state tiling");
    static_assert(DK % Path<T>::KS == 0 && C % Path<T>::KS == 0, "k steps");
};

template <typename T, int C, int DK, int BV>
struct PrefillSmem {
    typedef PrefillCfg<T, C, DK, BV> Cf;
    T Kr[C][Cf::LDK];      // K o e^{L}   (rows referenced to their sub-block start)
    T Qr[C][Cf::LDK];      // Q o e^{L}
    T Kd[C][Cf::LDK];      // K o e^{-L}  (diagonal-block columns)
    T KcT[DK][Cf::LDC];    // (K o e^{B - L})^T  (columns referenced to their sub-block end)
    T Tm[C][Cf::LDC];      // T = (I + A)^-1, lower triangular
    T P[C][Cf::LDC];       // Tril((Q o e^G)(K o e^-G)^T)
    T ST[BV][Cf::LDK];     // state slice, transposed, operand copy
    T RT[BV][Cf::LDC];     // R^T = (B(V - K e^G S))^T, then U^T
    T V[C][Cf::LDV];       // value slice, then the output staging tile
    float A[C][Cf::LDA];   // A, fp32
    float eB[Cf::NB][DK];  // e^{B_J}: decay across sub-block J
    float eE[Cf::NB][DK];  // e^{E_J}: decay from the chunk start to just before J
    float eT[Cf::NB][DK];  // decay from just after J to the chunk end
    float gam[DK];         // decay across the whole chunk
    float beta[C];
};

template <typename T, int CPT> struct ChanVec;
template <typename T> struct ChanVec<T, 1> { typedef T type; };
template <> struct ChanVec<bf16, 2> { typedef __bf16 type __attribute__((ext_vector_type(2))); };
template <> struct ChanVec<float, 2> { typedef f32x2 type; };
template <> struct ChanVec<bf16, 4> { typedef bf16x4 type; };
template <> struct ChanVec<float, 4> { typedef f32x4 type; };
template <int CPT> struct GVec;
template <> struct GVec<1> { typedef float type; };
template <> struct GVec<2> { typedef f32x2 type; };
template <> struct GVec<4> { typedef f32x4 type; };

// Raw inputs of one chunk held in registers (prefetched one chunk ahead).
template <typename T, int C, int DK, int BV>
struct ChunkRegs {
    typedef PrefillCfg<T, C, DK, BV> Cf;
    typename GVec<Cf::CPT>::type g[16];
    typename ChanVec<T, Cf::CPT>::type k[16], q[16];
    f32x4 v[Cf::NVV];
    float beta;
};

struct SeqView {
    int64_t bos, eos;   // token range of the sequence
    int head, H;
    int v0;             // first value column of the slice
};

template <typename T, int C, int DK, int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, C, DK, BV> &R, const SeqView &sv,
                                           int64_t t0, const T *__restrict__ q,
                                           const T *__restrict__ k, const T *__restrict__ v,
                                           const float *__restrict__ g,
                                           const float *__restrict__ beta, int DV)
{
    typedef PrefillCfg<T, C, DK, BV> Cf;
    typedef typename ChanVec<T, Cf::CPT>::type CV;
    typedef typename GVec<Cf::CPT>::type GV;
    const int t = threadIdx.x;
    if (t < Cf::NITEM) {
        const int I = t / (DK / Cf::CPT);
        const int c0 = (t % (DK / Cf::CPT)) * Cf::CPT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t tok = t0 + 16 * I + r;
            if (tok < sv.eos) {
                const int64_t off = (tok * sv.H + sv.head) * DK + c0;
                R.g[r] = *reinterpret_cast<const GV *>(g + off);
                R.k[r] = *reinterpret_cast<const CV *>(k + off);
                R.q[r] = *reinterpret_cast<const CV *>(q + off);
            } else {
                R.g[r] = GV{};
                R.k[r] = CV{};
                R.q[r] = CV{};
            }
        }
    }
#pragma unroll
    for (int m = 0; m < Cf::NVV; ++m) {
        const int vi = t + Cf::NT * m;
        const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
        const int64_t tok = t0 + row;
        R.v[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < C && tok < sv.eos) {
            const T *p = v + (tok * sv.H + sv.head) * DV + sv.v0 + cv * (16 / (int)sizeof(T));
            R.v[m] = *reinterpret_cast<const f32x4 *>(p);
        }
    }
    R.beta = 0.f;
    if (t < C && t0 + t < sv.eos) R.beta = beta[(t0 + t) * sv.H + sv.head];
}

template <typename V> __device__ __forceinline__ float vget(const V &x, int i) { return x[i]; }
__device__ __forceinline__ float vget(const float &x, int) { return x; }
__device__ __forceinline__ float vget(const bf16 &x, int) { return (float)x; }

// Sub-block-local decay factors and the operand tiles derived from them.
template <typename T, int C, int DK, int BV>
__device__ __forceinline__ void elementwise(const ChunkRegs<T, C, DK, BV> &R,
                                            PrefillSmem<T, C, DK, BV> &sm)
{
    typedef PrefillCfg<T, C, DK, BV> Cf;
    const int t = threadIdx.x;
    if (t < Cf::NITEM) {
        const int I = t / (DK / Cf::CPT);
        const int c0 = (t % (DK / Cf::CPT)) * Cf::CPT;
#pragma unroll
        for (int cc = 0; cc < Cf::CPT; ++cc) {
            const int c = c0 + cc;
            float a[16], eL[16], sfx[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = __expf(vget(R.g[r], cc));
            eL[0] = a[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) eL[r] = eL[r - 1] * a[r];
            sfx[15] = 1.f;
#pragma unroll
            for (int r = 14; r >= 0; --r) sfx[r] = sfx[r + 1] * a[r + 1];
            const float eb = eL[15];
            const float rb = __builtin_amdgcn_rcpf(eb);     // <= e^80
            T kc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float kk = vget(R.k[r], cc), qq = vget(R.q[r], cc);
                sm.Kr[16 * I + r][c] = from_f32<T>(kk * eL[r]);
                sm.Qr[16 * I + r][c] = from_f32<T>(qq * eL[r]);
                sm.Kd[16 * I + r][c] = from_f32<T>((kk * sfx[r]) * rb);
                kc[r] = from_f32<T>(kk * sfx[r]);
            }
            constexpr int EPV = 16 / (int)sizeof(T);   // elements per 16-byte store
#pragma unroll
            for (int r = 0; r < 16; r += EPV) {   // 16 contiguous tokens of one channel
                f32x4 w;
                __builtin_memcpy(&w, &kc[r], 16);
                *reinterpret_cast<f32x4 *>(&sm.KcT[c][16 * I + r]) = w;
            }
            sm.eB[I][c] = eb;
        }
    }
    if (t < C) sm.beta[t] = R.beta;
#pragma unroll
    for (int m = 0; m < Cf::NVV; ++m) {
        const int vi = t + Cf::NT * m;
        const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
        if (row < C)
            *reinterpret_cast<f32x4 *>(&sm.V[row][cv * (16 / (int)sizeof(T))]) = R.v[m];
    }
}

// B-operand fragment of the column factor for pair (I, J), channels kc.. .
template <typename T, int C, int DK, int BV>
__device__ __forceinline__ typename Path<T>::frag col_frag(const PrefillSmem<T, C, DK, BV> &sm,
                                                           int I, int J, int row, int kc)
{
    typedef Path<T> PT;
    typename PT::frag f = load_frag<T>(&sm.Kd[row][kc]);
    if (I == J) return f;
    float x[PT::KPL];
    PT::unpack(f, x);
#pragma unroll
    for (int e = 0; e < PT::KPL; ++e) {
        float s = x[e] * sm.eB[J][kc + e];                 // -> K o e^{B_J - L}, <= |k|
        for (int m = J + 1; m < I; ++m) s *= sm.eB[m][kc + e];
        x[e] = s;
    }
    return PT::pack(x);
}

template <typename T, int C, int DK, int BV, int DV>
__global__ __launch_bounds__(4 * C, 1) void prefill_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ s0, const int32_t *__restrict__ cu_seqlens, int num_seqs,
    int64_t seq_len, int H, T *__restrict__ o, float *__restrict__ sfinal)
{
    typedef PrefillCfg<T, C, DK, BV> Cf;
    typedef Path<T> PT;
    typedef PrefillSmem<T, C, DK, BV> Sm;
    constexpr int NB = Cf::NB, NW = Cf::NW, NT = Cf::NT;
    constexpr int NSLICE = DV / BV;
    __shared__ __align__(16) unsigned char smem_raw[sizeof(Sm)];
    Sm &sm = *reinterpret_cast<Sm *>(smem_raw);

    // ---- work item: (sequence, head, value slice), slices of a head adjacent
    // and, when the count allows, on the same XCD (blocks are dealt to the 8
    // XCDs round-robin) so that they share q, k, g through that XCD's L2.
    const int64_t nwork = (int64_t)num_seqs * H * NSLICE;
    int64_t b = blockIdx.x, w = b;
    if (nwork % 8 == 0) w = (b % 8) * (nwork / 8) + b / 8;
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

    // ---- state slice in registers, D layout: tile (ct, vt) holds
    // S[16 ct + 4 grp + i][16 vt + n16]
    const int ct0 = (wv / Cf::WPC) * Cf::CTW;
    const int vt0 = (wv % Cf::WPC) * Cf::VTW;
    f32x4 S[Cf::CTW][Cf::VTW];
    const int64_t sbase = ((int64_t)seq * H + head) * (int64_t)(DK * DV) + sv.v0;
#pragma unroll
    for (int a = 0; a < Cf::CTW; ++a)
#pragma unroll
        for (int bq = 0; bq < Cf::VTW; ++bq) {
            const int ct = ct0 + a, vt = vt0 + bq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ct + 4 * grp + i, cidx = 16 * vt + n16;
                S[a][bq][i] = s0 ? s0[sbase + (int64_t)r * DV + cidx] : 0.f;
            }
        }

    // constant zero blocks above the diagonal of Tm and P
    for (int e = t; e < C * C; e += NT) {
        const int r = e / C, j = e % C;
        if ((j >> 4) > (r >> 4)) {
            sm.Tm[r][j] = from_f32<T>(0.f);
            sm.P[r][j] = from_f32<T>(0.f);
        }
    }
    // operand copy of the state
#pragma unroll
    for (int a = 0; a < Cf::CTW; ++a)
#pragma unroll
        for (int bq = 0; bq < Cf::VTW; ++bq)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.ST[16 * (vt0 + bq) + n16][16 * (ct0 + a) + 4 * grp + i] =
                    from_f32<T>(S[a][bq][i]);

    const int64_t nchunks = (sv.eos - sv.bos + C - 1) / C;
    ChunkRegs<T, C, DK, BV> R;
    if (nchunks > 0) load_chunk(R, sv, sv.bos, q, k, v, g, beta, DV);

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = sv.bos + ch * C;
        elementwise(R, sm);
        __syncthreads();
        if (ch + 1 < nchunks) load_chunk(R, sv, t0 + C, q, k, v, g, beta, DV);

        // ---- chunk-level decay factors from the sub-block totals
        for (int c = t; c < DK; c += NT) {
            float e = 1.f;
#pragma unroll
            for (int J = 0; J < NB; ++J) { sm.eE[J][c] = e; e *= sm.eB[J][c]; }
            sm.gam[c] = e;
            float f = 1.f;
#pragma unroll
            for (int J = NB - 1; J >= 0; --J) { sm.eT[J][c] = f; f *= sm.eB[J][c]; }
        }

        // ---- A and P, 16x16 blocks (I, J <= I); pairs dealt round-robin to waves
        for (int p = wv; p < NB * (NB + 1) / 2; p += NW) {
            int I = 0, rem = p;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / PT::KS; ++ks) {
                const int kc = ks * PT::KS + grp * PT::KPL;
                const typename PT::frag ak = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
                const typename PT::frag aq = load_frag<T>(&sm.Qr[16 * I + n16][kc]);
                const typename PT::frag bk = col_frag(sm, I, J, 16 * J + n16, kc);
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
        __syncthreads();

        // ---- T = (I + A)^-1: diagonal blocks by forward substitution (fp32)
        {
            const int I = wv;
            float Tc[16];
            const int c = n16;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) acc -= sm.A[16 * I + r][16 * I + j] * Tc[j];
                Tc[r] = acc;
            }
            if (grp == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sm.Tm[16 * I + r][16 * I + c] = from_f32<T>(Tc[r]);
            }
        }
        __syncthreads();
        // off-diagonal blocks level by level: T_IJ = -T_II sum_{J<=M<I} A_IM T_MJ
        for (int d = 1; d < NB; ++d) {
            const int I = wv, J = wv - d;
            if (J >= 0) {
                f32x4 X = zero4();
                for (int M = J; M < I; ++M) {
                    float a4[4], b4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a4[i] = sm.A[16 * I + n16][16 * M + 4 * grp + i];
                        b4[i] = to_f32(sm.Tm[16 * M + 4 * grp + i][16 * J + n16]);
                    }
                    X = PT::mma16(a4, b4, X);
                }
                float a4[4], b4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a4[i] = to_f32(sm.Tm[16 * I + n16][16 * I + 4 * grp + i]);
                    b4[i] = X[i];
                }
                const f32x4 Y = PT::mma16(a4, b4, zero4());
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.Tm[16 * I + 4 * grp + i][16 * J + n16] = from_f32<T>(-Y[i]);
            }
            __syncthreads();
        }

        // ---- state-dependent part.  Wave wv owns token rows of sub-block I = wv.
        constexpr int NVTA = BV / 16;
        f32x4 accZ[NVTA];
        {
            const int I = wv;
            f32x4 accY[NVTA];
#pragma unroll
            for (int vt = 0; vt < NVTA; ++vt) { accY[vt] = zero4(); accZ[vt] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < DK / PT::KS; ++ks) {
                const int kc = ks * PT::KS + grp * PT::KPL;
                typename PT::frag ak = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
                typename PT::frag aq = load_frag<T>(&sm.Qr[16 * I + n16][kc]);
                if (I > 0) {   // rows referenced to the chunk start: times e^{E_I}
                    float xk[PT::KPL], xq[PT::KPL];
                    PT::unpack(ak, xk);
                    PT::unpack(aq, xq);
#pragma unroll
                    for (int e = 0; e < PT::KPL; ++e) {
                        const float f = sm.eE[I][kc + e];
                        xk[e] *= f;
                        xq[e] *= f;
                    }
                    ak = PT::pack(xk);
                    aq = PT::pack(xq);
                }
#pragma unroll
                for (int vt = 0; vt < NVTA; ++vt) {
                    const typename PT::frag bs = load_frag<T>(&sm.ST[16 * vt + n16][kc]);
                    accY[vt] = PT::mma(ak, bs, accY[vt]);
                    accZ[vt] = PT::mma(aq, bs, accZ[vt]);
                }
            }
            // R = B (V - Y), stored transposed
#pragma unroll
            for (int vt = 0; vt < NVTA; ++vt) {
                T rv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * grp + i;
                    rv[i] = from_f32<T>(sm.beta[r] * (to_f32(sm.V[r][16 * vt + n16]) - accY[vt][i]));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.RT[16 * vt + n16][16 * I + 4 * grp + i] = rv[i];
            }
        }
        __syncthreads();
        // U = T R  (rows of sub-block I; T is zero right of block I)
        f32x4 accU[NVTA];
        {
            const int I = wv;
#pragma unroll
            for (int vt = 0; vt < NVTA; ++vt) accU[vt] = zero4();
            const int nks = (16 * (I + 1) + PT::KS - 1) / PT::KS;
            for (int ks = 0; ks < nks; ++ks) {
                const int kj = ks * PT::KS + grp * PT::KPL;
                const typename PT::frag at = load_frag<T>(&sm.Tm[16 * I + n16][kj]);
#pragma unroll
                for (int vt = 0; vt < NVTA; ++vt)
                    accU[vt] = PT::mma(at, load_frag<T>(&sm.RT[16 * vt + n16][kj]), accU[vt]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int vt = 0; vt < NVTA; ++vt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.RT[16 * vt + n16][16 * wv + 4 * grp + i] = from_f32<T>(accU[vt][i]);
        __syncthreads();

        // O = Z + P U  -> staging tile (V region, consumed above)
        {
            const int I = wv;
            const int nks = (16 * (I + 1) + PT::KS - 1) / PT::KS;
            for (int ks = 0; ks < nks; ++ks) {
                const int kj = ks * PT::KS + grp * PT::KPL;
                const typename PT::frag ap = load_frag<T>(&sm.P[16 * I + n16][kj]);
#pragma unroll
                for (int vt = 0; vt < NVTA; ++vt)
                    accZ[vt] = PT::mma(ap, load_frag<T>(&sm.RT[16 * vt + n16][kj]), accZ[vt]);
            }
#pragma unroll
            for (int vt = 0; vt < NVTA; ++vt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.V[16 * I + 4 * grp + i][16 * vt + n16] = from_f32<T>(accZ[vt][i]);
        }

        // S' = Diag(gamma) S + (K o e^{G_n - G})^T U
#pragma unroll
        for (int a = 0; a < Cf::CTW; ++a) {
            const int ct = ct0 + a;
#pragma unroll
            for (int bq = 0; bq < Cf::VTW; ++bq)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[a][bq][i] *= sm.gam[16 * ct + 4 * grp + i];
#pragma unroll
            for (int ks = 0; ks < C / PT::KS; ++ks) {
                const int kj = ks * PT::KS + grp * PT::KPL;
                const int J = kj >> 4;
                const int c = 16 * ct + n16;
                typename PT::frag ak = load_frag<T>(&sm.KcT[c][kj]);
                {
                    float x[PT::KPL];
                    PT::unpack(ak, x);
                    const float f = sm.eT[J][c];
#pragma unroll
                    for (int e = 0; e < PT::KPL; ++e) x[e] *= f;
                    ak = PT::pack(x);
                }
#pragma unroll
                for (int bq = 0; bq < Cf::VTW; ++bq)
                    S[a][bq] = PT::mma(ak, load_frag<T>(&sm.RT[16 * (vt0 + bq) + n16][kj]),
                                       S[a][bq]);
            }
        }
        __syncthreads();   // all reads of RT, KcT, ST, V(O) staging writes done

        // operand copy of the new state; coalesced write of the output rows
#pragma unroll
        for (int a = 0; a < Cf::CTW; ++a)
#pragma unroll
            for (int bq = 0; bq < Cf::VTW; ++bq)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.ST[16 * (vt0 + bq) + n16][16 * (ct0 + a) + 4 * grp + i] =
                        from_f32<T>(S[a][bq][i]);
        for (int vi = t; vi < C * Cf::VPR; vi += NT) {
            const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
            const int64_t tok = t0 + row;
            if (tok < sv.eos) {
                T *p = o + (tok * H + head) * DV + sv.v0 + cv * (16 / (int)sizeof(T));
                *reinterpret_cast<f32x4 *>(p) =
                    *reinterpret_cast<const f32x4 *>(&sm.V[row][cv * (16 / (int)sizeof(T))]);
            }
        }
        __syncthreads();
    }

    if (sfinal) {
#pragma unroll
        for (int a = 0; a < Cf::CTW; ++a)
#pragma unroll
            for (int bq = 0; bq < Cf::VTW; ++bq)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * (ct0 + a) + 4 * grp + i, cidx = 16 * (vt0 + bq) + n16;
                    sfinal[sbase + (int64_t)r * DV + cidx] = S[a][bq][i];
                }
    }
}

template <typename T, int C, int D, int BV>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int H, void *o, float *sf,
                                   hipStream_t stream)
{
    typedef PrefillCfg<T, C, D, BV> Cf;
    const int64_t nwork = (int64_t)num_seqs * H * (D / BV);
    if (nwork == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_kernel<T, C, D, BV, D>), dim3((unsigned)nwork), dim3(Cf::NT), 0,
                       stream, (const T *)q, (const T *)k, (const T *)v, g, beta, s0, cu,
                       num_seqs, seq_len, H, (T *)o, sf);
    return hipGetLastError();
}

// Value-slice width: split d_v in two when there are too few (sequence, head)
// pairs to fill the 256 compute units.
hipError_t launch_prefill(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int H, int d, int chunk, bool is_bf16, void *o,
                          float *sf, hipStream_t stream)
{
    if (chunk != 64) return hipErrorInvalidValue;
    if (is_bf16) {
        switch (d) {
            case 32:
                return launch_prefill_t<bf16, 64, 32, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                          seq_len, H, o, sf, stream);
            case 64:
                return launch_prefill_t<bf16, 64, 64, 64>(q, k, v, g, beta, s0, cu, num_seqs,
                                                          seq_len, H, o, sf, stream);
            case 128:
                return launch_prefill_t<bf16, 64, 128, 64>(q, k, v, g, beta, s0, cu, num_seqs,
                                                           seq_len, H, o, sf, stream);
        }
    } else {
        switch (d) {
            case 32:
                return launch_prefill_t<float, 64, 32, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                           seq_len, H, o, sf, stream);
            case 64:
                return launch_prefill_t<float, 64, 64, 32>(q, k, v, g, beta, s0, cu, num_seqs,
                                                           seq_len, H, o, sf, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
