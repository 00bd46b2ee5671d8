// Fused chunkwise KDA prefill on gfx950 (CDNA4).
//
// What is computed (page "Notations mathematiques", table "Attention et KDA"):
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     alpha_t = exp(g_t),  o_t = S_t^T q_t,
// evaluated block by block: serial across chunks of C = 64 tokens, parallel
// inside a chunk ("Glossaire", entry "Chunkwise"; it is an exact rewrite).
// Inside a chunk of n <= C tokens entering with state S, with G the in-chunk
// inclusive cumulative sum of g (exp(G_r) is the cumulative decay gamma^{1->r}
// of the notation table) and B = Diag(beta):
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
// (N strictly lower 16 x 16, so N^16 = 0), evaluated with matrix-core products,
// and U follows by block forward substitution
//     U_I = (I + A_II)^-1 (R_I - sum_{J<I} A_IJ U_J),   R = B (V - (K o e^G) S).
//
// Decay factors never leave the float range.  With L the sub-block-local
// inclusive cumulative sum of g and B_J the total log decay of sub-block J:
//   rows of sub-block I:        e^{L_r}                          in [e^-80, 1]
//   diagonal-block columns:     e^{-L_j}                         in [1, e^80]
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
// fp32 accumulation; operands are rounded to the input type.  The next chunk's
// raw inputs are loaded into registers one chunk ahead.
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
    static constexpr int LD16 = 16 + PAD;             // 16 x 16 tiles
    // elementwise items: (sub-block, 4 channels, 4 rows); the four row
    // quarters of one channel quad sit in the four 16-lane groups of a wave
    static constexpr int QPW = (DK / 4 < 16) ? DK / 4 : 16;   // quads per lane group
    static constexpr int WPB = (DK / 64 > 1) ? DK / 64 : 1;   // waves per sub-block
    static constexpr int EWAVES = NB * WPB;                   // waves doing elementwise
    static constexpr int VPR = BV * (int)sizeof(T) / 16;      // 16-byte vectors per V row
    static constexpr int NVV = (C * VPR + NT - 1) / NT;
    static constexpr int NCT = DK / 16;               // state row tiles
    static constexpr int NVT = BV / 16;               // state column tiles
    static constexpr int SWPC = (NCT >= 4) ? 1 : 4 / NCT;   // state waves per row tile
    static constexpr int SCT = (NCT >= 4) ? NCT / 4 : 1;    // row tiles per state wave
    static constexpr int SVT = NVT / SWPC;                   // column tiles per state wave
    static_assert(EWAVES <= NW, "elementwise mapping");
    static_assert(SVT >= 1 && NVT % SWPC == 0, "state tiling");
    static_assert(DK % Path<T>::KS == 0 && C % Path<T>::KS == 0, "k steps");
};

template <typename T, int DK, int BV>
struct Smem64 {
    typedef Cfg64<T, DK, BV> Cf;
    T Kr[Cf::C][Cf::LDK];      // K o e^{L}        row operand
    T Qr[Cf::C][Cf::LDK];      // Q o e^{L}
    T Kc[Cf::C][Cf::LDK];      // K o e^{B - L}    column operand of blocks J < I
    T Kd[Cf::C][Cf::LDK];      // K o e^{-L}       column operand of diagonal blocks
    T P[Cf::C][Cf::LDC];       // Tril((Q o e^G)(K o e^-G)^T)
    T A[Cf::C][Cf::LDC];       // A (beta applied, strictly lower)
    T ST[BV][Cf::LDK];         // state slice, transposed operand copy
    T RT[BV][Cf::LDC];         // R^T, overwritten in place by U^T
    T V[Cf::C][BV];            // value slice
    T Tm[Cf::NB][16][Cf::LD16];      // diagonal blocks of (I + A)^-1
    T scr[4][2][16][Cf::LD16];       // per-wave N^2, N^4 for the diagonal inverses
    float eB[Cf::NB][DK];      // e^{B_J}
    float eE[Cf::NB + 1][DK];  // e^{E_J} = prod_{m<J} e^{B_m}; row NB: whole-chunk decay
    float eT[Cf::NB][DK];      // prod_{m>J} e^{B_m}
    float beta[Cf::C];
};

template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

// Raw inputs of one chunk, held in registers one chunk ahead: for the
// elementwise item of this thread, four rows of four channels of g, k, q;
// plus a share of the value slice and one beta.
template <typename T, int DK, int BV>
struct ChunkRegs {
    typedef Cfg64<T, DK, BV> Cf;
    f32x4 g[4];
    typename Quad<T>::type k[4], q[4];
    f32x4 v[Cf::NVV];
    float beta;
};

struct SeqView {
    int64_t bos, eos;   // token range of the sequence
    int head, H;
    int v0;             // first value column of the slice
};

// Elementwise item of thread t: sub-block I, channel quad c4 (channels
// 4 c4 .. 4 c4 + 3), row quarter qr (rows 4 qr .. 4 qr + 3 of the sub-block).
template <int DK, int QPW, int WPB>
__device__ __forceinline__ bool item_of(int t, int &I, int &c4, int &qr)
{
    const int w = t >> 6, l = t & 63;
    qr = l >> 4;
    const int qi = l & 15;
    I = w / WPB;
    c4 = (w % WPB) * QPW + qi;
    return qi < QPW && w < 4 * WPB;
}

// Offset (in elements) of row `row` of the chunk, clamped to the last row of
// the sequence: rows past the end read a valid address and are zeroed where
// the values are consumed.  Offsets are 32-bit and added to a wave-uniform
// base pointer, so that an access costs one VGPR.
__device__ __forceinline__ uint32_t row_off(int row, int64_t nvalid, int rowstride)
{
    const int r = row < nvalid ? row : (int)nvalid - 1;
    return (uint32_t)r * (uint32_t)rowstride;
}

// Loads are unconditional, so that no select on a loaded value makes the wave
// wait for it.  `parts` selects what to load (LOAD_G, LOAD_KQ, LOAD_VB) so that
// the next chunk's loads can be spread over the phases of the current one.
enum { LOAD_G = 1, LOAD_KQ = 2, LOAD_VB = 4, LOAD_ALL = 7 };

template <typename T, int DK, int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, DK, BV> &R, int parts, const SeqView &sv,
                                           int64_t t0, const T *__restrict__ q,
                                           const T *__restrict__ k, const T *__restrict__ v,
                                           const float *__restrict__ g,
                                           const float *__restrict__ beta, int DV)
{
    typedef Cfg64<T, DK, BV> Cf;
    typedef typename Quad<T>::type QV;
    const int t = threadIdx.x;
    const int64_t nvalid = sv.eos - t0;
    const int64_t cbase = (t0 * sv.H + sv.head) * DK;      // wave-uniform
    const int rs = sv.H * DK;                              // row stride, elements
    int I, c4, qr;
    if (item_of<DK, Cf::QPW, Cf::WPB>(t, I, c4, qr)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t off = row_off(16 * I + 4 * qr + r, nvalid, rs) + 4 * c4;
            if (parts & LOAD_G) R.g[r] = *reinterpret_cast<const f32x4 *>(g + cbase + off);
            if (parts & LOAD_KQ) {
                R.k[r] = *reinterpret_cast<const QV *>(k + cbase + off);
                R.q[r] = *reinterpret_cast<const QV *>(q + cbase + off);
            }
        }
    }
    if (parts & LOAD_VB) {
        const T *vb = v + (t0 * sv.H + sv.head) * DV + sv.v0;
#pragma unroll
        for (int m = 0; m < Cf::NVV; ++m) {
            const int vi = t + Cf::NT * m;
            const int row = (vi / Cf::VPR) < Cf::C ? vi / Cf::VPR : Cf::C - 1, cv = vi % Cf::VPR;
            R.v[m] = *reinterpret_cast<const f32x4 *>(vb + row_off(row, nvalid, sv.H * DV) +
                                                      cv * (16 / (int)sizeof(T)));
        }
        const float *bb = beta + t0 * sv.H + sv.head;
        R.beta = bb[row_off(t < Cf::C ? t : 0, nvalid, sv.H)];
    }
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

// Four consecutive elements, packed for one store.
template <typename T> __device__ __forceinline__ typename Quad<T>::type pack4(const float *x)
{
    typename Quad<T>::type r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = from_f32<T>(x[i]);
    return r;
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
    typedef typename Quad<T>::type QV;
    constexpr int C = Cf::C, NB = Cf::NB, NT = Cf::NT, KS = PT::KS, KPL = PT::KPL;
    constexpr int NSLICE = DV / BV;
    constexpr int NVT = Cf::NVT;
    __shared__ __align__(16) Sm sm;

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
    if (nchunks > 0) load_chunk(R, LOAD_ALL, sv, sv.bos, q, k, v, g, beta, DV);

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = sv.bos + ch * C;
        const int64_t nvalid = sv.eos - t0;              // rows of this chunk in the sequence
        const bool full = nvalid >= C;

        // ================= E: sub-block-local decays and operand tiles
        {
            int I, c4, qr;
            if (item_of<DK, Cf::QPW, Cf::WPB>(t, I, c4, qr)) {
                const int r0 = 16 * I + 4 * qr;
                float kr[4][4], qrw[4][4], kc[4][4], kd[4][4], ebv[4];
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) {
                    float a[4], pl[4], sl[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        a[r] = (full || r0 + r < nvalid) ? __expf(R.g[r][cc]) : 1.f;
                    pl[0] = a[0];
#pragma unroll
                    for (int r = 1; r < 4; ++r) pl[r] = pl[r - 1] * a[r];
                    sl[3] = 1.f;
#pragma unroll
                    for (int r = 2; r >= 0; --r) sl[r] = sl[r + 1] * a[r + 1];
                    // decays of the four row quarters of this sub-block
                    float qd[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) qd[j] = __shfl(pl[3], (lane & 15) + 16 * j);
                    float lead = 1.f, tail = 1.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (j < qr) lead *= qd[j];
                        if (j > qr) tail *= qd[j];
                    }
                    const float eb = ((qd[0] * qd[1]) * qd[2]) * qd[3];
                    const float rb = __builtin_amdgcn_rcpf(eb);     // <= e^80
                    ebv[cc] = eb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool in = full || r0 + r < nvalid;
                        const float kk = in ? to_f32(R.k[r][cc]) : 0.f;
                        const float qq = in ? to_f32(R.q[r][cc]) : 0.f;
                        const float eL = lead * pl[r];            // e^{L_r}
                        const float sfx = sl[r] * tail;           // e^{B - L_r}
                        kr[r][cc] = kk * eL;
                        qrw[r][cc] = qq * eL;
                        kc[r][cc] = kk * sfx;
                        kd[r][cc] = (kk * sfx) * rb;              // e^{-L_r}, <= e^80
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    *reinterpret_cast<QV *>(&sm.Kr[r0 + r][4 * c4]) = pack4<T>(kr[r]);
                    *reinterpret_cast<QV *>(&sm.Qr[r0 + r][4 * c4]) = pack4<T>(qrw[r]);
                    *reinterpret_cast<QV *>(&sm.Kc[r0 + r][4 * c4]) = pack4<T>(kc[r]);
                    *reinterpret_cast<QV *>(&sm.Kd[r0 + r][4 * c4]) = pack4<T>(kd[r]);
                }
                if (qr == 0)
                    *reinterpret_cast<f32x4 *>(&sm.eB[I][4 * c4]) =
                        f32x4{ebv[0], ebv[1], ebv[2], ebv[3]};
            }
        }
        if (t < C) sm.beta[t] = t < nvalid ? R.beta : 0.f;     // beta = 0 masks rows past the end
#pragma unroll
        for (int m = 0; m < Cf::NVV; ++m) {
            const int vi = t + NT * m;
            const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
            if (row < C)
                *reinterpret_cast<f32x4 *>(&sm.V[row][cv * (16 / (int)sizeof(T))]) = R.v[m];
        }
        __syncthreads();   // ---------------------------------------------- B1
        const bool more = ch + 1 < nchunks;
        if (more) load_chunk(R, LOAD_G, sv, t0 + C, q, k, v, g, beta, DV);

        // ================= AP: 16x16 blocks (I, J <= I) of A and P, computed
        // transposed so that each lane ends with four consecutive columns of
        // one row
        for (int p = wv; p < NB * (NB + 1) / 2; p += Cf::NW) {
            int I = 0, rem = p;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / KS; ++ks) {
                const int kc = ks * KS + grp * KPL;
                typename PT::frag ac;
                if (I == J) {
                    ac = load_frag<T>(&sm.Kd[16 * J + n16][kc]);
                } else if (I == J + 1) {
                    ac = load_frag<T>(&sm.Kc[16 * J + n16][kc]);
                } else {                                       // times prod_{J<m<I} e^{B_m}
                    float x[KPL], f[KPL];
                    PT::unpack(load_frag<T>(&sm.Kc[16 * J + n16][kc]), x);
                    load_f32<KPL>(f, &sm.eB[J + 1][kc]);
                    if (I == J + 3) {
                        float f2[KPL];
                        load_f32<KPL>(f2, &sm.eB[J + 2][kc]);
#pragma unroll
                        for (int e = 0; e < KPL; ++e) f[e] *= f2[e];
                    }
#pragma unroll
                    for (int e = 0; e < KPL; ++e) x[e] *= f[e];
                    ac = PT::pack(x);
                }
                accA = PT::mma(ac, load_frag<T>(&sm.Kr[16 * I + n16][kc]), accA);
                accP = PT::mma(ac, load_frag<T>(&sm.Qr[16 * I + n16][kc]), accP);
            }
            // lane holds A[r][j], P[r][j] for r = 16 I + n16, j = 16 J + 4 grp + i
            const int r = 16 * I + n16;
            const float br = sm.beta[r];
            float va[4], vp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int jl = 4 * grp + i;
                va[i] = (I != J || jl < n16) ? accA[i] * br : 0.f;
                vp[i] = (I != J || jl <= n16) ? accP[i] : 0.f;
            }
            *reinterpret_cast<QV *>(&sm.A[r][16 * J + 4 * grp]) = pack4<T>(va);
            *reinterpret_cast<QV *>(&sm.P[r][16 * J + 4 * grp]) = pack4<T>(vp);
        }
        // decay tables: e^{E_J}, whole-chunk decay, decay after J
        for (int e = t; e < (2 * NB + 1) * DK; e += NT) {
            const int J = e / DK, c = e % DK;
            float f = 1.f;
            if (J <= NB) {
#pragma unroll
                for (int m = 0; m < NB; ++m)
                    if (m < J) f *= sm.eB[m][c];
                sm.eE[J][c] = f;
            } else {
#pragma unroll
                for (int m = 0; m < NB; ++m)
                    if (m > J - NB - 1) f *= sm.eB[m][c];
                sm.eT[J - NB - 1][c] = f;
            }
        }
        __syncthreads();   // ---------------------------------------------- B2
        if (more) load_chunk(R, LOAD_KQ, sv, t0 + C, q, k, v, g, beta, DV);

        f32x4 accZ[NVT];
        if (state_wave) {
            // ============= diagonal-block inverses (I + N)^-1, N = A_II
            const int I = wv;
            float dN[4], aN[4], aN2[4], aN4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dN[i] = to_f32(sm.A[16 * I + 4 * grp + i][16 * I + n16]);
                aN[i] = to_f32(sm.A[16 * I + n16][16 * I + 4 * grp + i]);
            }
            const f32x4 N2 = PT::mma16(aN, dN, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.scr[I][0][4 * grp + i][n16] = from_f32<T>(N2[i]);
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) aN2[i] = to_f32(sm.scr[I][0][n16][4 * grp + i]);
            float bN2[4] = {N2[0], N2[1], N2[2], N2[3]};
            const f32x4 N4 = PT::mma16(aN2, bN2, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.scr[I][1][4 * grp + i][n16] = from_f32<T>(N4[i]);
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) aN4[i] = to_f32(sm.scr[I][1][n16][4 * grp + i]);
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
            for (int i = 0; i < 4; ++i) sm.Tm[I][4 * grp + i][n16] = from_f32<T>(X[i]);
        } else {
            // ============= state read-out for row block I: Y = K e^G S, Z = Q e^G S
            const int I = I_row;
            f32x4 accY[NVT];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) { accY[vt] = zero4(); accZ[vt] = zero4(); }
#pragma unroll
            for (int ks = 0; ks < DK / KS; ++ks) {
                const int kc = ks * KS + grp * KPL;
                typename PT::frag ak = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
                typename PT::frag aq = load_frag<T>(&sm.Qr[16 * I + n16][kc]);
                if (I > 0) {                                     // times e^{E_I}
                    float xk[KPL], xq[KPL], f[KPL];
                    PT::unpack(ak, xk);
                    PT::unpack(aq, xq);
                    load_f32<KPL>(f, &sm.eE[I][kc]);
#pragma unroll
                    for (int e = 0; e < KPL; ++e) { xk[e] *= f[e]; xq[e] *= f[e]; }
                    ak = PT::pack(xk);
                    aq = PT::pack(xq);
                }
#pragma unroll
                for (int vt = 0; vt < NVT; ++vt) {
                    const typename PT::frag bs = load_frag<T>(&sm.ST[16 * vt + n16][kc]);
                    accY[vt] = PT::mma(ak, bs, accY[vt]);
                    accZ[vt] = PT::mma(aq, bs, accZ[vt]);
                }
            }
            // R = B (V - Y), stored transposed
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                float rv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * grp + i;
                    rv[i] = sm.beta[r] * (to_f32(sm.V[r][16 * vt + n16]) - accY[vt][i]);
                }
                *reinterpret_cast<QV *>(&sm.RT[16 * vt + n16][16 * I + 4 * grp]) = pack4<T>(rv);
            }
        }
        __syncthreads();   // ---------------------------------------------- B3
        if (more) load_chunk(R, LOAD_VB, sv, t0 + C, q, k, v, g, beta, DV);

        if (!state_wave) {
            // ============= forward substitution U_I = T_II (R_I - sum_{J<I} A_IJ U_J),
            // one value-column tile at a time; U^T overwrites R^T in place
            for (int vt = I_row; vt < NVT; vt += 4) {
                f32x4 X[NB], Ub[NB];
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        X[I][i] = to_f32(sm.RT[16 * vt + n16][16 * I + 4 * grp + i]);
#pragma unroll
                for (int I = 0; I < NB; ++I) {
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        float aA[4], bU[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            aA[i] = -to_f32(sm.A[16 * I + n16][16 * J + 4 * grp + i]);
                            bU[i] = Ub[J][i];
                        }
                        X[I] = PT::mma16(aA, bU, X[I]);
                    }
                    float aT[4], bX[4] = {X[I][0], X[I][1], X[I][2], X[I][3]};
#pragma unroll
                    for (int i = 0; i < 4; ++i) aT[i] = to_f32(sm.Tm[I][n16][4 * grp + i]);
                    Ub[I] = PT::mma16(aT, bX, zero4());
                }
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    float u4[4] = {Ub[I][0], Ub[I][1], Ub[I][2], Ub[I][3]};
                    *reinterpret_cast<QV *>(&sm.RT[16 * vt + n16][16 * I + 4 * grp]) = pack4<T>(u4);
                }
            }
        }
        __syncthreads();   // ---------------------------------------------- B4

        if (state_wave) {
            // ============= S' = Diag(gamma) S + (K o e^{G_n - G})^T U
#pragma unroll
            for (int a = 0; a < Cf::SCT; ++a) {
                const int c = 16 * (ct0 + a) + n16;
                typename PT::frag kb[C / KS];                    // (K o e^{G_n - G})^T
#pragma unroll
                for (int ks = 0; ks < C / KS; ++ks) {
                    const int kj = ks * KS + grp * KPL;
                    const float f = sm.eT[kj >> 4][c];
                    float x[KPL];
#pragma unroll
                    for (int e = 0; e < KPL; ++e) x[e] = to_f32(sm.Kc[kj + e][c]) * f;
                    kb[ks] = PT::pack(x);
                }
                float gam[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) gam[i] = sm.eE[NB][16 * (ct0 + a) + 4 * grp + i];
#pragma unroll
                for (int bq = 0; bq < Cf::SVT; ++bq) {
                    f32x4 acc = S[a][bq];
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] *= gam[i];
#pragma unroll
                    for (int ks = 0; ks < C / KS; ++ks) {
                        const int kj = ks * KS + grp * KPL;
                        acc = PT::mma(kb[ks], load_frag<T>(&sm.RT[16 * (vt0 + bq) + n16][kj]),
                                      acc);
                    }
                    S[a][bq] = acc;
                    float s4[4] = {acc[0], acc[1], acc[2], acc[3]};
                    *reinterpret_cast<QV *>(
                        &sm.ST[16 * (vt0 + bq) + n16][16 * (ct0 + a) + 4 * grp]) = pack4<T>(s4);
                }
            }
        } else {
            // ============= O = Z + P U for row block I, written straight to o
            const int I = I_row;
            const int nks = (16 * (I + 1) + KS - 1) / KS;
            T *ob = o + (t0 * H + head) * DV + sv.v0;         // wave-uniform
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
                    const int row = 16 * I + 4 * grp + i;
                    if (row < nvalid)
                        ob[(uint32_t)row * (uint32_t)(H * DV) + 16 * vt + n16] =
                            from_f32<T>(acc[i]);
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
