// Two-pass chunkwise KDA prefill on gfx950 (CDNA4): a chunk-parallel intra
// pass and a persistent state pass.
//
// The recurrence (page "Notations mathematiques", table "Attention et KDA"):
//     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//     alpha_t = exp(g_t),  o_t = S_t^T q_t.
// Chunks of C = 64 or 128 tokens ("Dimensions du modele", row C) start at each
// sequence start.  Inside a chunk of n <= C tokens entering with state S, with
// G the in-chunk inclusive cumulative sum of g and B = Diag(beta)
// ("Glossaire", entries "Chunkwise" and "UT"):
//     A  = StrictTril( B (K o e^G)(K o e^-G)^T ),   T = (I + A)^-1
//     U  = T B (V - (K o e^G) S)
//     O  = (Q o e^G) S + Tril((Q o e^G)(K o e^-G)^T) U
//     S' = Diag(e^{G_n}) S + (K o e^{G_n - G})^T U
// Everything that does not depend on S is a function of the chunk alone, so it
// is formed for every chunk at once by the intra pass, which writes one
// packet per (chunk, head) to the workspace:
//     Kg = K o e^G, Qg = Q o e^G, Kbar^T = (K o e^{G_n - G})^T, TB = T B,
//     P = Tril((Q o e^G)(K o e^-G)^T), gamma = e^{G_n}.
// The state pass then walks the chunks of each (sequence, head, slice of BV
// value columns) in order, with the fp32 state in registers:
//     Y^T = S^T Kg^T, Z^T = S^T Qg^T, R = V - Y, U = TB R,
//     O^T = Z^T + U^T P^T, S' = gamma o S + Kbar^T U.
// U is carried as two bf16 halves (hi + lo) for bf16 inputs, so the products
// that use it see U to about 16 bits.
//
// Decays inside the intra pass follow the same sub-block scheme as the fused
// kernel: 16-token sub-blocks with local references, each factor within
// [e^-80, e^80] (the bound of "Glossaire", entry "Decroissance bornee", for
// g_min = -5), the diagonal blocks of T from recursive block inversion.
//
// Packet layout (element type of the inputs; gamma fp32 at the end), every
// matrix-core operand stored in the order the consumer's lanes read it:
//   KG, QG  [NB row blocks][DK/KS k steps][64 lanes][KPL]   A fragments of Kg, Qg
//   KB      [DK/16 row tiles][64 lanes][C/KS k steps][KPL]  A fragments of Kbar^T
//   TB, TL, PP [block (I, J <= I), I-major][64 lanes][4]    16x16 blocks, A layout
//           (TL, bf16 only: the low half of T Diag(beta), TB + TL = T Diag(beta)
//           to about 16 bits)
//   gamma   [DK] fp32
// (lane (n16, grp) of an A fragment holds row n16 and the KPL consecutive k
// indices KS ks + KPL grp ..; of a 16x16 block, row n16 and columns 4 grp ..).
// The packet of chunk c of sequence s sits at slot floor(bos_s / C) + s + c:
// slots are distinct, increase with (s, c), and stay below
// ceil(total / C) + num_seqs, so the host sizes the workspace without reading
// the sequence lengths.
#include "kda_common.hpp"

#include <mutex>
#include <type_traits>

namespace kda {
namespace cp {

template <typename T> struct V2T;
template <> struct V2T<bf16> { typedef bf16x2 two; typedef bf16x4 four; };
template <> struct V2T<float> { typedef f32x2 two; typedef f32x4 four; };

// packet geometry
template <typename T, int DK, int C>
struct Pk {
    typedef Path<T> PT;
    static constexpr int KS = PT::KS, KPL = PT::KPL;
    static constexpr int NB = C / 16;
    static constexpr int NKD = DK / KS;   // k steps over channels
    static constexpr int NKC = C / KS;    // k steps over tokens
    static constexpr int NBLK = NB * (NB + 1) / 2;
    static constexpr int FRAG = 64 * KPL;
    static constexpr int64_t KG = 0;
    static constexpr int64_t QG = KG + (int64_t)C * DK;
    static constexpr int64_t KB = QG + (int64_t)C * DK;
    // bf16: T Diag(beta) is stored as two bf16 halves, hi (TB) and lo (TL)
    static constexpr bool TLO = std::is_same<T, bf16>::value;
    static constexpr int64_t TB = KB + (int64_t)C * DK;
    static constexpr int64_t TL = TB + (int64_t)NBLK * 256;
    static constexpr int64_t PP = TL + (TLO ? (int64_t)NBLK * 256 : 0);
    static constexpr int64_t END = PP + (int64_t)NBLK * 256;
    static constexpr int64_t GAM_BYTE = END * (int64_t)sizeof(T);
    static constexpr int64_t BYTES = ((GAM_BYTE + DK * 4 + 255) / 256) * 256;
    static_assert(C % 32 == 0 && DK % 32 == 0, "tile sizes");
};

__host__ __device__ inline int blk(int I, int J) { return I * (I + 1) / 2 + J; }

// Token range of sequence s (packed offsets, or s equal lengths).
struct SeqRange {
    int64_t bos, eos;
};
__device__ __forceinline__ SeqRange seq_range(const int32_t *cu, int64_t seq_len, int s)
{
    SeqRange r;
    if (cu) {
        r.bos = cu[s];
        r.eos = cu[s + 1];
    } else {
        r.bos = (int64_t)s * seq_len;
        r.eos = r.bos + seq_len;
    }
    return r;
}

// Slot -> (sequence, chunk).  key(s) = floor(bos_s / C) + s increases strictly
// with s; the slot belongs to the largest s with key(s) <= slot, as its chunk
// slot - key(s) when that chunk exists.  False for a slot no chunk uses.
__device__ __forceinline__ bool slot_chunk(int64_t slot, const int32_t *cu, int num_seqs,
                                           int64_t seq_len, int C, int &seq, int64_t &t0, int &nv)
{
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const SeqRange r = seq_range(cu, seq_len, mid);
        if (r.bos / C + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const SeqRange r = seq_range(cu, seq_len, lo);
    const int64_t c = slot - (r.bos / C + lo);
    seq = lo;
    t0 = r.bos + c * C;
    if (c < 0 || t0 >= r.eos) return false;
    const int64_t n = r.eos - t0;
    nv = n < C ? (int)n : C;
    return true;
}

// ===========================================================================
// Intra pass
// ===========================================================================
template <typename T, int DK, int C>
struct ICfg {
    typedef Pk<T, DK, C> P;
    static constexpr int NW = 16, NT = 1024;
    static constexpr int NB = C / 16;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD;
    static constexpr int WPB = DK / 32;                 // elementwise units per sub-block
    static constexpr int NUNIT = NB * WPB;              // a unit is one wave's worth
    static constexpr int UPW = (NUNIT + NW - 1) / NW;   // units per wave
    static constexpr int NPAIR = NB * (NB - 1) / 2;
    static constexpr int NTAB = (DK + 63) / 64;
    static constexpr int NJOB = NB + NPAIR + NTAB;
};

template <typename T, int DK, int C>
struct ISmem {
    typedef ICfg<T, DK, C> Cf;
    typedef typename V2T<T>::four Q4;   // one lane's share of a 16x16 block
    T Kr[C][Cf::LDK];    // K o e^{L}       row operand (sub-block reference)
    T Qr[C][Cf::LDK];    // Q o e^{L}
    T Kc[C][Cf::LDK];    // K o e^{B - L}   column operand
    Q4 An[Cf::NPAIR > 0 ? Cf::NPAIR : 1][64];   // -B A_IJ, I > J, A layout
    Q4 Tma[Cf::NB][64];  // (I + A_II)^-1, A layout
    Q4 Tmd[Cf::NB][64];  // the same, D layout
    float eB[Cf::NB][DK];    // e^{B_J}
    float eBr[Cf::NB][DK];   // e^{-B_J}
    float eTx[Cf::NB][DK];   // prod_{m > J} e^{B_m}
    float eE[Cf::NB][DK];    // prod_{m < J} e^{B_m}
    float beta[C];
};

// Raw inputs of one elementwise unit (sub-block I, 16 channel pairs, four row
// quarters) for the next item, and one beta.
template <typename T, int DK, int C>
struct IRegs {
    typedef ICfg<T, DK, C> Cf;
    typedef typename V2T<T>::two V2;
    f32x2 g[Cf::UPW][4];
    V2 k[Cf::UPW][4], q[Cf::UPW][4];
    float beta;
};

// Loads of one item (unconditional, rows clamped to the chunk's last valid
// row; they are masked where consumed).
template <bool OUT, typename T, int DK, int C>
__device__ __forceinline__ void i_load(IRegs<T, DK, C> &R, const T *__restrict__ q,
                                       const T *__restrict__ k, const float *__restrict__ g,
                                       const float *__restrict__ beta, int64_t t0, int nv, int head,
                                       int H)
{
    typedef ICfg<T, DK, C> Cf;
    typedef typename V2T<T>::two V2;
    const int t = threadIdx.x, wv = wave_id(), lane = t & 63;
    const int n16 = lane & 15, qr = lane >> 4;
    const int64_t rs = (int64_t)H * DK;
    const int64_t base = (t0 * H + head) * DK;
#pragma unroll
    for (int u = 0; u < Cf::UPW; ++u) {
        const int unit = wv + Cf::NW * u;
        if (Cf::NUNIT % Cf::NW == 0 || unit < Cf::NUNIT) {
            const int I = unit / Cf::WPB, cp = (unit % Cf::WPB) * 16 + n16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = min(16 * I + 4 * qr + r, nv - 1);
                const int64_t off = base + row * rs + 2 * cp;
                R.g[u][r] = *reinterpret_cast<const f32x2 *>(g + off);
                R.k[u][r] = *reinterpret_cast<const V2 *>(k + off);
                if (OUT) R.q[u][r] = *reinterpret_cast<const V2 *>(q + off);
            }
        }
    }
    R.beta = beta[(t0 + min(t < C ? t : 0, nv - 1)) * H + head];
}

// Elementwise phase: sub-block-local decays e^{L}, e^{B - L}, the block totals
// e^{B}, e^{-B}, and the operand tiles K o e^L, Q o e^L, K o e^{B - L}.
template <bool OUT, typename T, int DK, int C>
__device__ __forceinline__ void i_elementwise(ISmem<T, DK, C> &sm, const IRegs<T, DK, C> &R, int nv)
{
    typedef ICfg<T, DK, C> Cf;
    typedef typename V2T<T>::two V2;
    const int t = threadIdx.x, wv = wave_id();
    const int lp = __lane_id(), n16 = lp & 15, qr = lp >> 4;
#pragma unroll
    for (int u = 0; u < Cf::UPW; ++u) {
        const int unit = wv + Cf::NW * u;
        if (Cf::NUNIT % Cf::NW == 0 || unit < Cf::NUNIT) {
            const int I = unit / Cf::WPB, cp = (unit % Cf::WPB) * 16 + n16;
            const int r0 = 16 * I + 4 * qr;
            float eL[2][4], sx[2][4], rb[2], ebv[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                float a[4], pl[4], sl[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = r0 + r < nv ? __expf(R.g[u][r][cc]) : 1.f;
                pl[0] = a[0];
#pragma unroll
                for (int r = 1; r < 4; ++r) pl[r] = pl[r - 1] * a[r];
                sl[3] = 1.f;
#pragma unroll
                for (int r = 2; r >= 0; --r) sl[r] = sl[r + 1] * a[r + 1];
                float qd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) qd[j] = __shfl(pl[3], n16 + 16 * j);
                const float lead = ((qr > 0 ? qd[0] : 1.f) * (qr > 1 ? qd[1] : 1.f)) * (qr > 2 ? qd[2] : 1.f);
                const float tail = ((qr < 1 ? qd[1] : 1.f) * (qr < 2 ? qd[2] : 1.f)) * (qr < 3 ? qd[3] : 1.f);
                ebv[cc] = ((qd[0] * qd[1]) * qd[2]) * qd[3];
                rb[cc] = __builtin_amdgcn_rcpf(ebv[cc]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    eL[cc][r] = lead * pl[r];
                    sx[cc][r] = sl[r] * tail;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool in = r0 + r < nv;
                float kk[2], qq[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    kk[cc] = in ? to_f32(R.k[u][r][cc]) : 0.f;
                    qq[cc] = (OUT && in) ? to_f32(R.q[u][r][cc]) : 0.f;
                }
                V2 x;
                x[0] = from_f32<T>(kk[0] * eL[0][r]);
                x[1] = from_f32<T>(kk[1] * eL[1][r]);
                *reinterpret_cast<V2 *>(&sm.Kr[r0 + r][2 * cp]) = x;
                if (OUT) {
                    x[0] = from_f32<T>(qq[0] * eL[0][r]);
                    x[1] = from_f32<T>(qq[1] * eL[1][r]);
                    *reinterpret_cast<V2 *>(&sm.Qr[r0 + r][2 * cp]) = x;
                }
                x[0] = from_f32<T>(kk[0] * sx[0][r]);
                x[1] = from_f32<T>(kk[1] * sx[1][r]);
                *reinterpret_cast<V2 *>(&sm.Kc[r0 + r][2 * cp]) = x;
            }
            if (qr == 0) {
                *reinterpret_cast<f32x2 *>(&sm.eB[I][2 * cp]) = f32x2{ebv[0], ebv[1]};
                *reinterpret_cast<f32x2 *>(&sm.eBr[I][2 * cp]) = f32x2{rb[0], rb[1]};
            }
        }
    }
    if (t < C) sm.beta[t] = t < nv ? R.beta : 0.f;   // beta = 0 masks rows past the end
}

template <typename T> __device__ __forceinline__ void store_quad(T *dst, const float *x);
template <> __device__ __forceinline__ void store_quad<bf16>(bf16 *dst, const float *x)
{
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
    *reinterpret_cast<bf16x4 *>(dst) = r;
}
template <> __device__ __forceinline__ void store_quad<float>(float *dst, const float *x)
{
    *reinterpret_cast<f32x4 *>(dst) = f32x4{x[0], x[1], x[2], x[3]};
}

template <int KPL> __device__ __forceinline__ void load_fk(float *dst, const float *src)
{
    if constexpr (KPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < KPL; i += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(src + i);
            dst[i] = x[0]; dst[i + 1] = x[1]; dst[i + 2] = x[2]; dst[i + 3] = x[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < KPL; ++i) dst[i] = src[i];
    }
}

// TB_IJ = T_IJ Diag(beta) of one lane (A layout) into the packet: the value
// rounded to the input type, and for bf16 also the rounding remainder.
template <typename T, int DK, int C>
__device__ __forceinline__ void store_tb(T *__restrict__ pk, int I, int J, const float *tb)
{
    typedef Pk<T, DK, C> P;
    const int lp = __lane_id();
    store_quad<T>(pk + P::TB + blk(I, J) * 256 + 4 * lp, tb);
    if constexpr (P::TLO) {
        float lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lo[i] = tb[i] - to_f32(from_f32<T>(tb[i]));
        store_quad<T>(pk + P::TL + blk(I, J) * 256 + 4 * lp, lo);
    }
}

// Diagonal block I: A_II (both layouts), P_II, and (I + A_II)^-1 by recursive
// block inversion (D_2b = D_b - D_b F_b D_b with F_b the part of N = A_II in
// the lower-left b x b block of each 2b x 2b diagonal block).  P_II and
// TB_II = T_II Diag(beta) go to the packet; T_II to LDS in both layouts.
template <bool OUT, typename T, int DK, int C>
__device__ __forceinline__ void i_diag(ISmem<T, DK, C> &sm, int I, T *__restrict__ pk)
{
    typedef Path<T> PT;
    typedef Pk<T, DK, C> P;
    typedef typename PT::quad Q4;
    constexpr int KS = PT::KS, KPL = PT::KPL;
    const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
    f32x4 accAt = zero4(), accA = zero4(), accPt = zero4();
#pragma unroll
    for (int ks = 0; ks < DK / KS; ++ks) {
        const int kc = ks * KS + grp * KPL;
        typename PT::frag fd = load_frag<T>(&sm.Kc[16 * I + n16][kc]);
        {
            float x[KPL], f[KPL];
            PT::unpack(fd, x);
            load_fk<KPL>(f, &sm.eBr[I][kc]);
#pragma unroll
            for (int e = 0; e < KPL; ++e) x[e] *= f[e];
            fd = PT::pack(x);
        }
        const typename PT::frag fk = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
        accAt = PT::mma(fd, fk, accAt);   // [r = n16][j = 4 grp + i]
        accA = PT::mma(fk, fd, accA);     // [r = 4 grp + i][j = n16]
        if (OUT) accPt = PT::mma(fd, load_frag<T>(&sm.Qr[16 * I + n16][kc]), accPt);
    }
    const float br = sm.beta[16 * I + n16];
    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * I + 4 * grp]);
    float Na[4], Nd[4], pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int jl = 4 * grp + i;
        Na[i] = jl < n16 ? br * accAt[i] : 0.f;
        Nd[i] = n16 < jl ? b4[i] * accA[i] : 0.f;
        pv[i] = jl <= n16 ? accPt[i] : 0.f;
    }
    if (OUT) store_quad<T>(pk + P::PP + blk(I, I) * 256 + 4 * lp, pv);
    auto in_f = [](int r, int c, int bs) { return (r ^ c) < 2 * bs && (r & bs) && !(c & bs); };
    f32x4 Da, Dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int jl = 4 * grp + i;
        Da[i] = (jl == n16 ? 1.f : 0.f) - (in_f(n16, jl, 1) ? Na[i] : 0.f);
        Dd[i] = (jl == n16 ? 1.f : 0.f) - (in_f(jl, n16, 1) ? Nd[i] : 0.f);
    }
#pragma unroll
    for (int bs = 2; bs < 16; bs *= 2) {
        float Fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) Fa[i] = in_f(n16, 4 * grp + i, bs) ? Na[i] : 0.f;
        const Q4 da = PT::to_quad(Da);
        const Q4 yd = PT::to_quad(PT::mma16q(PT::to_quad(Fa), PT::to_quad(Dd), zero4()));  // F D
        Da -= PT::mma16q(yd, da, zero4());                                                   // D F D
        Dd -= PT::mma16q(da, yd, zero4());
    }
    sm.Tma[I][lp] = PT::to_quad(Da);
    sm.Tmd[I][lp] = PT::to_quad(Dd);
    float tb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tb[i] = Da[i] * b4[i];
    store_tb<T, DK, C>(pk, I, I, tb);
}

// Off-diagonal block (I, J < I) of A (stored negated with beta, to LDS) and of
// P (to the packet).  The column operand K o e^{B_J - L_j} is brought to the
// reference of row block I by prod_{J<m<I} e^{B_m} (at most 1).
template <bool OUT, typename T, int DK, int C>
__device__ __forceinline__ void i_pair(ISmem<T, DK, C> &sm, int I, int J, T *__restrict__ pk)
{
    typedef Path<T> PT;
    typedef Pk<T, DK, C> P;
    constexpr int KS = PT::KS, KPL = PT::KPL;
    const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int ks = 0; ks < DK / KS; ++ks) {
        const int kc = ks * KS + grp * KPL;
        typename PT::frag col = load_frag<T>(&sm.Kc[16 * J + n16][kc]);
        if (I > J + 1) {
            float x[KPL], f[KPL];
            PT::unpack(col, x);
            load_fk<KPL>(f, &sm.eB[J + 1][kc]);
            for (int m = J + 2; m < I; ++m) {
                float f2[KPL];
                load_fk<KPL>(f2, &sm.eB[m][kc]);
#pragma unroll
                for (int e = 0; e < KPL; ++e) f[e] *= f2[e];
            }
#pragma unroll
            for (int e = 0; e < KPL; ++e) x[e] *= f[e];
            col = PT::pack(x);
        }
        accA = PT::mma(col, load_frag<T>(&sm.Kr[16 * I + n16][kc]), accA);
        if (OUT) accP = PT::mma(col, load_frag<T>(&sm.Qr[16 * I + n16][kc]), accP);
    }
    // lane holds X[16 I + n16][16 J + 4 grp + i]
    const float nb = -sm.beta[16 * I + n16];
    float wa[4], wp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wa[i] = nb * accA[i];
        wp[i] = accP[i];
    }
    sm.An[I * (I - 1) / 2 + J][lp] = PT::to_quad(wa);
    if (OUT) store_quad<T>(pk + P::PP + blk(I, J) * 256 + 4 * lp, wp);
}

// Column block J of T = (I + A)^-1 below the diagonal, by block forward
// substitution: T_IJ = T_II sum_{J <= M < I} (-A_IM) T_MJ for I > J.  Written
// to the packet as TB_IJ = T_IJ Diag(beta_J).  T_MJ stays in registers in the
// D layout (the B operand of the next products); T_IJ is also formed in the A
// layout for the store.
template <typename T, int DK, int C>
__device__ __forceinline__ void i_tcol(ISmem<T, DK, C> &sm, int J, T *__restrict__ pk)
{
    typedef Path<T> PT;
    typedef Pk<T, DK, C> P;
    typedef typename PT::quad Q4;
    constexpr int NB = C / 16;
    const int lp = __lane_id(), grp = lp >> 4;
    const f32x4 bJ = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * J + 4 * grp]);
    Q4 Td[NB];
#pragma unroll
    for (int M = 0; M < NB; ++M)
        if (M == J) Td[M] = sm.Tmd[M][lp];
#pragma unroll
    for (int I = 1; I < NB; ++I) {
        if (I <= J) continue;
        f32x4 X = zero4();
#pragma unroll
        for (int M = 0; M < I; ++M)
            if (M >= J) X = PT::mma16q(sm.An[I * (I - 1) / 2 + M][lp], Td[M], X);
        const Q4 xq = PT::to_quad(X), ta = sm.Tma[I][lp];
        Td[I] = PT::to_quad(PT::mma16q(ta, xq, zero4()));
        const f32x4 Ta = PT::mma16q(xq, ta, zero4());
        float tb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tb[i] = Ta[i] * bJ[i];
        store_tb<T, DK, C>(pk, I, J, tb);
    }
}

// Decay tables of channel c: prod_{m > J} e^{B_m}, prod_{m < J} e^{B_m}, and
// the whole-chunk decay gamma (to the packet).
template <typename T, int DK, int C>
__device__ __forceinline__ void i_tables(ISmem<T, DK, C> &sm, int c, float *__restrict__ gam)
{
    constexpr int NB = C / 16;
    float f = 1.f;
#pragma unroll
    for (int m = NB - 1; m >= 0; --m) {
        sm.eTx[m][c] = f;
        f *= sm.eB[m][c];
    }
    gam[c] = f;
    f = 1.f;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        sm.eE[m][c] = f;
        f *= sm.eB[m][c];
    }
}

__device__ __forceinline__ bf16x8 i_tr8(const bf16 *x, int ld, int k0, int c0, int n16, int grp)
{
    typedef short s4 __attribute__((ext_vector_type(4)));
    const bf16 *p = x + (k0 + 8 * grp + (n16 >> 2)) * ld + c0 + 4 * (n16 & 3);
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)p);
    const s4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(p + 4 * ld));
    const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Copy-out of Kg, Qg (from the row tiles times prod_{m<I} e^{B_m}) and Kbar^T
// (from the column tile times prod_{m>J} e^{B_m}) in the packet's fragment
// order, 16 bytes (bf16) or 4 bytes (fp32) a lane.
template <bool OUT, typename T, int DK, int C>
__device__ __forceinline__ void i_copyout(ISmem<T, DK, C> &sm, T *__restrict__ pk)
{
    typedef Path<T> PT;
    typedef Pk<T, DK, C> P;
    constexpr int KS = PT::KS, KPL = PT::KPL, NKD = P::NKD, NKC = P::NKC;
    constexpr int NT = ICfg<T, DK, C>::NT;
    const int t = threadIdx.x;
    const int lp = t & 63, n16 = lp & 15, grp = lp >> 4;
    constexpr int NF = C * DK / KPL;   // fragments-lanes of one C x DK tile
#pragma unroll
    for (int f0 = 0; f0 < NF; f0 += NT) {
        const int f = f0 + t;
        if (NF % NT == 0 || f < NF) {
            const int rb = f / (NKD * 64), ks = (f / 64) % NKD;
            const int row = 16 * rb + n16, col = ks * KS + grp * KPL;
            float e[KPL];
            load_fk<KPL>(e, &sm.eE[rb][col]);
            float x[KPL];
            PT::unpack(load_frag<T>(&sm.Kr[row][col]), x);
#pragma unroll
            for (int i = 0; i < KPL; ++i) x[i] *= e[i];
            *reinterpret_cast<typename PT::frag *>(pk + P::KG + (int64_t)f * KPL) = PT::pack(x);
            if (OUT) {
                PT::unpack(load_frag<T>(&sm.Qr[row][col]), x);
#pragma unroll
                for (int i = 0; i < KPL; ++i) x[i] *= e[i];
                *reinterpret_cast<typename PT::frag *>(pk + P::QG + (int64_t)f * KPL) = PT::pack(x);
            }
        }
    }
    // Kbar^T: fragment (ct, lane, ks) holds Kbar[KS ks + KPL grp + e][16 ct + n16],
    // one wave per (row tile, k step) so that the LDS transpose read sees its
    // own lanes
    constexpr int NKF = (DK / 16) * NKC;   // (row tile, k step) pairs; one wave each
    for (int p = wave_id(); p < NKF; p += ICfg<T, DK, C>::NW) {
        const int ct = p / NKC, ks = p % NKC;
        const int c = 16 * ct + n16, tok0 = ks * KS + grp * KPL;
        const float fct = sm.eTx[tok0 >> 4][c];
        float x[KPL];
        if constexpr (std::is_same<T, bf16>::value) {
            PT::unpack(i_tr8(&sm.Kc[0][0], ICfg<T, DK, C>::LDK, ks * KS, 16 * ct, n16, grp), x);
        } else {
            x[0] = to_f32(sm.Kc[tok0][c]);
        }
#pragma unroll
        for (int i = 0; i < KPL; ++i) x[i] *= fct;
        *reinterpret_cast<typename PT::frag *>(pk + P::KB + ((int64_t)(ct * 64 + lp) * NKC + ks) * KPL) =
            PT::pack(x);
    }
}

// One workgroup loops over (slot, head) items with a grid stride.
template <typename T, int DK, int C, bool OUT>
__global__ __launch_bounds__(1024, 1) void intra_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu_seqlens, int num_seqs,
    int64_t seq_len, int H, int64_t nitems, char *__restrict__ ws)
{
    typedef ICfg<T, DK, C> Cf;
    typedef Pk<T, DK, C> P;
    __shared__ __align__(16) ISmem<T, DK, C> sm;
    const int wv = wave_id();

    // find the first item of this workgroup that has a chunk
    int64_t item = blockIdx.x;
    int seq, nv = 0, head = 0;
    int64_t t0 = 0;
    auto next_valid = [&](int64_t it) -> int64_t {
        for (; it < nitems; it += gridDim.x) {
            head = (int)(it % H);
            if (slot_chunk(it / H, cu_seqlens, num_seqs, seq_len, C, seq, t0, nv)) return it;
        }
        return nitems;
    };
    item = next_valid(item);
    IRegs<T, DK, C> R;
    if (item < nitems) i_load<OUT>(R, q, k, g, beta, t0, nv, head, H);
    while (item < nitems) {
        T *pk = reinterpret_cast<T *>(ws + item * P::BYTES);
        float *gam = reinterpret_cast<float *>(ws + item * P::BYTES + P::GAM_BYTE);
        const int nv_cur = nv;
        i_elementwise<OUT>(sm, R, nv_cur);
        // the next item's loads fly during this item's products
        const int64_t nxt = next_valid(item + gridDim.x);
        if (nxt < nitems) i_load<OUT>(R, q, k, g, beta, t0, nv, head, H);
        __syncthreads();
        for (int job = wv; job < Cf::NJOB; job += Cf::NW) {
            if (job < Cf::NB) {
                i_diag<OUT>(sm, job, pk);
            } else if (job < Cf::NB + Cf::NPAIR) {
                const int p = job - Cf::NB;
                int I = 1;
                while ((I + 1) * I / 2 <= p) ++I;
                i_pair<OUT>(sm, I, p - I * (I - 1) / 2, pk);
            } else {
                const int c = 64 * (job - Cf::NB - Cf::NPAIR) + __lane_id();
                if (c < DK) i_tables(sm, c, gam);
            }
        }
        __syncthreads();
        if (wv < Cf::NB - 1) i_tcol(sm, wv, pk);
        i_copyout<OUT>(sm, pk);
        __syncthreads();
        item = nxt;
    }
}

// ===========================================================================
// State pass
// ===========================================================================
template <typename T, int DK, int C, int BV>
struct SCfg {
    typedef Pk<T, DK, C> P;
    static constexpr int NW = 16, NT = 1024;
    static constexpr int NB = C / 16;
    static constexpr int NVT = BV / 16;                 // value tiles
    static constexpr int NVJ = NB * NVT > 8 ? NB * NVT / 8 : 1;   // value tiles per read-out job
    static constexpr int NJOB = NB * NVT / NVJ;         // read-out / output jobs (<= 8)
    static constexpr int NCT = DK / 16;                 // state row tiles
    static constexpr int SW0 = 8;                       // first state wave
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDS2 = DK + 2 * PAD;           // S^T rows (32-byte pad)
    static constexpr int LDR = BV + PAD;                // R / U rows
    static constexpr bool HILO = std::is_same<T, bf16>::value;
    // staged packet parts, in 16-byte chunks
    static constexpr int KQ16 = (int)(2 * (int64_t)C * DK * sizeof(T) / 16);
    static constexpr int PP16 = (int)((int64_t)P::NBLK * 256 * sizeof(T) / 16);
    static constexpr int TB16 = (P::TLO ? 2 : 1) * PP16;   // TB and TL
    static constexpr int NKQ = (KQ16 + NT - 1) / NT;
    static constexpr int NTB = (TB16 + NT - 1) / NT;
    static constexpr int NPP = (PP16 + NT - 1) / NT;
    static_assert(NJOB <= 8 && NVT % NVJ == 0, "read-out jobs");
    static_assert(SW0 + NCT <= NW, "state waves");
    static_assert(NVT <= NW, "substitution waves");
};

template <typename T, int DK, int C, int BV>
struct SSmem {
    typedef SCfg<T, DK, C, BV> Cf;
    typedef Pk<T, DK, C> P;
    T kq[2 * C * DK];                 // Kg, Qg fragments
    T tb[(P::TLO ? 2 : 1) * P::NBLK * 256];   // TB (and TL) blocks
    T pp[P::NBLK * 256];              // P blocks
    T ST[BV][Cf::LDS2];               // S^T (operand copy)
    T R[C][Cf::LDR];                  // R, then U (hi part) in place
    T Ul[Cf::HILO ? C : 1][Cf::LDR];  // U lo part
};

// 16-byte staging of a packet part: thread t holds chunks t, t + NT, ...
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int N>
struct Stage {
    u32x4 x[N];
};
template <int N, int TOTAL>
__device__ __forceinline__ void stage_load(Stage<N> &s, const char *__restrict__ src)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = t + 1024 * i;
        if (TOTAL % 1024 == 0 || c < TOTAL) s.x[i] = reinterpret_cast<const u32x4 *>(src)[c];
    }
}
template <int N, int TOTAL>
__device__ __forceinline__ void stage_store(const Stage<N> &s, void *dst)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = t + 1024 * i;
        if (TOTAL % 1024 == 0 || c < TOTAL) reinterpret_cast<u32x4 *>(dst)[c] = s.x[i];
    }
}

// 4 rows r0 .. r0 + 3 of column c0 + n16 of a row-major tile (stride ld)
__device__ __forceinline__ void col4(const bf16 *x, int ld, int r0, int c0, int n16, float *out)
{
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4 *)(x + (r0 + (n16 >> 2)) * ld + c0 + 4 * (n16 & 3)));
    const bf16x4 b = __builtin_bit_cast(bf16x4, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (float)b[i];
}
__device__ __forceinline__ void col4(const float *x, int ld, int r0, int c0, int n16, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = x[(r0 + i) * ld + c0 + n16];
}

// B operand of a contraction over tokens from a token-major tile: lane
// (n16, grp) receives X[k0 + KPL grp + e][c0 + n16], e < KPL.
__device__ __forceinline__ bf16x8 tok_frag(const bf16 *x, int ld, int k0, int c0, int n16, int grp)
{
    return i_tr8(x, ld, k0, c0, n16, grp);
}
__device__ __forceinline__ float tok_frag(const float *x, int ld, int k0, int c0, int n16, int grp)
{
    return x[(k0 + grp) * ld + c0 + n16];
}

// One register block serves two roles that never share a wave: a state wave
// keeps its Kbar^T fragments in it, a read-out wave its value rows.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename T> struct RU;
template <> struct RU<bf16> {
    static constexpr int slots(int nfrag) { return nfrag; }
    __device__ __forceinline__ static bf16x8 frag(const u32x4 *X, int ks) { return __builtin_bit_cast(bf16x8, X[ks]); }
    __device__ __forceinline__ static void set_frag(u32x4 *X, int ks, bf16x8 f) { X[ks] = __builtin_bit_cast(u32x4, f); }
    __device__ __forceinline__ static bf16x4 val(const u32x4 *X, int j)
    {
        return __builtin_bit_cast(bf16x4, u32x2{X[j][0], X[j][1]});
    }
    __device__ __forceinline__ static void set_val(u32x4 *X, int j, bf16x4 v)
    {
        const u32x2 h = __builtin_bit_cast(u32x2, v);
        X[j][0] = h[0];
        X[j][1] = h[1];
    }
};
template <> struct RU<float> {
    static constexpr int slots(int nfrag) { return (nfrag + 3) / 4; }
    // (the element goes through a scalar first: a bit cast applied directly to
    // a vector-element expression reads element 0 of the vector)
    __device__ __forceinline__ static float frag(const u32x4 *X, int ks)
    {
        const uint32_t u = X[ks / 4][ks % 4];
        return __builtin_bit_cast(float, u);
    }
    __device__ __forceinline__ static void set_frag(u32x4 *X, int ks, float f) { X[ks / 4][ks % 4] = __builtin_bit_cast(uint32_t, f); }
    __device__ __forceinline__ static f32x4 val(const u32x4 *X, int j) { return __builtin_bit_cast(f32x4, X[j]); }
    __device__ __forceinline__ static void set_val(u32x4 *X, int j, f32x4 v) { X[j] = __builtin_bit_cast(u32x4, v); }
};

// Kbar^T fragments (lane-contiguous k steps) and gamma of state row tile ct.
// The lane's NKC fragments are contiguous, so they are read as 16-byte
// vectors straight into the register block.
template <typename T, int DK, int C>
__device__ __forceinline__ void s_load_state_side(u32x4 *X, f32x4 &gm, const char *__restrict__ p,
                                                  int ct, int lane, int grp)
{
    typedef Pk<T, DK, C> P;
    constexpr int KPL = Path<T>::KPL;
    constexpr int NV16 = (int)(P::NKC * KPL * sizeof(T) / 16);
    static_assert(P::NKC * KPL * sizeof(T) % 16 == 0, "fragment block");
    const u32x4 *kbp = reinterpret_cast<const u32x4 *>(reinterpret_cast<const T *>(p) + P::KB +
                                                       (int64_t)(ct * 64 + lane) * P::NKC * KPL);
#pragma unroll
    for (int m = 0; m < NV16; ++m) X[m] = kbp[m];
    gm = *reinterpret_cast<const f32x4 *>(p + P::GAM_BYTE + 4 * (16 * ct + 4 * grp));
}

// Values of a read-out job: row 16 jI + n16 of the chunk starting at tc (clamped
// to the sequence's last row), four columns at c0 + 16 j + 4 grp for each of
// the job's NVJ value tiles; zeros when v is NULL.
template <typename T, int NVJ>
__device__ __forceinline__ void s_load_values(u32x4 *X, const T *__restrict__ v,
                                              int64_t tc, int64_t eos, int H, int head, int DV,
                                              int c0, int jI, int n16, int grp)
{
    typedef typename V2T<T>::four V4;
    int64_t row = tc + 16 * jI + n16;
    row = row < eos - 1 ? row : eos - 1;
#pragma unroll
    for (int j = 0; j < NVJ; ++j)
        RU<T>::set_val(X, j, v ? *reinterpret_cast<const V4 *>(v + (row * H + head) * DV + c0 + 16 * j + 4 * grp) : V4{});
}

template <typename T, int DK, int C, int BV, bool OUT, typename TO>
__global__ __launch_bounds__(1024, 1) void state_kernel(
    const T *__restrict__ v, const float *__restrict__ s0, const int32_t *__restrict__ cu_seqlens,
    int num_seqs, int64_t seq_len, int H, TO *__restrict__ o, float *__restrict__ sfinal,
    const char *__restrict__ ws)
{
    typedef SCfg<T, DK, C, BV> Cf;
    typedef Pk<T, DK, C> P;
    typedef Path<T> PT;
    typedef typename PT::quad Q4;
    typedef typename V2T<T>::four V4;
    constexpr int KS = PT::KS, KPL = PT::KPL, NB = Cf::NB, NVT = Cf::NVT, NVJ = Cf::NVJ;
    constexpr int NSLICE = DK / BV, DV = DK;
    __shared__ __align__(16) SSmem<T, DK, C, BV> sm;

    // work item: (sequence, head, slice); the slices of a head on one XCD
    const int64_t b = blockIdx.x;
    int64_t w = b;
    if (H % 8 == 0) {
        const int64_t x = b % 8, slot = b / 8, per_seq = (int64_t)(H / 8) * NSLICE;
        w = ((slot / per_seq) * H + x * (H / 8)) * NSLICE + slot % per_seq;
    }
    const int seq = (int)(w / ((int64_t)H * NSLICE));
    const int head = (int)((w / NSLICE) % H);
    const int v0 = (int)(w % NSLICE) * BV;
    const SeqRange sr = seq_range(cu_seqlens, seq_len, seq);
    const int64_t nch = (sr.eos - sr.bos + C - 1) / C;
    const int64_t slot0 = sr.bos / C + seq;
#define KDA_PKT(c) (ws + ((slot0 + (c)) * H + head) * P::BYTES)

    const int t = threadIdx.x, lane = t & 63, wv = wave_id();
    const int n16 = lane & 15, grp = lane >> 4;
    const bool state_wave = wv >= Cf::SW0 && wv < Cf::SW0 + Cf::NCT;
    const int ct = wv - Cf::SW0;
    const bool has_job = wv < Cf::NJOB;
    const int jI = wv / (NVT / NVJ), jvt = (wv % (NVT / NVJ)) * NVJ;

    // W: on a state wave its state slice S[16 ct + 4 grp + i][v0 + 16 vt + n16]
    // (D layout, vt < NVT); on a read-out wave the Z^T tiles of its job
    constexpr int NWR = NVT > NVJ ? NVT : NVJ;
    f32x4 W[NWR];
#define S W
    const int64_t sbase = ((int64_t)seq * H + head) * (int64_t)(DK * DV) + v0;
    if (state_wave) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[vt][i] = s0 ? s0[sbase + (int64_t)(16 * ct + 4 * grp + i) * DV + 16 * vt + n16] : 0.f;
            float s4[4] = {S[vt][0], S[vt][1], S[vt][2], S[vt][3]};
            store_quad<T>(&sm.ST[16 * vt + n16][16 * ct + 4 * grp], s4);
        }
    }

    // per-role registers, one chunk ahead: the Kbar^T fragments and gamma of a
    // state wave's row tile, the values of a read-out job's rows
    typedef typename PT::frag Frag;
    // bf16: one register block for both roles; fp32: the state waves' fragments
    // apart (four to a 16-byte slot)
    constexpr bool SHARE = std::is_same<T, bf16>::value;
    constexpr int NKB = RU<T>::slots(P::NKC);
    constexpr int NX = SHARE ? (NKB > NVJ ? NKB : NVJ) : NVJ;
    u32x4 X[NX];
    u32x4 Xk[SHARE ? 1 : NKB];
    u32x4 *XK = SHARE ? X : Xk;
    f32x4 gm = zero4();
    Stage<Cf::NKQ> stKQ;
    Stage<Cf::NTB> stTB;
    Stage<Cf::NPP> stP;
    if (nch > 0) {
        stage_load<Cf::NKQ, Cf::KQ16>(stKQ, KDA_PKT(0) + P::KG * sizeof(T));
        stage_load<Cf::NTB, Cf::TB16>(stTB, KDA_PKT(0) + P::TB * sizeof(T));
        if (OUT) stage_load<Cf::NPP, Cf::PP16>(stP, KDA_PKT(0) + P::PP * sizeof(T));
        if (state_wave) s_load_state_side<T, DK, C>(XK, gm, KDA_PKT(0), ct, lane, grp);
        if (has_job) s_load_values<T, NVJ>(X, v, sr.bos, sr.eos, H, head, DV, v0 + 16 * jvt, jI, n16, grp);
        stage_store<Cf::NKQ, Cf::KQ16>(stKQ, sm.kq);
        stage_store<Cf::NTB, Cf::TB16>(stTB, sm.tb);
        if (OUT) stage_store<Cf::NPP, Cf::PP16>(stP, sm.pp);
        if (nch > 1) {
            stage_load<Cf::NKQ, Cf::KQ16>(stKQ, KDA_PKT(1) + P::KG * sizeof(T));
            stage_load<Cf::NTB, Cf::TB16>(stTB, KDA_PKT(1) + P::TB * sizeof(T));
            if (OUT) stage_load<Cf::NPP, Cf::PP16>(stP, KDA_PKT(1) + P::PP * sizeof(T));
        }
    }
    __syncthreads();

    for (int64_t ch = 0; ch < nch; ++ch) {
        const int64_t tc = sr.bos + ch * C;
        const int64_t nrem = sr.eos - tc;
        const int nv = nrem < C ? (int)nrem : C;
        // P of this chunk (P of the previous one was last read before the barrier)
        if (OUT && ch > 0) {
            stage_store<Cf::NPP, Cf::PP16>(stP, sm.pp);
            if (ch + 1 < nch) stage_load<Cf::NPP, Cf::PP16>(stP, KDA_PKT(ch + 1) + P::PP * sizeof(T));
        }

        // ============ YZ: Y^T = S^T Kg^T, Z^T = S^T Qg^T; R = V - Y
#define Zt W
        if (has_job) {
            f32x4 Yt[NVJ];
#pragma unroll
            for (int j = 0; j < NVJ; ++j) {
                Yt[j] = zero4();
                Zt[j] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < P::NKD; ++ks) {
                const int64_t fo = ((int64_t)(jI * P::NKD + ks) * 64 + lane) * KPL;
                const Frag kg = load_frag<T>(&sm.kq[P::KG + fo]);
                Frag qg{};
                if (OUT) qg = load_frag<T>(&sm.kq[P::QG + fo]);
#pragma unroll
                for (int j = 0; j < NVJ; ++j) {
                    const Frag sf = load_frag<T>(&sm.ST[16 * (jvt + j) + n16][ks * KS + grp * KPL]);
                    Yt[j] = PT::mma(sf, kg, Yt[j]);
                    if (OUT) Zt[j] = PT::mma(sf, qg, Zt[j]);
                }
            }
            // lane holds Y[16 jI + n16][16 (jvt + j) + 4 grp + i]
#pragma unroll
            for (int j = 0; j < NVJ; ++j) {
                float r[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = to_f32(RU<T>::val(X, j)[i]) - Yt[j][i];
                store_quad<T>(&sm.R[16 * jI + n16][16 * (jvt + j) + 4 * grp], r);
            }
            if (ch + 1 < nch)
                s_load_values<T, NVJ>(X, v, tc + C, sr.eos, H, head, DV, v0 + 16 * jvt, jI, n16, grp);
        }
        __syncthreads();   // ------------------------------------------- B1

        // ============ U = TB R, one wave per value tile (in place over R)
        if (wv < NVT) {
            const int vt = wv;
            Q4 Rd[NB];
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                float x[4];
                col4(&sm.R[0][0], Cf::LDR, 16 * J + 4 * grp, 16 * vt, n16, x);
                Rd[J] = PT::to_quad(x);
            }
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 X = zero4();
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    X = PT::mma16q(Rd[J], *reinterpret_cast<const Q4 *>(&sm.tb[blk(I, J) * 256 + 4 * lane]), X);
                    if constexpr (P::TLO)
                        X = PT::mma16q(Rd[J],
                                       *reinterpret_cast<const Q4 *>(&sm.tb[(P::NBLK + blk(I, J)) * 256 + 4 * lane]), X);
                }
                // lane holds U[16 I + n16][16 vt + 4 grp + i]
                float hi[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    hi[i] = to_f32(from_f32<T>(X[i]));
                    lo[i] = X[i] - hi[i];
                }
                store_quad<T>(&sm.R[16 * I + n16][16 * vt + 4 * grp], hi);
                if constexpr (Cf::HILO) store_quad<T>(&sm.Ul[16 * I + n16][16 * vt + 4 * grp], lo);
            }
        }
        // the next chunk's Kg, Qg (this chunk's were last read before B1)
        if (ch + 1 < nch) {
            stage_store<Cf::NKQ, Cf::KQ16>(stKQ, sm.kq);
            if (ch + 2 < nch) stage_load<Cf::NKQ, Cf::KQ16>(stKQ, KDA_PKT(ch + 2) + P::KG * sizeof(T));
        }
        __syncthreads();   // ------------------------------------------- B2

        // ============ SO: S' = gamma o S + Kbar^T U;  O^T = Z^T + U^T P^T
        if (state_wave) {
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = S[vt] * gm;
#pragma unroll
                for (int ks = 0; ks < P::NKC; ++ks) {
                    acc = PT::mma(RU<T>::frag(XK, ks), tok_frag(&sm.R[0][0], Cf::LDR, ks * KS, 16 * vt, n16, grp), acc);
                    if constexpr (Cf::HILO)
                        acc = PT::mma(RU<T>::frag(XK, ks), tok_frag(&sm.Ul[0][0], Cf::LDR, ks * KS, 16 * vt, n16, grp), acc);
                }
                S[vt] = acc;
                float s4[4] = {acc[0], acc[1], acc[2], acc[3]};
                store_quad<T>(&sm.ST[16 * vt + n16][16 * ct + 4 * grp], s4);
            }
            if (ch + 1 < nch) s_load_state_side<T, DK, C>(XK, gm, KDA_PKT(ch + 1), ct, lane, grp);
        }
        if (OUT && has_job) {
            const int row = 16 * jI + n16;
#pragma unroll
            for (int j = 0; j < NVJ; ++j) {
                f32x4 acc = Zt[j];
                const int vt = jvt + j;
#pragma unroll
                for (int J = 0; J < NB; ++J) {
                    if (J > jI) break;
                    const Q4 pb = *reinterpret_cast<const Q4 *>(&sm.pp[blk(jI, J) * 256 + 4 * lane]);
                    float u[4];
                    col4(&sm.R[0][0], Cf::LDR, 16 * J + 4 * grp, 16 * vt, n16, u);
                    acc = PT::mma16q(PT::to_quad(u), pb, acc);
                    if constexpr (Cf::HILO) {
                        col4(&sm.Ul[0][0], Cf::LDR, 16 * J + 4 * grp, 16 * vt, n16, u);
                        acc = PT::mma16q(PT::to_quad(u), pb, acc);
                    }
                }
                // lane holds O[16 jI + n16][v0 + 16 vt + 4 grp + i]
                if (row < nv) {
                    typedef typename V2T<TO>::four VO;
                    VO ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i) ov[i] = from_f32<TO>(acc[i]);
                    *reinterpret_cast<VO *>(o + ((tc + row) * H + head) * DV + v0 + 16 * vt + 4 * grp) = ov;
                }
            }
        }
        // the next chunk's TB (this chunk's were last read before B2)
        if (ch + 1 < nch) {
            stage_store<Cf::NTB, Cf::TB16>(stTB, sm.tb);
            if (ch + 2 < nch) stage_load<Cf::NTB, Cf::TB16>(stTB, KDA_PKT(ch + 2) + P::TB * sizeof(T));
        }
        __syncthreads();   // ------------------------------------------- B3
    }

    if (sfinal && state_wave) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sfinal[sbase + (int64_t)(16 * ct + 4 * grp + i) * DV + 16 * vt + n16] = S[vt][i];
    }
}

#undef KDA_PKT
#undef S
#undef Zt
}  // namespace cp

// ---------------------------------------------------------------------------
// Static scratch of the no-allocation entry point: the two-pass workspace for
// callers that cannot allocate device memory.  Every GPU the library runs on
// holds one copy until the process ends; all calls on a GPU share it, so calls
// that overlap on one GPU race.  Nothing in it has to start at zero: every
// packet slot the state pass reads is written first by the intra pass of the
// same call.
constexpr size_t kStaticScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// Device address of this device's copy of `scratch` (looked up once per device,
// with that device current).  In host code the array's name is a host-side
// stand-in, never a device address.
hipError_t static_scratch_ptr(void **ptr)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Host side

// Value-slice width of the state pass.
template <typename T, int D, int C> constexpr int state_bv()
{
    return std::is_same<T, bf16>::value ? (C == 128 ? 32 : (D < 64 ? D : 64))
                                        : (C == 128 ? 16 : (D < 32 ? D : 32));
}

size_t chunked_packet_bytes(int d, int chunk, bool is_bf16)
{
#define KDA_PK(T, D, C) \
    if (d == D && chunk == C) return (size_t)cp::Pk<T, D, C>::BYTES;
    if (is_bf16) {
        KDA_PK(bf16, 32, 64) KDA_PK(bf16, 64, 64) KDA_PK(bf16, 128, 64)
        KDA_PK(bf16, 32, 128) KDA_PK(bf16, 64, 128) KDA_PK(bf16, 128, 128)
    } else {
        KDA_PK(float, 32, 64) KDA_PK(float, 64, 64) KDA_PK(float, 128, 64)
        KDA_PK(float, 32, 128) KDA_PK(float, 64, 128)
    }
#undef KDA_PK
    return 0;
}

template <typename T, int D, int C, bool OUT, typename TO>
static hipError_t launch_chunked_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int64_t total_tokens, int H,
                                   void *o, float *sf, void *ws, hipStream_t stream)
{
    constexpr int BV = state_bv<T, D, C>();
    const int64_t nslots = (total_tokens + C - 1) / C + num_seqs;
    const int64_t nitems = nslots * H;
    if (nitems > 0 && total_tokens > 0) {
        int dev = 0, ncu = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int x = 0;
            if (hipDeviceGetAttribute(&x, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && x > 0)
                ncu = x;
        }
        const int64_t grid = nitems < ncu ? nitems : ncu;
        hipLaunchKernelGGL((cp::intra_kernel<T, D, C, OUT>), dim3((unsigned)grid), dim3(1024), 0,
                           stream, (const T *)q, (const T *)k, g, beta, cu, num_seqs, seq_len, H,
                           nitems, (char *)ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t nwork = (int64_t)num_seqs * H * (D / BV);
    if (nwork == 0) return hipSuccess;
    hipLaunchKernelGGL((cp::state_kernel<T, D, C, BV, OUT, TO>), dim3((unsigned)nwork), dim3(1024), 0,
                       stream, (const T *)v, s0, cu, num_seqs, seq_len, H, (TO *)o, sf,
                       (const char *)ws);
    return hipGetLastError();
}

template <typename T, int D, int C>
static hipError_t launch_chunked_o(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int64_t total_tokens, int H,
                                   void *o, bool o_f32, float *sf, void *ws, hipStream_t stream)
{
    if (!o)
        return launch_chunked_t<T, D, C, false, T>(q, k, v, g, beta, s0, cu, num_seqs, seq_len,
                                                   total_tokens, H, o, sf, ws, stream);
    if (std::is_same<T, bf16>::value && o_f32)
        return launch_chunked_t<T, D, C, true, float>(q, k, v, g, beta, s0, cu, num_seqs, seq_len,
                                                      total_tokens, H, o, sf, ws, stream);
    return launch_chunked_t<T, D, C, true, T>(q, k, v, g, beta, s0, cu, num_seqs, seq_len,
                                              total_tokens, H, o, sf, ws, stream);
}

hipError_t launch_chunked(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int64_t total_tokens, int H, int d, int chunk,
                          bool is_bf16, void *o, bool o_f32, float *sf, void *ws,
                          hipStream_t stream)
{
#define KDA_CH(T, D, C)                                                                        \
    if (d == D && chunk == C)                                                                  \
        return launch_chunked_o<T, D, C>(q, k, v, g, beta, s0, cu, num_seqs, seq_len,          \
                                         total_tokens, H, o, o_f32, sf, ws, stream);
    if (is_bf16) {
        KDA_CH(bf16, 32, 64) KDA_CH(bf16, 64, 64) KDA_CH(bf16, 128, 64)
        KDA_CH(bf16, 32, 128) KDA_CH(bf16, 64, 128) KDA_CH(bf16, 128, 128)
    } else {   // fp32 inputs: o is fp32 whatever o_f32 says
        KDA_CH(float, 32, 64) KDA_CH(float, 64, 64) KDA_CH(float, 128, 64)
        KDA_CH(float, 32, 128) KDA_CH(float, 64, 128)
    }
#undef KDA_CH
    return hipErrorInvalidValue;
}

}  // namespace kda
