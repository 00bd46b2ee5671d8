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
// (N strictly lower 16 x 16, so N^16 = 0), evaluated on the matrix cores, and U
// follows by block forward substitution
//     U_I = (I + A_II)^-1 (R_I - sum_{J<I} A_IJ U_J),   R = B (V - (K o e^G) S).
//
// Decay factors never leave the float range.  With L the sub-block-local
// inclusive cumulative sum of g, B_J the total log decay of sub-block J and E_I
// the log decay from the chunk start to sub-block I:
//   rows of sub-block I (row operand):   e^{L_r}                     in [e^-80, 1]
//   columns of the diagonal blocks:      e^{-L_j}                    in [1, e^80]
//   column operand of block (I, J < I):  e^{-L_j} prod_{J<=m<I} e^{B_m}   <= 1
//   state read-out rows (Kg, Qg):        e^{G_r} = e^{E_I} e^{L_r}   <= 1
// e^80 is the bound the "Glossaire" entry "Decroissance bornee" gives for
// g_min = -5 (16 tokens times 5; see also the box "Limite importante" of page
// "Vecteurs, embeddings, espaces de representation").  A factor that
// underflows is a product of true decays below 1e-38: no significant term is
// lost.  Products are taken in an order in which no intermediate overflows.
//
// Work split: 16 waves, each with a fixed job in every phase of a chunk.
//   E    all waves: decays of a (16-token sub-block, channel pair, 4 rows) item
//        and the operand tiles K o e^L, Q o e^L, K o e^{B-L} and e^{B_I},
//        e^{-B_I}; it runs in the previous chunk's U phase.
//   AP   waves 0-3: diagonal block I of A and P (column operand K o e^{-L},
//        formed from K o e^{B-L} and e^{-B_I}) and the inverse of I + A_II,
//        kept in registers; waves 4-8, 10: one pair of off-diagonal
//        blocks of A and P; waves 12-13: the decay tables.  It runs beside the
//        previous chunk's SO phase, with no barrier between them: three
//        barriers a chunk.
//   YZ   one wave per (row block I, pair of value tiles): (K o e^G) S and
//        (Q o e^G) S for its 16 rows and 32 value columns, from the tiles
//        Kg, Qg built one chunk ahead, then R = B (V - (K o e^G) S); the state
//        waves take their Kbar^T fragments (K o e^{B-L} through the LDS
//        transpose read, times the decay to the chunk end) into registers,
//        where they stay until the state update.
//   U    one wave per 16 value columns: the forward substitution (for d <= 64
//        on waves that have no elementwise work).
//   SO   the read-out waves: their two blocks of O = (Q o e^G) S + P U,
//        stored to o; waves 8 ..: one state row tile each,
//        S' = Diag(gamma) S + Kbar^T U, the state staying in their registers
//        across chunks; then every wave a share of the next chunk's Kg, Qg
//        (diagonal scalings on the matrix cores).
// Contractions run on the matrix cores (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x16_bf16, or v_mfma_f32_16x16x4_f32 for fp32 inputs) with
// fp32 accumulation; operands are rounded to the input type.  The fp32 state
// stays in registers across the chunk loop.  The next chunk's raw inputs are
// loaded into registers one chunk ahead.
#include "kda_common.hpp"

#include <type_traits>

namespace kda {

template <typename T, int DK, int BV>
struct Cfg {
    static constexpr int C = 64;
    static constexpr int NB = 4;                      // 16-token sub-blocks
    static constexpr int NW = 16;
    static constexpr int NT = 64 * NW;
    static constexpr int PAD = 16 / (int)sizeof(T);   // 16-byte row padding
    static constexpr int LDK = DK + PAD;              // [token][channel] tiles
    static constexpr int LDC = C + PAD;               // [.][token] tiles
    static constexpr int LDV = BV + PAD;              // value slice rows
    // Tiles read mostly as 16-byte MFMA fragments (lane (n16, grp): row n16,
    // chunk grp) get rows padded by 32 bytes: with 64 four-byte banks that
    // read is then free of bank conflicts (a 16-byte pad makes it two-way),
    // at the price of two-way conflicts on their 8-byte accesses.
    static constexpr int LDK2 = DK + 2 * PAD;
    static constexpr int LDC2 = C + 2 * PAD;
    static constexpr int LD16 = 16 + PAD;             // 16 x 16 tiles
    static constexpr int WPB = DK / 32;               // E waves per sub-block
    static constexpr int EWAVES = NB * WPB;
    static constexpr int NCT = DK / 16;               // state row tiles
    static constexpr int NVT = BV / 16;               // state column tiles
    static constexpr int SW0 = NW / 2;                // first state wave
    static constexpr int NREG = NVT > 2 ? NVT : 2;    // f32x4 tiles held per wave
    static constexpr int NJOB = NB * NVT;             // (row block, value tile) jobs
    static constexpr int VEC = 8 / (int)sizeof(T);    // elements per 8-byte vector
    static constexpr int VPR = BV / VEC;              // 8-byte vectors per value row
    static constexpr int NVV = (C * VPR + NT - 1) / NT;
    static_assert(DK % 32 == 0 && DK <= 128, "head size");
    static_assert(BV % 16 == 0 && NJOB <= NW, "value slice");
    static_assert(EWAVES <= NW, "elementwise mapping");
    static_assert(NCT <= NW - SW0, "state tiling");
    static_assert(DK % Path<T>::KS == 0 && C % Path<T>::KS == 0, "k steps");
};

template <typename T, int DK, int BV>
struct Smem {
    typedef Cfg<T, DK, BV> Cf;
    T Kr[Cf::C][Cf::LDK];       // K o e^{L}         row operand
    T Qr[Cf::C][Cf::LDK];       // Q o e^{L}
    T Kc[Cf::C][Cf::LDK];       // K o e^{B - L}     column operand; times e^{-B}, that
                                //                   of the diagonal blocks
    T Kg[Cf::C - 16][Cf::LDK];  // K o e^{G}, rows 16 ..: read-out row operand on the
    T Qg[Cf::C - 16][Cf::LDK];  // Q o e^{G}          chunk-start reference
    T P[Cf::C][Cf::LDC];        // Tril((Q o e^G)(K o e^-G)^T)
    T An[Cf::C - 16][Cf::LDC];  // -A, blocks J < I (row r at r - 16: block 0 has none)
    T Tm[Cf::NB][16][Cf::LD16]; // (I + A_II)^-1
    T ST[BV][Cf::LDK2];         // state slice, transposed operand copy
    T RT[BV][Cf::LDC2];         // R^T, overwritten in place by U^T
    T V[Cf::C][Cf::LDV];        // value slice
    float eB[Cf::NB][DK];       // e^{B_J}
    float eBr[Cf::NB][DK];      // e^{-B_J}
    float eE[2][DK];            // whole-chunk decay prod_m e^{B_m}, by chunk parity
    float eTx[Cf::NB][DK];      // prod_{m>J} e^{B_m}
    float beta[Cf::C];
    float nrm[2][Cf::C][Cf::WPB];  // fused prologue: partial sums of squares of k, q rows
    float bA[DK];                  // fused prologue: decay bias b_alpha^h of the head
};

// two and four elements; `eight_bytes` is the 8-byte vector of the value loads
template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x2 two; typedef bf16x4 four; typedef bf16x4 eight_bytes; };
template <> struct Vec<float> { typedef f32x2 two; typedef f32x4 four; typedef f32x2 eight_bytes; };

// Raw inputs of one chunk, held in registers one chunk ahead: for the
// elementwise item of this thread, four rows of two channels of g, k, q;
// plus a share of the value slice and one beta.
template <typename T, int DK, int BV>
struct ChunkRegs {
    typedef Cfg<T, DK, BV> Cf;
    f32x2 g[4];                         // fused prologue: the gate alpha, once computed
    typename Vec<T>::two z[4];          // fused prologue: decay logits instead of g
    typename Vec<T>::two k[4], q[4];
    typename Vec<T>::eight_bytes v[Cf::NVV];
    float beta;
};

struct SeqView {
    int64_t bos, eos;   // token range of the sequence
    int head, H;
    int v0;             // first value column of the slice
};

// Byte offset of element `col` of row `row` of the chunk, the row clamped to
// `last`, the chunk's last row in the sequence: rows past the end read a valid
// address and are zeroed where the values are consumed.  Offsets are 32-bit
// and added to a wave-uniform 64-bit base, so that an access costs one VGPR
// and no 64-bit vector arithmetic; the row stride in bytes is below 2^24 (the
// launcher checks it), so that the product is one 24-bit multiply-add.
template <typename E>
__device__ __forceinline__ uint32_t row_byte_off(int row, int last, uint32_t stride_bytes, int col)
{
    const uint32_t r = (uint32_t)min(row, last);
    return __umul24(r, stride_bytes) + (uint32_t)col * (uint32_t)sizeof(E);
}

template <typename V, typename E>
__device__ __forceinline__ V load_at(const E *base, uint32_t byte_off)
{
    return *reinterpret_cast<const V *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Loads are unconditional, so that no select on a loaded value makes the wave
// wait for it.  `parts` selects what to load (LOAD_G, LOAD_KQ, LOAD_VB) so that
// the next chunk's loads can be spread over the phases of the current one.
enum { LOAD_G = 1, LOAD_KQ = 2, LOAD_VB = 4, LOAD_ALL = 7 };

// The layer's front end inside the kernel (template argument FUSED): none (q,
// k and g given), the bounded gate and the L2Norm of q and k (raw q, k and
// decay logits z given), or the bounded gate only (q, k given L2-normalised,
// z instead of g).
enum { FE_NONE = 0, FE_GATE_NORM = 1, FE_GATE = 2 };

// OUT = false (state only): q is not read.  v == nullptr: the values are zero.
template <int FUSED, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, DK, BV> &R, int parts, const SeqView &sv,
                                           int64_t t0, const T *__restrict__ q,
                                           const T *__restrict__ k, const T *__restrict__ v,
                                           const float *__restrict__ g, const T *__restrict__ z,
                                           const float *__restrict__ beta, int DV)
{
    typedef Cfg<T, DK, BV> Cf;
    typedef typename Vec<T>::two V2;
    typedef typename Vec<T>::eight_bytes V8;
    const int t = threadIdx.x, wv = wave_id(), lane = t & 63;
    const int64_t nvalid = sv.eos - t0;                    // >= 1
    const int last = nvalid < Cf::C ? (int)nvalid - 1 : Cf::C - 1;
    const int64_t cbase = (t0 * sv.H + sv.head) * DK;      // wave-uniform
    const uint32_t rs = (uint32_t)(sv.H * DK);             // row stride, elements
    const uint32_t rsT = rs * (uint32_t)sizeof(T), rsG = rs * 4u;
    if (wv < Cf::EWAVES) {
        const int I = wv / Cf::WPB, cp = (wv % Cf::WPB) * 16 + (lane & 15), qr = lane >> 4;
        const float *gb = g + cbase;
        const T *zb = z + cbase, *kb = k + cbase, *qb = q + cbase;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * I + 4 * qr + r;
            if (parts & LOAD_G) {
                if (FUSED) R.z[r] = load_at<V2>(zb, row_byte_off<T>(row, last, rsT, 2 * cp));
                else R.g[r] = load_at<f32x2>(gb, row_byte_off<float>(row, last, rsG, 2 * cp));
            }
            if (parts & LOAD_KQ) {
                const uint32_t bo = row_byte_off<T>(row, last, rsT, 2 * cp);
                R.k[r] = load_at<V2>(kb, bo);
                if (OUT) R.q[r] = load_at<V2>(qb, bo);
            }
        }
    }
    if (parts & LOAD_VB) {
        if (v) {
            const T *vb = v + (t0 * sv.H + sv.head) * DV + sv.v0;
#pragma unroll
            for (int m = 0; m < Cf::NVV; ++m) {
                const int vi = t + Cf::NT * m;
                const int row = min(vi / Cf::VPR, Cf::C - 1), cv = vi % Cf::VPR;
                R.v[m] = load_at<V8>(vb, row_byte_off<T>(row, last, (uint32_t)(sv.H * DV * sizeof(T)),
                                                          cv * Cf::VEC));
            }
        } else {
#pragma unroll
            for (int m = 0; m < Cf::NVV; ++m) R.v[m] = V8{};
        }
        const float *bb = beta + t0 * sv.H + sv.head;
        R.beta = load_at<float>(bb, row_byte_off<float>(t < Cf::C ? t : 0, last, (uint32_t)sv.H * 4u, 0));
    }
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

template <typename T> __device__ __forceinline__ typename Vec<T>::two pack2(float a, float b)
{
    typename Vec<T>::two r;
    r[0] = from_f32<T>(a);
    r[1] = from_f32<T>(b);
    return r;
}

template <typename T> __device__ __forceinline__ typename Vec<T>::four pack4(const float *x)
{
    typename Vec<T>::four r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = from_f32<T>(x[i]);
    return r;
}

template <typename T> __device__ __forceinline__ void unpack4(typename Vec<T>::four v, float *x)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f32(v[i]);
}


// Per-workgroup constant of the fused prologue: e^{A_h} (the decay bias is in
// LDS).
struct GateCtx {
    float eA;
};

// g = g_min sigma(e^{A_h} (z + b_alpha^h)) ("Glossaire", entry "Decroissance
// bornee", with the per-head bias of the notation table), returned as
// alpha = e^g.
__device__ __forceinline__ float bounded_alpha(float z, float eA, float b)
{
    constexpr float kGMin = -5.f;
    const float x = eA * (z + b);
    const float s = __builtin_amdgcn_rcpf(1.f + __expf(-x));
    return __expf(kGMin * s);
}

// Elementwise phase for one chunk: from the raw g, k, q of this thread's item
// (sub-block I, channels 2 cp and 2 cp + 1, rows 4 qr .. 4 qr + 3 of the
// sub-block), the sub-block-local decays, the operand tiles K o e^L, Q o e^L,
// K o e^{B-L}, and e^{B_I}, e^{-B_I}; then this thread's share of beta and of
// the value slice.  FULL: every row of the
// chunk lies in the sequence.  FUSED: g comes from decay logits through the
// bounded gate, and k and q are divided by their row norms (L2Norm of the
// function table), whose partial sums of squares are in sm.nrm.
template <bool FULL, int FUSED, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void e_phase(Smem<T, DK, BV> &sm, const ChunkRegs<T, DK, BV> &R, int nv,
                                        const GateCtx &gc, bool pre)
{
    typedef Cfg<T, DK, BV> Cf;
    typedef typename Vec<T>::two V2;
    typedef typename Vec<T>::eight_bytes V8;
    const int wv = wave_id();
    if (wv < Cf::EWAVES) {
        const int lp = __lane_id(), n16 = lp & 15, qr = lp >> 4;
        const int I = wv / Cf::WPB, cp = (wv % Cf::WPB) * 16 + n16;
        const int r0 = 16 * I + 4 * qr;
        float bb[2] = {0.f, 0.f};
        if (FUSED) {
            const f32x2 b2 = *reinterpret_cast<const f32x2 *>(&sm.bA[2 * cp]);
            bb[0] = b2[0];
            bb[1] = b2[1];
        }
        // per channel: e^{L_r} (eL) and e^{B - L_r} (sx) for the four rows, e^{-B}
        float eL[2][4], sx[2][4], rb[2], ebv[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            float a[4], pl[4], sl[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = FUSED ? (pre ? R.g[r][cc] : bounded_alpha(to_f32(R.z[r][cc]), gc.eA, bb[cc]))
                                       : __expf(R.g[r][cc]);
                a[r] = (FULL || r0 + r < nv) ? ar : 1.f;
            }
            pl[0] = a[0];
#pragma unroll
            for (int r = 1; r < 4; ++r) pl[r] = pl[r - 1] * a[r];
            sl[3] = 1.f;
#pragma unroll
            for (int r = 2; r >= 0; --r) sl[r] = sl[r + 1] * a[r + 1];
            // decays of the four row quarters of this sub-block
            float qd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) qd[j] = __shfl(pl[3], n16 + 16 * j);
            const float lead = ((qr > 0 ? qd[0] : 1.f) * (qr > 1 ? qd[1] : 1.f)) * (qr > 2 ? qd[2] : 1.f);
            const float tail = ((qr < 1 ? qd[1] : 1.f) * (qr < 2 ? qd[2] : 1.f)) * (qr < 3 ? qd[3] : 1.f);
            ebv[cc] = ((qd[0] * qd[1]) * qd[2]) * qd[3];
            rb[cc] = __builtin_amdgcn_rcpf(ebv[cc]);                 // e^{-B} <= e^80
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                eL[cc][r] = lead * pl[r];
                sx[cc][r] = sl[r] * tail;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool in = FULL || r0 + r < nv;
            // fused prologue: 1 / ||k_r||, 1 / ||q_r|| (0 for a zero row)
            float ik = 1.f, iq = 1.f;
            if (FUSED == FE_GATE_NORM) {
                float s2k = 0.f, s2q = 0.f;
#pragma unroll
                for (int w = 0; w < Cf::WPB; ++w) {
                    s2k += sm.nrm[0][r0 + r][w];
                    s2q += sm.nrm[1][r0 + r][w];
                }
                ik = s2k > 0.f ? __builtin_amdgcn_rsqf(s2k) : 0.f;
                iq = s2q > 0.f ? __builtin_amdgcn_rsqf(s2q) : 0.f;
            }
            float kk[2], qq[2], kc[2];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                kk[cc] = in ? to_f32(R.k[r][cc]) : 0.f;
                qq[cc] = (OUT && in) ? to_f32(R.q[r][cc]) : 0.f;
                if (FUSED == FE_GATE_NORM) {
                    kk[cc] *= ik;
                    qq[cc] *= iq;
                }
                kc[cc] = kk[cc] * sx[cc][r];              // e^{B - L_r} <= 1
            }
            *reinterpret_cast<V2 *>(&sm.Kr[r0 + r][2 * cp]) =
                pack2<T>(kk[0] * eL[0][r], kk[1] * eL[1][r]);
            if (OUT)
                *reinterpret_cast<V2 *>(&sm.Qr[r0 + r][2 * cp]) =
                    pack2<T>(qq[0] * eL[0][r], qq[1] * eL[1][r]);
            *reinterpret_cast<V2 *>(&sm.Kc[r0 + r][2 * cp]) = pack2<T>(kc[0], kc[1]);
        }
        if (qr == 0) {
            *reinterpret_cast<f32x2 *>(&sm.eB[I][2 * cp]) = f32x2{ebv[0], ebv[1]};
            *reinterpret_cast<f32x2 *>(&sm.eBr[I][2 * cp]) = f32x2{rb[0], rb[1]};
        }
    }
    const int to = 64 * wv + __lane_id();
    if (to < Cf::C) sm.beta[to] = (FULL || to < nv) ? R.beta : 0.f;   // beta = 0 masks rows past the end
#pragma unroll
    for (int m = 0; m < Cf::NVV; ++m) {
        const int vi = to + Cf::NT * m;
        const int row = vi / Cf::VPR, cv = vi % Cf::VPR;
        if (row < Cf::C) *reinterpret_cast<V8 *>(&sm.V[row][cv * Cf::VEC]) = R.v[m];
    }
}

template <int FUSED, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void e_phase(Smem<T, DK, BV> &sm, const ChunkRegs<T, DK, BV> &R, int nv,
                                        const GateCtx &gc, bool pre = false)
{
    if (nv >= Cfg<T, DK, BV>::C) e_phase<true, FUSED, OUT>(sm, R, nv, gc, pre);
    else e_phase<false, FUSED, OUT>(sm, R, nv, gc, pre);
}

// Fused prologue: the gate alpha of this thread's elementwise item, computed
// ahead (on waves that are idle when it runs) into the registers g is not
// using.  Rows past the end of the sequence are masked later, by the
// elementwise phase.
template <typename T, int DK, int BV>
__device__ __forceinline__ void gate_items(const Smem<T, DK, BV> &sm, ChunkRegs<T, DK, BV> &R,
                                           const GateCtx &gc)
{
    typedef Cfg<T, DK, BV> Cf;
    const int wv = wave_id();
    const int cp = (wv % Cf::WPB) * 16 + (__lane_id() & 15);
    const f32x2 b2 = *reinterpret_cast<const f32x2 *>(&sm.bA[2 * cp]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) R.g[r][cc] = bounded_alpha(to_f32(R.z[r][cc]), gc.eA, b2[cc]);
}

// Fused prologue: partial sums of squares of the raw k and q rows of this
// thread's item, over the wave's 32 channels; lane 0 of each row quarter
// stores them for the elementwise phase, which adds the WPB partials of a row.
template <typename T, int DK, int BV>
__device__ __forceinline__ void norm_partials(Smem<T, DK, BV> &sm, const ChunkRegs<T, DK, BV> &R)
{
    typedef Cfg<T, DK, BV> Cf;
    const int wv = wave_id();
    if (wv < Cf::EWAVES) {
        const int lp = __lane_id(), n16 = lp & 15, qr = lp >> 4;
        const int I = wv / Cf::WPB, part = wv % Cf::WPB;
        const int r0 = 16 * I + 4 * qr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float k0 = to_f32(R.k[r][0]), k1 = to_f32(R.k[r][1]);
            const float q0 = to_f32(R.q[r][0]), q1 = to_f32(R.q[r][1]);
            const float sk = row16_sum(k0 * k0 + k1 * k1);
            const float sq = row16_sum(q0 * q0 + q1 * q1);
            if (n16 == 0) {
                sm.nrm[0][r0 + r][part] = sk;
                sm.nrm[1][r0 + r][part] = sq;
            }
        }
    }
}

// Off-diagonal blocks (I, J < I) of A (stored negated, beta applied) and of P.
// The column operand K o e^{B_J - L_j} is brought to the reference of row
// block I by prod_{J<m<I} e^{B_m} (nothing for adjacent blocks), once for
// both products.  The products are taken transposed so that each lane ends
// with four consecutive columns of one row.
template <int I, int J, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void ap_pair(Smem<T, DK, BV> &sm, int n16, int grp)
{
    typedef Path<T> PT;
    typedef typename Vec<T>::four V4;
    constexpr int KS = PT::KS, KPL = PT::KPL;
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int ks = 0; ks < DK / KS; ++ks) {
        const int kc = ks * KS + grp * KPL;
        typename PT::frag col = load_frag<T>(&sm.Kc[16 * J + n16][kc]);
        if (I > J + 1) {
            float x[KPL], f[KPL];
            PT::unpack(col, x);
            load_f32<KPL>(f, &sm.eB[J + 1][kc]);
#pragma unroll
            for (int m = J + 2; m < I; ++m) {
                float f2[KPL];
                load_f32<KPL>(f2, &sm.eB[m][kc]);
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
    // lane holds X[r][j], r = 16 I + n16, j = 16 J + 4 grp + i
    const int r = 16 * I + n16;
    const float nb = -sm.beta[r];
    float wa[4], wp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wa[i] = nb * accA[i];
        wp[i] = accP[i];
    }
    *reinterpret_cast<V4 *>(&sm.An[r - 16][16 * J + 4 * grp]) = pack4<T>(wa);
    if (OUT) *reinterpret_cast<V4 *>(&sm.P[r][16 * J + 4 * grp]) = pack4<T>(wp);
}

// Decay tables of the chunk for channel c: prod_{m>J} e^{B_m} for each
// sub-block J, and the whole-chunk decay prod_m e^{B_m} (into buffer par of
// two: the previous chunk's state update may still read the other).
template <typename T, int DK, int BV>
__device__ __forceinline__ void decay_tables(Smem<T, DK, BV> &sm, int c, int par)
{
    constexpr int NB = Cfg<T, DK, BV>::NB;
    float f = 1.f;
#pragma unroll
    for (int m = NB - 1; m >= 0; --m) {
        sm.eTx[m][c] = f;
        f *= sm.eB[m][c];
    }
    sm.eE[par][c] = f;
}

// Row operands of the state read-out for sub-blocks I >= 1 on the reference of
// the chunk start: Kg = (K o e^{L}) e^{E_I} = K o e^{G} with e^{E_I} =
// prod_{m<I} e^{B_m}, and Qg likewise.  Every factor here is at most 1, so a
// product can only underflow, and one that does is a term below 1e-38 of its
// row: nothing significant is lost.  A 16 x 16 block is one K = 16 product on
// the matrix cores, Kg_blk^T = Diag(e^{E_I}) Kr_blk^T: the transposed block is
// read in the layout of its rows, and the result lands as four consecutive
// channels of a row per lane.  All waves share the (sub-block, channel
// block) pairs, waves 0 .. 7 taking the extra ones.
template <bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void chunk_ref_rows(Smem<T, DK, BV> &sm, int wv)
{
    typedef Cfg<T, DK, BV> Cf;
    typedef Path<T> PT;
    typedef typename PT::quad Q4;
    constexpr int NCB = DK / 16;                      // channel blocks
    constexpr int NPAIR = (Cf::NB - 1) * NCB;
    constexpr int NWK = Cf::NW;
    if (wv >= NWK) return;
    constexpr int NIT = (NPAIR + NWK - 1) / NWK;
    const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
    // every load first (the compiler cannot tell that the stores do not alias
    // them), then the products and stores
    Q4 da[NIT], kx[NIT], qx[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int p = it * NWK + wv;
        if (NPAIR % NWK == 0 || p < NPAIR) {
            const int I = 1 + p / NCB, cb = p % NCB;
            const int c = 16 * cb + n16;                  // channel of this lane's diagonal entry
            float e = sm.eB[0][c];
            for (int m = 1; m < I; ++m) e *= sm.eB[m][c];
            float a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = 4 * grp + i == n16 ? e : 0.f;
            da[it] = PT::to_quad(a);
            const int col = 16 * cb + 4 * grp;
            kx[it] = *reinterpret_cast<const Q4 *>(&sm.Kr[16 * I + n16][col]);
            if (OUT) qx[it] = *reinterpret_cast<const Q4 *>(&sm.Qr[16 * I + n16][col]);
        }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int p = it * NWK + wv;
        if (NPAIR % NWK == 0 || p < NPAIR) {
            const int I = 1 + p / NCB, cb = p % NCB;
            const int col = 16 * cb + 4 * grp;
            const f32x4 ky = PT::mma16q(da[it], kx[it], zero4());
            *reinterpret_cast<Q4 *>(&sm.Kg[16 * (I - 1) + n16][col]) = PT::to_quad(ky);
            if (OUT) {
                const f32x4 qy = PT::mma16q(da[it], qx[it], zero4());
                *reinterpret_cast<Q4 *>(&sm.Qg[16 * (I - 1) + n16][col]) = PT::to_quad(qy);
            }
        }
    }
}

// Operand fragment of X^T for a contraction over tokens, X stored token-major
// in LDS (row stride ld): lane (n16, grp) receives X[k][c0 + n16] for the KPL
// tokens k of its k group at k step k0.  For 16-bit data the LDS transpose
// read of gfx950 (ds_read_b64_tr_b16) does it: within each group of 16 lanes,
// lane n receives element i of lane 4 i + n / 4 at position n % 4, so lane
// s = 4 i + j supplies the four channels c0 + 4 j .. c0 + 4 j + 3 of token i.
__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16 *p)
{
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)p);
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 load_frag_tr(const bf16 *x, int ld, int k0, int c0, int n16, int grp)
{
    const bf16 *p = x + (k0 + 8 * grp + (n16 >> 2)) * ld + c0 + 4 * (n16 & 3);
    const bf16x4 lo = ds_read_tr4(p), hi = ds_read_tr4(p + 4 * ld);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float load_frag_tr(const float *x, int ld, int k0, int c0, int n16, int grp)
{
    return x[(k0 + grp) * ld + c0 + n16];
}

// Rows r0 .. r0 + 3 of column c0 + n16 of a row-major tile (row stride ld).
// For 16-bit data it is one LDS transpose read, lane s = 4 i + j of each group
// of 16 supplying the columns c0 + 4 j .. c0 + 4 j + 3 of row r0 + i.
__device__ __forceinline__ void load_col4(const bf16 *x, int ld, int r0, int c0, int n16, float *out)
{
    const bf16x4 v = ds_read_tr4(x + (r0 + (n16 >> 2)) * ld + c0 + 4 * (n16 & 3));
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (float)v[i];
}

__device__ __forceinline__ void load_col4(const float *x, int ld, int r0, int c0, int n16, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = x[(r0 + i) * ld + c0 + n16];
}

// (K o e^G) S and (Q o e^G) S for row block I and the NV value tiles
// vt0 .. vt0 + NV - 1, from the row operands kx, qx (16 rows, stride LDK: the
// chunk-start-referenced Kg, Qg for I >= 1, K o e^L and Q o e^L for I = 0,
// where L = G); the K, Q fragments of a k step serve every value tile, and one
// state fragment serves both products.  Y comes back in the D layout (rows of
// the block in 4 grp + i, value columns in n16); Z transposed (value columns in
// 4 grp + i, rows in n16), as the output's transposed product needs it.
template <int NV, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void yz_block(Smem<T, DK, BV> &sm, const T *kx, const T *qx, int vt0,
                                         int n16, int grp, f32x4 (&Y)[NV], f32x4 *Zt)
{
    typedef Cfg<T, DK, BV> Cf;
    typedef Path<T> PT;
    constexpr int KS = PT::KS, KPL = PT::KPL;
#pragma unroll
    for (int ks = 0; ks < DK / KS; ++ks) {
        const int kc = ks * KS + grp * KPL;
        const typename PT::frag kr = load_frag<T>(kx + n16 * Cf::LDK + kc);
        typename PT::frag qr{};
        if (OUT) qr = load_frag<T>(qx + n16 * Cf::LDK + kc);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const typename PT::frag s = load_frag<T>(&sm.ST[16 * (vt0 + v) + n16][kc]);
            Y[v] = PT::mma(kr, s, Y[v]);
            if (OUT) Zt[v] = PT::mma(s, qr, Zt[v]);
        }
    }
}

// State read-out of job (I, value tiles vt0 .. vt0 + NV - 1): Y and Z^T by
// yz_block, then R = B (V - Y) stored transposed for the substitution.
template <int NV, bool OUT, typename T, int DK, int BV>
__device__ __forceinline__ void readout_r(Smem<T, DK, BV> &sm, int I, int vt0, f32x4 *Zt)
{
    typedef typename Vec<T>::four V4;
    const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
    f32x4 Y[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) Y[v] = zero4();
    const T *kx = I > 0 ? &sm.Kg[16 * (I - 1)][0] : &sm.Kr[0][0];
    const T *qx = I > 0 ? &sm.Qg[16 * (I - 1)][0] : &sm.Qr[0][0];
    yz_block<NV, OUT>(sm, kx, qx, vt0, n16, grp, Y, Zt);
    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * I + 4 * grp]);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int vt = vt0 + v;
        float rv[4];
        load_col4(&sm.V[0][0], Cfg<T, DK, BV>::LDV, 16 * I + 4 * grp, 16 * vt, n16, rv);
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = b4[i] * (rv[i] - Y[v][i]);
        *reinterpret_cast<V4 *>(&sm.RT[16 * vt + n16][16 * I + 4 * grp]) = pack4<T>(rv);
    }
}

// Rows of the chunk starting at t0 that lie in the sequence, at most C.
__device__ __forceinline__ int rows_in(int64_t t0, int64_t eos, int C)
{
    const int64_t n = eos - t0;
    return n < C ? (int)n : C;
}

// (I + N)^-1 of diagonal block I by recursive block inversion, N = A_II (with
// beta) given in both layouts.  Let D_b be the block-diagonal matrix of the
// inverses of the b x b diagonal blocks of I + N, and F_b the part of N that
// lies in the lower-left b x b block of each 2b x 2b diagonal block.  Then
// D_2b = D_b - D_b F_b D_b; D_1 = I gives D_2 = I - F_1, and three more levels
// reach D_16.  Every intermediate is a block of the true inverse, whose entries
// stay small when the keys of a sub-block are alike (the power-series product
// (I - N)(I + N^2)(I + N^4)(I + N^8) instead forms powers that grow like
// binomial coefficients and cancel).  Layouts: a lane's values of X in the A
// layout (X[n16][4 grp + i]) are those of X^T in the D layout
// (X[4 grp + i][n16]), so a product X Y comes in the D layout from
// mma16(X in A, Y in D) and in the A layout from mma16(Y in D, X in A).  D_b is
// kept in both layouts (fp32; rounded to the input type only as an operand).
//
// Masks: with dl = n16 - 4 grp, the A-layout element i of a lane is the
// diagonal where dl = i and lies in F_1 where i is even and dl = i + 1 (the
// D-layout element in F_1 where i is odd and dl = i - 1).  F_2 holds elements
// 0 and 1 of the lanes with n16 / 4 = grp and bit 1 of n16 set; F_4 all four of
// the lanes with n16 / 8 = grp / 2, bit 2 of n16 set and grp even; F_8 all four
// of the lanes with bit 3 of n16 set and grp < 2.
template <typename T, int DK, int BV>
__device__ __forceinline__ void diag_inverse(Smem<T, DK, BV> &sm, int I, const float *Na,
                                             const float *Nd)
{
    typedef Path<T> PT;
    typedef typename PT::quad Q4;
    typedef typename Vec<T>::four V4;
    const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
    const int dl = n16 - 4 * grp;
    f32x4 Da, Dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float one = dl == i ? 1.f : 0.f;
        Da[i] = one - ((i & 1) == 0 && dl == i + 1 ? Na[i] : 0.f);
        Dd[i] = one - ((i & 1) == 1 && dl == i - 1 ? Nd[i] : 0.f);
    }
    const bool f2 = (n16 >> 2) == grp && (n16 & 2);
    const bool f4 = (n16 >> 3) == (grp >> 1) && (n16 & 4) && !(grp & 1);
    const bool f8 = (n16 & 8) && grp < 2;
#pragma unroll
    for (int bs = 2; bs < 16; bs *= 2) {
        const bool f = bs == 2 ? f2 : (bs == 4 ? f4 : f8);
        float Fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) Fa[i] = (f && (bs > 2 || i < 2)) ? Na[i] : 0.f;
        const Q4 da = PT::to_quad(Da);
        const Q4 yd = PT::to_quad(PT::mma16q(PT::to_quad(Fa), PT::to_quad(Dd), zero4()));  // F D
        Da -= PT::mma16q(yd, da, zero4());                                                   // D F D
        if (bs < 8) Dd -= PT::mma16q(da, yd, zero4());
    }
    // the lane ends with T[n16][4 grp + i], T = (I + A_II)^-1
    *reinterpret_cast<V4 *>(&sm.Tm[I][n16][4 * grp]) = PT::to_quad(Da);
}

// FUSED (FE_GATE, FE_GATE_NORM): g is replaced by decay logits z with the
// per-head gate parameters A_log [H] and b_alpha [H][DK]; with FE_GATE_NORM q
// and k also arrive unnormalised.  OUT = false:
// only the final state is computed (no o, q not read, and neither P nor
// (Q o e^G) S is formed); v == nullptr stands for zero values.  TO: the type
// of o (the input type, or fp32 for bf16 inputs).
// KCP (with OUT = false): a segment's two summaries in one launch ("Glossaire",
// entry "KCP"; notation table rows M_t and S~).  The value slices are doubled:
// those of the first half run the transition product, from S = I with zero
// values, and write M to mfinal; those of the second half run from S = 0 with
// the values and write S~ to sfinal.  s0 is not read.
template <typename T, int DK, int BV, int DV, int FUSED, bool OUT, typename TO, bool KCP = false>
__global__ __launch_bounds__(1024, 1) void prefill_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ s0, const int32_t *__restrict__ cu_seqlens, int num_seqs,
    int64_t seq_len, int H, TO *__restrict__ o, float *__restrict__ sfinal,
    const T *__restrict__ z, const float *__restrict__ A_log, const float *__restrict__ b_alpha,
    float *__restrict__ mfinal)
{
    typedef Cfg<T, DK, BV> Cf;
    typedef Path<T> PT;
    typedef Smem<T, DK, BV> Sm;
    typedef typename Vec<T>::four V4;
    constexpr int C = Cf::C, NB = Cf::NB, NT = Cf::NT, KS = PT::KS, KPL = PT::KPL;
    static_assert(!KCP || (!OUT && !FUSED), "summaries are state-only");
    constexpr int NSLICE = (KCP ? 2 : 1) * DV / BV;
    constexpr int NVT = Cf::NVT, NCT = Cf::NCT;
    __shared__ __align__(16) Sm sm;

    // ---- work item w = NSLICE (sequence H + head) + slice.  Workgroups are
    // dealt to the 8 XCDs round-robin (block b to XCD b mod 8).  When H divides
    // by 8, XCD x takes heads [x H/8, (x + 1) H/8) of every sequence in turn:
    // the slices of a head share q, k, g through one L2, an XCD reads
    // contiguous row segments, and every XCD gets a share of every sequence
    // whatever the mix of sequence lengths.
    const int64_t b = blockIdx.x;
    int64_t w = b;
    if (H % 8 == 0) {
        const int64_t x = b % 8, slot = b / 8, per_seq = (int64_t)(H / 8) * NSLICE;
        w = ((slot / per_seq) * H + x * (H / 8)) * NSLICE + slot % per_seq;
    }
    const int seq = (int)(w / ((int64_t)H * NSLICE));
    const int head = (int)((w / NSLICE) % H);
    const int slice = (int)(w % NSLICE);
    const bool trans = KCP && slice < DV / BV;      // a transition-product slice
    const T *const vsrc = trans ? nullptr : v;
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
    sv.v0 = (slice % (DV / BV)) * BV;

    const int t = threadIdx.x;
    const int lane = lane_id(), wv = wave_id();

    // ---- register tiles W.  The state waves SW0 .. SW0 + NCT - 1 hold the
    // state row tile ct = wv - SW0 for every value tile vt in W[vt], D layout:
    // S[16 ct + 4 grp + i][16 vt + n16].  The read-out waves hold the
    // transposed (Q o e^G) S of their two output blocks in W[0], W[1].
    const bool state_wave = wv >= Cf::SW0 && wv < Cf::SW0 + NCT;
    const int ct = wv - Cf::SW0;
    f32x4 W[Cf::NREG];
#pragma unroll
    for (int v = 0; v < Cf::NREG; ++v) W[v] = zero4();
    const int64_t sbase = ((int64_t)seq * H + head) * (int64_t)(DK * DV) + sv.v0;
    if (state_wave) {
        const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            if (KCP) {
                if (trans) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        W[vt][i] = 16 * ct + 4 * grp + i == sv.v0 + 16 * vt + n16 ? 1.f : 0.f;
                }
            } else if (s0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    W[vt][i] = s0[sbase + (int64_t)(16 * ct + 4 * grp + i) * DV + 16 * vt + n16];
            }
            float s4[4] = {W[vt][0], W[vt][1], W[vt][2], W[vt][3]};
            *reinterpret_cast<V4 *>(&sm.ST[16 * vt + n16][16 * ct + 4 * grp]) = pack4<T>(s4);
        }
    }
    // constant zero blocks above the diagonal of P
    if (OUT) {
        for (int e = t; e < C * C; e += NT) {
            const int r = e / C, j = e % C;
            if ((j >> 4) > (r >> 4)) sm.P[r][j] = from_f32<T>(0.f);
        }
    }

    // (row block, pair of value tiles) job of this wave for the state read-out
    // and the output, on waves 0 .. NB NP - 1: row blocks 1 .. NB - 1 first,
    // row block 0 (which needs no decay scaling) last.  Waves w and w + 4 share
    // a SIMD, so with 64-column value slices (eight jobs) two SIMDs get two
    // rescaled jobs and the other two one rescaled and one light job.
    constexpr int NP = NVT / 2;
    static_assert(NVT % 2 == 0 && NB * NP <= Cf::SW0, "job mapping");
    static_assert(NB == 4 && Cf::NW == 16, "AP-phase wave roles: 4 diagonal, 6 pair, 2 table waves");
    const bool has_job = wv < NB * NP;
    const int jI = wv < (NB - 1) * NP ? 1 + wv / NP : 0;
    const int jvt = 2 * (wv % NP);                        // first of the two value tiles

    GateCtx gc;
    gc.eA = 1.f;
    if (FUSED) {
        gc.eA = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                              __builtin_bit_cast(int, __expf(A_log[head]))));
        for (int c = t; c < DK; c += NT) sm.bA[c] = b_alpha[(int64_t)head * DK + c];
        __syncthreads();
    }

    const int64_t nchunks = (sv.eos - sv.bos + C - 1) / C;
    ChunkRegs<T, DK, BV> R;
    if (nchunks > 0) {
        load_chunk<FUSED, OUT>(R, LOAD_ALL, sv, sv.bos, q, k, vsrc, g, z, beta, DV);
        if (FUSED == FE_GATE_NORM) {
            norm_partials(sm, R);
            __syncthreads();
        }
        e_phase<FUSED, OUT>(sm, R, rows_in(sv.bos, sv.eos, C), gc);
    }
    __syncthreads();
    // the first chunk's Kg, Qg; read after B1
    if (nchunks > 0) chunk_ref_rows<OUT>(sm, wv);

    // Per chunk: AP | YZ | U and the next chunk's E | SO, with no barrier
    // between SO and the next chunk's AP (three barriers a chunk).  The
    // elementwise phase of chunk c + 1 writes only tiles that chunk c no longer
    // reads.
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = sv.bos + ch * C;
        const int nv = rows_in(t0, sv.eos, C);           // rows of this chunk in the sequence
        const bool more = ch + 1 < nchunks;
        if (more) load_chunk<FUSED, OUT>(R, LOAD_G | LOAD_KQ, sv, t0 + C, q, k, vsrc, g, z, beta, DV);

        // ================= AP
        // (lane indices inside the loop come from __lane_id(), which the
        // compiler recomputes in each phase rather than keeping every per-lane
        // LDS address live across the loop)
        if (wv < NB) {
            // diagonal block I: A_II both ways round, P_II, then (I + A_II)^-1
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            const int I = wv;
            f32x4 accAt = zero4(), accA = zero4(), accPt = zero4();
#pragma unroll
            for (int ks = 0; ks < DK / KS; ++ks) {
                const int kc = ks * KS + grp * KPL;
                // K o e^{-L} = (K o e^{B - L}) e^{-B}, each factor <= e^80
                typename PT::frag fd = load_frag<T>(&sm.Kc[16 * I + n16][kc]);
                {
                    float x[KPL], f[KPL];
                    PT::unpack(fd, x);
                    load_f32<KPL>(f, &sm.eBr[I][kc]);
#pragma unroll
                    for (int e = 0; e < KPL; ++e) x[e] *= f[e];
                    fd = PT::pack(x);
                }
                const typename PT::frag fk = load_frag<T>(&sm.Kr[16 * I + n16][kc]);
                accAt = PT::mma(fd, fk, accAt);   // [r = n16][j = 4 grp + i]
                accA = PT::mma(fk, fd, accA);     // [r = 4 grp + i][j = n16]
                if (OUT) {
                    const typename PT::frag fq = load_frag<T>(&sm.Qr[16 * I + n16][kc]);
                    accPt = PT::mma(fd, fq, accPt);   // [r = n16][j = 4 grp + i]
                }
            }
            // N = A_II in the A-operand layout (Na: N[n16][4 grp + i]) and in the
            // D layout (Nd: N[4 grp + i][n16])
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
            if (OUT) *reinterpret_cast<V4 *>(&sm.P[16 * I + n16][16 * I + 4 * grp]) = pack4<T>(pv);
            diag_inverse(sm, I, Na, Nd);
        } else if (wv < 9 || wv == 10) {
            // off-diagonal block pairs.  Wave w runs on SIMD w mod 4: the three
            // pairs whose column needs a decay factor go to SIMDs 1, 2, 3, one
            // each, and the three adjacent ones to SIMDs 0, 0, 2 (SIMDs 0 and 1
            // also have the decay tables).  This phase also runs the previous
            // chunk's output blocks, the heaviest (row block 3) on waves 4 and 5
            // and the lightest (row block 0) on 6 and 7, so the farthest pair
            // (3, 0) goes to wave 7
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            switch (wv) {
                case 4: ap_pair<1, 0, OUT>(sm, n16, grp); break;
                case 5: ap_pair<2, 0, OUT>(sm, n16, grp); break;
                case 6: ap_pair<3, 1, OUT>(sm, n16, grp); break;
                case 7: ap_pair<3, 0, OUT>(sm, n16, grp); break;
                case 8: ap_pair<2, 1, OUT>(sm, n16, grp); break;
                default: ap_pair<3, 2, OUT>(sm, n16, grp); break;
            }
        } else if (wv == 12 || wv == 13) {
            // decay tables, one channel per thread
            const int c = 64 * (wv - 12) + __lane_id();
            if (c < DK) decay_tables(sm, c, (int)(ch & 1));
        }
        __syncthreads();   // ---------------------------------------------- B1
        if (more) load_chunk<FUSED, OUT>(R, LOAD_VB, sv, t0 + C, q, k, vsrc, g, z, beta, DV);

        // ================= YZ: state read-out and R = B (V - Y); the state
        // waves take their Kbar^T fragments before the next chunk's E
        // overwrites K o e^{B - L}
        if (has_job) {
            W[0] = zero4();   // Z^T of the two blocks accumulates in W[0], W[1]
            W[1] = zero4();
            readout_r<2, OUT>(sm, jI, jvt, W);
        }
        // (K o e^{G_n - G})^T fragments of a state wave's row tile, kept in its
        // registers until its state update (the next chunk's E overwrites
        // K o e^{B - L} before then)
        typename PT::frag kbr[C / KS];
        if (state_wave) {
            // (K o e^{B - L}) read transposed, times prod_{m>J} e^{B_m}
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            const int c = 16 * ct + n16;
#pragma unroll
            for (int ks = 0; ks < C / KS; ++ks) {
                const int kj = ks * KS + grp * KPL;
                const float f = sm.eTx[kj >> 4][c];
                float x[KPL];
                PT::unpack(load_frag_tr(&sm.Kc[0][0], Cf::LDK, ks * KS, 16 * ct, n16, grp), x);
#pragma unroll
                for (int e = 0; e < KPL; ++e) x[e] *= f;
                kbr[ks] = PT::pack(x);
            }
        }
        // fused prologue: the next chunk's row norms, read by its E after B2
        if (FUSED == FE_GATE_NORM && more) norm_partials(sm, R);
        // fused prologue: the state waves take their items' gate ahead
        const bool pre = FUSED && state_wave && wv < Cf::EWAVES;
        if (pre && more) gate_items(sm, R, gc);
        __syncthreads();   // ---------------------------------------------- B2

        // ================= U: forward substitution, one wave per value tile;
        // U^T overwrites R^T in place.  On waves the elementwise phase leaves
        // free when there are enough (d <= 64), else on waves 0 ..
        constexpr int UW0 = Cf::EWAVES + NVT <= Cf::NW ? Cf::EWAVES : 0;
        if (wv >= UW0 && wv < UW0 + NVT) {
            typedef typename PT::quad Q4;
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            const int vt = wv - UW0;
            Q4 Ub[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                float xr[4];
                unpack4<T>(*reinterpret_cast<const V4 *>(&sm.RT[16 * vt + n16][16 * I + 4 * grp]), xr);
                f32x4 X = f32x4{xr[0], xr[1], xr[2], xr[3]};
#pragma unroll
                for (int J = 0; J < I; ++J)
                    X = PT::mma16q(*reinterpret_cast<const Q4 *>(&sm.An[16 * I - 16 + n16][16 * J + 4 * grp]),
                                   Ub[J], X);
                Ub[I] = PT::to_quad(
                    PT::mma16q(*reinterpret_cast<const Q4 *>(&sm.Tm[I][n16][4 * grp]), PT::to_quad(X),
                               zero4()));
            }
#pragma unroll
            for (int I = 0; I < NB; ++I)
                *reinterpret_cast<Q4 *>(&sm.RT[16 * vt + n16][16 * I + 4 * grp]) = Ub[I];
        }
        // ================= the next chunk's elementwise phase (the substituting
        // waves do their share after their substitution)
        if (more) e_phase<FUSED, OUT>(sm, R, rows_in(t0 + C, sv.eos, C), gc, pre);
        // the P fragments of this wave's output blocks, read before B3: the
        // next chunk's AP work rewrites P beside the output
        const int nks = (16 * (jI + 1) + KS - 1) / KS;
        typename PT::frag pfr[(C + KS - 1) / KS];
        if (OUT && has_job) {
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
#pragma unroll
            for (int ks = 0; ks < (C + KS - 1) / KS; ++ks)
                if (ks < nks) pfr[ks] = load_frag<T>(&sm.P[16 * jI + n16][ks * KS + grp * KPL]);
        }
        __syncthreads();   // ---------------------------------------------- B3

        // ================= SO: S' = Diag(gamma) S + Kbar^T U; O = Z + P U
        if (state_wave) {
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sm.eE[ch & 1][16 * ct + 4 * grp]);
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                f32x4 acc = W[vt] * gam;
#pragma unroll
                for (int ks = 0; ks < C / KS; ++ks) {
                    const int kj = ks * KS + grp * KPL;
                    acc = PT::mma(kbr[ks], load_frag<T>(&sm.RT[16 * vt + n16][kj]), acc);
                }
                W[vt] = acc;
                float s4[4] = {acc[0], acc[1], acc[2], acc[3]};
                *reinterpret_cast<V4 *>(&sm.ST[16 * vt + n16][16 * ct + 4 * grp]) = pack4<T>(s4);
            }
        }
        if (OUT && has_job) {
            const int lp = __lane_id(), n16 = lp & 15, grp = lp >> 4;
            // transposed blocks: lane holds O[16 jI + n16][16 (jvt + v) + 4 grp + i]
            f32x4 acc[2] = {W[0], W[1]};
#pragma unroll
            for (int ks = 0; ks < (C + KS - 1) / KS; ++ks) {
                if (ks >= nks) break;
                const int kj = ks * KS + grp * KPL;
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    acc[v] = PT::mma(load_frag<T>(&sm.RT[16 * (jvt + v) + n16][kj]), pfr[ks], acc[v]);
            }
            const int row = 16 * jI + n16;
            if (row < nv) {
                typedef typename Vec<TO>::four VO;
                TO *ob = o + (t0 * H + head) * DV + sv.v0;        // wave-uniform
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    float o4[4] = {acc[v][0], acc[v][1], acc[v][2], acc[v][3]};
                    const uint32_t bo = __umul24((uint32_t)row, (uint32_t)(H * DV * sizeof(TO))) +
                                        (uint32_t)((16 * (jvt + v) + 4 * grp) * sizeof(TO));
                    *reinterpret_cast<VO *>(reinterpret_cast<char *>(ob) + bo) = pack4<TO>(o4);
                }
            }
        }
        // the next chunk's Kg, Qg (its E ran before B3).  No barrier follows:
        // the next chunk's AP work runs beside this output and state update,
        // which read P from registers and the whole-chunk decay from the other
        // buffer, and it writes nothing else they read
        if (more) chunk_ref_rows<OUT>(sm, wv);
    }

    float *const sf = trans ? mfinal : sfinal;
    if (sf && state_wave) {
        const int n16 = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sf[sbase + (int64_t)(16 * ct + 4 * grp + i) * DV + 16 * vt + n16] = W[vt][i];
        }
    }
}

template <typename T, int D, int BV, int FUSED, bool OUT, typename TO>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int H, void *o, float *sf,
                                   const void *z, const float *A_log, const float *b_alpha,
                                   hipStream_t stream)
{
    const int64_t nwork = (int64_t)num_seqs * H * (D / BV);
    if (nwork == 0) return hipSuccess;
    // token row strides in bytes (fp32 g, or an fp32 o, is the widest) must fit 24 bits
    if ((int64_t)H * D * 4 >= (int64_t)1 << 24) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<T, D, BV, D, FUSED, OUT, TO>), dim3((unsigned)nwork),
                       dim3(Cfg<T, D, BV>::NT), 0, stream, (const T *)q, (const T *)k,
                       (const T *)v, g, beta, s0, cu, num_seqs, seq_len, H, (TO *)o, sf,
                       (const T *)z, A_log, b_alpha, (float *)nullptr);
    return hipGetLastError();
}

// Segment summaries (M, S~) of packed segments in one launch.
template <typename T, int D, int BV>
static hipError_t launch_kcp_t(const void *k, const void *v, const float *g, const float *beta,
                               const int32_t *cu, int num_seqs, int64_t seq_len, int H, float *M,
                               float *St, hipStream_t stream)
{
    const int64_t nwork = (int64_t)num_seqs * H * (2 * D / BV);
    if (nwork == 0) return hipSuccess;
    if ((int64_t)H * D * 4 >= (int64_t)1 << 24) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<T, D, BV, D, FE_NONE, false, T, true>), dim3((unsigned)nwork),
                       dim3(Cfg<T, D, BV>::NT), 0, stream, (const T *)nullptr, (const T *)k,
                       (const T *)v, g, beta, (const float *)nullptr, cu, num_seqs, seq_len, H,
                       (T *)nullptr, St, (const T *)nullptr, (const float *)nullptr,
                       (const float *)nullptr, M);
    return hipGetLastError();
}

hipError_t launch_kcp_summaries(const void *k, const void *v, const float *g, const float *beta,
                                const int32_t *cu, int num_seqs, int64_t seq_len, int H, int d,
                                bool is_bf16, float *M, float *St, hipStream_t stream)
{
#define KDA_KCP_ARGS k, v, g, beta, cu, num_seqs, seq_len, H, M, St, stream
    if (is_bf16) {
        switch (d) {
            case 32: return launch_kcp_t<bf16, 32, 32>(KDA_KCP_ARGS);
            case 64: return launch_kcp_t<bf16, 64, 64>(KDA_KCP_ARGS);
            case 128: return launch_kcp_t<bf16, 128, 64>(KDA_KCP_ARGS);
        }
    } else {
        switch (d) {
            case 32: return launch_kcp_t<float, 32, 32>(KDA_KCP_ARGS);
            case 64: return launch_kcp_t<float, 64, 32>(KDA_KCP_ARGS);
        }
    }
#undef KDA_KCP_ARGS
    return hipErrorInvalidValue;
}

// O32: o in fp32 for bf16 inputs (only the unfused kernel with an output).
template <int FUSED, bool OUT, bool O32>
static hipError_t launch_prefill_f(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *s0, const int32_t *cu,
                                   int num_seqs, int64_t seq_len, int H, int d, bool is_bf16,
                                   void *o, float *sf, const void *z, const float *A_log,
                                   const float *b_alpha, hipStream_t stream)
{
#define KDA_PREFILL_ARGS q, k, v, g, beta, s0, cu, num_seqs, seq_len, H, o, sf, z, A_log, b_alpha, stream
    typedef typename std::conditional<O32, float, bf16>::type TOB;
    if (is_bf16) {
        switch (d) {
            case 32: return launch_prefill_t<bf16, 32, 32, FUSED, OUT, TOB>(KDA_PREFILL_ARGS);
            case 64: return launch_prefill_t<bf16, 64, 64, FUSED, OUT, TOB>(KDA_PREFILL_ARGS);
            case 128: return launch_prefill_t<bf16, 128, 64, FUSED, OUT, TOB>(KDA_PREFILL_ARGS);
        }
    } else if (!O32) {
        switch (d) {
            case 32: return launch_prefill_t<float, 32, 32, FUSED, OUT, float>(KDA_PREFILL_ARGS);
            case 64: return launch_prefill_t<float, 64, 32, FUSED, OUT, float>(KDA_PREFILL_ARGS);
        }
    }
#undef KDA_PREFILL_ARGS
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *s0, const int32_t *cu, int num_seqs,
                          int64_t seq_len, int H, int d, int chunk, bool is_bf16, void *o,
                          bool o_f32, float *sf, hipStream_t stream)
{
    if (chunk != 64) return hipErrorInvalidValue;
    if (!o)   // state only
        return launch_prefill_f<FE_NONE, false, false>(q, k, v, g, beta, s0, cu, num_seqs, seq_len, H,
                                                     d, is_bf16, o, sf, nullptr, nullptr, nullptr,
                                                     stream);
    if (is_bf16 && o_f32)
        return launch_prefill_f<FE_NONE, true, true>(q, k, v, g, beta, s0, cu, num_seqs, seq_len, H, d,
                                                   is_bf16, o, sf, nullptr, nullptr, nullptr,
                                                   stream);
    return launch_prefill_f<FE_NONE, true, false>(q, k, v, g, beta, s0, cu, num_seqs, seq_len, H, d,
                                                is_bf16, o, sf, nullptr, nullptr, nullptr, stream);
}

// norm: q, k arrive unnormalised (FE_GATE_NORM), else normalised (FE_GATE).
hipError_t launch_prefill_fused(const void *q_raw, const void *k_raw, const void *v,
                                const void *z, const float *A_log, const float *b_alpha,
                                const float *beta, const float *s0, const int32_t *cu,
                                int num_seqs, int64_t seq_len, int H, int d, int chunk,
                                bool is_bf16, bool norm, void *o, float *sf, hipStream_t stream)
{
    if (chunk != 64) return hipErrorInvalidValue;
    if (!o) return hipErrorInvalidValue;
    if (norm)
        return launch_prefill_f<FE_GATE_NORM, true, false>(q_raw, k_raw, v, nullptr, beta, s0, cu,
                                                           num_seqs, seq_len, H, d, is_bf16, o, sf,
                                                           z, A_log, b_alpha, stream);
    return launch_prefill_f<FE_GATE, true, false>(q_raw, k_raw, v, nullptr, beta, s0, cu, num_seqs,
                                                  seq_len, H, d, is_bf16, o, sf, z, A_log, b_alpha,
                                                  stream);
}

}  // namespace kda
