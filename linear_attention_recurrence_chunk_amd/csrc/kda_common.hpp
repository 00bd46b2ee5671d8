// Shared device helpers for the gfx950 (CDNA4) KDA kernels: element types,
// matrix-core (MFMA) wrappers and small vector utilities.
//
// Matrix-core conventions used throughout (wave64):
//   lane l, n16 = l % 16, grp = l / 16.
//   A 16x16 fp32 accumulator tile D holds, in lane l, D[4*grp + i][n16],
//   i = 0..3 (the "D layout").
//   An A-operand fragment holds row n16 of A; a B-operand fragment holds
//   column n16 of B; both hold the same set of k indices for a given grp, so
//   the contraction pairs A[m][k] with B[k][n] whatever order the hardware
//   sums them in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index within the workgroup, read as a scalar: it is uniform in a wave,
// so role branches on it are scalar branches and addresses derived from it
// live in scalar registers
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Matrix-core paths.  Path<bf16>: v_mfma_f32_16x16x32_bf16 (K = 32 per
// instruction, 8 k values per lane).  Path<float>: v_mfma_f32_16x16x4_f32
// (K = 4 per instruction, 1 k value per lane).  Both accumulate in fp32.
template <typename T> struct Path;

template <> struct Path<bf16> {
    static constexpr int KS = 32;   // k per instruction
    static constexpr int KPL = 8;   // k values held per lane
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // frag from KPL fp32 values
    __device__ __forceinline__ static frag pack(const float *x) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (bf16)x[e];
        return f;
    }
    __device__ __forceinline__ static void unpack(frag f, float *x) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)f[e];
    }
    // K = 16 product: a holds A[n16][4*grp + i], b holds B[4*grp + i][n16], i = 0..3
    typedef bf16x4 quad;
    __device__ __forceinline__ static quad to_quad(const float *x) {
        quad r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
        return r;
    }
    __device__ __forceinline__ static quad to_quad(f32x4 x) {
        quad r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
        return r;
    }
    __device__ __forceinline__ static f32x4 mma16q(quad a, quad b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(short4v, a), __builtin_bit_cast(short4v, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 mma16(const float *a, const float *b, f32x4 c) {
        return mma16q(to_quad(a), to_quad(b), c);
    }
};

template <> struct Path<float> {
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag pack(const float *x) { return x[0]; }
    __device__ __forceinline__ static void unpack(frag f, float *x) { x[0] = f; }
    typedef f32x4 quad;
    __device__ __forceinline__ static quad to_quad(const float *x) {
        return f32x4{x[0], x[1], x[2], x[3]};
    }
    __device__ __forceinline__ static quad to_quad(f32x4 x) { return x; }
    __device__ __forceinline__ static f32x4 mma16q(quad a, quad b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
        return c;
    }
    __device__ __forceinline__ static f32x4 mma16(const float *a, const float *b, f32x4 c) {
        return mma16q(to_quad(a), to_quad(b), c);
    }
};

// Load KPL contiguous elements (one fragment) from LDS or global memory.
template <typename T>
__device__ __forceinline__ typename Path<T>::frag load_frag(const T *p) {
    return *reinterpret_cast<const typename Path<T>::frag *>(p);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Sum over the 16 lanes of a row of the wave (lanes 16 j .. 16 j + 15), with
// DPP moves: swap neighbours, swap pairs, then rotate the row by 4 and by 8.
__device__ __forceinline__ float row16_sum(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
    return x;
}

}  // namespace kda
