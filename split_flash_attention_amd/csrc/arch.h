// gfx950 wave-level primitives used by the matrix-core kernels.
//
// v_mfma_f32_16x16x32_{bf16,f16} lane layout (wave64), as relied on below:
//   A (16 x 32, rows m, contraction k): lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B (32 x 16, contraction k, cols n): lane l holds B[8 * (l / 16) + j][l % 16]
//   C/D (16 x 16):                      lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace selattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// D = A * B + C for 16x16x32 operands held as 8 packed 16-bit values per lane.
template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

// v_mfma_f32_16x16x16_{bf16,f16}: the same layout with 4 packed 16-bit values per
// lane: A[l % 16][4 * (l / 16) + j], B[4 * (l / 16) + j][l % 16], j = 0..3.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    if constexpr (F16) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                         __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
    }
}

// Butterfly exchange within the wave.
__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }
// max(x[l], x[l ^ 32]) and max(x[l], x[l ^ 16]) without a trip through LDS: one
// v_permlane32_swap / v_permlane16_swap of x with itself leaves each lane holding its
// own value and its partner's in the two results (in some order); the maximum of
// the two is the pair's (v_max_f32: a NaN operand gives the other one)
__device__ __forceinline__ float wave_max_x32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max_x16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x[l ^ 32] (x[l ^ 16]) itself: of the two results, the one whose bits differ from
// the lane's own value (either, when they are equal)
__device__ __forceinline__ float wave_partner_x32(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0] == u ? r[1] : r[0]);
}
__device__ __forceinline__ float wave_partner_x16(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0] == u ? r[1] : r[0]);
}
// x[l] + x[l ^ 32] (x[l ^ 16]) and x[l] | x[l ^ 32] (x[l ^ 16]) the same way (addition
// is commutative, so the sum is the one a lane exchange gives, bit for bit)
__device__ __forceinline__ float wave_sum_x32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum_x16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int wave_or_x32(int x) {
    const auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return static_cast<int>(r[0] | r[1]);
}
__device__ __forceinline__ int wave_or_x16(int x) {
    const auto r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(x), static_cast<unsigned>(x), false, false);
    return static_cast<int>(r[0] | r[1]);
}
__device__ __forceinline__ int wave_xor_i(int x, int mask) { return __shfl_xor(x, mask, 64); }

// Lane `src`'s 64-bit value (two 32-bit exchanges).
__device__ __forceinline__ unsigned long long wave_read64(unsigned long long x, int src) {
    const unsigned lo = static_cast<unsigned>(__shfl(static_cast<int>(x & 0xffffffffull), src, 64));
    const unsigned hi = static_cast<unsigned>(__shfl(static_cast<int>(x >> 32), src, 64));
    return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Wave-uniform "does any lane hold true".
__device__ __forceinline__ bool wave_any(bool x) { return __any(x); }

}  // namespace selattn
