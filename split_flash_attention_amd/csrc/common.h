// Device helpers shared by the attention kernels of this library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/sel_attn.h"

namespace selattn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// ---------------------------------------------------------------------------
// storage decoding (exact widening to fp32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t x) {
    return __half2float(__ushort_as_half(x));
}

// e4m3 byte -> fp32 (exact): sign, exponent field with bias 7 (0: subnormal
// m * 2^-9), 3 mantissa bits, 0x7f / 0xff NaN, no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float mag;
    if (e == 15u && m == 7u) mag = __builtin_nanf("");
    else if (e == 0u) mag = static_cast<float>(m) * 0x1p-9f;
    else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -mag : mag;
}

// Widen element i of a K/V row of storage type `dt` (the row scale of int8 and
// e4m3 rows is applied by the caller).
__device__ __forceinline__ float load_kv_elem(const void* base, int64_t idx, int dt) {
    switch (dt) {
    case SEL_ATTN_F32: return static_cast<const float*>(base)[idx];
    case SEL_ATTN_F16: return f16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    case SEL_ATTN_BF16: return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
    case SEL_ATTN_FP8: return e4m3_to_f32(static_cast<const uint8_t*>(base)[idx]);
    default: return static_cast<float>(static_cast<const int8_t*>(base)[idx]);
    }
}

// ---------------------------------------------------------------------------
// score pipeline: scale, softcap (tanh), ALiBi, additive mask (natural units).
// Scores stay in natural units: folding log2(e) into a score would overflow a
// finite sentinel such as -FLT_MAX into -inf; only differences s - m, which
// are small, are scaled by log2(e) before exp2.
// ---------------------------------------------------------------------------
struct ScoreParams {
    float scale;
    float softcap;       // 0 = off
    bool has_alibi;
};

__device__ __forceinline__ float score_pipeline(float dot, float scale, float softcap,
                                                float slope, int rel, float maskv) {
    float s = dot * scale;
    if (softcap > 0.f) s = softcap * tanhf(s / softcap);
    s += slope * static_cast<float>(rel);   // slope 0 when ALiBi is off
    s += maskv;                              // 0 when there is no mask
    return s;
}

// A NaN-aware "is a greater than b": NaN is tracked separately, so a plain
// ordered compare (false for NaN) keeps the running max finite.
__device__ __forceinline__ float max_keep(float a, float b) { return a > b ? a : b; }

// exp(x - m) for a score x and running max m (x == -inf gives 0 even when m == -inf).
__device__ __forceinline__ float exp_diff(float x, float m) {
    return (x == kNegInf) ? 0.f : exp2f((x - m) * kLog2e);
}

// Correction factor exp(m_old - m_new); 0 while nothing has been seen.
__device__ __forceinline__ float rescale_factor(float m_old, float m_new) {
    return (m_old == kNegInf) ? 0.f : exp2f((m_old - m_new) * kLog2e);
}

}  // namespace selattn
