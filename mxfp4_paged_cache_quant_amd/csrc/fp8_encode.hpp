// FP8 (E4M3) row encode rule shared by the FP8 row encoders (fp8.hip) and the
// pooled insert (kpool.hip): one fp32 scale per 128-element row and the
// hardware E4M3 conversion.  Format: the FP8 indexer cache that P1 "[Kernel]
// MXFP4 indexer cache for GLM-5.2 / DSA", section "Benefit", compares against
// (132 bytes per token); OCP OFP8 for E4M3.
#pragma once

#include "common.hpp"

namespace mxidx {

constexpr int kF8Row = 128;                        // value bytes per token
constexpr int kF8PageValues = kPage * kF8Row;      // 8192: value rows first ...
constexpr int kF8PageBytes = kPage * (kF8Row + 4); // 8448: ... then the scale words
constexpr float kE4M3Max = 448.0f;

// Per-row scale from the amax bits (a non-negative finite fp32): amax / 448
// rounded to fp32 and floored at 2^-126, or (pow2) 2^E with E the smallest
// integer such that amax <= 448 * 2^E, clamped to [-126, 127].
__device__ __forceinline__ float fp8_row_scale(uint32_t a, bool pow2) {
  if (pow2) {
    // amax = 1.f * 2^e: 448 * 2^E = 1.75 * 2^(E+8) >= amax first at E = e - 8
    // when 1.f <= 1.75 (mantissa field <= 0x600000), else at e - 7; amax below
    // 2^-126 (subnormal or zero) clamps to -126
    const uint32_t ex = a >> 23;
    int E = -126;
    if (ex != 0u) {
      const int e = (int)ex - 127;
      E = max(((a & 0x7fffffu) <= 0x600000u) ? e - 8 : e - 7, -126);
    }
    return __uint_as_float((uint32_t)(E + 127) << 23);
  }
  const float s = __uint_as_float(a) / kE4M3Max;   // correctly rounded fp32 division
  return fmaxf(s, __uint_as_float(0x00800000u));   // floor: 2^-126
}

// Four E4M3 bytes of y0..y3 (byte i = y_i), hardware round to nearest even.
__device__ __forceinline__ uint32_t pack_fp8x4(float y0, float y1, float y2, float y3) {
  int out = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  out = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, out, true);
  return (uint32_t)out;
}

}  // namespace mxidx
