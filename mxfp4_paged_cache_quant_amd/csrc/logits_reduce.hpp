// Epilogue shared by the two logits kernels: ReLU-weighted head sums of
// block-scaled FP4 MFMA tiles and the cross-lane reduction that turns four
// 16-token tiles of per-lane partial sums into 64 per-token logits.
#pragma once

#include "common.hpp"

namespace mxidx {

// max(x, 0) for a finite float as one integer max: negative values (sign bit
// set, including -0.0) compare below 0 as int32 and become +0.0.  (A float max
// would also canonicalize its operand, costing a second instruction.)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// acc += sum_i w[i] * max(d[i], 0) over the 4 heads a lane holds in one
// 16x16 MFMA output tile (heads 4*(lane/16) + i of the 16-head group).
__device__ __forceinline__ float relu_weighted(const v4f d, const float4 w, float acc) {
  acc = fmaf(w.x, relu(d[0]), acc);
  acc = fmaf(w.y, relu(d[1]), acc);
  acc = fmaf(w.z, relu(d[2]), acc);
  acc = fmaf(w.w, relu(d[3]), acc);
  return acc;
}

// Lane (g = lane/16, n = lane%16) holds acc[j] = partial logit of token 16*j + n
// over the heads of lane group g.  Returns, in lane (g, n), the full sum over
// the 4 lane groups for token 16*g + n, i.e. token `lane` of the 64.
// gfx950's lane swaps do the two exchanges without LDS: v_permlane32_swap(x, y)
// yields [x lanes 0-31 | y lanes 0-31] and [x lanes 32-63 | y lanes 32-63];
// v_permlane16_swap(x, y) yields [x row 0 | y row 0 | x row 2 | y row 2] and
// the same with rows 1 and 3 (a row is 16 lanes).
// Fixed summation order: ((g=0) + (g=2)) + ((g=1) + (g=3)).
__device__ __forceinline__ float reduce_tiles(const float acc[4]) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0]),
                                                    __float_as_uint(acc[2]), false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[1]),
                                                    __float_as_uint(acc[3]), false, false);
  // p0: tile 0 (lanes 0-31) / tile 2 (lanes 32-63) summed over g and g^2; p1: tiles 1 / 3
  const float p0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float p1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1),
                                                  false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

}  // namespace mxidx
