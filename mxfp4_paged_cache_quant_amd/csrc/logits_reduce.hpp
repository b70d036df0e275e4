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
// Fixed summation order: ((g) + (g^2)) + ((g^1) + (g^3)).
__device__ __forceinline__ float reduce_tiles(const float acc[4], int lane) {
  const int g = lane >> 4;
  const bool lo_half = g < 2;
  const float keep0 = lo_half ? acc[0] : acc[2];
  const float keep1 = lo_half ? acc[1] : acc[3];
  const float send0 = lo_half ? acc[2] : acc[0];
  const float send1 = lo_half ? acc[3] : acc[1];
  const float p0 = keep0 + __shfl_xor(send0, 32);
  const float p1 = keep1 + __shfl_xor(send1, 32);
  const bool odd = g & 1;
  const float keep = odd ? p1 : p0;
  const float send = odd ? p0 : p1;
  return keep + __shfl_xor(send, 16);
}

}  // namespace mxidx
