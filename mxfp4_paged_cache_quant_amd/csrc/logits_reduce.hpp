// Epilogue shared by the two logits kernels: ReLU-weighted head sums of
// block-scaled FP4 MFMA tiles and the cross-lane reduction that turns four
// 16-token tiles of per-lane partial sums into 64 per-token logits.
#pragma once

#include "common.hpp"

namespace mxidx {

// acc += sum_i w[i] * max(d[i], 0) over the 4 heads a lane holds in one
// 16x16 MFMA output tile (heads 4*(lane/16) + i of the 16-head group).
__device__ __forceinline__ float relu_weighted(const v4f d, const float4 w, float acc) {
  acc = fmaf(w.x, fmaxf(d[0], 0.0f), acc);
  acc = fmaf(w.y, fmaxf(d[1], 0.0f), acc);
  acc = fmaf(w.z, fmaxf(d[2], 0.0f), acc);
  acc = fmaf(w.w, fmaxf(d[3], 0.0f), acc);
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
