// MXFP4 row encoder: contiguous output (query quantization) and paged scatter
// (indexer K quant-and-cache).
//
// Format: P1 "[Kernel] MXFP4 indexer cache for GLM-5.2 / DSA", sections
// "Changes" (E2M1 values + UE8M0 block-32 scales, written through an int64
// slot mapping) and "Benefit" (68 bytes per token); the block-split page
// layout of its live-validation comment; OCP MX v1.0 for E2M1 / E8M0.
//
// Work mapping: 16 lanes per 128-wide row, 8 consecutive elements per lane
// (one 16-byte load for bf16, two for fp32), so 4 lanes cover one 32-element
// block and a wave encodes 4 rows per step.  The block amax is an integer max
// over the magnitude bits (monotone for finite floats) reduced across the 4
// lanes with two xor-shuffles; the UE8M0 exponent is read off the amax bit
// fields; the elements are converted by the gfx950 scaled FP4 conversion,
// which divides by the power-of-two scale and rounds to nearest even, keeping
// the sign of zero.  Each lane stores 4 code bytes (a row's 64 code bytes are
// one coalesced 64-byte segment); lanes 0,4,8,12 of a row store the 4 scale bytes.
// The query encoder can rotate the rows first (RoPE, in fp32).
#include "common.hpp"
#include "launch.hpp"
#include "mxfp4_encode.hpp"

namespace mxidx {
namespace {

struct Bf16In {
  uint4 v;
  __device__ __forceinline__ void load(const void* base, int64_t row, int64_t stride, int sub) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row * stride + 8 * sub;
    v = *reinterpret_cast<const uint4*>(p);
  }
  // integer max over the 8 magnitudes, as fp32 bit patterns
  __device__ __forceinline__ uint32_t amax_bits() const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = max(m, w[i] & 0x7fffu);
      m = max(m, (w[i] >> 16) & 0x7fffu);
    }
    return m << 16;
  }
  // the 8 elements as fp32 values (exact)
  __device__ __forceinline__ void values(float (&f)[8]) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ uint32_t encode(float scale) const {
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
    return out;
  }
};

struct F32In {
  uint4 lo, hi;
  __device__ __forceinline__ void load(const void* base, int64_t row, int64_t stride, int sub) {
    const float* p = static_cast<const float*>(base) + row * stride + 8 * sub;
    lo = *reinterpret_cast<const uint4*>(p);
    hi = *reinterpret_cast<const uint4*>(p + 4);
  }
  __device__ __forceinline__ void values(float (&f)[8]) const {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(w[i]);
  }
  __device__ __forceinline__ uint32_t amax_bits() const {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, w[i] & 0x7fffffffu);
    return m;
  }
  __device__ __forceinline__ uint32_t encode(float scale) const {
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(lo.x), __uint_as_float(lo.y), scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(lo.z), __uint_as_float(lo.w), scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(hi.x), __uint_as_float(hi.y), scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(hi.z), __uint_as_float(hi.w), scale, 3);
    return out;
  }
};

constexpr int kRowsPerBlock = 16;   // 256 threads, 16 lanes per row

// Encode row `row` of x (16 lanes, lane `sub` takes elements 8*sub..8*sub+7)
// into 64 code bytes at cdst and 4 scale bytes at sdst.
template <typename In>
__device__ __forceinline__ void encode_loaded(const In& in, int sub, uint8_t* cdst, uint8_t* sdst) {
  uint32_t a = in.amax_bits();
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  const int E = block_exponent(a);
  const float scale = block_divisor(a, E);
  const uint32_t codes = in.encode(scale);
  *reinterpret_cast<uint32_t*>(cdst + 4 * sub) = codes;
  if ((sub & 3) == 0) sdst[sub >> 2] = (uint8_t)(E + 127);
}

template <typename In>
__device__ __forceinline__ void encode_row(const void* __restrict__ x, int64_t row, int64_t stride,
                                           int sub, uint8_t* cdst, uint8_t* sdst) {
  In in;
  in.load(x, row, stride, sub);
  encode_loaded(in, sub, cdst, sdst);
}

// Fused query RoPE + MXFP4 encode (P1 "Notes": a fused q-rope-mxfp4 kernel).
// Row r = t*H + h of q; the first rope_dim of its 128 elements are rotated in
// pairs -- (j, j + rope_dim/2) (neox) or (2j, 2j+1) (interleaved) -- by the
// angle j of table row positions[t] (t when positions is null):
//   a' = a*cos - b*sin,  b' = b*cos + a*sin,
// each product and each sum rounded to fp32 (no fused multiply-add), then the
// row is encoded as an fp32 row.  A row whose position lies outside the table
// is encoded unrotated.  rope_dim is a multiple of 16, so each lane's 8
// elements are all rotated or all not, and a neox lane's partner elements sit
// in one other lane of the row (lane sub +- rope_dim/16), fetched by shuffles.
__device__ __forceinline__ float rot_a(float a, float b, float c, float s) {
#pragma clang fp contract(off)
  return a * c - b * s;
}
__device__ __forceinline__ float rot_b(float a, float b, float c, float s) {
#pragma clang fp contract(off)
  return b * c + a * s;
}

// Rotates the row that 16 lanes hold (lane sub: elements 8sub..8sub+7) by the
// angles of table row p; a position outside the table leaves it unrotated.
// Every lane of the row calls it: a neox lane's partners come by shuffles.
__device__ __forceinline__ void rope_row8(float (&v)[8], int sub, int64_t p, const RopeSpec& rs) {
  const int half = rs.rope_dim >> 1;
  const int hl = half >> 3;                     // lanes per half of the rotated range
  const bool ok = p >= 0 && p < rs.table_rows;  // same for the row's 16 lanes
  float pv[8];
  if (!rs.interleaved) {
    const int partner = sub < hl ? sub + hl : sub - hl;
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = __shfl(v[i], partner, 16);
  }
  if (!ok || sub >= (rs.rope_dim >> 3)) return;
  const float* cr = rs.cos_t + p * half;
  const float* sr = rs.sin_t + p * half;
  if (rs.interleaved) {
    // pairs (8sub + 2i, 8sub + 2i + 1), angle index 4sub + i
    const float4 c = *reinterpret_cast<const float4*>(cr + 4 * sub);
    const float4 s = *reinterpret_cast<const float4*>(sr + 4 * sub);
    const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = v[2 * i], b = v[2 * i + 1];
      v[2 * i] = rot_a(a, b, cc[i], ss[i]);
      v[2 * i + 1] = rot_b(a, b, cc[i], ss[i]);
    }
  } else {
    // this lane holds elements 8sub..8sub+7: the a's of angles 8sub.. (sub < hl)
    // or the b's of angles 8(sub - hl).. ; the partner lane holds the others
    const int j0 = 8 * (sub < hl ? sub : sub - hl);
    const float4 c0 = *reinterpret_cast<const float4*>(cr + j0);
    const float4 c1 = *reinterpret_cast<const float4*>(cr + j0 + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(sr + j0);
    const float4 s1 = *reinterpret_cast<const float4*>(sr + j0 + 4);
    const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    if (sub < hl) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = rot_a(v[i], pv[i], cc[i], ss[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = rot_b(pv[i], v[i], cc[i], ss[i]);
    }
  }
}

// Row `row` of q (token row / H) rotated, then encoded as an fp32 row.
template <typename In>
__device__ __forceinline__ void rope_encode_row(const void* __restrict__ x, int64_t row,
                                                int64_t stride, int H, const RopeSpec& rs,
                                                int sub, uint8_t* cdst, uint8_t* sdst) {
  In in;
  in.load(x, row, stride, sub);
  float v[8];
  in.values(v);
  if (rs.rope_dim > 0) {   // uniform over the launch; no table or position read at 0
    const int64_t t = row / H;
    rope_row8(v, sub, rs.positions ? rs.positions[t] : t, rs);
  }
  F32In r;
  r.lo = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
  r.hi = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                    __float_as_uint(v[7]));
  encode_loaded(r, sub, cdst, sdst);
}

template <typename In>
__global__ __launch_bounds__(256) void mxfp4_rope_rows_kernel(const void* __restrict__ x,
                                                               int64_t rows, int64_t stride, int H,
                                                               RopeSpec rs,
                                                               uint8_t* __restrict__ dst_codes,
                                                               uint8_t* __restrict__ dst_scales) {
  const int sub = threadIdx.x & 15;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * kRowsPerBlock)
    rope_encode_row<In>(x, row, stride, H, rs, sub, dst_codes + row * kCodeBytes,
                        dst_scales + row * kScaleBytes);
}

// Paged destination of a slot: codes at page*4352 + off*64, scales at
// page*4352 + 4096 + off*4.  False (write nothing) unless 0 <= slot < num_slots.
__device__ __forceinline__ bool slot_dst(const int64_t* __restrict__ slot_mapping, int64_t row,
                                         int64_t num_slots, uint8_t* cache, uint8_t*& cdst,
                                         uint8_t*& sdst) {
  const int64_t slot = slot_mapping[row];
  if (slot < 0 || slot >= num_slots) return false;
  const int64_t page = slot / kPage;
  const int64_t off = slot % kPage;
  cdst = cache + page * kPageBytes + off * kCodeBytes;
  sdst = cache + page * kPageBytes + kPageCodeBytes + off * kScaleBytes;
  return true;
}

// kPaged = false: row r -> values[r*64], scales[r*4].
// kPaged = true:  row r -> the paged slot slot_mapping[r] (see slot_dst).
template <typename In, bool kPaged>
__global__ __launch_bounds__(256) void mxfp4_rows_kernel(const void* __restrict__ x, int64_t rows,
                                                          int64_t stride,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          int64_t num_slots,
                                                          uint8_t* __restrict__ dst_codes,
                                                          uint8_t* __restrict__ dst_scales) {
  const int sub = threadIdx.x & 15;
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
    uint8_t* cdst;
    uint8_t* sdst;
    if constexpr (kPaged) {
      // same decision for all 16 lanes of the row
      if (!slot_dst(slot_mapping, row, num_slots, dst_codes, cdst, sdst)) continue;
    } else {
      cdst = dst_codes + row * kCodeBytes;
      sdst = dst_scales + row * kScaleBytes;
    }
    encode_row<In>(x, row, stride, sub, cdst, sdst);
  }
}

// Both encodes of a decode step in one launch: workgroups [0, k_blocks) put
// the K rows into their cache slots, the others write the query rows
// contiguously.  Each part is a grid-stride loop over its own workgroups.
template <typename KIn, typename QIn, bool kRope>
__global__ __launch_bounds__(256) void insert_quantize_kernel(
    const void* __restrict__ k, int64_t k_rows, int64_t k_stride,
    const int64_t* __restrict__ slot_mapping, int64_t num_slots, uint8_t* __restrict__ cache,
    int k_blocks, const void* __restrict__ q, int64_t q_rows, int64_t q_stride,
    uint8_t* __restrict__ q_values, uint8_t* __restrict__ q_scales, int q_heads, RopeSpec rs) {
  const int sub = threadIdx.x & 15;
  if ((int)blockIdx.x < k_blocks) {
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4); row < k_rows;
         row += (int64_t)k_blocks * kRowsPerBlock) {
      uint8_t* cdst;
      uint8_t* sdst;
      if (!slot_dst(slot_mapping, row, num_slots, cache, cdst, sdst)) continue;
      encode_row<KIn>(k, row, k_stride, sub, cdst, sdst);
    }
  } else {
    const int64_t qb = (int64_t)blockIdx.x - k_blocks;
    const int64_t q_blocks = (int64_t)gridDim.x - k_blocks;
    for (int64_t row = qb * kRowsPerBlock + (threadIdx.x >> 4); row < q_rows;
         row += q_blocks * kRowsPerBlock) {
      if constexpr (kRope)
        rope_encode_row<QIn>(q, row, q_stride, q_heads, rs, sub, q_values + row * kCodeBytes,
                             q_scales + row * kScaleBytes);
      else
        encode_row<QIn>(q, row, q_stride, sub, q_values + row * kCodeBytes,
                        q_scales + row * kScaleBytes);
    }
  }
}

int grid_for_rows(int64_t rows) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t cap = 256 * 32;   // grid-stride beyond ~32 resident blocks per CU
  return (int)(blocks < cap ? blocks : cap);
}

template <typename KIn, typename QIn, bool kRope>
hipError_t launch_iq(const void* k, int64_t num_tokens, int64_t k_stride, const int64_t* slots,
                     uint8_t* cache, int64_t num_pages, const void* q, int64_t q_rows,
                     int64_t q_stride, uint8_t* q_values, uint8_t* q_scales, int q_heads,
                     const RopeSpec& rs, hipStream_t stream) {
  const int kb = grid_for_rows(num_tokens);
  const int qb = grid_for_rows(q_rows);
  hipLaunchKernelGGL((insert_quantize_kernel<KIn, QIn, kRope>), dim3(kb + qb), dim3(256), 0,
                     stream, k, num_tokens, k_stride, slots, num_pages * kPage, cache, kb, q,
                     q_rows, q_stride, q_values, q_scales, q_heads, rs);
  return hipGetLastError();
}

template <bool kRope>
hipError_t launch_iq_types(const void* k, bool k_f32, int64_t num_tokens, int64_t k_row_stride,
                           const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                           const void* q, bool q_f32, int64_t q_rows, int64_t q_row_stride,
                           uint8_t* q_values, uint8_t* q_scales, int q_heads, const RopeSpec& rs,
                           hipStream_t stream) {
#define MXIDX_IQ(KT, QT)                                                                        \
  launch_iq<KT, QT, kRope>(k, num_tokens, k_row_stride, slot_mapping, cache, num_pages, q,     \
                           q_rows, q_row_stride, q_values, q_scales, q_heads, rs, stream)
  if (k_f32) return q_f32 ? MXIDX_IQ(F32In, F32In) : MXIDX_IQ(F32In, Bf16In);
  return q_f32 ? MXIDX_IQ(Bf16In, F32In) : MXIDX_IQ(Bf16In, Bf16In);
#undef MXIDX_IQ
}

}  // namespace

hipError_t launch_quantize(const void* x, bool f32, int64_t rows, int64_t row_stride,
                           uint8_t* values, uint8_t* scales, hipStream_t stream) {
  const int grid = grid_for_rows(rows);
  if (f32)
    hipLaunchKernelGGL((mxfp4_rows_kernel<F32In, false>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, nullptr, 0, values, scales);
  else
    hipLaunchKernelGGL((mxfp4_rows_kernel<Bf16In, false>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, nullptr, 0, values, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_rope(const void* x, bool f32, int64_t rows, int64_t row_stride, int H,
                                const RopeSpec& rope, uint8_t* values, uint8_t* scales,
                                hipStream_t stream) {
  const int grid = grid_for_rows(rows);
  if (f32)
    hipLaunchKernelGGL((mxfp4_rope_rows_kernel<F32In>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, H, rope, values, scales);
  else
    hipLaunchKernelGGL((mxfp4_rope_rows_kernel<Bf16In>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, H, rope, values, scales);
  return hipGetLastError();
}

hipError_t launch_insert(const void* k, bool f32, int64_t num_tokens, int64_t row_stride,
                         const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                         hipStream_t stream) {
  const int grid = grid_for_rows(num_tokens);
  const int64_t num_slots = num_pages * kPage;
  if (f32)
    hipLaunchKernelGGL((mxfp4_rows_kernel<F32In, true>), dim3(grid), dim3(256), 0, stream, k,
                       num_tokens, row_stride, slot_mapping, num_slots, cache, nullptr);
  else
    hipLaunchKernelGGL((mxfp4_rows_kernel<Bf16In, true>), dim3(grid), dim3(256), 0, stream, k,
                       num_tokens, row_stride, slot_mapping, num_slots, cache, nullptr);
  return hipGetLastError();
}

hipError_t launch_insert_quantize(const void* k, bool k_f32, int64_t num_tokens,
                                  int64_t k_row_stride, const int64_t* slot_mapping,
                                  uint8_t* cache, int64_t num_pages, const void* q, bool q_f32,
                                  int64_t q_rows, int64_t q_row_stride, uint8_t* q_values,
                                  uint8_t* q_scales, hipStream_t stream) {
  const RopeSpec none{};
  return launch_iq_types<false>(k, k_f32, num_tokens, k_row_stride, slot_mapping, cache, num_pages,
                                q, q_f32, q_rows, q_row_stride, q_values, q_scales, 1, none,
                                stream);
}

hipError_t launch_insert_quantize_rope(const void* k, bool k_f32, int64_t num_tokens,
                                       int64_t k_row_stride, const int64_t* slot_mapping,
                                       uint8_t* cache, int64_t num_pages, const void* q,
                                       bool q_f32, int64_t q_rows, int64_t q_row_stride,
                                       int q_heads, const RopeSpec& rope, uint8_t* q_values,
                                       uint8_t* q_scales, hipStream_t stream) {
  return launch_iq_types<true>(k, k_f32, num_tokens, k_row_stride, slot_mapping, cache, num_pages,
                               q, q_f32, q_rows, q_row_stride, q_values, q_scales, q_heads, rope,
                               stream);
}

}  // namespace mxidx
