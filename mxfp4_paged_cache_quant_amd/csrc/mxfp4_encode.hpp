// MXFP4 encode rule shared by the row encoders (insert.hip) and the fused
// decode kernel (logits_paged.hip): UE8M0 exponent from the block amax, and
// one 32-element block per lane for the MFMA operand layout.
//
// Format: P1 "[Kernel] MXFP4 indexer cache for GLM-5.2 / DSA", "Changes"
// (E2M1 values + UE8M0 block-32 scales); OCP MX v1.0 for E2M1 / E8M0.
#pragma once

#include "common.hpp"

namespace mxidx {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Smallest E with amax <= 6 * 2^E, clamped to [-127, 127], from the bits of a
// non-negative finite fp32 amax = 1.f * 2^e:  E = e - 2 when f <= 0.5, else
// e - 1.  Exponent fields 0 and 1 (amax < 2^-125) always clamp to -127.
__device__ __forceinline__ int block_exponent(uint32_t a) {
  const uint32_t ex = a >> 23;
  if (ex <= 1u) return -127;
  const int e = (int)ex - 127;
  return ((a & 0x7fffffu) <= 0x400000u) ? e - 2 : e - 1;
}

// 2^E as an fp32 value (E in [-127, 126]; 2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2f(int E) {
  return __uint_as_float(E >= -126 ? (uint32_t)(E + 127) << 23 : 0x00400000u);
}

// Divisor handed to the scaled conversion for a block with amax bits `a` and
// exponent E.  An all-zero block needs no division (its codes are the sign
// bits alone); dividing by 1 keeps the subnormal scale out of the common case.
__device__ __forceinline__ float block_divisor(uint32_t a, int E) {
  return (a == 0u) ? 1.0f : pow2f(E);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(c.x, c.y, c.z, c.w);
}

// An empty asm that reads x: x is computed here (its loads have returned) and
// is not deferred past this point.
__device__ __forceinline__ void pin(const uint4& x) {
  asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
}
__device__ __forceinline__ void pin(int x) { asm volatile("" ::"v"(x)); }

// One 32-element bf16 block held by one lane: 64 bytes, four 16-byte loads.
struct Bf16Block {
  static constexpr int kElemBytes = 2;
  static constexpr int kPerWord = 2;   // elements per 32-bit word
  uint4 v[4];
  // word k (elements 2k, 2k+1) and element h of a word, as fp32 (exact)
  __device__ __forceinline__ uint32_t word(int k) const {
    const uint4& q = v[k >> 2];
    return (k & 3) == 0 ? q.x : (k & 3) == 1 ? q.y : (k & 3) == 2 ? q.z : q.w;
  }
  static __device__ __forceinline__ float elem(uint32_t w, int h) {
    return __uint_as_float(h ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = load16(rs, off + 16u * i);
  }
  __device__ __forceinline__ void pin() const {
#pragma unroll
    for (int i = 0; i < 4; ++i) mxidx::pin(v[i]);
  }
  // integer max over the 32 magnitudes, as fp32 bit patterns
  __device__ __forceinline__ uint32_t amax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
    }
    return m << 16;
  }
  // 16 code bytes: element 2j in the low nibble of byte j
  __device__ __forceinline__ uint4 encode(float scale) const {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t out = 0;
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v[i].x), scale, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v[i].y), scale, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v[i].z), scale, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2_t, v[i].w), scale, 3);
      o[i] = out;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
};

// One 32-element fp32 block held by one lane: 128 bytes, eight 16-byte loads.
struct F32Block {
  static constexpr int kElemBytes = 4;
  static constexpr int kPerWord = 1;
  uint4 v[8];
  __device__ __forceinline__ uint32_t word(int k) const {
    const uint4& q = v[k >> 2];
    return (k & 3) == 0 ? q.x : (k & 3) == 1 ? q.y : (k & 3) == 2 ? q.z : q.w;
  }
  static __device__ __forceinline__ float elem(uint32_t w, int) { return __uint_as_float(w); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = load16(rs, off + 16u * i);
  }
  __device__ __forceinline__ void pin() const {
#pragma unroll
    for (int i = 0; i < 8; ++i) mxidx::pin(v[i]);
  }
  __device__ __forceinline__ uint32_t amax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m = max(max(m, max(v[i].x & 0x7fffffffu, v[i].y & 0x7fffffffu)),
              max(v[i].z & 0x7fffffffu, v[i].w & 0x7fffffffu));
    return m;
  }
  __device__ __forceinline__ uint4 encode(float scale) const {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = v[2 * i], b = v[2 * i + 1];
      uint32_t out = 0;
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(a.x), __uint_as_float(a.y), scale, 0);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(a.z), __uint_as_float(a.w), scale, 1);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(b.x), __uint_as_float(b.y), scale, 2);
      out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(b.z), __uint_as_float(b.w), scale, 3);
      o[i] = out;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
};

}  // namespace mxidx
