// Shared device-side definitions for the gfx950 kernels of the MXFP4 indexer path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxidx {

constexpr int kHeadDim = 128;
constexpr int kBlock = 32;            // elements per UE8M0 scale
constexpr int kCodeBytes = 64;        // 128 E2M1 nibbles
constexpr int kScaleBytes = 4;        // 4 block scales
constexpr int kRowBytes = 68;
constexpr int kPage = 64;             // tokens per cache page
constexpr int kPageCodeBytes = kPage * kCodeBytes;   // 4096: code rows first ...
constexpr int kPageBytes = kPage * kRowBytes;        // 4352: ... then scale rows
constexpr int kWave = 64;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Block-scaled FP4 x FP4 MFMA, 16x16 output, K = 128 (gfx950).
// Lane l supplies A row (l % 16) and B column (l % 16), elements
// 32*(l/16) .. 32*(l/16)+31 of the 128-long contraction as 16 packed bytes,
// and the UE8M0 scale of exactly that 32-element block (byte 0 of the scale
// register).  Output: lane l holds D[4*(l/16) + i][l % 16] in element i.
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, int sa, int sb, v4f c) {
  v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = 4 / blgp = 4 select E2M1 for A / B; opsel 0 picks scale byte 0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key),
// with -0.0 and +0.0 mapped to the same key: non-negative u -> u | 2^31,
// negative u -> (~u) + 1 = 2^32 - u (so -0.0 -> 2^31, and -x below +0 for every
// negative x).  Four branch-free instructions: shift, or, shift, xor-add.
__device__ __forceinline__ uint32_t f32_key(uint32_t u) {
  const uint32_t m = (uint32_t)((int32_t)u >> 31);           // all ones for negative
  return (u ^ (m | 0x80000000u)) + (u >> 31);
}

// Raw buffer descriptors over a wave-uniform base (kept in scalar registers):
// a load outside [0, bytes) reads 0 and a store there is dropped, with no
// memory access.  Dword 3 holds data format 32 (bits 18:15 = 4); raw loads and
// stores move bytes and ignore the format otherwise.
constexpr int kBufferFormat = 0x00020000;
constexpr int kNonTemporal = 2;                 // cache-policy bits of buffer ops: nt
constexpr uint32_t kDropOffset = 0x40000000u;   // beyond any descriptor: the access is dropped

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFormat);
}

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }

}  // namespace mxidx
