// Pooled ("kpool") indexer-K insert (P3 "vllm.models.glm5next.nvidia.
// sparse_indexer", section "_kpool_compress_insert"): kpool consecutive tokens
// are pooled into one K row, which is quantized and written at a pool slot.
//
// Bookkeeping, as P3 prints it: slot_mapping is pool-granular (only the last
// token of a complete pool carries a slot >= 0); every position i is a
// candidate pool end and is written iff slot_mapping[i] >= 0 and
// i >= kpool - 1; its pool is tokens i - kpool + 1 .. i; nothing completes when
// n < kpool.  Pooling (not printed; the reading taken): per dimension d,
//   pooled[d] = sum_j softmax_j(gate[i-kpool+1+j, d] + ape[j, d]) * k[i-kpool+1+j, d],
// in fp32: z = gate + ape, the pool's maximum subtracted, exp, and the two
// sums accumulated over j in order, then one division.  The row is then
// encoded as the cache's format -- MXFP4 (the block-scaled rule of
// mxfp4_encode.hpp) or FP8 (fp8_encode.hpp, with P3's round_scale as the
// power-of-two scale) -- and written to its slot; slots outside the cache
// write nothing.  The pooled fp32 rows can also be returned (P3's
// return_compressed).
//
// Work mapping: 16 lanes per written row, 8 dimensions per lane (the row
// encoders' layout); each lane streams its 8 dims of the pool's kpool tokens
// twice (maximum, then the weighted sums; the second read hits the cache).
// Only one position in kpool ends a pool, so positions are not mapped to lane
// groups directly: each wave reads the slots of 64 consecutive positions,
// ballots the ones that write, and its four 16-lane groups take those four at
// a time (mapped directly, kpool 4 left three groups in four idle and the
// kernel bound by the idle groups' issue slots).
#include "common.hpp"
#include "fp8_encode.hpp"
#include "launch.hpp"
#include "mxfp4_encode.hpp"

namespace mxidx {
namespace {

constexpr int kKpPositionsPerBlock = 256;   // 4 waves x 64 positions per step
constexpr int kKpHeld = 4;                   // pools up to this size are held in registers

template <bool kF32>
__device__ __forceinline__ void load8(const void* base, int64_t row, int64_t stride, int sub,
                                      float (&v)[8]) {
  if constexpr (kF32) {
    const float* p = static_cast<const float*>(base) + row * stride + 8 * sub;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) +
                                                    row * stride + 8 * sub);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The pooled row of the pool ending at position i, encoded and written to
// `slot` (in the cache); run by the 16 lanes of one group, lane `sub` holding
// dimensions 8*sub .. 8*sub+7.  kFmt 0: MXFP4 cache (68 B rows), 1: FP8 cache
// (132 B rows).
template <bool kF32, int kFmt>
__device__ __forceinline__ void pool_row(const void* __restrict__ k, int64_t stride,
                                         const float* __restrict__ gate,
                                         const float* __restrict__ ape, int kpool, int64_t i,
                                         int64_t slot, int sub, int pow2,
                                         uint8_t* __restrict__ cache,
                                         float* __restrict__ compressed) {
  const int64_t first = i - kpool + 1;
  float m[8], ssum[8], acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    m[d] = neg_inf();
    ssum[d] = acc[d] = 0.f;
  }
  if (kpool <= kKpHeld) {
    // the whole pool's rows loaded before any is used: one memory round trip
    float z[kKpHeld][8], kv[kKpHeld][8];
#pragma unroll
    for (int j = 0; j < kKpHeld; ++j)
      if (j < kpool) {
        float a[8];
        load8f(gate + (first + j) * kHeadDim + 8 * sub, z[j]);
        load8f(ape + (int64_t)j * kHeadDim + 8 * sub, a);
        load8<kF32>(k, first + j, stride, sub, kv[j]);
#pragma unroll
        for (int d = 0; d < 8; ++d) z[j][d] = z[j][d] + a[d];
      }
#pragma unroll
    for (int j = 0; j < kKpHeld; ++j)
      if (j < kpool)
#pragma unroll
        for (int d = 0; d < 8; ++d) m[d] = fmaxf(m[d], z[j][d]);
#pragma unroll
    for (int j = 0; j < kKpHeld; ++j)
      if (j < kpool)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const float e = expf(z[j][d] - m[d]);
          ssum[d] += e;
          acc[d] += e * kv[j][d];
        }
  } else {
    for (int j = 0; j < kpool; ++j) {
      float g[8], a[8];
      load8f(gate + (first + j) * kHeadDim + 8 * sub, g);
      load8f(ape + (int64_t)j * kHeadDim + 8 * sub, a);
#pragma unroll
      for (int d = 0; d < 8; ++d) m[d] = fmaxf(m[d], g[d] + a[d]);
    }
    for (int j = 0; j < kpool; ++j) {
      float g[8], a[8], kv[8];
      load8f(gate + (first + j) * kHeadDim + 8 * sub, g);
      load8f(ape + (int64_t)j * kHeadDim + 8 * sub, a);
      load8<kF32>(k, first + j, stride, sub, kv);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float e = expf((g[d] + a[d]) - m[d]);
        ssum[d] += e;
        acc[d] += e * kv[d];
      }
    }
  }
  float v[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = acc[d] / ssum[d];
  if (compressed) {
    float* c = compressed + i * kHeadDim + 8 * sub;
    *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(c + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  const int64_t page = slot / kPage, off = slot % kPage;
  uint32_t amax = 0;
#pragma unroll
  for (int d = 0; d < 8; ++d) amax = max(amax, __float_as_uint(v[d]) & 0x7fffffffu);
  if constexpr (kFmt == 0) {
    // MXFP4: 4 lanes per 32-element block
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    const int E = block_exponent(amax);
    const float sc = block_divisor(amax, E);
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[0], v[1], sc, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[2], v[3], sc, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[4], v[5], sc, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, v[6], v[7], sc, 3);
    uint8_t* base = cache + page * kPageBytes;
    *reinterpret_cast<uint32_t*>(base + off * kCodeBytes + 4 * sub) = out;
    if ((sub & 3) == 0) base[kPageCodeBytes + off * kScaleBytes + (sub >> 2)] = (uint8_t)(E + 127);
  } else {
    // FP8: one scale for the row's 16 lanes
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, msk));
    const float s = fp8_row_scale(amax, pow2 != 0);
    float y[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) y[d] = v[d] / s;
    uint8_t* base = cache + page * kF8PageBytes;
    *reinterpret_cast<uint2*>(base + off * kF8Row + 8 * sub) =
        make_uint2(pack_fp8x4(y[0], y[1], y[2], y[3]), pack_fp8x4(y[4], y[5], y[6], y[7]));
    if (sub == 0) *reinterpret_cast<float*>(base + kF8PageValues + off * 4) = s;
  }
}

template <bool kF32, int kFmt>
__global__ __launch_bounds__(256) void kpool_insert_kernel(
    const void* __restrict__ k, int64_t n, int64_t stride, const float* __restrict__ gate,
    const float* __restrict__ ape, const int64_t* __restrict__ slot_mapping, int kpool,
    int64_t num_slots, int pow2, uint8_t* __restrict__ cache, float* __restrict__ compressed) {
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane >> 4;                     // lane group: 16 lanes per written row
  const int sub = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t base = wave * kWave; base < n; base += waves * kWave) {
    // the slots of 64 consecutive positions, one per lane; the writing ones balloted
    const int64_t i = base + lane;
    const int64_t slot = i < n ? slot_mapping[i] : -1;
    uint64_t todo = __ballot(i >= kpool - 1 && slot >= 0 && slot < num_slots);
    while (todo) {                               // wave-uniform
      // the next four writing positions, one per group (bit < 0: none left)
      int bit = -1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int b = todo ? __builtin_ctzll(todo) : -1;
        if (g == grp) bit = b;
        todo &= todo - 1;
      }
      // the group's slot, from the lane that read it (every lane takes part)
      const int src = bit < 0 ? lane : bit;
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)slot, src);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)slot >> 32), src);
      if (bit >= 0)                              // uniform over the group
        pool_row<kF32, kFmt>(k, stride, gate, ape, kpool, base + bit,
                             (int64_t)(((uint64_t)hi << 32) | lo), sub, pow2, cache, compressed);
    }
  }
}

// Pipelined form for pools of KP <= kKpHeld tokens and caches (and compressed
// outputs) below 2 GiB: the loop issues the next four pools' loads, then the
// previous four rows' stores, then computes.  gfx9 counts loads and stores in one
// in-order vmcnt, so in the form above every step's loads waited for the last
// step's store acknowledgements (the stores cost 23 of 171 us at 1M tokens, kpool
// 4).  Loads and stores are branch-free -- a group with no row loads pool 0 and
// its stores go to a dropped buffer offset -- so the compiler's waits are exact;
// the ape rows are loaded once per wave.  Same arithmetic, in the same order, as
// pool_row.
constexpr uint32_t kKpDrop = 0x80000000u;   // beyond a buffer of < 2 GiB: dropped

template <bool kF32>
struct KRaw {
  uint4 v[kF32 ? 2 : 1];
  __device__ __forceinline__ void load(const void* base, int64_t row, int64_t stride, int sub) {
    if constexpr (kF32) {
      const float* p = static_cast<const float*>(base) + row * stride + 8 * sub;
      v[0] = *reinterpret_cast<const uint4*>(p);
      v[1] = *reinterpret_cast<const uint4*>(p + 4);
    } else {
      v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * stride + 8 * sub);
    }
  }
  __device__ __forceinline__ void values(float (&f)[8]) const {
    if constexpr (kF32) {
      const uint32_t u[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(u[i]);
    } else {
      const uint32_t u[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    }
  }
};

template <bool kF32, int kFmt, int KP>
__global__ __launch_bounds__(256) void kpool_insert_pipe_kernel(
    const void* __restrict__ k, int64_t n, int64_t stride, const float* __restrict__ gate,
    const float* __restrict__ ape, const int64_t* __restrict__ slot_mapping, int64_t num_slots,
    int pow2, uint8_t* cache, int cache_bytes, float* compressed, int compressed_bytes) {
  const int lane = threadIdx.x & (kWave - 1);
  const int grp = lane >> 4;
  const int sub = lane & 15;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  const auto rc = buffer_rsrc(cache, cache_bytes);
  const auto rz = buffer_rsrc(compressed, compressed ? compressed_bytes : 0);
  float a[KP][8];
#pragma unroll
  for (int j = 0; j < KP; ++j) load8f(ape + (int64_t)j * kHeadDim + 8 * sub, a[j]);
  // the previous step's row: its encoded words, their offsets, its fp32 values
  uint32_t w0 = 0, w1 = 0, w2 = 0, o0 = kKpDrop, o1 = kKpDrop, oz = kKpDrop;
  float pv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto store_prev = [&]() {
    if constexpr (kFmt == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(w0, rc, o0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)w1, rc, o1, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(w0, rc, o0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(w1, rc, o0 == kKpDrop ? kKpDrop : o0 + 4u, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(w2, rc, o1, 0, 0);
    }
    const u32x4 z0 = {__float_as_uint(pv[0]), __float_as_uint(pv[1]), __float_as_uint(pv[2]),
                      __float_as_uint(pv[3])};
    const u32x4 z1 = {__float_as_uint(pv[4]), __float_as_uint(pv[5]), __float_as_uint(pv[6]),
                      __float_as_uint(pv[7])};
    __builtin_amdgcn_raw_buffer_store_b128(z0, rz, oz, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(z1, rz, oz == kKpDrop ? kKpDrop : oz + 16u, 0, 0);
  };
  for (int64_t base = wave * kWave; base < n; base += waves * kWave) {
    const int64_t i = base + lane;
    const int64_t slot = i < n ? slot_mapping[i] : -1;
    uint64_t todo = __ballot(i >= KP - 1 && slot >= 0 && slot < num_slots);
    while (todo) {                               // wave-uniform
      int bit = -1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int b = todo ? __builtin_ctzll(todo) : -1;
        if (g == grp) bit = b;
        todo &= todo - 1;
      }
      const int src = bit < 0 ? lane : bit;
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)slot, src);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)slot >> 32), src);
      const bool live = bit >= 0;
      const int64_t pos = live ? base + bit : KP - 1;   // a group with no row loads pool 0
      const int64_t first = pos - KP + 1;
      float4 gr[KP][2];
      KRaw<kF32> kr[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const float* gp = gate + (first + j) * kHeadDim + 8 * sub;
        gr[j][0] = *reinterpret_cast<const float4*>(gp);
        gr[j][1] = *reinterpret_cast<const float4*>(gp + 4);
        kr[j].load(k, first + j, stride, sub);
      }
      __builtin_amdgcn_sched_barrier(0);         // these loads ahead of the stores below
      store_prev();
      __builtin_amdgcn_sched_barrier(0);
      float m[8], ssum[8], acc[8], z[KP][8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        m[d] = neg_inf();
        ssum[d] = acc[d] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const float g8[8] = {gr[j][0].x, gr[j][0].y, gr[j][0].z, gr[j][0].w,
                             gr[j][1].x, gr[j][1].y, gr[j][1].z, gr[j][1].w};
#pragma unroll
        for (int d = 0; d < 8; ++d) z[j][d] = g8[d] + a[j][d];
      }
#pragma unroll
      for (int j = 0; j < KP; ++j)
#pragma unroll
        for (int d = 0; d < 8; ++d) m[d] = fmaxf(m[d], z[j][d]);
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        float kv[8];
        kr[j].values(kv);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const float e = expf(z[j][d] - m[d]);
          ssum[d] += e;
          acc[d] += e * kv[d];
        }
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) pv[d] = acc[d] / ssum[d];
      const int64_t wslot = (int64_t)(((uint64_t)hi << 32) | lo);
      const uint32_t page = (uint32_t)(wslot / kPage), off = (uint32_t)(wslot % kPage);
      uint32_t amax = 0;
#pragma unroll
      for (int d = 0; d < 8; ++d) amax = max(amax, __float_as_uint(pv[d]) & 0x7fffffffu);
      if constexpr (kFmt == 0) {
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
        const int E = block_exponent(amax);
        const float sc = block_divisor(amax, E);
        uint32_t out = 0;
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, pv[0], pv[1], sc, 0);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, pv[2], pv[3], sc, 1);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, pv[4], pv[5], sc, 2);
        out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, pv[6], pv[7], sc, 3);
        const uint32_t pb = page * (uint32_t)kPageBytes;
        w0 = out;
        w1 = (uint32_t)(E + 127);
        o0 = live ? pb + off * kCodeBytes + 4u * sub : kKpDrop;
        o1 = (live && (sub & 3) == 0) ? pb + kPageCodeBytes + off * kScaleBytes + (sub >> 2) : kKpDrop;
      } else {
#pragma unroll
        for (int msk = 1; msk < 16; msk <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, msk));
        const float s = fp8_row_scale(amax, pow2 != 0);
        float y[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) y[d] = pv[d] / s;
        const uint32_t pb = page * (uint32_t)kF8PageBytes;
        w0 = pack_fp8x4(y[0], y[1], y[2], y[3]);
        w1 = pack_fp8x4(y[4], y[5], y[6], y[7]);
        w2 = __float_as_uint(s);
        o0 = live ? pb + off * kF8Row + 8u * sub : kKpDrop;
        o1 = (live && sub == 0) ? pb + kF8PageValues + off * 4u : kKpDrop;
      }
      oz = live ? (uint32_t)(pos * kHeadDim * 4 + 32 * sub) : kKpDrop;
    }
  }
  store_prev();
}

template <bool kF32, int kFmt>
hipError_t launch_kp(const void* k, int64_t n, int64_t stride, const float* gate, const float* ape,
                     const int64_t* slots, int kpool, int64_t num_pages, bool pow2, uint8_t* cache,
                     float* compressed, hipStream_t stream) {
  const int64_t blocks = (n + kKpPositionsPerBlock - 1) / kKpPositionsPerBlock;
  const int grid = (int)(blocks < 256 * 32 ? blocks : 256 * 32);
  const int64_t cache_bytes = num_pages * (kFmt == 0 ? kPageBytes : kF8PageBytes);
  const int64_t comp_bytes = compressed ? n * kHeadDim * 4 : 0;
  if (kpool <= kKpHeld && cache_bytes <= 0x7fffffffLL && comp_bytes <= 0x7fffffffLL) {
#define MXIDX_KPP(kp)                                                                         \
  case kp:                                                                                    \
    hipLaunchKernelGGL((kpool_insert_pipe_kernel<kF32, kFmt, kp>), dim3(grid), dim3(256), 0,  \
                       stream, k, n, stride, gate, ape, slots, num_pages * kPage,              \
                       pow2 ? 1 : 0, cache, (int)cache_bytes, compressed, (int)comp_bytes);   \
    return hipGetLastError();
    switch (kpool) {
      MXIDX_KPP(1)
      MXIDX_KPP(2)
      MXIDX_KPP(3)
      MXIDX_KPP(4)
      default:
        break;
    }
#undef MXIDX_KPP
  }
  hipLaunchKernelGGL((kpool_insert_kernel<kF32, kFmt>), dim3(grid), dim3(256), 0, stream, k, n,
                     stride, gate, ape, slots, kpool, num_pages * kPage, pow2 ? 1 : 0, cache,
                     compressed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kpool_insert(const void* k, bool f32, int64_t n, int64_t row_stride,
                               const float* gate, const float* ape, const int64_t* slot_mapping,
                               int kpool, bool fp8, bool pow2, uint8_t* cache, int64_t num_pages,
                               float* compressed, hipStream_t stream) {
  if (f32)
    return fp8 ? launch_kp<true, 1>(k, n, row_stride, gate, ape, slot_mapping, kpool, num_pages,
                                    pow2, cache, compressed, stream)
               : launch_kp<true, 0>(k, n, row_stride, gate, ape, slot_mapping, kpool, num_pages,
                                    pow2, cache, compressed, stream);
  return fp8 ? launch_kp<false, 1>(k, n, row_stride, gate, ape, slot_mapping, kpool, num_pages,
                                   pow2, cache, compressed, stream)
             : launch_kp<false, 0>(k, n, row_stride, gate, ape, slot_mapping, kpool, num_pages,
                                   pow2, cache, compressed, stream);
}

}  // namespace mxidx
