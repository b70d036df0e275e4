// FP8 (E4M3) indexer cache: the format the MXFP4 cache replaces (P1 "[Kernel]
// MXFP4 indexer cache for GLM-5.2 / DSA", section "Benefit": 132 bytes per
// token per head against 68), with the same roles -- quantize, insert through
// a slot mapping, gather, dense and paged logits -- on gfx950's FP8 MFMA.
//
// Row format (132 bytes): 128 OCP E4M3 values and one fp32 scale.  Encode rule:
// s = amax / 448 in fp32 (floored at 2^-126), or with power-of-two scales
// (P3 "_kpool_compress_insert": round_scale) s = 2^E, E the smallest integer
// with amax <= 448 * 2^E; each element is x / s rounded to fp32, then to the
// nearest E4M3 value (ties to even) by the hardware conversion.  Pages keep
// the block-split layout: 64 value rows (8192 bytes), then 64 scale words.
//
// Query (P3 "forward_cuda": FP8 q is a single tensor, its per-token scale
// folded into the weights): the row encoder can also write w' = w * s_q, and
// the logits kernels take q's E4M3 values with w' as given:
//
//   logits[t, s] = s_k[s] * sum_h w'[t,h] * max(0, q8[t,h] . k8[s]),
//
// the positive K scale applied after the head sum.  Heads are the M dimension
// of v_mfma_scale_f32_16x16x128_f8f6f4 in its E4M3 x E4M3 form (unit scales):
// lane (g, n) supplies the 32 bytes 32g..32g+31 of row n, i.e. the whole
// 128-wide dot in one instruction; the ReLU-weighted head sum and the
// cross-lane reduction are the MXFP4 kernels' (logits_reduce.hpp).
//
// At equal throughput the FP8 MFMA takes twice the FP4 instruction's cycles
// for the same 65,536 flops, so here the 8 VALU instructions of the epilogue
// per MFMA no longer bound the prefill kernel: it is MFMA-bound at the FP8
// peak (half the FP4 one), which is where the FP4 kernel's VALU co-bound
// already holds that one.
#include "common.hpp"
#include "launch.hpp"
#include "fp8_encode.hpp"
#include "logits_reduce.hpp"

namespace mxidx {
namespace {

constexpr int kF8RowsPerBlock = 16;                // 256 threads, 16 lanes per row

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a row as fp32 values.
struct Bf16x8 {
  static __device__ __forceinline__ void load(const void* base, int64_t row, int64_t stride,
                                              int sub, float (&v)[8]) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) +
                                                    row * stride + 8 * sub);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
struct F32x8 {
  static __device__ __forceinline__ void load(const void* base, int64_t row, int64_t stride,
                                              int sub, float (&v)[8]) {
    const float* p = static_cast<const float*>(base) + row * stride + 8 * sub;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// kPaged = false: row r -> values[r*128], scales[r] (and w_out[r] = w_in[r] * s when given).
// kPaged = true:  row r -> slot slot_mapping[r]: values at page*8448 + off*128, the
//                 scale at page*8448 + 8192 + off*4; slots outside the cache write nothing.
// 16 lanes per row, 8 elements per lane; the row amax is an integer max over
// the magnitude bits reduced over the row's 16 lanes.
template <typename In, bool kPaged>
__global__ __launch_bounds__(256) void fp8_rows_kernel(const void* __restrict__ x, int64_t rows,
                                                       int64_t stride,
                                                       const int64_t* __restrict__ slot_mapping,
                                                       int64_t num_slots,
                                                       uint8_t* __restrict__ dst_values,
                                                       float* __restrict__ dst_scales, int pow2,
                                                       const float* __restrict__ w_in,
                                                       float* __restrict__ w_out) {
  const int sub = threadIdx.x & 15;
  for (int64_t row = (int64_t)blockIdx.x * kF8RowsPerBlock + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * kF8RowsPerBlock) {
    uint8_t* vdst;
    float* sdst;
    if constexpr (kPaged) {
      const int64_t slot = slot_mapping[row];       // same for the row's 16 lanes
      if (slot < 0 || slot >= num_slots) continue;
      const int64_t page = slot / kPage, off = slot % kPage;
      vdst = dst_values + page * kF8PageBytes + off * kF8Row;
      sdst = reinterpret_cast<float*>(dst_values + page * kF8PageBytes + kF8PageValues + off * 4);
    } else {
      vdst = dst_values + row * kF8Row;
      sdst = dst_scales + row;
    }
    float v[8];
    In::load(x, row, stride, sub, v);
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = max(a, __float_as_uint(v[i]) & 0x7fffffffu);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) a = max(a, (uint32_t)__shfl_xor((int)a, m));
    const float s = fp8_row_scale(a, pow2 != 0);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] / s;      // correctly rounded fp32 division
    const uint2 packed = make_uint2(pack_fp8x4(y[0], y[1], y[2], y[3]),
                                    pack_fp8x4(y[4], y[5], y[6], y[7]));
    *reinterpret_cast<uint2*>(vdst + 8 * sub) = packed;
    if (sub == 0) {
      *sdst = s;
      if constexpr (!kPaged)
        if (w_out) w_out[row] = w_in[row] * s;
    }
  }
}

int f8_grid(int64_t rows) {
  const int64_t blocks = (rows + kF8RowsPerBlock - 1) / kF8RowsPerBlock;
  const int64_t cap = 256 * 32;
  return (int)(blocks < cap ? blocks : cap);
}

// Paged FP8 cache -> contiguous rows: one 512-thread workgroup per (sequence,
// page), 8 lanes of 16 bytes per token, the first of them also moving the scale.
__global__ __launch_bounds__(512) void gather_fp8_kernel(const uint8_t* __restrict__ cache,
                                                         int64_t num_pages,
                                                         const int32_t* __restrict__ block_table,
                                                         int64_t bt_row_stride,
                                                         const int32_t* __restrict__ seq_lens,
                                                         const int64_t* __restrict__ cu_seq_offsets,
                                                         int64_t total_tokens,
                                                         uint8_t* __restrict__ k_values,
                                                         float* __restrict__ k_scales) {
  const int b = blockIdx.y;
  const int64_t lp = blockIdx.x;
  const int64_t j = lp * kPage + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  // the three index loads in one round trip, as vector loads (as in the MXFP4
  // gather); the table entry exists for every launched page
  const int32_t len = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(seq_lens + b, 4), 0, 0, 0);
  const int32_t page32 = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_rsrc(block_table + (int64_t)b * bt_row_stride + lp, 4), 0, 0, 0);
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(cu_seq_offsets + b, 8);
  const uint32_t f_lo = __builtin_amdgcn_raw_buffer_load_b32(ro, 0, 0, 0);
  const uint32_t f_hi = __builtin_amdgcn_raw_buffer_load_b32(ro, 4, 0, 0);
  const int64_t page = __builtin_amdgcn_readfirstlane(page32);
  const int64_t row = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)f_hi) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((int)f_lo)) + j;
  if (j >= __builtin_amdgcn_readfirstlane(len) || page < 0 || page >= num_pages || row < 0 ||
      row >= total_tokens)
    return;
  const int off = (int)(j % kPage);
  const uint8_t* pbase = cache + page * kF8PageBytes;
  *reinterpret_cast<uint4*>(k_values + row * kF8Row + part * 16) =
      *reinterpret_cast<const uint4*>(pbase + off * kF8Row + part * 16);
  if (part == 0) k_scales[row] = *reinterpret_cast<const float*>(pbase + kF8PageValues + off * 4);
}

// E4M3 x E4M3 MFMA (unit scales): 16 heads x 16 keys, the full 128-wide dot.
__device__ __forceinline__ v4f mfma_fp8(const uint4 (&a)[2], const uint4 (&b)[2], v4f c) {
  const v8i av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                  (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
  const v8i bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                  (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
  // cbsz = blgp = 0: E4M3 operands; scale bytes 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

template <int kAux>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kAux);
  return make_uint4(c.x, c.y, c.z, c.w);
}

template <int NH>
struct F8Query {
  uint4 a[NH][2];     // group grp: bytes 32g..32g+31 of head 16*grp + n
  float4 w[NH];       // w' of heads 16*grp + 4g .. +3
};

template <int NH>
__device__ __forceinline__ F8Query<NH> load_f8_query(const uint8_t* __restrict__ q_values,
                                                     const float* __restrict__ weights, int64_t r,
                                                     int g, int n) {
  constexpr int H = 16 * NH;
  F8Query<NH> q;
#pragma unroll
  for (int grp = 0; grp < NH; ++grp) {
    const uint8_t* p = q_values + (r * H + 16 * grp + n) * kF8Row + 32 * g;
    q.a[grp][0] = *reinterpret_cast<const uint4*>(p);
    q.a[grp][1] = *reinterpret_cast<const uint4*>(p + 16);
    q.w[grp] = *reinterpret_cast<const float4*>(weights + r * H + 16 * grp + 4 * g);
  }
  return q;
}

// 64 keys: tile j = keys 16j + n, lane (g, n) holding bytes 32g..32g+31; lane l
// also holds the scale of key l.
struct F8Tile {
  uint4 v[4][2];
  float scale;
};

// Scores of the 64 keys against the query's heads.  The next head group's four
// MFMAs are issued before the current group's ReLU-weighted sums, so the matrix
// core works while the vector ALU runs the epilogue; the sums keep the head
// order, so the result is the same bits as one group at a time.
template <int NH>
__device__ __forceinline__ float f8_tile_score(const F8Tile& t, const F8Query<NH>& q) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  v4f d[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) d[0][j] = mfma_fp8(q.a[0], t.v[j], zero);
#pragma unroll
  for (int grp = 0; grp < NH; ++grp) {
    if (grp + 1 < NH)
#pragma unroll
      for (int j = 0; j < 4; ++j) d[(grp + 1) & 1][j] = mfma_fp8(q.a[grp + 1], t.v[j], zero);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = relu_weighted(d[grp & 1][j], q.w[grp], acc[j]);
  }
  return reduce_tiles(acc) * t.scale;
}

// ---------------------------------------------------------------------------
// Query sources of the paged kernel.  F8Packed: rows encoded beforehand (E4M3
// values and the folded weights).
struct F8Packed {
  const uint8_t* q_values;
  const float* weights;
  static constexpr bool kInsert = false;
  static constexpr int kPages = 2;
  template <int NH>
  using Fetched = F8Query<NH>;
  template <int NH>
  __device__ __forceinline__ F8Query<NH> fetch(int64_t r, int g, int n) const {
    return load_f8_query<NH>(q_values, weights, r, g, n);
  }
  template <int NH>
  __device__ __forceinline__ F8Query<NH> finish(const F8Query<NH>& f) const {
    return f;
  }
};

// The 32 elements 32g..32g+31 of a 128-wide row: loaded as 16-byte words
// (bf16 or fp32), then read as fp32 values.
template <bool kF32>
struct Raw32 {
  uint4 v[kF32 ? 8 : 4];
  __device__ __forceinline__ void load(const void* base, int64_t row, int g) {
    const uint4* p = kF32 ? reinterpret_cast<const uint4*>(static_cast<const float*>(base) +
                                                            row * kHeadDim + 32 * g)
                          : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) +
                                                           row * kHeadDim + 32 * g);
#pragma unroll
    for (int i = 0; i < (kF32 ? 8 : 4); ++i) v[i] = p[i];
  }
  __device__ __forceinline__ void values(float (&o)[32]) const {
#pragma unroll
    for (int i = 0; i < (kF32 ? 8 : 4); ++i) {
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (kF32) {
          o[4 * i + k] = __uint_as_float(u[k]);
        } else {
          o[8 * i + 2 * k] = __uint_as_float(u[k] << 16);
          o[8 * i + 2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
      }
    }
  }
};

// E4M3 encode of the row whose 4 blocks the lanes g = 0..3 of one column n
// hold (every lane of the wave takes part): the row encoder's rule -- the scale
// from the amax over the row, each element x / s correctly rounded in fp32
// (with power-of-two scales a multiply by the exact reciprocal, the same
// value), the hardware conversion -- packed in element order.  Returns s.
__device__ __forceinline__ float encode_block32(const float (&v)[32], bool pow2, uint4 (&out)[2]) {
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = max(a, __float_as_uint(v[i]) & 0x7fffffffu);
  a = max(a, (uint32_t)__shfl_xor((int)a, 16));
  a = max(a, (uint32_t)__shfl_xor((int)a, 32));
  const float s = fp8_row_scale(a, pow2);
  float y[32];
  if (pow2) {
    const float r = 1.0f / s;                      // exact: s is a power of two
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = v[i] * r;
  } else if (s >= 0x1p-64f) {
    // x / s correctly rounded without a division per element (Markstein's
    // theorem: with y = 1/s rounded, q0 = x*y within an ulp and the remainder
    // e = x - s*q0 exact under an FMA, fma(e, y, q0) is the rounded quotient when
    // nothing underflows).  For s >= 2^-64 that holds wherever |x/s| >= 2^-11;
    // smaller quotients round to an E4M3 zero either way, and x's sign bit is
    // copied so that -0 stays -0.  The host check tests/c/fp8_quotient_check.c
    // holds the route to the division bit for bit.
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float q0 = v[i] * r;
      const float q = fmaf(fmaf(-s, q0, v[i]), r, q0);
      y[i] = __uint_as_float((__float_as_uint(q) & 0x7fffffffu) | (__float_as_uint(v[i]) & 0x80000000u));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = v[i] / s;
  }
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = pack_fp8x4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
  out[0] = make_uint4(p[0], p[1], p[2], p[3]);
  out[1] = make_uint4(p[4], p[5], p[6], p[7]);
  return s;
}

// F8Raw: bf16 / fp32 query rows encoded in the wave -- lane (g, n) encodes
// block g of head 16*grp + n, the 32 bytes it supplies to the MFMA -- with the
// weights folded there (w' = w * s of the head's row, fetched from the lane
// that holds that row), so the operands equal the separate encode's; the new
// tokens' K rows come with it (kInsert).
template <bool kF32>
struct F8Raw {
  const void* q;          // [rows, H, 128]
  const void* k_new;      // [rows, 128]: row b*next_n + i is token L_b - next_n + i
  const float* weights;   // [rows, H], not folded
  int pow2;
  static constexpr bool kInsert = true;
  static constexpr bool kF32In = kF32;
  static constexpr int kPages = 3;
  template <int NH>
  struct Fetched {
    Raw32<kF32> blk[NH];
    float4 w[NH];
  };
  template <int NH>
  __device__ __forceinline__ Fetched<NH> fetch(int64_t r, int g, int n) const {
    constexpr int H = 16 * NH;
    Fetched<NH> f;
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      f.blk[grp].load(q, r * H + 16 * grp + n, g);
      f.w[grp] = *reinterpret_cast<const float4*>(weights + r * H + 16 * grp + 4 * g);
    }
    return f;
  }
  template <int NH>
  __device__ __forceinline__ F8Query<NH> finish(const Fetched<NH>& f) const {
    F8Query<NH> q8;
    const int g = (int)(threadIdx.x & 63) >> 4;
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      float v[32];
      f.blk[grp].values(v);
      const float s = encode_block32(v, pow2 != 0, q8.a[grp]);
      const float s0 = __shfl(s, 4 * g), s1 = __shfl(s, 4 * g + 1);
      const float s2 = __shfl(s, 4 * g + 2), s3 = __shfl(s, 4 * g + 3);
      q8.w[grp] = make_float4(f.w[grp].x * s0, f.w[grp].y * s1, f.w[grp].z * s2, f.w[grp].w * s3);
    }
    return q8;
  }
};

// ---------------------------------------------------------------------------
// Paged decode: one wave per workgroup over PPW (the query source's kPages)
// consecutive pages of one sequence (17 KB of cache in flight per wave at 2
// pages), pages read through buffer descriptors with a wave-uniform base (a
// missing page reads zeros, no access), query rows one at a time.  With a raw
// query source the wave that holds a new token's page first encodes that token
// and writes it to its slot.

template <int NH, int PPW, typename QS>
__global__ __launch_bounds__(kWave) void logits_paged_fp8_kernel(
    QS qs, const uint8_t* cache, int64_t num_pages,   // written when inserting: no restrict
    const int32_t* __restrict__ block_table,
    int64_t bt_row_stride, const int32_t* __restrict__ context_lens, int next_n, int64_t width,
    float* __restrict__ logits, int64_t ld, int clean, int stream_out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int g = lane >> 4, n = lane & 15;
  const int64_t lp0 = (int64_t)blockIdx.x * PPW;
  const int64_t wpages = (width + kPage - 1) / kPage;
  const int64_t row0 = (int64_t)b * next_n;
  const int bt_count = (int)min((int64_t)PPW, wpages - lp0);
  const int bt_lane = (int)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_rsrc(block_table + (int64_t)b * bt_row_stride + lp0, 4 * bt_count), 4u * lane, 0, 0);
  const int64_t ctx = (int32_t)__builtin_amdgcn_readfirstlane(
      (int)__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(context_lens + b, 4), 0, 0, 0));
  const int64_t L = min(ctx, width);

  auto store = [&](int64_t r, int64_t tok0, int64_t ke, float v) {
    const int64_t col = tok0 + lane;
    const bool scored = col < ke;
    const bool keep = scored || (clean && col < width);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(logits + r * ld + tok0, kPage * 4);
    const uint32_t bits = __float_as_uint(scored ? v : neg_inf());
    const uint32_t off = keep ? 4u * lane : kDropOffset;
    if (stream_out)
      __builtin_amdgcn_raw_buffer_store_b32(bits, rs, off, 0, kNonTemporal);
    else
      __builtin_amdgcn_raw_buffer_store_b32(bits, rs, off, 0, 0);
  };

  if (lp0 * kPage >= L) {
    if (clean)
      for (int i = 0; i < next_n; ++i)
#pragma unroll
        for (int p = 0; p < PPW; ++p) store(row0 + i, (lp0 + p) * kPage, 0, 0.f);
    return;
  }
  const int np = (int)min((int64_t)PPW, (L - lp0 * kPage + kPage - 1) / kPage);
  // a raw source's row 0 fetched ahead of the insert and the page loads (and
  // pinned there): its latency runs under the pages', and it is encoded while
  // the pages are still in flight (encoded rows keep the compiler's order)
  typename QS::template Fetched<NH> qf0;
  if constexpr (QS::kInsert) {
    qf0 = qs.template fetch<NH>(row0, g, n);
    asm volatile("" ::: "memory");
  }

  if constexpr (QS::kInsert) {
    // New token i sits at position P = context_len - next_n + i.  The wave whose
    // live pages hold it encodes it and writes it to the cache before loading
    // its pages: lane (g, n_t) later loads exactly the 32 value bytes it stores
    // here and lane `off` the scale word it stores, so the page loads see the
    // new token (program order of one lane, one address).  Pages past the row
    // width belong to no wave: tokens there are not written.
    for (int i = 0; i < next_n; ++i) {
      const int64_t P = ctx - next_n + i;
      const int64_t wp = P - lp0 * kPage;
      if (P < 0 || wp < 0 || wp >= (int64_t)np * kPage) continue;   // uniform
      const int p_t = (int)(wp / kPage), off = (int)(wp % kPage);
      const int64_t dst = __builtin_amdgcn_readlane(bt_lane, p_t);
      if (dst < 0 || dst >= num_pages) continue;   // invalid table entry: not written
      Raw32<QS::kF32In> kr;
      kr.load(qs.k_new, row0 + i, g);
      float v[32];
      kr.values(v);
      uint4 code[2];
      const float sc = encode_block32(v, qs.pow2 != 0, code);
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(const_cast<uint8_t*>(cache) + dst * kF8PageBytes, kF8PageBytes);
      const bool col = n == off % 16;
      const uint32_t voff = (uint32_t)(off * kF8Row + 32 * g);
      const u32x4 c0 = {code[0].x, code[0].y, code[0].z, code[0].w};
      const u32x4 c1 = {code[1].x, code[1].y, code[1].z, code[1].w};
      __builtin_amdgcn_raw_buffer_store_b128(c0, rs, col ? voff : kDropOffset, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(c1, rs, col ? voff + 16u : kDropOffset, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rs,
                                            lane == off ? (uint32_t)(kF8PageValues + 4 * off)
                                                        : kDropOffset,
                                            0, 0);
    }
    asm volatile("" ::: "memory");   // the page loads stay behind the stores
  }

  F8Tile pg[PPW];
  bool page_ok[PPW];
  const uint32_t off_v = (uint32_t)(kF8Row * n + 32 * g);
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int pid = __builtin_amdgcn_readlane(bt_lane, p);
    const bool valid = pid >= 0 && pid < num_pages;
    page_ok[p] = p >= np || valid;
    const int live = __builtin_amdgcn_readfirstlane((p < np && valid) ? 1 : 0);
    const int64_t page = __builtin_amdgcn_readfirstlane(live ? pid : 0);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(cache + page * kF8PageBytes, live ? kF8PageBytes : 0);
    // Lane (g, n) takes the 32 bytes 32g.. of key n as two 16-byte loads, so each
    // load instruction touches every 64-byte line of the 2 KB tile at half width
    // and the next touches the same lines.  Large batches load through the caches
    // (as non-temporal loads the second touch refetched the lines: 153 -> 134 us
    // on the long-context batch); small ones, whose logits stay in the caches for
    // the top-k, keep the non-temporal loads (cached, the 16 x 8192 decode step
    // took 18.2 us instead of 16.8).
    if (stream_out) {                            // wave-uniform
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pg[p].v[j][0] = ld16<0>(rs, off_v + 2048u * j);
        pg[p].v[j][1] = ld16<0>(rs, off_v + 2048u * j + 16u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pg[p].v[j][0] = ld16<kNonTemporal>(rs, off_v + 2048u * j);
        pg[p].v[j][1] = ld16<kNonTemporal>(rs, off_v + 2048u * j + 16u);
      }
    }
    pg[p].scale = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(kF8PageValues + 4 * lane), 0, kNonTemporal));
  }
  for (int i = 0; i < next_n; ++i) {
    const int64_t r = row0 + i;
    const int64_t ke = L - next_n + i + 1;
    const F8Query<NH> q = (QS::kInsert && i == 0)
                              ? qs.template finish<NH>(qf0)
                              : qs.template finish<NH>(qs.template fetch<NH>(r, g, n));
#pragma unroll
    for (int p = 0; p < PPW; ++p)
      if (page_ok[p]) store(r, (lp0 + p) * kPage, ke, f8_tile_score<NH>(pg[p], q));
  }
}

// ---------------------------------------------------------------------------
// Dense prefill: 4 waves x RW query rows per workgroup over a chunk of keys, 64
// keys per step, as the MXFP4 kernel (logits_prefill.hip) does; K rows are 128
// bytes and each key's scale is applied to its logit after the head sum.  Unlike
// the MXFP4 kernel, the K tiles go through LDS once per workgroup: a lane's 32
// bytes of a key are two 16-byte loads at half a line's width, and with every wave
// loading each tile itself the vector-memory path, not the matrix core, set the
// pace (one row per wave instead of two nearly doubled the time).  Staged tiles
// also free the registers of two tile buffers, so 3 waves fit per SIMD.
constexpr int kF8KeyChunkSmallS = 512;
constexpr int kF8KeyChunk = 4096;
constexpr int64_t kF8SmallS = 16384;

constexpr int kF8TileLds = 64 * 128 + 64 * 4;   // one 64-key tile: values, then scales

template <int NH, int RW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void logits_prefill_fp8_kernel(
    const uint8_t* __restrict__ q_values, const float* __restrict__ weights,
    const uint8_t* __restrict__ k_values, const float* __restrict__ k_scales,
    const int32_t* __restrict__ ks, const int32_t* __restrict__ ke, int64_t T, int S,
    float* __restrict__ logits, int64_t ld, int clean, int64_t n_qb, int64_t n_kc, int key_chunk) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, n = lane & 15;
  // Workgroup order as in the MXFP4 kernel: key-chunk-major for long inputs (the
  // resident workgroups share a K chunk in L2), XCD-aware for short ones
  int64_t qb, kc;
  if (key_chunk == kF8KeyChunk) {
    kc = n_kc - 1 - (int64_t)blockIdx.x / n_qb;
    qb = n_qb - 1 - (int64_t)blockIdx.x % n_qb;
  } else if (n_qb % 8 == 0) {
    const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
    qb = n_qb - 1 - ((j / n_kc) * 8 + x);
    kc = j % n_kc;
  } else {
    qb = n_qb - 1 - blockIdx.x / n_kc;
    kc = blockIdx.x % n_kc;
  }
  const int64_t t0 = qb * (4 * RW) + wave * RW;
  const int c_begin = (int)kc * key_chunk;
  const int c_end = (int)min((int64_t)c_begin + key_chunk, (int64_t)S);
  int lo[RW], hi[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t t = t0 + i;
    lo[i] = 0;
    hi[i] = 0;
    if (t < T) {
      lo[i] = ks ? max(ks[t], 0) : 0;
      hi[i] = min(ke[t], S);
    }
  }
  // the window of the whole workgroup: its 4 waves share the K tiles
  int need_lo = c_end, need_hi = c_begin;
  for (int r = 0; r < 4 * RW; ++r) {
    const int64_t t = qb * (4 * RW) + r;
    if (t >= T) break;
    const int l = ks ? max(ks[t], 0) : 0, h = min(ke[t], S);
    if (l < h) {
      need_lo = min(need_lo, max(l, c_begin));
      need_hi = max(need_hi, min(h, c_end));
    }
  }
  need_lo = __builtin_amdgcn_readfirstlane(need_lo);
  need_hi = __builtin_amdgcn_readfirstlane(need_hi);
  float* lrow[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) lrow[i] = logits + min(t0 + i, T - 1) * ld;
  auto store = [&](int i, int c0, float v, bool live = true) {
    c0 = __builtin_amdgcn_readfirstlane(max(c0, 0));
    uint32_t off = 4u * lane;
    if (t0 + i >= T || !live) off = kDropOffset;
    if (!(c0 >= lo[i] && c0 + 64 <= hi[i])) {          // a tile that straddles [ks, ke)
      const int col = c0 + lane;
      const bool scored = col >= lo[i] && col < hi[i];
      if (!scored) v = neg_inf();
      if (!scored && !(clean && col < c_end)) off = kDropOffset;
    }
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), buffer_rsrc(lrow[i] + c0, 64 * 4), off,
                                          0, kNonTemporal);
  };
  const int k_first = c_begin + ((need_lo - c_begin) & ~63);
  if (clean) {
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
      if (need_lo < need_hi && c0 >= k_first && c0 < need_hi) continue;
#pragma unroll
      for (int i = 0; i < RW; ++i) store(i, c0, neg_inf());
    }
  }
  if (need_lo >= need_hi) return;

  F8Query<NH> q[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) q[i] = load_f8_query<NH>(q_values, weights, min(t0 + i, T - 1), g, n);

  // K tiles staged once per workgroup in LDS, two buffers.  A tile's 8 KB of
  // values are 8 slices of 1 KB, slice 2j + h holding, for lane (g, n), bytes
  // 32g + 16h .. +15 of key 16j + n (the 16 bytes that lane supplies as half h of
  // MFMA tile j); wave w copies slices 2w and 2w + 1 with 16-byte buffer-to-LDS
  // loads and every wave the 64 key scales (identical data).  Keys at or past S
  // read as zeros.  A tile's results are stored one step later, and one barrier
  // per step publishes the next tile and frees the current one.
  __shared__ __attribute__((aligned(16))) uint8_t kb0[kF8TileLds];
  __shared__ __attribute__((aligned(16))) uint8_t kb1[kF8TileLds];
  const uint32_t src0 = (uint32_t)((16 * wave + n) * kF8Row + 32 * g);
  auto dma = [&](uint8_t* kb, int c0) {
    c0 = __builtin_amdgcn_readfirstlane(c0);
    const int keys = __builtin_amdgcn_readfirstlane(max(min(S - c0, 64), 0));
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(k_values + (int64_t)c0 * kF8Row, keys * kF8Row);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(k_scales + (int64_t)c0, keys * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (__attribute__((address_space(3))) void*)(kb + 2048 * wave), 16, src0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (__attribute__((address_space(3))) void*)(kb + 2048 * wave + 1024), 16, src0 + 16u, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(kb + 8192), 4, 4u * lane, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // the copy stays ahead of the step's stores
  };
  // Scores of the 64 keys of an LDS tile for the wave's rows, tile j outermost:
  // acc[i][j] sums the head groups in order, so the bits equal f8_tile_score's.
  auto score_lds = [&](const uint8_t* kb, float (&out)[RW]) {
    constexpr int P = RW * NH;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    float acc[RW][4];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 v[2];
      v[0] = *reinterpret_cast<const uint4*>(kb + 2048 * j + 16 * lane);
      v[1] = *reinterpret_cast<const uint4*>(kb + 2048 * j + 1024 + 16 * lane);
      v4f d[3];
      d[0] = mfma_fp8(q[0].a[0], v, zero);
      if (P > 1) d[1] = mfma_fp8(q[1 / NH].a[1 % NH], v, zero);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (p + 2 < P) d[(p + 2) % 3] = mfma_fp8(q[(p + 2) / NH].a[(p + 2) % NH], v, zero);
        acc[p / NH][j] = relu_weighted(d[p % 3], q[p / NH].w[p % NH], acc[p / NH][j]);
      }
    }
    const float sc = *reinterpret_cast<const float*>(kb + 8192 + 4 * lane);
#pragma unroll
    for (int i = 0; i < RW; ++i) out[i] = reduce_tiles(acc[i]) * sc;
  };
  // vmcnt counts loads and stores in issue order: after a step only its RW
  // stores may still be outstanding, so the wait covers the tile copy alone
  constexpr int kWaitCopy = (RW & 15) | (0x7 << 4) | (0xF << 8);
  float res[RW] = {};
  int prev = -1;
  auto step_from = [&](const uint8_t* kb, int c0) {
#pragma unroll
    for (int i = 0; i < RW; ++i) store(i, prev, res[i], prev >= 0);
    score_lds(kb, res);
#pragma unroll
    for (int i = 0; i < RW; ++i) asm volatile("" ::"v"(res[i]));   // done before the barrier
    prev = c0;
    __builtin_amdgcn_s_waitcnt(kWaitCopy);
    asm volatile("s_barrier" ::: "memory");
  };
  dma(kb0, k_first);
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("s_barrier" ::: "memory");
  for (int c0 = k_first; c0 < need_hi; c0 += 128) {
    dma(kb1, c0 + 64);
    step_from(kb0, c0);
    if (c0 + 64 >= need_hi) break;
    dma(kb0, c0 + 128);
    step_from(kb1, c0 + 64);
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) store(i, prev, res[i], true);
}

template <int NH, typename QS>
hipError_t launch_paged_fp8_nh(QS qs, const uint8_t* cache, int64_t num_pages, const int32_t* bt,
                               int64_t bt_stride, const int32_t* ctx, int B, int next_n,
                               int64_t width, float* logits, int64_t ld, int clean,
                               hipStream_t stream) {
  const int64_t pages = (width + kPage - 1) / kPage;
  const int stream_out = (int64_t)B * next_n * width * 4 > (4 << 20) ? 1 : 0;
  constexpr int P = QS::kPages;
  const dim3 grid((unsigned)((pages + P - 1) / P), (unsigned)B);
  hipLaunchKernelGGL((logits_paged_fp8_kernel<NH, P, QS>), grid, dim3(kWave), 0, stream,
                     qs, cache, num_pages, bt, bt_stride, ctx, next_n, width, logits, ld, clean,
                     stream_out);
  return hipGetLastError();
}

template <typename QS>
hipError_t launch_paged_fp8_source(QS qs, const uint8_t* cache, int64_t num_pages,
                                   const int32_t* block_table, int64_t bt_row_stride,
                                   const int32_t* context_lens, int B, int next_n, int H,
                                   int64_t max_context_len, float* logits, int64_t ld, int clean,
                                   hipStream_t stream) {
#define MXIDX_F8P(nh)                                                                          \
  case nh:                                                                                     \
    return launch_paged_fp8_nh<nh>(qs, cache, num_pages, block_table, bt_row_stride,           \
                                   context_lens, B, next_n, max_context_len, logits, ld, clean, \
                                   stream);
  switch (H / 16) {
    MXIDX_F8P(1)
    MXIDX_F8P(2)
    MXIDX_F8P(3)
    MXIDX_F8P(4)
    MXIDX_F8P(5)
    MXIDX_F8P(6)
    MXIDX_F8P(7)
    MXIDX_F8P(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MXIDX_F8P
}

template <int NH, int RW>
hipError_t launch_prefill_fp8_cfg(const uint8_t* qv, const float* w, const uint8_t* kv,
                                  const float* ksc, const int32_t* ks, const int32_t* ke, int64_t T,
                                  int64_t S, float* logits, int64_t ld, int clean,
                                  hipStream_t stream) {
  const int64_t n_qb = (T + 4 * RW - 1) / (4 * RW);
  const int key_chunk = S <= kF8SmallS ? kF8KeyChunkSmallS : kF8KeyChunk;
  const int64_t n_kc = (S + key_chunk - 1) / key_chunk;
  hipLaunchKernelGGL((logits_prefill_fp8_kernel<NH, RW>), dim3((unsigned)(n_qb * n_kc)), dim3(256), 0,
                     stream, qv, w, kv, ksc, ks, ke, T, (int)S, logits, ld, clean, n_qb, n_kc,
                     key_chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, bool f32, int64_t rows, int64_t row_stride, bool pow2,
                               uint8_t* values, float* scales, const float* w_in, float* w_out,
                               hipStream_t stream) {
  const int grid = f8_grid(rows);
  if (f32)
    hipLaunchKernelGGL((fp8_rows_kernel<F32x8, false>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, nullptr, 0, values, scales, pow2 ? 1 : 0, w_in, w_out);
  else
    hipLaunchKernelGGL((fp8_rows_kernel<Bf16x8, false>), dim3(grid), dim3(256), 0, stream, x, rows,
                       row_stride, nullptr, 0, values, scales, pow2 ? 1 : 0, w_in, w_out);
  return hipGetLastError();
}

hipError_t launch_insert_fp8(const void* k, bool f32, int64_t num_tokens, int64_t row_stride,
                             bool pow2, const int64_t* slot_mapping, uint8_t* cache,
                             int64_t num_pages, hipStream_t stream) {
  const int grid = f8_grid(num_tokens);
  const int64_t num_slots = num_pages * kPage;
  if (f32)
    hipLaunchKernelGGL((fp8_rows_kernel<F32x8, true>), dim3(grid), dim3(256), 0, stream, k,
                       num_tokens, row_stride, slot_mapping, num_slots, cache, nullptr,
                       pow2 ? 1 : 0, nullptr, nullptr);
  else
    hipLaunchKernelGGL((fp8_rows_kernel<Bf16x8, true>), dim3(grid), dim3(256), 0, stream, k,
                       num_tokens, row_stride, slot_mapping, num_slots, cache, nullptr,
                       pow2 ? 1 : 0, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_gather_fp8(const uint8_t* cache, int64_t num_pages, const int32_t* block_table,
                             int64_t bt_row_stride, const int32_t* seq_lens,
                             const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                             int64_t total_tokens, uint8_t* k_values, float* k_scales,
                             hipStream_t stream) {
  const int64_t pages = (max_seq_len + kPage - 1) / kPage;
  hipLaunchKernelGGL(gather_fp8_kernel, dim3((unsigned)pages, (unsigned)batch), dim3(512), 0,
                     stream, cache, num_pages, block_table, bt_row_stride, seq_lens,
                     cu_seq_offsets, total_tokens, k_values, k_scales);
  return hipGetLastError();
}

hipError_t launch_logits_paged_fp8(const uint8_t* q_values, const float* weights,
                                   const uint8_t* cache, int64_t num_pages,
                                   const int32_t* block_table, int64_t bt_row_stride,
                                   const int32_t* context_lens, int B, int next_n, int H,
                                   int64_t max_context_len, float* logits, int64_t ld, int clean,
                                   hipStream_t stream) {
  return launch_paged_fp8_source(F8Packed{q_values, weights}, cache, num_pages, block_table,
                                 bt_row_stride, context_lens, B, next_n, H, max_context_len,
                                 logits, ld, clean, stream);
}

hipError_t launch_logits_paged_insert_fp8(const void* q, const void* k_new, bool f32,
                                          const float* weights, bool pow2, uint8_t* cache,
                                          int64_t num_pages, const int32_t* block_table,
                                          int64_t bt_row_stride, const int32_t* context_lens,
                                          int B, int next_n, int H, int64_t max_context_len,
                                          float* logits, int64_t ld, int clean,
                                          hipStream_t stream) {
  if (f32)
    return launch_paged_fp8_source(F8Raw<true>{q, k_new, weights, pow2 ? 1 : 0}, cache,
                                   num_pages, block_table, bt_row_stride, context_lens, B, next_n,
                                   H, max_context_len, logits, ld, clean, stream);
  return launch_paged_fp8_source(F8Raw<false>{q, k_new, weights, pow2 ? 1 : 0}, cache, num_pages,
                                 block_table, bt_row_stride, context_lens, B, next_n, H,
                                 max_context_len, logits, ld, clean, stream);
}

hipError_t launch_logits_prefill_fp8(const uint8_t* q_values, const float* weights,
                                     const uint8_t* k_values, const float* k_scales,
                                     const int32_t* ks, const int32_t* ke, int64_t T, int H,
                                     int64_t S, float* logits, int64_t ld, int clean,
                                     hipStream_t stream) {
#define MXIDX_F8X(nh, rw)                                                                        \
  case nh:                                                                                       \
    return launch_prefill_fp8_cfg<nh, rw>(q_values, weights, k_values, k_scales, ks, ke, T, S,  \
                                          logits, ld, clean, stream);
  switch (H / 16) {
    MXIDX_F8X(1, 4)
    MXIDX_F8X(2, 4)
    MXIDX_F8X(3, 2)
    MXIDX_F8X(4, 2)
    MXIDX_F8X(5, 1)
    MXIDX_F8X(6, 1)
    MXIDX_F8X(7, 1)
    MXIDX_F8X(8, 1)
    default:
      return hipErrorInvalidValue;
  }
#undef MXIDX_F8X
}

}  // namespace mxidx
