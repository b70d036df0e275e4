// Paged decode indexer logits (paged_mqa_logits of P3
// "SparseAttnIndexerKpool"; P2 "Summary": paged-decode MQA-logits kernel):
//
//   logits[r, s] = sum_h w[r,h] * max(0, qhat[r,h] . khat[s]),   s < L_b - next_n + i + 1
//
// with row r = b*next_n + i and token s read from page block_table[b, s/64]
// of the block-split MXFP4 cache (P1 live-validation comment).
//
// Design (HBM-bound: 68 bytes of K per scored token, 4 bytes of logit out):
//  * grid = (logical pages / 3, sequences), one wave per workgroup, so the
//    dispatcher balances ragged sequence lengths at a fine grain; each wave
//    owns three consecutive pages of one sequence (13 KB of cache) and has
//    every page's loads in flight before it computes any.  Three measured
//    faster than two (more bytes in flight per wave) and than four (fewer
//    waves) on long contexts.
//  * A page's base address is wave-uniform: it goes into a buffer descriptor
//    in scalar registers and every lane keeps one fixed offset, so a page
//    costs no vector address arithmetic.  A missing page (past the context,
//    or an invalid block-table entry) gets a zero-length descriptor: its
//    loads return zeros without touching memory.
//  * Lane l takes 16 bytes (block l/16 of token 16*j + l%16) for each of the
//    page's 4 token tiles j -- the page's 4096 code bytes as one contiguous
//    sweep -- plus each token's 4 scale bytes.  The cache streams through
//    once per call, so the loads are non-temporal; logit stores are too when
//    the output exceeds a few MB (else they stay cached for the top-k).
//  * Heads are the MFMA M dimension: per 16-head group one
//    v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1, UE8M0 scale per 32-wide
//    block and lane) per token tile gives the exact scaled head dots.  An
//    output column depends on its own token only, so tokens past the context
//    need no masking of operands, only of stores.
//  * ReLU and the head weights are applied on the fp32 MFMA output; lane-pair
//    swaps across the wave halves and quarters combine the four lane groups'
//    partial sums, after which lane l owns token l of the page and the wave
//    stores 64 consecutive floats.
//  * The fused decode step (query source RawQuery) takes q and the new
//    tokens' K in bf16 / fp32: each wave encodes its query rows itself, and
//    the wave whose pages hold a new token encodes it, writes it to the cache
//    and patches its page registers, so one launch does insert, quantize and
//    logits.  Only the sequence's own pages are written, and no other wave
//    reads them.
//  * Vector memory counters retire in issue order, so a wait for a load also
//    waits for every store issued before it: for up to NN query rows per
//    sequence (NN * heads/16 <= 8) every row's query is loaded up front and
//    all logit stores are issued after the wave's last load; more rows take a
//    general loop (one row at a time).
#include "common.hpp"
#include "launch.hpp"
#include "logits_reduce.hpp"
#include "mxfp4_encode.hpp"

namespace mxidx {
namespace {

// Pages per wave: 3 (13 KB of cache in flight) for batches that fill the chip;
// a small batch (at most ~2 waves per SIMD at 3 pages) runs one-row decode with
// the query source's kSmallPages (fewer pages: less work after the last page
// arrives; 16 x 8192, one launch: 4.65 -> 4.47 us at 2 pages).
constexpr int kPagesPerWave = 3;
constexpr int64_t kSmallGrid = 2048;
constexpr int64_t kCachedLogitsBytes = 4 << 20;
struct PageRegs {
  uint4 code[4];      // tile j: block g of token 16*j + n
  uint32_t scale[4];  // tile j: the 4 scale bytes of token 16*j + n
};

template <int NH>
struct QueryRegs {
  uint4 a[NH];        // group grp: block g of head 16*grp + n
  int sa[NH];         // its UE8M0 scale byte
  float4 w[NH];       // weights of heads 16*grp + 4*g .. +3
};

template <int NH>
__device__ __forceinline__ QueryRegs<NH> load_query(const uint8_t* __restrict__ q_values,
                                                    const uint8_t* __restrict__ q_scales,
                                                    const float* __restrict__ weights, int64_t r,
                                                    int g, int n) {
  constexpr int H = 16 * NH;
  QueryRegs<NH> q;
#pragma unroll
  for (int grp = 0; grp < NH; ++grp) {
    const int64_t qrow = r * H + 16 * grp + n;
    q.a[grp] = *reinterpret_cast<const uint4*>(q_values + qrow * kCodeBytes + g * 16);
    q.sa[grp] = q_scales[qrow * kScaleBytes + g];
    q.w[grp] = *reinterpret_cast<const float4*>(weights + r * H + 16 * grp + 4 * g);
  }
  return q;
}

// Query source of the paged kernel: MXFP4 rows encoded beforehand.  fetch()
// issues the loads, finish() turns fetched registers into MFMA operands.
struct PackedQuery {
  const uint8_t* q_values;
  const uint8_t* q_scales;
  const float* weights;
  static constexpr bool kInsert = false;
  template <int NH>
  using Fetched = QueryRegs<NH>;
  static constexpr bool kRope = false;
  static constexpr int kSmallPages = 1;    // 16 x 8192: 4.33 -> 4.24 us
  template <int NH>
  __device__ __forceinline__ QueryRegs<NH> fetch(int64_t r, int g, int n, int64_t) const {
    return load_query<NH>(q_values, q_scales, weights, r, g, n);
  }
  template <int NH>
  __device__ __forceinline__ QueryRegs<NH> finish(const QueryRegs<NH>& f) const {
    return f;
  }
};

// Angle operands of one query row for a lane's 32-element block: cosines and
// sines of the block's angles (neox: 32 consecutive angles, interleaved: 16)
// and whether the row is rotated (its position lies inside the table).
template <bool kOn>
struct RopeRegs {};
template <>
struct RopeRegs<true> {
  float4 c[8];
  float4 s[8];
  int on;
};

__device__ __forceinline__ float comp(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The word of lane l ^ 16 (K 16) or l ^ 32 (K 32), by gfx950's lane swaps
// (see reduce_tiles for their lane mapping).
template <int K>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int g) {
  if constexpr (K == 32) {
    const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return g < 2 ? s[1] : s[0];
  } else {
    const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (g & 1) ? s[0] : s[1];
  }
}

// One product pair of a rotation, each product and the sum rounded to fp32:
// x*c + y*s.  With s negated this is a*cos - b*sin exactly (a negated
// product is exact), so both halves of a pair take this one form.
__device__ __forceinline__ float rot_sum(float x, float c, float y, float s) {
#pragma clang fp contract(off)
  return x * c + y * s;
}

// Neox pairs (j, j + rope_dim/2) with rope_dim 64 (K 16: blocks 0 and 1) or
// 128 (K 32: blocks g and g ^ 2): element e of this lane's block pairs with
// element e of the partner lane's, at the e-th of the lane's angles.
template <int K, typename Blk>
__device__ __forceinline__ void rope_neox(const Blk& b, const RopeRegs<true>& r, int g, float (&o)[32]) {
  const bool rot = K == 32 || g < 2;           // rope_dim 64: blocks 2, 3 pass
  const bool is_a = K == 32 ? g < 2 : g == 0;  // this lane holds the pairs' first elements
  const uint32_t flip = is_a ? 0x80000000u : 0u;
#pragma unroll
  for (int k = 0; k < 32 / Blk::kPerWord; ++k) {
    const uint32_t w = b.word(k);
    const uint32_t pw = lane_xor<K>(w, g);
#pragma unroll
    for (int h = 0; h < Blk::kPerWord; ++h) {
      const int e = k * Blk::kPerWord + h;
      const float x = Blk::elem(w, h), y = Blk::elem(pw, h);
      const float c = comp(r.c[e >> 2], e & 3);
      const float s = __uint_as_float(__float_as_uint(comp(r.s[e >> 2], e & 3)) ^ flip);
      o[e] = rot ? rot_sum(x, c, y, s) : x;
    }
  }
}

// Interleaved pairs (2j, 2j + 1): pair m of this lane's block is angle
// 16g + m, rotated while that angle is below rope_dim/2.
template <typename Blk>
__device__ __forceinline__ void rope_interleaved(const Blk& b, const RopeRegs<true>& r, int g,
                                                 int half, float (&o)[32]) {
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    float a, bb;
    if constexpr (Blk::kPerWord == 2) {
      const uint32_t w = b.word(m);
      a = Blk::elem(w, 0);
      bb = Blk::elem(w, 1);
    } else {
      a = Blk::elem(b.word(2 * m), 0);
      bb = Blk::elem(b.word(2 * m + 1), 0);
    }
    const float c = comp(r.c[m >> 2], m & 3), s = comp(r.s[m >> 2], m & 3);
    const bool rot = 16 * g + m < half;
    o[2 * m] = rot ? rot_sum(a, c, bb, -s) : a;
    o[2 * m + 1] = rot ? rot_sum(bb, c, a, s) : bb;
  }
}

// Query source of the fused decode step: q rows in bf16 / fp32 (Blk), encoded
// to MXFP4 in the wave -- lane (g, n) encodes block g of head 16*grp + n, the
// block it supplies to the MFMA -- with the rule and conversion of the row
// encoders, so the operands equal those of the separate encode.  The new
// tokens' K rows come with it (kInsert).  With kRopeOn the rows are first
// rotated (RopeSpec; neox needs rope_dim 64 or 128) at position P, in fp32,
// and encoded as fp32 rows: the bytes of the separate RoPE encode.  The angle
// loads are issued with the query rows, ahead of the page loads.
template <bool kOn>
struct RopeField {};      // empty without RoPE: the kernel arguments stay as they were
template <>
struct RopeField<true> {
  RopeSpec rope;
};

template <typename Blk, bool kRopeOn = false>
struct RawQuery : RopeField<kRopeOn> {
  const void* q;          // [rows, H, 128]
  const void* k_new;      // [rows, 128]: row b*next_n + i is token L_b - next_n + i
  const float* weights;
  static constexpr bool kInsert = true;
  static constexpr bool kRope = kRopeOn;
  // each wave also encodes the query rows: 2 pages per wave for small batches,
  // 3 with RoPE, whose per-wave rotation more waves would repeat (6.74 / 6.83 us)
  static constexpr int kSmallPages = kRopeOn ? 3 : 2;
  using Block = Blk;
  template <int NH>
  struct Fetched {
    Blk blk[NH];
    float4 w[NH];
    RopeRegs<kRopeOn> r;
  };
  template <int NH>
  __device__ __forceinline__ Fetched<NH> fetch(int64_t r, int g, int n, int64_t P) const {
    constexpr int H = 16 * NH;
    constexpr int kRow = kHeadDim * Blk::kElemBytes;
    Fetched<NH> f;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(static_cast<const uint8_t*>(q) + r * H * kRow, H * kRow);
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      f.blk[grp].load(rs, (uint32_t)((16 * grp + n) * kRow + g * kBlock * Blk::kElemBytes));
      f.w[grp] = *reinterpret_cast<const float4*>(weights + r * H + 16 * grp + 4 * g);
    }
    if constexpr (kRopeOn) {
      // the table row P, bounded at rope_dim/2 angles (angles past it read 0,
      // without an access); a position outside the table rotates nothing
      const int half = this->rope.rope_dim >> 1;
      const bool on = P >= 0 && P < this->rope.table_rows;   // wave-uniform
      f.r.on = on ? 1 : 0;
      const int64_t prow = on ? P : 0;
      const int bytes = on ? 4 * half : 0;
      const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(this->rope.cos_t + prow * half, bytes);
      const __amdgpu_buffer_rsrc_t rn = buffer_rsrc(this->rope.sin_t + prow * half, bytes);
      const int base = this->rope.interleaved ? 16 * g
                                              : (this->rope.rope_dim == 128 ? 32 * (g & 1) : 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint4 c = load16(rc, 4u * (uint32_t)(base + 4 * k));
        const uint4 s = load16(rn, 4u * (uint32_t)(base + 4 * k));
        f.r.c[k] = make_float4(__uint_as_float(c.x), __uint_as_float(c.y), __uint_as_float(c.z),
                               __uint_as_float(c.w));
        f.r.s[k] = make_float4(__uint_as_float(s.x), __uint_as_float(s.y), __uint_as_float(s.z),
                               __uint_as_float(s.w));
      }
    }
    return f;
  }
  template <int NH>
  __device__ __forceinline__ QueryRegs<NH> finish(const Fetched<NH>& f) const {
    QueryRegs<NH> q;
    if constexpr (kRopeOn) {
      if (f.r.on) {                      // wave-uniform
        const int g = (int)(threadIdx.x & 63) >> 4;
#pragma unroll
        for (int grp = 0; grp < NH; ++grp) {
          float o[32];
          if (this->rope.interleaved)
            rope_interleaved(f.blk[grp], f.r, g, this->rope.rope_dim >> 1, o);
          else if (this->rope.rope_dim == 128)
            rope_neox<32>(f.blk[grp], f.r, g, o);
          else
            rope_neox<16>(f.blk[grp], f.r, g, o);
          F32Block ob;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            ob.v[i] = make_uint4(__float_as_uint(o[4 * i]), __float_as_uint(o[4 * i + 1]),
                                 __float_as_uint(o[4 * i + 2]), __float_as_uint(o[4 * i + 3]));
          const uint32_t a = ob.amax_bits();
          const int E = block_exponent(a);
          q.a[grp] = ob.encode(block_divisor(a, E));
          q.sa[grp] = E + 127;
          q.w[grp] = f.w[grp];
        }
        return q;
      }
    }
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      const uint32_t a = f.blk[grp].amax_bits();
      const int E = block_exponent(a);
      q.a[grp] = f.blk[grp].encode(block_divisor(a, E));
      q.sa[grp] = E + 127;
      q.w[grp] = f.w[grp];
    }
    return q;
  }
};

// The new token's K block a wave preloads with its table entries: one bf16
// row (64 bytes per lane) for a single held row; more would cost registers
// that the fp32 and multi-row kernels do not have.  An empty stand-in
// otherwise (those load the K row when they insert).
template <typename QS, int NN, bool = QS::kInsert>
struct NewRows {
  static constexpr bool kPreload = false;
  struct type {};
};
template <typename QS, int NN>
struct NewRows<QS, NN, true> {
  static constexpr bool kPreload = NN > 0 && NN * QS::Block::kElemBytes <= 2;
  using type = typename QS::Block;
};

// Weighted ReLU head sum for the 64 tokens of one page; lane l returns token l.
template <int NH>
__device__ __forceinline__ float page_score(const PageRegs& pg, const QueryRegs<NH>& q, int lane) {
  const int g = lane >> 4;
  int bs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bs[j] = (int)((pg.scale[j] >> (8 * g)) & 0xffu);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int grp = 0; grp < NH; ++grp)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = relu_weighted(mfma_fp4(q.a[grp], pg.code[j], q.sa[grp], bs[j], zero), q.w[grp], acc[j]);
  return reduce_tiles(acc);
}

// NN > 0: exactly NN query rows per sequence, all held in registers;
// NN == 0: any next_n, one row at a time.  QS: the query source; with
// QS::kInsert the wave holding a new token's page also encodes that token,
// writes it to its cache slot and scores the page with it.
template <int NH, int NN, int PPW, typename QS>
__global__ __launch_bounds__(kWave) void logits_paged_kernel(
    QS qs, const uint8_t* cache, int64_t num_pages,   // written when inserting: no restrict
    const int32_t* __restrict__ block_table, int64_t bt_row_stride,
    const int32_t* __restrict__ context_lens, int next_n, int64_t width,
    float* __restrict__ logits, int64_t ld, int clean, int stream_out) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int g = lane >> 4;       // 32-element block this lane supplies / head quad it receives
  const int n = lane & 15;       // token within a 16-token tile / head within a group
  const int64_t lp0 = (int64_t)blockIdx.x * PPW;
  const int64_t wpages = (width + kPage - 1) / kPage;
  const int64_t row0 = (int64_t)b * next_n;

  // Context length and the wave's block-table entries in one round trip: both
  // as vector loads (a scalar load of the length would have to retire before
  // the table load could issue).  Lane p < PPW reads the entry of page lp0 + p;
  // the other lanes fall outside the descriptor and read 0 without an access.
  const int bt_count = (int)min((int64_t)PPW, wpages - lp0);
  const int bt_lane = (int)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_rsrc(block_table + (int64_t)b * bt_row_stride + lp0, 4 * bt_count), 4u * lane, 0, 0);
  const uint32_t ctx_raw =
      __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(context_lens + b, 4), 0, 0, 0);
  // RoPE positions of the sequence's rows, in the same round trip: lane i <
  // next_n reads positions[row0 + i] (null: row i is at its token's position
  // context_len - next_n + i).
  uint32_t pos_lo = 0, pos_hi = 0;
  if constexpr (QS::kRope) {
    if (qs.rope.positions) {   // uniform
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(qs.rope.positions + row0, 8 * next_n);
      pos_lo = __builtin_amdgcn_raw_buffer_load_b32(rs, 8u * lane, 0, 0);
      pos_hi = __builtin_amdgcn_raw_buffer_load_b32(rs, 8u * lane + 4u, 0, 0);
    }
  }
  auto row_pos = [&](int i) -> int64_t {
    if constexpr (QS::kRope) {
      if (qs.rope.positions)
        return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)pos_hi, i) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)pos_lo, i));
      return (int64_t)(int32_t)__builtin_amdgcn_readfirstlane(ctx_raw) - next_n + i;
    } else {
      return 0;
    }
  };
  // The new token's K row is issued right behind the table loads.  The asm
  // below waits for the table only (counters retire in order, later loads stay
  // in flight) and, clobbering memory when inserting, keeps every load on its
  // side.
  constexpr int kRowsHeld = NN > 0 ? NN : 1;
  typename QS::template Fetched<NH> qf[kRowsHeld];
  constexpr int kNewHeld = NN > 0 ? NN : 1;
  constexpr bool kPreload = NewRows<QS, NN>::kPreload;
  typename NewRows<QS, NN>::type kpre[kNewHeld];
  if constexpr (kPreload) {
    constexpr int kRow = kHeadDim * QS::Block::kElemBytes;
#pragma unroll
    for (int i = 0; i < NN; ++i)
      kpre[i].load(buffer_rsrc(static_cast<const uint8_t*>(qs.k_new) + (row0 + i) * kRow, kRow),
                   (uint32_t)(g * kBlock * QS::Block::kElemBytes));
  }
  // Raw held query rows: fetched after the table wait and pinned ahead of the
  // page loads by a second memory clobber (left alone, the compiler issues
  // them behind the pages, and their encode would wait for the pages; issued
  // with the table, their 8 KB per wave slow the table loads).  Encoded rows
  // are fetched after the table wait with no clobbers: the compiler's order
  // (behind the weights, ahead of the pages) measured fastest for them.
  if constexpr (QS::kInsert) {
    asm volatile("" ::"v"(bt_lane) : "memory");
    if (NN > 0)
#pragma unroll
      for (int i = 0; i < kRowsHeld; ++i) qf[i] = qs.template fetch<NH>(row0 + i, g, n, row_pos(i));
    asm volatile("" ::: "memory");
  } else {
    asm volatile("" ::"v"(bt_lane));   // keeps the table load here, not sunk past the branch below
    if (NN > 0)
#pragma unroll
      for (int i = 0; i < kRowsHeld; ++i) qf[i] = qs.template fetch<NH>(row0 + i, g, n, 0);
  }
  const int64_t ctx = (int32_t)__builtin_amdgcn_readfirstlane(ctx_raw);
  // context lengths beyond the row width are a precondition violation; clamp so
  // that no store leaves the row
  const int64_t L = min(ctx, width);

  // Store of one page-row: scored columns get v, other columns of the row
  // width get -inf when cleaning, the rest is left untouched.
  auto store = [&](int64_t r, int64_t tok0, int64_t ke, float v) {
    const int64_t col = tok0 + lane;
    const bool scored = col < ke;
    const bool keep = scored || (clean && col < width);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(logits + r * ld + tok0, kPage * 4);
    const uint32_t bits = __float_as_uint(scored ? v : neg_inf());
    const uint32_t off = keep ? 4u * lane : kDropOffset;
    if (stream_out)   // wave-uniform
      __builtin_amdgcn_raw_buffer_store_b32(bits, rs, off, 0, kNonTemporal);
    else
      __builtin_amdgcn_raw_buffer_store_b32(bits, rs, off, 0, 0);
  };

  if (lp0 * kPage >= L) {        // every page lies past the context: -inf fill only
    if (clean)
      for (int i = 0; i < next_n; ++i)
#pragma unroll
        for (int p = 0; p < PPW; ++p) store(row0 + i, (lp0 + p) * kPage, 0, 0.f);
    return;
  }
  const int np = (int)min((int64_t)PPW, (L - lp0 * kPage + kPage - 1) / kPage);

  if constexpr (QS::kInsert) {
    // New token i sits at position P = context_len - next_n + i.  The wave
    // whose live pages hold it encodes it -- every lane block g of the row --
    // and writes its 68 bytes to the cache before loading the pages: lane
    // (g, n) later loads exactly the 16 code bytes it stores here, and every
    // lane of the token's column stores the 4 scale bytes it later loads, so
    // the page loads see the new token (program order of one lane, one
    // address).  Pages past the row width belong to no wave: tokens there are
    // not written.
    using Blk = typename QS::Block;
    constexpr int kRow = kHeadDim * Blk::kElemBytes;
    auto insert_one = [&](int i, const Blk* pre) {   // pre: the preloaded row, or null
      const int64_t P = ctx - next_n + i;
      const int64_t wp = P - lp0 * kPage;        // position within the wave's pages
      if (P < 0 || wp < 0 || wp >= (int64_t)np * kPage) return;   // uniform
      const int p_t = (int)(wp / kPage), off = (int)(wp % kPage);
      const int n_t = off % 16;
      const int64_t dst = __builtin_amdgcn_readlane(bt_lane, p_t);
      if (dst < 0 || dst >= num_pages) return;    // invalid table entry: not written
      Blk kb;
      if (pre)
        kb = *pre;
      else
        kb.load(buffer_rsrc(static_cast<const uint8_t*>(qs.k_new) + (row0 + i) * kRow, kRow),
                (uint32_t)(g * kBlock * Blk::kElemBytes));
      const uint32_t a = kb.amax_bits();
      const int E = block_exponent(a);
      const uint4 code = kb.encode(block_divisor(a, E));
      // the row's 4 scale bytes, one per lane group (all lanes of a group agree)
      const uint32_t sword = (uint32_t)(E + 127) & 0xffu;
      const uint32_t srow = (uint32_t)__builtin_amdgcn_readlane((int)sword, 0) |
                            ((uint32_t)__builtin_amdgcn_readlane((int)sword, 16) << 8) |
                            ((uint32_t)__builtin_amdgcn_readlane((int)sword, 32) << 16) |
                            ((uint32_t)__builtin_amdgcn_readlane((int)sword, 48) << 24);
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(const_cast<uint8_t*>(cache) + dst * kPageBytes, kPageBytes);
      const u32x4 cv = {code.x, code.y, code.z, code.w};
      __builtin_amdgcn_raw_buffer_store_b128(
          cv, rs, n == n_t ? (uint32_t)(off * kCodeBytes + 16 * g) : kDropOffset, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(
          srow, rs, n == n_t ? (uint32_t)(kPageCodeBytes + off * kScaleBytes) : kDropOffset, 0,
          0);
    };
    if constexpr (kPreload) {
#pragma unroll
      for (int i = 0; i < NN; ++i) insert_one(i, &kpre[i]);
    } else {
      for (int i = 0; i < next_n; ++i) insert_one(i, nullptr);
    }
  }

  PageRegs pg[PPW];
  bool page_ok[PPW];   // false: invalid block-table entry, the page is skipped
  const uint32_t off_code = 64u * n + 16u * g;
  const uint32_t off_scale = kPageCodeBytes + 4u * n;
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int pid = __builtin_amdgcn_readlane(bt_lane, p);
    const bool valid = pid >= 0 && pid < num_pages;
    page_ok[p] = p >= np || valid;
    const int live = __builtin_amdgcn_readfirstlane((p < np && valid) ? 1 : 0);
    const int64_t page = __builtin_amdgcn_readfirstlane(live ? pid : 0);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(cache + page * kPageBytes, live ? kPageBytes : 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, off_code + 1024u * j, 0, kNonTemporal);
      pg[p].code[j] = make_uint4(c.x, c.y, c.z, c.w);
      pg[p].scale[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, off_scale + 64u * j, 0, kNonTemporal);
    }
  }
  // The RoPE encode below branches on the row's position: without a clobber the
  // compiler sinks the page loads past it, behind the wait for the angles.
  if constexpr (QS::kRope) asm volatile("" ::: "memory");
  // Keep the preloaded K rows live until here in every wave: a wave without a
  // new token would otherwise reuse their registers while the loads are in
  // flight, which waits for every load before the page loads can issue.
  if constexpr (kPreload)
#pragma unroll
    for (int i = 0; i < NN; ++i) kpre[i].pin();
  __builtin_amdgcn_sched_barrier(0);   // every page load issues before any compute

  // held rows' operands first: a raw query is encoded while the pages load
  // (pinned, or the compiler defers the encode into the scoring code, behind
  // the waits for the pages)
  QueryRegs<NH> qr[kRowsHeld];
  if (NN > 0)
#pragma unroll
    for (int i = 0; i < kRowsHeld; ++i) {
      qr[i] = qs.template finish<NH>(qf[i]);
      if constexpr (QS::kInsert)
#pragma unroll
        for (int grp = 0; grp < NH; ++grp) {
          pin(qr[i].a[grp]);
          pin(qr[i].sa[grp]);
        }
    }

  if (NN > 0) {
    float out[kRowsHeld][PPW];
#pragma unroll
    for (int i = 0; i < kRowsHeld; ++i)
#pragma unroll
      for (int p = 0; p < PPW; ++p) out[i][p] = page_score<NH>(pg[p], qr[i], lane);
#pragma unroll
    for (int i = 0; i < kRowsHeld; ++i)
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        if (page_ok[p]) store(row0 + i, (lp0 + p) * kPage, L - NN + i + 1, out[i][p]);
  } else {
    for (int i = 0; i < next_n; ++i) {
      const int64_t r = row0 + i;
      const int64_t ke = L - next_n + i + 1;
      const QueryRegs<NH> q = qs.template finish<NH>(qs.template fetch<NH>(r, g, n, row_pos(i)));
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        if (page_ok[p]) store(r, (lp0 + p) * kPage, ke, page_score<NH>(pg[p], q, lane));
    }
  }
}

template <int NH, typename QS>
hipError_t launch_nh(QS qs, const uint8_t* cache, int64_t num_pages, const int32_t* bt,
                     int64_t bt_stride, const int32_t* ctx, int B, int next_n, int64_t width,
                     float* logits, int64_t ld, int clean, hipStream_t stream) {
  const int64_t pages = (width + kPage - 1) / kPage;
  // Logits of a few MB (a decode batch) are stored through the caches, where
  // the top-k that reads them next finds them (decode step 11.10 -> 10.84 us);
  // larger outputs stream past them (cached, the 33.5 MB of the 64 x 131072
  // batch slowed the logits from 64.7 to 69.3 us).
  const int stream_out = (int64_t)B * next_n * width * 4 > kCachedLogitsBytes ? 1 : 0;
  const int64_t groups = (pages + kPagesPerWave - 1) / kPagesPerWave;
  if constexpr (!QS::kRope || NH <= 4) {        // (RoPE holds one row up to 4 head groups)
    if (next_n == 1 && (int64_t)B * groups < kSmallGrid) {
      constexpr int P = QS::kSmallPages;
      const dim3 small_grid((unsigned)((pages + P - 1) / P), (unsigned)B);
      hipLaunchKernelGGL((logits_paged_kernel<NH, 1, P, QS>), small_grid, dim3(kWave), 0, stream,
                         qs, cache, num_pages, bt, bt_stride, ctx, next_n, width, logits, ld,
                         clean, stream_out);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)groups, (unsigned)B);
#define MXIDX_PAGED_ROWS(nn)                                                                   \
  hipLaunchKernelGGL((logits_paged_kernel<NH, nn, kPagesPerWave, QS>), grid, dim3(kWave), 0,     \
                     stream, qs, cache, num_pages, bt, bt_stride, ctx, next_n, width, logits, ld, \
                     clean, stream_out)
  // rows held in registers while rows * NH <= 8 (the query operands of 8 head
  // groups); <= 4 with RoPE, whose angle registers are held per row too
  bool held = true;
  if constexpr (QS::kRope) {
    if constexpr (NH <= 2) {
      if (next_n == 1)
        MXIDX_PAGED_ROWS(1);
      else if (next_n == 2)
        MXIDX_PAGED_ROWS(2);
      else
        held = false;
    } else if constexpr (NH <= 4) {
      if (next_n == 1)
        MXIDX_PAGED_ROWS(1);
      else
        held = false;
    } else {
      held = false;
    }
  } else if (next_n == 1) {
    MXIDX_PAGED_ROWS(1);
  } else if constexpr (NH <= 4) {
    if (next_n == 2) {
      MXIDX_PAGED_ROWS(2);
    } else if constexpr (NH <= 2) {
      if (next_n == 3)
        MXIDX_PAGED_ROWS(3);
      else if (next_n == 4)
        MXIDX_PAGED_ROWS(4);
      else
        held = false;
    } else {
      held = false;
    }
  } else {
    held = false;
  }
  if (!held) MXIDX_PAGED_ROWS(0);
#undef MXIDX_PAGED_ROWS
  return hipGetLastError();
}

template <typename QS>
hipError_t launch_source(QS qs, const uint8_t* cache, int64_t num_pages,
                         const int32_t* block_table, int64_t bt_row_stride,
                         const int32_t* context_lens, int B, int next_n, int H,
                         int64_t max_context_len, float* logits, int64_t ld, int clean,
                         hipStream_t stream) {
#define MXIDX_PAGED_CASE(nh)                                                                     \
  case nh:                                                                                       \
    return launch_nh<nh>(qs, cache, num_pages, block_table, bt_row_stride, context_lens, B,     \
                         next_n, max_context_len, logits, ld, clean, stream);
  switch (H / 16) {
    MXIDX_PAGED_CASE(1)
    MXIDX_PAGED_CASE(2)
    MXIDX_PAGED_CASE(3)
    MXIDX_PAGED_CASE(4)
    MXIDX_PAGED_CASE(5)
    MXIDX_PAGED_CASE(6)
    MXIDX_PAGED_CASE(7)
    MXIDX_PAGED_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MXIDX_PAGED_CASE
}

}  // namespace

hipError_t launch_logits_paged(const uint8_t* q_values, const uint8_t* q_scales,
                               const float* weights, const uint8_t* cache, int64_t num_pages,
                               const int32_t* block_table, int64_t bt_row_stride,
                               const int32_t* context_lens, int B, int next_n, int H,
                               int64_t max_context_len, float* logits, int64_t ld, int clean,
                               hipStream_t stream) {
  return launch_source(PackedQuery{q_values, q_scales, weights}, cache, num_pages, block_table,
                       bt_row_stride, context_lens, B, next_n, H, max_context_len, logits, ld,
                       clean, stream);
}

hipError_t launch_logits_paged_insert(const void* q, const void* k_new, bool f32,
                                      const float* weights, uint8_t* cache, int64_t num_pages,
                                      const int32_t* block_table, int64_t bt_row_stride,
                                      const int32_t* context_lens, int B, int next_n, int H,
                                      int64_t max_context_len, float* logits, int64_t ld,
                                      int clean, hipStream_t stream) {
  if (f32)
    return launch_source(RawQuery<F32Block>{{}, q, k_new, weights}, cache, num_pages, block_table,
                         bt_row_stride, context_lens, B, next_n, H, max_context_len, logits, ld,
                         clean, stream);
  return launch_source(RawQuery<Bf16Block>{{}, q, k_new, weights}, cache, num_pages, block_table,
                       bt_row_stride, context_lens, B, next_n, H, max_context_len, logits, ld,
                       clean, stream);
}

hipError_t launch_logits_paged_insert_rope(const void* q, const void* k_new, bool f32,
                                           const float* weights, uint8_t* cache,
                                           int64_t num_pages, const int32_t* block_table,
                                           int64_t bt_row_stride, const int32_t* context_lens,
                                           int B, int next_n, int H, int64_t max_context_len,
                                           float* logits, int64_t ld, int clean,
                                           const RopeSpec& rope, hipStream_t stream) {
  if (rope.rope_dim == 0)
    return launch_logits_paged_insert(q, k_new, f32, weights, cache, num_pages, block_table,
                                      bt_row_stride, context_lens, B, next_n, H, max_context_len,
                                      logits, ld, clean, stream);
  if (f32)
    return launch_source(RawQuery<F32Block, true>{{rope}, q, k_new, weights}, cache, num_pages,
                         block_table, bt_row_stride, context_lens, B, next_n, H, max_context_len,
                         logits, ld, clean, stream);
  return launch_source(RawQuery<Bf16Block, true>{{rope}, q, k_new, weights}, cache, num_pages,
                       block_table, bt_row_stride, context_lens, B, next_n, H, max_context_len,
                       logits, ld, clean, stream);
}

}  // namespace mxidx
