// Dense indexer logits over contiguous MXFP4 K (mqa_logits of P3
// "SparseAttnIndexerKpool"; P2 "Summary": prefill MQA-logits kernel):
//
//   logits[t, s] = sum_h w[t,h] * max(0, qhat[t,h] . khat[s]),   ks[t] <= s < ke[t]
//
// The one dense contraction of the path (256*H flops per scored pair), so it
// is built on the block-scaled FP4 MFMA: v_mfma_scale_f32_16x16x128_f8f6f4
// with heads as M, 16 keys as N and the full 128-wide dot as K; each lane
// feeds one 32-element MX block of its row/column with that block's UE8M0
// scale, so the MFMA returns the exact scaled head dots in fp32.
//
// Tiling: a workgroup = 4 waves x RW query rows, over a chunk of KC keys.
// Each wave keeps its rows' q operands, scales and head weights in registers
// for the whole chunk and sweeps the keys 64 at a time (4 MFMA B tiles loaded
// straight from the contiguous K rows, 16 bytes per lane).  Per 16-head group
// and 16-key tile: one MFMA, then ReLU + weight FMA on the 4 outputs of each
// lane; a cross-lane reduction (two lane-swap steps) leaves logit
// (t, c0+lane) in lane `lane`, so each row's 64 results are one coalesced
// 256-byte store.  Keys past the key window or past S cost nothing unless
// clean output asks for -inf fill.
//
// The kernel is bound by its vector ALU, not by the MFMA: the ReLU and the
// weight FMA are 2 wave-wide VALU instructions (4 cycles each on a 16-lane
// SIMD) per MFMA output register, i.e. 32 VALU cycles per 16-cycle MFMA, so
// every other VALU instruction is kept out of the loop: tile loads and logit
// stores go through buffer descriptors whose base (key tile, logits row) is
// wave-uniform and lives in scalar registers, and lane masks are computed only
// for the tiles that straddle a row's [ks, ke) boundary.
//
// Block order: workgroup id i runs on XCD i % 8; the j-th workgroup of an XCD
// gets query block (j / n_kc) * 8 + i % 8 and key chunk j % n_kc, so one XCD's
// resident workgroups share a query block in its L2, and the causal work is
// spread evenly over the 8 XCDs.  Query blocks are taken last to first: under
// causal masking the late rows see the most keys, so the longest workgroups
// are dispatched first and the short ones fill the tail.
#include "common.hpp"
#include "launch.hpp"
#include "logits_reduce.hpp"

namespace mxidx {
namespace {

// Keys per workgroup: 4096, or 512 when S <= 16384 -- short causal inputs
// (the 8192 chunk) have too little work per workgroup to hide its start-up,
// and more workgroups balance better (measured at 8192 x 8192: 512 keys 119.5 us,
// 1024 129, 2048 156, 8192 136); long inputs amortize each workgroup's q and
// weight loads over more keys (16384 x 122880: 1024 keys 9.86-9.90 ms, 4096
// 9.64-9.68, 8192 9.63).
constexpr int kKeyChunkSmallS = 512;
constexpr int kKeyChunk = 4096;
constexpr int64_t kSmallS = 16384;

// B operands of 64 consecutive keys c0..c0+63: lane (g, n) takes the 16 code
// bytes of block g of key c0 + 16*j + n for each tile j, and that key's 4
// scale bytes (the block's byte is extracted when the tile is used).  Keys at
// or past S lie outside the descriptors and read as zeros; their columns are
// never stored.
struct KTile {
  uint4 code[4];
  uint32_t scale[4];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ kv, const uint8_t* __restrict__ ksc,
                                       int c0, int S, uint32_t off_code, uint32_t off_scale) {
    c0 = __builtin_amdgcn_readfirstlane(c0);   // wave-uniform: descriptors stay in scalar registers
    const int keys = __builtin_amdgcn_readfirstlane(max(min(S - c0, 64), 0));
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(kv + (int64_t)c0 * kCodeBytes, keys * kCodeBytes);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(ksc + (int64_t)c0 * kScaleBytes, keys * kScaleBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rc, off_code + 1024u * j, 0, 0);
      code[j] = make_uint4(c.x, c.y, c.z, c.w);
      scale[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, off_scale + 64u * j, 0, 0);
    }
  }
};

template <int NH, int RW>
__global__ __launch_bounds__(256) void logits_prefill_kernel(
    const uint8_t* __restrict__ q_values, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_values, const uint8_t* __restrict__ k_scales,
    const float* __restrict__ weights, const int32_t* __restrict__ ks,
    const int32_t* __restrict__ ke, int64_t T, int S, float* __restrict__ logits, int64_t ld,
    int clean, int64_t n_qb, int64_t n_kc, int key_chunk) {
  constexpr int H = 16 * NH;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;

  // Workgroup order.  Long inputs (4096-key chunks) go key chunk by key chunk, so
  // the workgroups resident at one time share one chunk of K, which stays in L2,
  // while their query blocks stream; the last chunks, which the causal diagonal
  // leaves uneven, run first.  Short inputs are XCD-aware (workgroup i runs on
  // XCD i % 8): one XCD's resident workgroups share a query block, causal work
  // spreads over the XCDs, and query blocks run last to first (the longest
  // causal rows first).
  int64_t qb, kc;
  if (key_chunk == kKeyChunk) {
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
  const int c_end = (int)min((int64_t)c_begin + key_chunk, (int64_t)S);   // no int32 overflow near S = 2^31

  // visible range of each row (empty for rows past T), and the key window
  // [need_lo, need_hi) inside this chunk that any of the rows needs
  int lo[RW], hi[RW];
  int need_lo = c_end, need_hi = c_begin;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t t = t0 + i;
    lo[i] = 0;
    hi[i] = 0;
    if (t < T) {
      lo[i] = ks ? max(ks[t], 0) : 0;
      hi[i] = min(ke[t], S);
      if (lo[i] < hi[i]) {
        need_lo = min(need_lo, max(lo[i], c_begin));
        need_hi = max(need_hi, min(hi[i], c_end));
      }
    }
  }
  float* lrow[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) lrow[i] = logits + min(t0 + i, T - 1) * ld;
  // Store of row i's 64 results for keys c0..c0+63: scored columns get v,
  // other columns of the chunk get -inf when cleaning, the rest is untouched.
  auto store = [&](int i, int c0, float v) {
    c0 = __builtin_amdgcn_readfirstlane(c0);
    uint32_t off = 4u * lane;
    if (t0 + i >= T) off = kDropOffset;
    if (!(c0 >= lo[i] && c0 + 64 <= hi[i])) {        // a tile that straddles [ks, ke)
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
    // -inf for the keys of this chunk that the computed window below does not
    // cover (inside the window, masked columns are written at store time)
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
      if (need_lo < need_hi && c0 >= k_first && c0 < need_hi) continue;
#pragma unroll
      for (int i = 0; i < RW; ++i) store(i, c0, neg_inf());
    }
  }
  if (need_lo >= need_hi) return;

  uint4 a[RW][NH];
  int sa[RW][NH];
  float4 wv[RW][NH];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t t = min(t0 + i, T - 1);     // rows past T are never stored
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      const int64_t qrow = t * H + 16 * grp + n;
      a[i][grp] = *reinterpret_cast<const uint4*>(q_values + qrow * kCodeBytes + g * 16);
      sa[i][grp] = q_scales[qrow * kScaleBytes + g];
      wv[i][grp] = *reinterpret_cast<const float4*>(weights + t * H + 16 * grp + 4 * g);
    }
  }

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const uint32_t off_code = 64u * n + 16u * g;
  const uint32_t off_scale = 4u * n;
  // One 64-key step over the wave's rows.  All rows x head groups x tiles,
  // no per-row branches: rows that see nothing of these keys are masked at the
  // store.  The MFMAs of the next (row, group) are issued before the epilogue
  // of the current one.
  auto step = [&](int c0, const KTile& kt) {
    int bs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bs[j] = (int)((kt.scale[j] >> (8 * g)) & 0xffu);
    float acc[RW][4];
    v4f d[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[0][j] = mfma_fp4(a[0][0], kt.code[j], sa[0][0], bs[j], zero);
#pragma unroll
    for (int p = 0; p < RW * NH; ++p) {
      const int i = p / NH, grp = p % NH;
      if (p + 1 < RW * NH) {
        const int i1 = (p + 1) / NH, g1 = (p + 1) % NH;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d[(p + 1) & 1][j] = mfma_fp4(a[i1][g1], kt.code[j], sa[i1][g1], bs[j], zero);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = relu_weighted(d[p & 1][j], wv[i][grp], grp == 0 ? 0.f : acc[i][j]);
      if (grp == NH - 1) store(i, c0, reduce_tiles(acc[i]));
    }
  };
  // Two tile buffers, the next tile's loads in flight during a step (a
  // prefetch past the window reads keys nobody stores, or nothing past S).
  KTile kt0, kt1;
  kt0.load(k_values, k_scales, k_first, S, off_code, off_scale);
  for (int c0 = k_first; c0 < need_hi; c0 += 128) {
    kt1.load(k_values, k_scales, c0 + 64, S, off_code, off_scale);
    step(c0, kt0);
    if (c0 + 64 >= need_hi) break;
    kt0.load(k_values, k_scales, c0 + 128, S, off_code, off_scale);
    step(c0 + 64, kt1);
  }
}

template <int NH, int RW>
hipError_t launch_cfg(const uint8_t* qv, const uint8_t* qs, const uint8_t* kv, const uint8_t* ksc,
                      const float* w, const int32_t* ks, const int32_t* ke, int64_t T, int64_t S,
                      float* logits, int64_t ld, int clean, hipStream_t stream) {
  // column indices are int32 inside the kernel (S < 2^31 is checked by the ABI)
  const int64_t n_qb = (T + 4 * RW - 1) / (4 * RW);
  const int key_chunk = S <= kSmallS ? kKeyChunkSmallS : kKeyChunk;
  const int64_t n_kc = (S + key_chunk - 1) / key_chunk;
  const int64_t grid = n_qb * n_kc;
  hipLaunchKernelGGL((logits_prefill_kernel<NH, RW>), dim3((unsigned)grid), dim3(256), 0, stream,
                     qv, qs, kv, ksc, w, ks, ke, T, (int)S, logits, ld, clean, n_qb, n_kc,
                     key_chunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logits_prefill(const uint8_t* q_values, const uint8_t* q_scales,
                                 const uint8_t* k_values, const uint8_t* k_scales,
                                 const float* weights, const int32_t* ks, const int32_t* ke,
                                 int64_t T, int H, int64_t S, float* logits, int64_t ld,
                                 int clean, hipStream_t stream) {
#define MXIDX_PREFILL_CASE(nh, rw)                                                               \
  case nh:                                                                                       \
    return launch_cfg<nh, rw>(q_values, q_scales, k_values, k_scales, weights, ks, ke, T, S,     \
                              logits, ld, clean, stream);
  switch (H / 16) {
    MXIDX_PREFILL_CASE(1, 4)
    MXIDX_PREFILL_CASE(2, 4)
    MXIDX_PREFILL_CASE(3, 4)
    MXIDX_PREFILL_CASE(4, 4)
    MXIDX_PREFILL_CASE(5, 2)
    MXIDX_PREFILL_CASE(6, 2)
    MXIDX_PREFILL_CASE(7, 2)
    MXIDX_PREFILL_CASE(8, 2)
    default:
      return hipErrorInvalidValue;
  }
#undef MXIDX_PREFILL_CASE
}

}  // namespace mxidx
