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
// lane; a 2-step xor-shuffle reduction leaves logit (t, c0+lane) in lane
// `lane`, so each row's 64 results are one coalesced 256-byte store.
// Rows whose visible range misses the 64 keys skip their MFMAs (causal tiles
// above the diagonal cost nothing unless clean output asks for -inf fill).
//
// Block order: workgroup id i runs on XCD i % 8; the j-th workgroup of an XCD
// gets query block (j / n_kc) * 8 + i % 8 and key chunk j % n_kc, so one XCD's
// resident workgroups share a query block in its L2, and the causal work is
// spread evenly over the 8 XCDs.
#include "common.hpp"
#include "launch.hpp"
#include "logits_reduce.hpp"

namespace mxidx {
namespace {

constexpr int kKeyChunk = 1024;

// B operands of 64 consecutive keys: lane (g, n) takes the 16 code bytes of
// block g of key c0 + 16*j + n for each tile j, and that key's 4 scale bytes
// (the block's byte is extracted when the tile is used).  Keys past the last
// one are clamped to it: their columns are never stored.
struct KTile {
  uint4 code[4];
  uint32_t scale[4];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ kv, const uint8_t* __restrict__ ksc,
                                       int c0, int last, int g, int n) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(c0 + 16 * j + n, last);
      code[j] = *reinterpret_cast<const uint4*>(kv + (int64_t)key * kCodeBytes + g * 16);
      scale[j] = *reinterpret_cast<const uint32_t*>(ksc + (int64_t)key * kScaleBytes);
    }
  }
};

template <int NH, int RW>
__global__ __launch_bounds__(256) void logits_prefill_kernel(
    const uint8_t* __restrict__ q_values, const uint8_t* __restrict__ q_scales,
    const uint8_t* __restrict__ k_values, const uint8_t* __restrict__ k_scales,
    const float* __restrict__ weights, const int32_t* __restrict__ ks,
    const int32_t* __restrict__ ke, int64_t T, int S, float* __restrict__ logits, int64_t ld,
    int clean, int64_t n_qb, int64_t n_kc) {
  constexpr int H = 16 * NH;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;

  int64_t qb, kc;
  if (n_qb % 8 == 0) {
    const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
    qb = (j / n_kc) * 8 + x;
    kc = j % n_kc;
  } else {
    qb = blockIdx.x / n_kc;
    kc = blockIdx.x % n_kc;
  }
  const int64_t t0 = qb * (4 * RW) + wave * RW;
  const int c_begin = (int)kc * kKeyChunk;
  const int c_end = min(c_begin + kKeyChunk, S);

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
  const int k_first = c_begin + ((need_lo - c_begin) & ~63);
  if (clean) {
    // -inf for the keys of this chunk that the computed window below does not
    // cover (inside the window, masked columns are written at store time)
    for (int c0 = c_begin; c0 < c_end; c0 += 64) {
      if (need_lo < need_hi && c0 >= k_first && c0 < need_hi) continue;
      const int col = c0 + lane;
#pragma unroll
      for (int i = 0; i < RW; ++i)
        if (t0 + i < T && col < c_end) lrow[i][col] = neg_inf();
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
  const int last = S - 1;
  KTile nxt;
  nxt.load(k_values, k_scales, k_first, last, g, n);
  for (int c0 = k_first; c0 < need_hi; c0 += 64) {
    const KTile cur = nxt;
    if (c0 + 64 < need_hi) nxt.load(k_values, k_scales, c0 + 64, last, g, n);   // prefetch
    int bs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bs[j] = (int)((cur.scale[j] >> (8 * g)) & 0xffu);
    const int col = c0 + lane;
    // All rows x head groups x tiles, no per-row branches: rows that see
    // nothing of these 64 keys are masked at the store.  The MFMAs of the next
    // (row, group) are issued before the epilogue of the current one.
    float acc[RW][4];
    v4f d[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) d[0][j] = mfma_fp4(a[0][0], cur.code[j], sa[0][0], bs[j], zero);
#pragma unroll
    for (int p = 0; p < RW * NH; ++p) {
      const int i = p / NH, grp = p % NH;
      if (p + 1 < RW * NH) {
        const int i1 = (p + 1) / NH, g1 = (p + 1) % NH;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d[(p + 1) & 1][j] = mfma_fp4(a[i1][g1], cur.code[j], sa[i1][g1], bs[j], zero);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = relu_weighted(d[p & 1][j], wv[i][grp], grp == 0 ? 0.f : acc[i][j]);
      if (grp == NH - 1) {
        const float out = reduce_tiles(acc[i], lane);
        if (t0 + i < T) {
          if (col >= lo[i] && col < hi[i])
            lrow[i][col] = out;
          else if (clean && col < c_end)
            lrow[i][col] = neg_inf();
        }
      }
    }
  }
}

template <int NH, int RW>
hipError_t launch_cfg(const uint8_t* qv, const uint8_t* qs, const uint8_t* kv, const uint8_t* ksc,
                      const float* w, const int32_t* ks, const int32_t* ke, int64_t T, int64_t S,
                      float* logits, int64_t ld, int clean, hipStream_t stream) {
  // column indices are int32 inside the kernel (S < 2^31 is checked by the ABI)
  const int64_t n_qb = (T + 4 * RW - 1) / (4 * RW);
  const int64_t n_kc = (S + kKeyChunk - 1) / kKeyChunk;
  const int64_t grid = n_qb * n_kc;
  hipLaunchKernelGGL((logits_prefill_kernel<NH, RW>), dim3((unsigned)grid), dim3(256), 0, stream,
                     qv, qs, kv, ksc, w, ks, ke, T, (int)S, logits, ld, clean, n_qb, n_kc);
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
