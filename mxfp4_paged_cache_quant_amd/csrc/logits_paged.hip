// Paged decode indexer logits (paged_mqa_logits of P3
// "SparseAttnIndexerKpool"; P2 "Summary": paged-decode MQA-logits kernel):
//
//   logits[r, s] = sum_h w[r,h] * max(0, qhat[r,h] . khat[s]),   s < L_b - next_n + i + 1
//
// with row r = b*next_n + i and token s read from page block_table[b, s/64]
// of the block-split MXFP4 cache (P1 live-validation comment).
//
// Design (HBM-bound: 68 bytes of K per scored token):
//  * grid = (logical pages / 4, sequences); each wave owns one 64-token page.
//  * The page's codes are loaded straight into MFMA B operands: lane l takes
//    16 bytes (block l/16 of token 16*j + l%16) for each of the 4 token tiles
//    j, so a wave reads the page's 4096 code bytes as one contiguous 4 KB
//    sweep, plus each token's 4 scale bytes.
//  * Heads are the MFMA M dimension: per 16-head group one
//    v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1, UE8M0 scale per 32-wide
//    block and lane) per token tile gives the exact scaled head dots.
//  * ReLU and the head weights are applied on the fp32 MFMA output; the four
//    lane groups' partial sums are combined by two xor-shuffles, after which
//    lane l owns token l of the page and the wave stores 64 consecutive floats.
#include "common.hpp"
#include "launch.hpp"
#include "logits_reduce.hpp"

namespace mxidx {
namespace {

constexpr int kPagesPerBlock = 4;   // 4 waves, one page each

template <int NH>
__global__ __launch_bounds__(256) void logits_paged_kernel(
    const uint8_t* __restrict__ q_values, const uint8_t* __restrict__ q_scales,
    const float* __restrict__ weights, const uint8_t* __restrict__ cache, int64_t num_pages,
    const int32_t* __restrict__ block_table, int64_t bt_row_stride,
    const int32_t* __restrict__ context_lens, int next_n, int64_t width,
    float* __restrict__ logits, int64_t ld, int clean) {
  constexpr int H = 16 * NH;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;       // 32-element block this lane supplies / head quad it receives
  const int n = lane & 15;       // token within a 16-token tile / head within a group
  const int64_t lp = (int64_t)blockIdx.x * kPagesPerBlock + (threadIdx.x >> 6);
  const int64_t tok0 = lp * kPage;
  if (tok0 >= width) return;
  // context lengths beyond the row width are a precondition violation; clamp so
  // that no store leaves the row
  const int64_t L = min((int64_t)context_lens[b], width);
  const int64_t col = tok0 + lane;
  const int64_t row0 = (int64_t)b * next_n;

  if (tok0 >= L) {               // the whole page lies past the context
    if (clean && col < width)
      for (int i = 0; i < next_n; ++i) logits[(row0 + i) * ld + col] = neg_inf();
    return;
  }
  const int64_t page = block_table[(int64_t)b * bt_row_stride + lp];
  if (page < 0 || page >= num_pages) return;
  const uint8_t* pbase = cache + page * kPageBytes;

  // the cache streams through once per call: non-temporal loads
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  uint4 bk[4];
  int bs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tk = 16 * j + n;
    const u32x4 c = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(pbase + tk * kCodeBytes + g * 16));
    bk[j] = make_uint4(c.x, c.y, c.z, c.w);
    const uint32_t s4 = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(pbase + kPageCodeBytes + tk * kScaleBytes));
    bs[j] = (int)((s4 >> (8 * g)) & 0xffu);
    if (tok0 + tk >= L) {        // unwritten slots past the context: neutral operands
      bk[j] = make_uint4(0, 0, 0, 0);
      bs[j] = 127;
    }
  }

  for (int i = 0; i < next_n; ++i) {
    const int64_t r = row0 + i;
    const int64_t ke = L - next_n + i + 1;
    if (tok0 >= ke) {
      if (clean && col < width) logits[r * ld + col] = neg_inf();
      continue;
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int grp = 0; grp < NH; ++grp) {
      const int64_t qrow = r * H + 16 * grp + n;
      const uint4 a = *reinterpret_cast<const uint4*>(q_values + qrow * kCodeBytes + g * 16);
      const int sa = q_scales[qrow * kScaleBytes + g];
      const float4 w = *reinterpret_cast<const float4*>(weights + r * H + 16 * grp + 4 * g);
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = relu_weighted(mfma_fp4(a, bk[j], sa, bs[j], zero), w, acc[j]);
    }
    const float out = reduce_tiles(acc, lane);
    if (col < ke)
      logits[r * ld + col] = out;
    else if (clean && col < width)
      logits[r * ld + col] = neg_inf();
  }
}

template <int NH>
hipError_t launch_nh(const uint8_t* qv, const uint8_t* qs, const float* w, const uint8_t* cache,
                     int64_t num_pages, const int32_t* bt, int64_t bt_stride, const int32_t* ctx,
                     int B, int next_n, int64_t width, float* logits, int64_t ld, int clean,
                     hipStream_t stream) {
  const int64_t pages = (width + kPage - 1) / kPage;
  const int64_t gx = (pages + kPagesPerBlock - 1) / kPagesPerBlock;
  hipLaunchKernelGGL((logits_paged_kernel<NH>), dim3((unsigned)gx, (unsigned)B), dim3(256), 0, stream,
                     qv, qs, w, cache, num_pages, bt, bt_stride, ctx, next_n, width, logits, ld,
                     clean);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_logits_paged(const uint8_t* q_values, const uint8_t* q_scales,
                               const float* weights, const uint8_t* cache, int64_t num_pages,
                               const int32_t* block_table, int64_t bt_row_stride,
                               const int32_t* context_lens, int B, int next_n, int H,
                               int64_t max_context_len, float* logits, int64_t ld, int clean,
                               hipStream_t stream) {
#define MXIDX_PAGED_CASE(nh)                                                                     \
  case nh:                                                                                       \
    return launch_nh<nh>(q_values, q_scales, weights, cache, num_pages, block_table,             \
                         bt_row_stride, context_lens, B, next_n, max_context_len, logits, ld,    \
                         clean, stream);
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

}  // namespace mxidx
