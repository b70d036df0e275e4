// Paged MXFP4 cache -> contiguous K rows (the shared cp_gather of P1's
// live-validation comment, which reads the same block-split pages as the
// paged logits reader).
//
// One workgroup per (sequence, page): 256 lanes = 64 tokens x 4 lanes, each
// lane moving 16 of the token's 64 code bytes; the first lane of a token also
// moves its 4 scale bytes.  A page's 4352 bytes are read as contiguous 16-byte
// and 4-byte segments and written to two contiguous output arrays.
#include "common.hpp"
#include "launch.hpp"

namespace mxidx {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ cache,
                                                     int64_t num_pages,
                                                     const int32_t* __restrict__ block_table,
                                                     int64_t bt_row_stride,
                                                     const int32_t* __restrict__ seq_lens,
                                                     const int64_t* __restrict__ cu_seq_offsets,
                                                     int64_t total_tokens,
                                                     uint8_t* __restrict__ k_values,
                                                     uint8_t* __restrict__ k_scales) {
  const int b = blockIdx.y;
  const int64_t lp = blockIdx.x;               // logical page of sequence b
  const int64_t j = lp * kPage + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  // the three index loads in one round trip, as vector loads (scalar loads
  // return out of order, so each test would wait for every load before it);
  // the table entry exists for every launched page: the row stride covers
  // max_seq_len's pages
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
  const uint8_t* pbase = cache + page * kPageBytes;
  const uint4 c = *reinterpret_cast<const uint4*>(pbase + off * kCodeBytes + part * 16);
  *reinterpret_cast<uint4*>(k_values + row * kCodeBytes + part * 16) = c;
  if (part == 0) {
    const uint32_t s = *reinterpret_cast<const uint32_t*>(pbase + kPageCodeBytes + off * kScaleBytes);
    *reinterpret_cast<uint32_t*>(k_scales + row * kScaleBytes) = s;
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* cache, int64_t num_pages, const int32_t* block_table,
                         int64_t bt_row_stride, const int32_t* seq_lens,
                         const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                         int64_t total_tokens, uint8_t* k_values, uint8_t* k_scales,
                         hipStream_t stream) {
  const int64_t pages = (max_seq_len + kPage - 1) / kPage;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)pages, (unsigned)batch), dim3(256), 0, stream,
                     cache, num_pages, block_table, bt_row_stride, seq_lens, cu_seq_offsets,
                     total_tokens, k_values, k_scales);
  return hipGetLastError();
}

}  // namespace mxidx
