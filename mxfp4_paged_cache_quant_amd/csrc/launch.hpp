// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI layer (abi.hip) before these are called; each launcher only sizes the
// grid and enqueues on `stream`, returning the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxidx {

hipError_t launch_quantize(const void* x, bool f32, int64_t rows, int64_t row_stride,
                           uint8_t* values, uint8_t* scales, hipStream_t stream);

// Query RoPE of a fused encode: fp32 angle tables [table_rows, rope_dim/2],
// per-token table rows (null: the call's default position), the rotated
// prefix of the 128 dims (a multiple of 16) and the pairing.
struct RopeSpec {
  const float* cos_t;
  const float* sin_t;
  int64_t table_rows;
  const int64_t* positions;
  int rope_dim;
  bool interleaved;
};

// Query RoPE (first rope_dim dims, neox or interleaved pairs, fp32) fused into
// the MXFP4 encode; rows = T*H, row r of token r / H (default position: t).
hipError_t launch_quantize_rope(const void* x, bool f32, int64_t rows, int64_t row_stride, int H,
                                const RopeSpec& rope, uint8_t* values, uint8_t* scales,
                                hipStream_t stream);

hipError_t launch_insert(const void* k, bool f32, int64_t num_tokens, int64_t row_stride,
                         const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                         hipStream_t stream);

hipError_t launch_insert_quantize(const void* k, bool k_f32, int64_t num_tokens,
                                  int64_t k_row_stride, const int64_t* slot_mapping,
                                  uint8_t* cache, int64_t num_pages, const void* q, bool q_f32,
                                  int64_t q_rows, int64_t q_row_stride, uint8_t* q_values,
                                  uint8_t* q_scales, hipStream_t stream);
// The same with the query rows (q_rows = T * q_heads) rotated first.
hipError_t launch_insert_quantize_rope(const void* k, bool k_f32, int64_t num_tokens,
                                       int64_t k_row_stride, const int64_t* slot_mapping,
                                       uint8_t* cache, int64_t num_pages, const void* q,
                                       bool q_f32, int64_t q_rows, int64_t q_row_stride,
                                       int q_heads, const RopeSpec& rope, uint8_t* q_values,
                                       uint8_t* q_scales, hipStream_t stream);

hipError_t launch_gather(const uint8_t* cache, int64_t num_pages, const int32_t* block_table,
                         int64_t bt_row_stride, const int32_t* seq_lens,
                         const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                         int64_t total_tokens, uint8_t* k_values, uint8_t* k_scales,
                         hipStream_t stream);

hipError_t launch_logits_prefill(const uint8_t* q_values, const uint8_t* q_scales,
                                 const uint8_t* k_values, const uint8_t* k_scales,
                                 const float* weights, const int32_t* ks, const int32_t* ke,
                                 int64_t T, int H, int64_t S, float* logits, int64_t ld,
                                 int clean, hipStream_t stream);

hipError_t launch_logits_paged(const uint8_t* q_values, const uint8_t* q_scales,
                               const float* weights, const uint8_t* cache, int64_t num_pages,
                               const int32_t* block_table, int64_t bt_row_stride,
                               const int32_t* context_lens, int B, int next_n, int H,
                               int64_t max_context_len, float* logits, int64_t ld, int clean,
                               hipStream_t stream);

// The decode step's encodes fused into the paged logits: q rows and the new
// tokens' K rows in bf16 (f32 = false) or fp32, encoded in the kernel.
hipError_t launch_logits_paged_insert(const void* q, const void* k_new, bool f32,
                                      const float* weights, uint8_t* cache, int64_t num_pages,
                                      const int32_t* block_table, int64_t bt_row_stride,
                                      const int32_t* context_lens, int B, int next_n, int H,
                                      int64_t max_context_len, float* logits, int64_t ld,
                                      int clean, hipStream_t stream);
// The same with the query rows rotated before their encode (neox pairs need
// rope_dim 64 or 128; default position of row b*next_n + i: its token's
// position context_lens[b] - next_n + i).
hipError_t launch_logits_paged_insert_rope(const void* q, const void* k_new, bool f32,
                                           const float* weights, uint8_t* cache,
                                           int64_t num_pages, const int32_t* block_table,
                                           int64_t bt_row_stride, const int32_t* context_lens,
                                           int B, int next_n, int H, int64_t max_context_len,
                                           float* logits, int64_t ld, int clean,
                                           const RopeSpec& rope, hipStream_t stream);

// FP8 (E4M3) indexer cache (fp8.hip): rows of 128 E4M3 values + an fp32 scale.
hipError_t launch_quantize_fp8(const void* x, bool f32, int64_t rows, int64_t row_stride, bool pow2,
                               uint8_t* values, float* scales, const float* w_in, float* w_out,
                               hipStream_t stream);
hipError_t launch_insert_fp8(const void* k, bool f32, int64_t num_tokens, int64_t row_stride,
                             bool pow2, const int64_t* slot_mapping, uint8_t* cache,
                             int64_t num_pages, hipStream_t stream);
hipError_t launch_gather_fp8(const uint8_t* cache, int64_t num_pages, const int32_t* block_table,
                             int64_t bt_row_stride, const int32_t* seq_lens,
                             const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                             int64_t total_tokens, uint8_t* k_values, float* k_scales,
                             hipStream_t stream);
hipError_t launch_logits_paged_fp8(const uint8_t* q_values, const float* weights,
                                   const uint8_t* cache, int64_t num_pages,
                                   const int32_t* block_table, int64_t bt_row_stride,
                                   const int32_t* context_lens, int B, int next_n, int H,
                                   int64_t max_context_len, float* logits, int64_t ld, int clean,
                                   hipStream_t stream);
hipError_t launch_logits_paged_insert_fp8(const void* q, const void* k_new, bool f32,
                                          const float* weights, bool pow2, uint8_t* cache,
                                          int64_t num_pages, const int32_t* block_table,
                                          int64_t bt_row_stride, const int32_t* context_lens,
                                          int B, int next_n, int H, int64_t max_context_len,
                                          float* logits, int64_t ld, int clean,
                                          hipStream_t stream);
hipError_t launch_logits_prefill_fp8(const uint8_t* q_values, const float* weights,
                                     const uint8_t* k_values, const float* k_scales,
                                     const int32_t* ks, const int32_t* ke, int64_t T, int H,
                                     int64_t S, float* logits, int64_t ld, int clean,
                                     hipStream_t stream);

// Pooled (kpool) insert: softmax(gate + ape)-weighted pool of kpool tokens,
// encoded as MXFP4 (fp8 = false) or FP8 rows, written at pool-end slots.
hipError_t launch_kpool_insert(const void* k, bool f32, int64_t n, int64_t row_stride,
                               const float* gate, const float* ape, const int64_t* slot_mapping,
                               int kpool, bool fp8, bool pow2, uint8_t* cache, int64_t num_pages,
                               float* compressed, hipStream_t stream);

hipError_t launch_topk_merge(const float* values, const int32_t* indices, int world, int k_in,
                             int64_t rows, int interleave, int k, int32_t* out_idx,
                             hipStream_t stream);

hipError_t launch_topk(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                       const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream);
// Workspace bytes of launch_topk_ws (0: it runs launch_topk, no workspace).
int64_t topk_workspace_bytes(int64_t rows, int64_t ld);
hipError_t launch_topk_ws(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                          const int32_t* ke, int k, int32_t* out_idx, void* workspace,
                          hipStream_t stream);
// launch_topk_ws with the workspace in the library's static device array
// (kNoAllocScratchBytes per device); hipErrorInvalidValue when the call needs more.
constexpr int64_t kNoAllocScratchBytes = 36ll << 20;
hipError_t launch_topk_noalloc(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                               const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream);

}  // namespace mxidx
