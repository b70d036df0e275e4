// C ABI of the MXFP4 indexer-cache library (declared in include/mxidx.h):
// host-side argument validation, the fail-closed gfx950 gate, and dispatch to
// the kernel launchers.  No allocation, no synchronization, no exceptions.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "mxidx.h"
#include "launch.hpp"

static_assert(IDX_TOPK_NOALLOC_MAX_WORKSPACE == mxidx::kNoAllocScratchBytes,
              "the header's scratch limit is the size of the library's scratch array");

extern "C" int idx_arch_supported(const char* gcn_arch_name);

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = another architecture
std::atomic<int> g_gate[kMaxDevices];

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int gate_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return IDX_ERR_NO_DEVICE;
  const int st = g_gate[dev].load(std::memory_order_acquire);
  if (st == 1) return IDX_OK;
  if (st == 2) return IDX_ERR_UNSUPPORTED_ARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return IDX_ERR_NO_DEVICE;
  const char* arch = prop.gcnArchName;
  // Test hook: pretend the device reports another architecture.
  if (const char* forced = std::getenv("MXIDX_FORCE_ARCH")) arch = forced;
  const bool ok = idx_arch_supported(arch) == IDX_OK;
  g_gate[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? IDX_OK : IDX_ERR_UNSUPPORTED_ARCH;
}

int gate_current() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return IDX_ERR_NO_DEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return IDX_ERR_NO_DEVICE;
  return gate_device(dev);
}

int launched(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_ERR_LAUNCH; }

bool heads_ok(int H) { return H >= 16 && H <= IDX_MAX_HEADS && H % 16 == 0; }

int check_rows_input(const void* x, int dtype, int64_t rows, int64_t row_stride) {
  if (rows < 0) return IDX_ERR_ARG;
  if (dtype != IDX_BF16 && dtype != IDX_F32) return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!x || !aligned(x, 16)) return IDX_ERR_ARG;
  if (row_stride < IDX_HEAD_DIM) return IDX_ERR_ARG;
  if (row_stride % (dtype == IDX_BF16 ? 8 : 4) != 0) return IDX_ERR_ARG;
  return IDX_OK;
}

}  // namespace

extern "C" {

int idx_version(void) { return 107; }

int idx_arch_supported(const char* gcn_arch_name) {
  // "gfx950" alone or followed by target features ("gfx950:sramecc+:xnack-")
  if (!gcn_arch_name) return IDX_ERR_UNSUPPORTED_ARCH;
  const bool ok = std::strncmp(gcn_arch_name, "gfx950", 6) == 0 &&
                  (gcn_arch_name[6] == '\0' || gcn_arch_name[6] == ':');
  return ok ? IDX_OK : IDX_ERR_UNSUPPORTED_ARCH;
}

const char* idx_strerror(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_ERR_ARG: return "invalid argument";
    case IDX_ERR_NO_DEVICE: return "no HIP device";
    case IDX_ERR_UNSUPPORTED_ARCH: return "device is not gfx950 (MI355X)";
    case IDX_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int idx_init(int device) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
    return IDX_ERR_NO_DEVICE;
  return gate_device(device);
}

int idx_quantize(const void* x, int dtype, int64_t rows, int64_t row_stride, uint8_t* values,
                 uint8_t* scales, hipStream_t stream) {
  int st = check_rows_input(x, dtype, rows, row_stride);
  if (st != IDX_OK) return st;
  if (rows == 0) return IDX_OK;
  if (!values || !scales || !aligned(values, 4)) return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_quantize(x, dtype == IDX_F32, rows, row_stride, values, scales, stream));
}

int idx_quantize_rope(const void* x, int dtype, int64_t T, int H, int64_t row_stride,
                      const float* cos_table, const float* sin_table, int64_t table_rows,
                      const int64_t* positions, int rope_dim, int rope_mode, uint8_t* values,
                      uint8_t* scales, hipStream_t stream) {
  if (T < 0 || H < 1 || T > ((int64_t)1 << 40)) return IDX_ERR_ARG;
  const int64_t rows = T * H;
  int st = check_rows_input(x, dtype, rows, row_stride);
  if (st != IDX_OK) return st;
  if (rope_dim < 0 || rope_dim > IDX_HEAD_DIM || rope_dim % 16 != 0) return IDX_ERR_ARG;
  if (rope_mode != IDX_ROPE_NEOX && rope_mode != IDX_ROPE_INTERLEAVED) return IDX_ERR_ARG;
  if (table_rows < 0) return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!values || !scales || !aligned(values, 4)) return IDX_ERR_ARG;
  if (rope_dim > 0) {
    if (!cos_table || !sin_table || !aligned(cos_table, 16) || !aligned(sin_table, 16))
      return IDX_ERR_ARG;
    if (positions ? !aligned(positions, 8) : table_rows < T) return IDX_ERR_ARG;
  }
  if ((st = gate_current()) != IDX_OK) return st;
  const mxidx::RopeSpec rs{cos_table, sin_table, table_rows, positions, rope_dim,
                          rope_mode == IDX_ROPE_INTERLEAVED};
  return launched(mxidx::launch_quantize_rope(x, dtype == IDX_F32, rows, row_stride, H, rs, values,
                                              scales, stream));
}

// The checks of an idx_rope block common to the fused calls: the rotated
// prefix, the pairing, and the tables when something is rotated.
static int check_rope(const idx_rope* r) {
  if (!r) return IDX_ERR_ARG;
  if (r->rope_dim < 0 || r->rope_dim > IDX_HEAD_DIM || r->rope_dim % 16 != 0) return IDX_ERR_ARG;
  if (r->rope_mode != IDX_ROPE_NEOX && r->rope_mode != IDX_ROPE_INTERLEAVED) return IDX_ERR_ARG;
  if (r->table_rows < 0) return IDX_ERR_ARG;
  if (r->rope_dim > 0) {
    if (!r->cos_table || !r->sin_table || !aligned(r->cos_table, 16) ||
        !aligned(r->sin_table, 16))
      return IDX_ERR_ARG;
    if (r->positions && !aligned(r->positions, 8)) return IDX_ERR_ARG;
  }
  return IDX_OK;
}

static mxidx::RopeSpec rope_spec(const idx_rope* r) {
  return mxidx::RopeSpec{r->cos_table, r->sin_table, r->table_rows, r->positions, r->rope_dim,
                         r->rope_mode == IDX_ROPE_INTERLEAVED};
}

int idx_insert(const void* k, int dtype, int64_t num_tokens, int64_t k_row_stride,
               const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages, int page_size,
               hipStream_t stream) {
  int st = check_rows_input(k, dtype, num_tokens, k_row_stride);
  if (st != IDX_OK) return st;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0) return IDX_ERR_ARG;
  if (num_tokens == 0) return IDX_OK;
  if (!slot_mapping || !aligned(slot_mapping, 8)) return IDX_ERR_ARG;
  if (num_pages > 0 && (!cache || !aligned(cache, 4))) return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_insert(k, dtype == IDX_F32, num_tokens, k_row_stride, slot_mapping,
                                       cache, num_pages, stream));
}

int idx_insert_quantize(const void* k, int k_dtype, int64_t num_tokens, int64_t k_row_stride,
                        const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                        int page_size, const void* q, int q_dtype, int64_t q_rows,
                        int64_t q_row_stride, uint8_t* q_values, uint8_t* q_scales,
                        hipStream_t stream) {
  // exactly the checks of idx_insert and of idx_quantize
  int st = check_rows_input(k, k_dtype, num_tokens, k_row_stride);
  if (st != IDX_OK) return st;
  if ((st = check_rows_input(q, q_dtype, q_rows, q_row_stride)) != IDX_OK) return st;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0) return IDX_ERR_ARG;
  if (num_tokens > 0) {
    if (!slot_mapping || !aligned(slot_mapping, 8)) return IDX_ERR_ARG;
    if (num_pages > 0 && (!cache || !aligned(cache, 4))) return IDX_ERR_ARG;
  }
  if (q_rows > 0 && (!q_values || !q_scales || !aligned(q_values, 4))) return IDX_ERR_ARG;
  if (num_tokens == 0 && q_rows == 0) return IDX_OK;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_insert_quantize(k, k_dtype == IDX_F32, num_tokens, k_row_stride,
                                                slot_mapping, cache, num_pages, q,
                                                q_dtype == IDX_F32, q_rows, q_row_stride, q_values,
                                                q_scales, stream));
}

int idx_insert_quantize_rope(const void* k, int k_dtype, int64_t num_tokens,
                             int64_t k_row_stride, const int64_t* slot_mapping, uint8_t* cache,
                             int64_t num_pages, int page_size, const void* q, int q_dtype,
                             int64_t q_rows, int64_t q_row_stride, int q_heads,
                             const idx_rope* rope, uint8_t* q_values, uint8_t* q_scales,
                             hipStream_t stream) {
  int st = check_rows_input(k, k_dtype, num_tokens, k_row_stride);
  if (st != IDX_OK) return st;
  if ((st = check_rows_input(q, q_dtype, q_rows, q_row_stride)) != IDX_OK) return st;
  if ((st = check_rope(rope)) != IDX_OK) return st;
  if (q_heads < 1 || q_rows % q_heads != 0) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0) return IDX_ERR_ARG;
  if (num_tokens > 0) {
    if (!slot_mapping || !aligned(slot_mapping, 8)) return IDX_ERR_ARG;
    if (num_pages > 0 && (!cache || !aligned(cache, 4))) return IDX_ERR_ARG;
  }
  if (q_rows > 0 && (!q_values || !q_scales || !aligned(q_values, 4))) return IDX_ERR_ARG;
  // default positions (token t at table row t) need a row for every token
  if (rope->rope_dim > 0 && !rope->positions && rope->table_rows < q_rows / q_heads)
    return IDX_ERR_ARG;
  if (num_tokens == 0 && q_rows == 0) return IDX_OK;
  if ((st = gate_current()) != IDX_OK) return st;
  if (rope->rope_dim == 0)
    return launched(mxidx::launch_insert_quantize(k, k_dtype == IDX_F32, num_tokens, k_row_stride,
                                                  slot_mapping, cache, num_pages, q,
                                                  q_dtype == IDX_F32, q_rows, q_row_stride,
                                                  q_values, q_scales, stream));
  return launched(mxidx::launch_insert_quantize_rope(
      k, k_dtype == IDX_F32, num_tokens, k_row_stride, slot_mapping, cache, num_pages, q,
      q_dtype == IDX_F32, q_rows, q_row_stride, q_heads, rope_spec(rope), q_values, q_scales,
      stream));
}

int idx_gather(const uint8_t* cache, int64_t num_pages, int page_size, const int32_t* block_table,
               int64_t bt_row_stride, const int32_t* seq_lens, const int64_t* cu_seq_offsets,
               int batch, int64_t max_seq_len, int64_t total_tokens, uint8_t* k_values,
               uint8_t* k_scales, hipStream_t stream) {
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || batch < 0 || batch > 65535 ||
      max_seq_len < 0 || total_tokens < 0)
    return IDX_ERR_ARG;
  if (batch == 0 || max_seq_len == 0 || total_tokens == 0 || num_pages == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_seq_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq) return IDX_ERR_ARG;
  if (!cache || !aligned(cache, 16) || !block_table || !seq_lens || !cu_seq_offsets ||
      !aligned(cu_seq_offsets, 8) || !k_values || !aligned(k_values, 16) || !k_scales ||
      !aligned(k_scales, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_gather(cache, num_pages, block_table, bt_row_stride, seq_lens,
                                       cu_seq_offsets, batch, max_seq_len, total_tokens, k_values,
                                       k_scales, stream));
}

int idx_logits_prefill(const uint8_t* q_values, const uint8_t* q_scales, const uint8_t* k_values,
                       const uint8_t* k_scales, const float* weights, const int32_t* ks,
                       const int32_t* ke, int64_t T, int H, int64_t S, float* logits,
                       int64_t logits_row_stride, int clean, hipStream_t stream) {
  if (T < 0 || S < 0 || S > 0x7fffffffLL - 1024 || !heads_ok(H)) return IDX_ERR_ARG;
  if (T == 0 || S == 0) return IDX_OK;
  if (logits_row_stride < S) return IDX_ERR_ARG;
  if (!q_values || !aligned(q_values, 16) || !q_scales || !k_values || !aligned(k_values, 16) ||
      !k_scales || !aligned(k_scales, 4) || !weights || !aligned(weights, 16) || !ke || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_prefill(q_values, q_scales, k_values, k_scales, weights, ks,
                                               ke, T, H, S, logits, logits_row_stride, clean,
                                               stream));
}

int idx_logits_paged(const uint8_t* q_values, const uint8_t* q_scales, const float* weights,
                     const uint8_t* cache, int64_t num_pages, int page_size,
                     const int32_t* block_table, int64_t bt_row_stride,
                     const int32_t* context_lens, int B, int next_n, int H,
                     int64_t max_context_len, float* logits, int64_t logits_row_stride, int clean,
                     hipStream_t stream) {
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || B < 0 || B > IDX_MAX_DECODE_SEQS ||
      next_n < 1 || next_n > 16 || !heads_ok(H) || max_context_len < 0 ||
      max_context_len > 0x7fffffffLL - IDX_PAGE_SIZE)
    return IDX_ERR_ARG;
  if (B == 0 || max_context_len == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_context_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq || logits_row_stride < max_context_len || num_pages < 1 ||
      (int64_t)B * pages_per_seq > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (!q_values || !aligned(q_values, 16) || !q_scales || !weights || !aligned(weights, 16) ||
      !cache || !aligned(cache, 16) || !block_table || !context_lens || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_paged(q_values, q_scales, weights, cache, num_pages,
                                             block_table, bt_row_stride, context_lens, B, next_n,
                                             H, max_context_len, logits, logits_row_stride, clean,
                                             stream));
}

int idx_logits_paged_insert(const void* q, const void* k_new, int dtype, const float* weights,
                            uint8_t* cache, int64_t num_pages, int page_size,
                            const int32_t* block_table, int64_t bt_row_stride,
                            const int32_t* context_lens, int B, int next_n, int H,
                            int64_t max_context_len, float* logits, int64_t logits_row_stride,
                            int clean, hipStream_t stream) {
  if (dtype != IDX_BF16 && dtype != IDX_F32) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || B < 0 || B > IDX_MAX_DECODE_SEQS ||
      next_n < 1 || next_n > 16 || !heads_ok(H) || max_context_len < 0 ||
      max_context_len > 0x7fffffffLL - IDX_PAGE_SIZE)
    return IDX_ERR_ARG;
  if (B == 0 || max_context_len == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_context_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq || logits_row_stride < max_context_len || num_pages < 1 ||
      (int64_t)B * pages_per_seq > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (!q || !aligned(q, 16) || !k_new || !aligned(k_new, 16) || !weights || !aligned(weights, 16) ||
      !cache || !aligned(cache, 16) || !block_table || !context_lens || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_paged_insert(
      q, k_new, dtype == IDX_F32, weights, cache, num_pages, block_table, bt_row_stride,
      context_lens, B, next_n, H, max_context_len, logits, logits_row_stride, clean, stream));
}

int idx_logits_paged_insert_rope(const void* q, const void* k_new, int dtype,
                                 const float* weights, uint8_t* cache, int64_t num_pages,
                                 int page_size, const int32_t* block_table, int64_t bt_row_stride,
                                 const int32_t* context_lens, int B, int next_n, int H,
                                 int64_t max_context_len, float* logits,
                                 int64_t logits_row_stride, int clean, const idx_rope* rope,
                                 hipStream_t stream) {
  int st = check_rope(rope);
  if (st != IDX_OK) return st;
  // the in-wave rotation takes neox partners from one other lane block
  if (rope->rope_mode == IDX_ROPE_NEOX && rope->rope_dim != 0 && rope->rope_dim != 64 &&
      rope->rope_dim != 128)
    return IDX_ERR_ARG;
  if (dtype != IDX_BF16 && dtype != IDX_F32) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || B < 0 || B > IDX_MAX_DECODE_SEQS ||
      next_n < 1 || next_n > 16 || !heads_ok(H) || max_context_len < 0 ||
      max_context_len > 0x7fffffffLL - IDX_PAGE_SIZE)
    return IDX_ERR_ARG;
  if (B == 0 || max_context_len == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_context_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq || logits_row_stride < max_context_len || num_pages < 1 ||
      (int64_t)B * pages_per_seq > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (!q || !aligned(q, 16) || !k_new || !aligned(k_new, 16) || !weights || !aligned(weights, 16) ||
      !cache || !aligned(cache, 16) || !block_table || !context_lens || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_logits_paged_insert_rope(
      q, k_new, dtype == IDX_F32, weights, cache, num_pages, block_table, bt_row_stride,
      context_lens, B, next_n, H, max_context_len, logits, logits_row_stride, clean,
      rope_spec(rope), stream));
}

int idx_topk_merge(const float* values, const int32_t* indices, int world, int64_t rows, int k_in,
                   int interleave, int k, int32_t* out_idx, hipStream_t stream) {
  if (world < 1 || rows < 0 || k_in < 1 || interleave < 1 || k < 1 || k > IDX_TOPK_MAX ||
      (int64_t)world * k_in > IDX_MERGE_MAX_CANDIDATES || rows > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!values || !aligned(values, 4) || !indices || !aligned(indices, 4) || !out_idx) return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_topk_merge(values, indices, world, k_in, rows, interleave, k,
                                           out_idx, stream));
}

int idx_topk(const float* logits, int64_t rows, int64_t logits_row_stride, const int32_t* ks,
             const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream) {
  if (rows < 0 || k < 1 || k > IDX_TOPK_MAX || logits_row_stride < 0 ||
      rows > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!logits || !aligned(logits, 4) || !ke || !out_idx) return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_topk(logits, rows, logits_row_stride, ks, ke, k, out_idx, stream));
}

size_t idx_topk_workspace_bytes(int64_t rows, int64_t logits_row_stride) {
  if (rows < 0 || logits_row_stride < 0 || rows > 0x7fffffffLL) return 0;
  return (size_t)mxidx::topk_workspace_bytes(rows, logits_row_stride);
}

int idx_topk_ws(const float* logits, int64_t rows, int64_t logits_row_stride, const int32_t* ks,
                const int32_t* ke, int k, int32_t* out_idx, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (rows < 0 || k < 1 || k > IDX_TOPK_MAX || logits_row_stride < 0 ||
      rows > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!logits || !aligned(logits, 4) || !ke || !out_idx) return IDX_ERR_ARG;
  const size_t need = idx_topk_workspace_bytes(rows, logits_row_stride);
  if (need > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < need))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_topk_ws(logits, rows, logits_row_stride, ks, ke, k, out_idx,
                                        workspace, stream));
}

int idx_quantize_fp8(const void* x, int dtype, int64_t rows, int64_t row_stride, int scale_fmt,
                     uint8_t* values, float* scales, const float* w_in, float* w_out,
                     hipStream_t stream) {
  int st = check_rows_input(x, dtype, rows, row_stride);
  if (st != IDX_OK) return st;
  if (scale_fmt != IDX_FP8_SCALE_F32 && scale_fmt != IDX_FP8_SCALE_POW2) return IDX_ERR_ARG;
  if ((w_in == nullptr) != (w_out == nullptr)) return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!values || !aligned(values, 16) || !scales || !aligned(scales, 4)) return IDX_ERR_ARG;
  if (w_in && (!aligned(w_in, 4) || !aligned(w_out, 4))) return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_quantize_fp8(x, dtype == IDX_F32, rows, row_stride,
                                             scale_fmt == IDX_FP8_SCALE_POW2, values, scales, w_in,
                                             w_out, stream));
}

int idx_insert_fp8(const void* k, int dtype, int64_t num_tokens, int64_t k_row_stride,
                   int scale_fmt, const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                   int page_size, hipStream_t stream) {
  int st = check_rows_input(k, dtype, num_tokens, k_row_stride);
  if (st != IDX_OK) return st;
  if (scale_fmt != IDX_FP8_SCALE_F32 && scale_fmt != IDX_FP8_SCALE_POW2) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0) return IDX_ERR_ARG;
  if (num_tokens == 0) return IDX_OK;
  if (!slot_mapping || !aligned(slot_mapping, 8)) return IDX_ERR_ARG;
  if (num_pages > 0 && (!cache || !aligned(cache, 16))) return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_insert_fp8(k, dtype == IDX_F32, num_tokens, k_row_stride,
                                           scale_fmt == IDX_FP8_SCALE_POW2, slot_mapping, cache,
                                           num_pages, stream));
}

int idx_gather_fp8(const uint8_t* cache, int64_t num_pages, int page_size,
                   const int32_t* block_table, int64_t bt_row_stride, const int32_t* seq_lens,
                   const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                   int64_t total_tokens, uint8_t* k_values, float* k_scales, hipStream_t stream) {
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || batch < 0 || batch > 65535 ||
      max_seq_len < 0 || total_tokens < 0)
    return IDX_ERR_ARG;
  if (batch == 0 || max_seq_len == 0 || total_tokens == 0 || num_pages == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_seq_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq) return IDX_ERR_ARG;
  if (!cache || !aligned(cache, 16) || !block_table || !seq_lens || !cu_seq_offsets ||
      !aligned(cu_seq_offsets, 8) || !k_values || !aligned(k_values, 16) || !k_scales ||
      !aligned(k_scales, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_gather_fp8(cache, num_pages, block_table, bt_row_stride, seq_lens,
                                           cu_seq_offsets, batch, max_seq_len, total_tokens,
                                           k_values, k_scales, stream));
}

int idx_logits_prefill_fp8(const uint8_t* q_values, const float* weights, const uint8_t* k_values,
                           const float* k_scales, const int32_t* ks, const int32_t* ke, int64_t T,
                           int H, int64_t S, float* logits, int64_t logits_row_stride, int clean,
                           hipStream_t stream) {
  if (T < 0 || S < 0 || S > 0x7fffffffLL - 1024 || !heads_ok(H)) return IDX_ERR_ARG;
  if (T == 0 || S == 0) return IDX_OK;
  if (logits_row_stride < S) return IDX_ERR_ARG;
  if (!q_values || !aligned(q_values, 16) || !weights || !aligned(weights, 16) || !k_values ||
      !aligned(k_values, 16) || !k_scales || !aligned(k_scales, 4) || !ke || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_prefill_fp8(q_values, weights, k_values, k_scales, ks, ke, T,
                                                   H, S, logits, logits_row_stride, clean, stream));
}

int idx_logits_paged_fp8(const uint8_t* q_values, const float* weights, const uint8_t* cache,
                         int64_t num_pages, int page_size, const int32_t* block_table,
                         int64_t bt_row_stride, const int32_t* context_lens, int B, int next_n,
                         int H, int64_t max_context_len, float* logits, int64_t logits_row_stride,
                         int clean, hipStream_t stream) {
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || B < 0 || B > IDX_MAX_DECODE_SEQS ||
      next_n < 1 || next_n > 16 || !heads_ok(H) || max_context_len < 0 ||
      max_context_len > 0x7fffffffLL - IDX_PAGE_SIZE)
    return IDX_ERR_ARG;
  if (B == 0 || max_context_len == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_context_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq || logits_row_stride < max_context_len || num_pages < 1 ||
      (int64_t)B * pages_per_seq > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (!q_values || !aligned(q_values, 16) || !weights || !aligned(weights, 16) || !cache ||
      !aligned(cache, 16) || !block_table || !context_lens || !logits || !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_paged_fp8(q_values, weights, cache, num_pages, block_table,
                                                 bt_row_stride, context_lens, B, next_n, H,
                                                 max_context_len, logits, logits_row_stride, clean,
                                                 stream));
}

int idx_logits_paged_insert_fp8(const void* q, const void* k_new, int dtype, const float* weights,
                                int scale_fmt, uint8_t* cache, int64_t num_pages, int page_size,
                                const int32_t* block_table, int64_t bt_row_stride,
                                const int32_t* context_lens, int B, int next_n, int H,
                                int64_t max_context_len, float* logits,
                                int64_t logits_row_stride, int clean, hipStream_t stream) {
  if (dtype != IDX_BF16 && dtype != IDX_F32) return IDX_ERR_ARG;
  if (scale_fmt != IDX_FP8_SCALE_F32 && scale_fmt != IDX_FP8_SCALE_POW2) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0 || B < 0 || B > IDX_MAX_DECODE_SEQS ||
      next_n < 1 || next_n > 16 || !heads_ok(H) || max_context_len < 0 ||
      max_context_len > 0x7fffffffLL - IDX_PAGE_SIZE)
    return IDX_ERR_ARG;
  if (B == 0 || max_context_len == 0) return IDX_OK;
  const int64_t pages_per_seq = (max_context_len + IDX_PAGE_SIZE - 1) / IDX_PAGE_SIZE;
  if (bt_row_stride < pages_per_seq || logits_row_stride < max_context_len || num_pages < 1 ||
      (int64_t)B * pages_per_seq > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (!q || !aligned(q, 16) || !k_new || !aligned(k_new, 16) || !weights || !aligned(weights, 16) ||
      !cache || !aligned(cache, 16) || !block_table || !context_lens || !logits ||
      !aligned(logits, 4))
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_logits_paged_insert_fp8(
      q, k_new, dtype == IDX_F32, weights, scale_fmt == IDX_FP8_SCALE_POW2, cache, num_pages,
      block_table, bt_row_stride, context_lens, B, next_n, H, max_context_len, logits,
      logits_row_stride, clean, stream));
}

int idx_kpool_insert(const void* k, int dtype, int64_t n, int64_t k_row_stride,
                     const float* gate_score, const float* ape, const int64_t* slot_mapping,
                     int kpool, int cache_format, int fp8_scale_fmt, uint8_t* cache,
                     int64_t num_pages, int page_size, float* compressed, hipStream_t stream) {
  int st = check_rows_input(k, dtype, n, k_row_stride);
  if (st != IDX_OK) return st;
  if (kpool < 1 || kpool > IDX_KPOOL_MAX) return IDX_ERR_ARG;
  if (cache_format != IDX_CACHE_MXFP4 && cache_format != IDX_CACHE_FP8) return IDX_ERR_ARG;
  if (fp8_scale_fmt != IDX_FP8_SCALE_F32 && fp8_scale_fmt != IDX_FP8_SCALE_POW2) return IDX_ERR_ARG;
  if (page_size != IDX_PAGE_SIZE || num_pages < 0) return IDX_ERR_ARG;
  if (n < kpool) return IDX_OK;                 // no pool completes
  if (!gate_score || !aligned(gate_score, 16) || !ape || !aligned(ape, 16) || !slot_mapping ||
      !aligned(slot_mapping, 8))
    return IDX_ERR_ARG;
  if (compressed && !aligned(compressed, 16)) return IDX_ERR_ARG;
  if (num_pages > 0 && (!cache || !aligned(cache, 16))) return IDX_ERR_ARG;
  if ((st = gate_current()) != IDX_OK) return st;
  return launched(mxidx::launch_kpool_insert(k, dtype == IDX_F32, n, k_row_stride, gate_score, ape,
                                             slot_mapping, kpool, cache_format == IDX_CACHE_FP8,
                                             fp8_scale_fmt == IDX_FP8_SCALE_POW2, cache, num_pages,
                                             compressed, stream));
}

int idx_topk_noalloc(const float* logits, int64_t rows, int64_t logits_row_stride,
                     const int32_t* ks, const int32_t* ke, int k, int32_t* out_idx,
                     hipStream_t stream) {
  if (rows < 0 || k < 1 || k > IDX_TOPK_MAX || logits_row_stride < 0 || rows > 0x7fffffffLL)
    return IDX_ERR_ARG;
  if (rows == 0) return IDX_OK;
  if (!logits || !aligned(logits, 4) || !ke || !out_idx) return IDX_ERR_ARG;
  // the library's scratch holds at most IDX_TOPK_NOALLOC_MAX_WORKSPACE bytes
  if (idx_topk_workspace_bytes(rows, logits_row_stride) > (size_t)IDX_TOPK_NOALLOC_MAX_WORKSPACE)
    return IDX_ERR_ARG;
  int st = gate_current();
  if (st != IDX_OK) return st;
  return launched(mxidx::launch_topk_noalloc(logits, rows, logits_row_stride, ks, ke, k, out_idx,
                                             stream));
}

}  // extern "C"
