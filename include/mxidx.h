/*
 * mxidx.h -- C ABI of the MXFP4 paged indexer-cache library for MI355X (gfx950).
 *
 * The library implements the hot path of a DSA lightning indexer whose K cache
 * is stored in MXFP4:
 *
 *   idx_quantize        rows of 128 values -> MXFP4 rows (the FP4 query)
 *   idx_quantize_rope   the same after the query's RoPE (fused)
 *   idx_kpool_insert    kpool tokens pooled into one K row, then inserted
 *   idx_insert          K rows -> MXFP4 -> paged cache through a slot mapping
 *   idx_gather          paged cache -> contiguous MXFP4 K (prefill)
 *   idx_logits_prefill  logit[t,s] = sum_h w[t,h] * max(0, q[t,h] . k[s]), dense K
 *   idx_logits_paged    the same score, K read through a block table (decode)
 *   idx_topk            per-row top-k column indices over [ks, ke)
 *   idx_topk_ws         the same with a workspace: few long rows split over
 *                       workgroups
 *   idx_insert_quantize, idx_logits_paged_insert (and their _rope forms, with
 *                       the query RoPE): a decode step's calls in fewer launches
 *   idx_*_fp8           the FP8 (E4M3) indexer cache the MXFP4 one replaces:
 *                       quantize, insert, gather, dense and paged logits,
 *                       and idx_logits_paged_insert_fp8, its decode step's
 *                       quantize + insert + paged logits in one launch
 *
 * Sources: P1 = "[Kernel] MXFP4 indexer cache for GLM-5.2 / DSA (glm_moe_dsa)"
 * (vLLM pull request 48558); P2 = "Enable SM86 MXFP4 sparse-indexer cache"
 * (Whamp/vllm pull request 14); P3 = API page
 * "vllm.models.glm5next.nvidia.sparse_indexer".  MXFP4 itself is the OCP
 * Microscaling Formats (MX) v1.0 format: E2M1 elements, E8M0 block scales.
 *
 * MXFP4 row (P1 "Changes", "Benefit": 68 bytes per token per head):
 *   128 values = 4 blocks of 32.  64 code bytes: element 2j in the low nibble
 *   of byte j, element 2j+1 in the high nibble; nibble = sign<<3 | code, code
 *   c in 0..7 has magnitude {0,0.5,1,1.5,2,3,4,6}[c].  4 scale bytes: byte b
 *   is E_b + 127 for block b, the value of an element being
 *   (-1)^s * grid[c] * 2^E_b.
 *   Encode rule: E_b = the smallest integer with amax_b <= 6 * 2^E_b
 *   (amax_b = 0 gives -127; clamped to [-127, 127]); each element is
 *   x * 2^-E_b rounded to the nearest grid value, ties to the even code; the
 *   sign bit is the input's sign bit (so -0.0 encodes as 0x8).
 *
 * Paged cache (P1 live-validation comment: block-split value/scale layout):
 *   num_pages pages of page_size * 68 bytes.  Within a page, the page_size
 *   code rows (64 B each) come first in token order, then the page_size scale
 *   rows (4 B each).  Slot s = page * page_size + offset.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers allocated and owned by the
 *     caller.  The library never allocates, frees or synchronizes; every call
 *     only enqueues work on `stream` (0 = the null stream) and returns.
 *   - Shapes are row-major; "stride" arguments count elements of the array's
 *     own type.
 *   - Arguments that the host can check (null pointers with non-zero sizes,
 *     unsupported sizes, misaligned pointers or strides) return IDX_ERR_ARG
 *     before any device work.  Zero-sized work returns IDX_OK and enqueues
 *     nothing.
 *   - Device-side preconditions (slots, block-table entries and ks/ke within
 *     range, finite inputs) are not checked on the host.  Kernels skip slots
 *     and page ids outside the cache instead of touching memory out of range,
 *     and clamp ke to the row width.
 *   - The first call on a device checks that it is a gfx950 device
 *     (fail-closed gate, as P2 "Summary" asks of its kernels); on other
 *     devices every call returns IDX_ERR_UNSUPPORTED_ARCH.
 *   - No exception crosses this boundary; launch failures return IDX_ERR_LAUNCH.
 *   - Calls are thread-safe: the library's only global state is the gate's
 *     per-device result and per-device "attribute set" flags, all atomics.
 *     Calls on one stream execute in order.
 */
#ifndef MXIDX_H
#define MXIDX_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IDX_OK = 0,
  IDX_ERR_ARG = 1,               /* invalid argument (checked on the host) */
  IDX_ERR_NO_DEVICE = 2,         /* no HIP device / device index out of range */
  IDX_ERR_UNSUPPORTED_ARCH = 3,  /* device is not gfx950 */
  IDX_ERR_LAUNCH = 4             /* kernel launch failed */
} idx_status;

typedef enum { IDX_BF16 = 0, IDX_F32 = 1 } idx_dtype;

#define IDX_HEAD_DIM 128
#define IDX_BLOCK 32
#define IDX_ROW_CODE_BYTES 64
#define IDX_ROW_SCALE_BYTES 4
#define IDX_ROW_BYTES 68
#define IDX_PAGE_SIZE 64
#define IDX_MAX_HEADS 128
#define IDX_TOPK_MAX 2048
#define IDX_MAX_DECODE_SEQS 65535
#define IDX_MERGE_MAX_CANDIDATES 8192

/* Version of this ABI (major * 100 + minor). */
int idx_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* idx_strerror(int status);

/* The architecture rule of the gate, on a device's gcnArchName string (host
 * only; no device is touched): IDX_OK for "gfx950", alone or followed by
 * ':'-separated target features, IDX_ERR_UNSUPPORTED_ARCH for any other
 * string or NULL.  Every call runs this rule on the current device's name
 * before its first launch there (P2 "Summary": fail-closed capability gates);
 * the environment variable MXIDX_FORCE_ARCH, read at that first check,
 * replaces the device's name (a test hook). */
int idx_arch_supported(const char* gcn_arch_name);

/* Run the architecture gate for `device` now (it otherwise runs on the first
 * call that enqueues work on that device).  Returns IDX_OK on gfx950,
 * IDX_ERR_UNSUPPORTED_ARCH on another GPU, IDX_ERR_NO_DEVICE when `device`
 * does not exist. */
int idx_init(int device);

/* idx_quantize -- MXFP4-encode `rows` rows of 128 values into contiguous output
 * (the FP4 query of P1 "Changes"/"Notes" and P2 "Summary"; P3 "forward_cuda"
 * takes FP4 q as a (values, scales) pair).
 *   x:        [rows, row_stride] of bf16 (dtype IDX_BF16) or fp32 (IDX_F32);
 *             the first 128 elements of each row are encoded.  16-byte aligned;
 *             row_stride >= 128 and a multiple of 8 (bf16) or 4 (fp32).
 *   values:   [rows, 64] uint8 out (code bytes).
 *   scales:   [rows, 4] uint8 out (scale bytes).
 * Bytes are bit-exact to the encode rule above. */
int idx_quantize(const void* x, int dtype, int64_t rows, int64_t row_stride,
                 uint8_t* values, uint8_t* scales, hipStream_t stream);

/* idx_quantize_rope -- the query's rotary position embedding fused into its
 * MXFP4 encode (the fused q-rope-mxfp4 kernel that P1 "Notes" proposes; the
 * pages give no RoPE layout, so this call takes the following one).
 *   x: [T*H, row_stride] rows as for idx_quantize; row r = t*H + h belongs to
 *      query token t = r / H.
 *   cos_table, sin_table: [table_rows, rope_dim/2] fp32, contiguous, 16-byte
 *      aligned; positions: [T] int64 choosing token t's table row (NULL: row t,
 *      which needs table_rows >= T).  A row whose position lies outside
 *      [0, table_rows) is encoded unrotated.
 *   rope_dim: the first rope_dim of the 128 dims are rotated, 0 <= rope_dim <=
 *      128, a multiple of 16 (0: idx_quantize's bytes).
 *   rope_mode: IDX_ROPE_NEOX rotates the pairs (j, j + rope_dim/2),
 *      IDX_ROPE_INTERLEAVED the pairs (2j, 2j+1), each by angle j:
 *      a' = a*cos - b*sin, b' = b*cos + a*sin, every product and sum rounded to
 *      fp32 (no fused multiply-add); the rotated row is then encoded as an
 *      fp32 row by the rule above.
 *   values [T*H, 64], scales [T*H, 4] uint8 out. */
typedef enum { IDX_ROPE_NEOX = 0, IDX_ROPE_INTERLEAVED = 1 } idx_rope_mode;
int idx_quantize_rope(const void* x, int dtype, int64_t T, int H, int64_t row_stride,
                      const float* cos_table, const float* sin_table, int64_t table_rows,
                      const int64_t* positions, int rope_dim, int rope_mode, uint8_t* values,
                      uint8_t* scales, hipStream_t stream);

/* idx_rope -- the query RoPE of the fused decode-step calls below, with the
 * meaning of idx_quantize_rope's arguments of the same names (caller-owned
 * device tables; the struct itself is host memory, read during the call only).
 * The position of a query token when positions is NULL is stated by each call. */
typedef struct {
  const float* cos_table;     /* [table_rows, rope_dim/2] fp32, 16-byte aligned */
  const float* sin_table;     /* [table_rows, rope_dim/2] fp32, 16-byte aligned */
  int64_t table_rows;
  const int64_t* positions;   /* per query token, or NULL */
  int rope_dim;               /* 0..128, a multiple of 16; 0 rotates nothing */
  int rope_mode;              /* idx_rope_mode */
} idx_rope;

/* idx_insert -- quantize K rows and scatter them into the paged cache
 * (the indexer K quant-and-cache kernel of P1 "Changes"; slot -1 = no write,
 * P3 "_kpool_compress_insert").
 *   k:            [num_tokens, k_row_stride] bf16 or fp32, as for idx_quantize.
 *   slot_mapping: [num_tokens] int64; token i goes to slot_mapping[i];
 *                 negative slots (and slots >= num_pages*page_size) write
 *                 nothing.  Non-negative slots must be distinct.
 *   cache:        [num_pages, page_size * 68] uint8, updated in place; only the
 *                 68 bytes of each written slot change.
 *   page_size:    must be 64. */
int idx_insert(const void* k, int dtype, int64_t num_tokens, int64_t k_row_stride,
               const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
               int page_size, hipStream_t stream);

/* idx_insert_quantize -- idx_insert and idx_quantize in one launch: the new
 * tokens' K rows into their cache slots and the query rows into contiguous
 * MXFP4, the two encodes of a decode step (P1 "Changes": K quant-and-cache;
 * P3 "forward_cuda": FP4 q).  For callers whose decode step is launch-bound.
 *   k, k_dtype, num_tokens, k_row_stride, slot_mapping, cache, num_pages,
 *   page_size: as for idx_insert (num_tokens may be 0).
 *   q, q_dtype, q_rows, q_row_stride, q_values, q_scales: as x, dtype, rows,
 *   row_stride, values, scales of idx_quantize (q_rows may be 0).
 * Every argument is checked as the two calls check it; the outputs are
 * byte-identical to idx_insert followed by idx_quantize.  The query output must
 * not overlap the cache. */
int idx_insert_quantize(const void* k, int k_dtype, int64_t num_tokens, int64_t k_row_stride,
                        const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                        int page_size, const void* q, int q_dtype, int64_t q_rows,
                        int64_t q_row_stride, uint8_t* q_values, uint8_t* q_scales,
                        hipStream_t stream);

/* idx_insert_quantize_rope -- idx_insert_quantize with the query rows rotated
 * before their encode (the fused q-rope-mxfp4 step of P1 "Notes" inside the
 * decode step's one encode launch).
 *   q_rows = T * q_heads: row r belongs to query token t = r / q_heads;
 *   rope: required; token t takes table row positions[t] (NULL: row t, which
 *         needs table_rows >= T); rows outside the table are not rotated.
 * The outputs are byte-identical to idx_insert followed by idx_quantize_rope
 * (rope_dim 0: to idx_insert_quantize).  Errors: those of idx_insert_quantize,
 * plus IDX_ERR_ARG for a missing or invalid rope block or q_rows not a
 * multiple of q_heads. */
int idx_insert_quantize_rope(const void* k, int k_dtype, int64_t num_tokens,
                             int64_t k_row_stride, const int64_t* slot_mapping, uint8_t* cache,
                             int64_t num_pages, int page_size, const void* q, int q_dtype,
                             int64_t q_rows, int64_t q_row_stride, int q_heads,
                             const idx_rope* rope, uint8_t* q_values, uint8_t* q_scales,
                             hipStream_t stream);

/* idx_gather -- paged cache -> contiguous MXFP4 K (the cp_gather that P1's
 * live-validation comment names as sharing the cache layout).
 *   block_table:    [batch, bt_row_stride] int32 page ids, bt_row_stride >=
 *                   ceil(max_seq_len / page_size); the first that many entries of
 *                   each row are read (those past a sequence's pages are unused).
 *   seq_lens:       [batch] int32; token j < seq_lens[b] of sequence b is read
 *                   from page block_table[b, j / page_size], offset j % page_size.
 *   cu_seq_offsets: [batch] int64; that token lands in output row
 *                   cu_seq_offsets[b] + j (rows >= total_tokens are skipped).
 *   max_seq_len:    host-side upper bound of seq_lens (sizes the grid; tokens
 *                   beyond it are not gathered).
 *   k_values:       [total_tokens, 64] uint8 out;  k_scales: [total_tokens, 4] uint8 out.
 *   Output rows that no token maps to are left untouched. */
int idx_gather(const uint8_t* cache, int64_t num_pages, int page_size,
               const int32_t* block_table, int64_t bt_row_stride,
               const int32_t* seq_lens, const int64_t* cu_seq_offsets, int batch,
               int64_t max_seq_len, int64_t total_tokens,
               uint8_t* k_values, uint8_t* k_scales, hipStream_t stream);

/* idx_logits_prefill -- dense indexer logits (mqa_logits, P3
 * "SparseAttnIndexerKpool"; the prefill MQA-logits kernel of P2 "Summary"):
 *   logits[t, s] = sum_h weights[t,h] * max(0, sum_i qhat[t,h,i] * khat[s,i])
 * for ks[t] <= s < ke[t] (ke clamped to S), qhat/khat the exact MXFP4 values.
 *   q_values [T, H, 64], q_scales [T, H, 4]  (idx_quantize output);
 *   k_values [S, 64],    k_scales [S, 4]     (idx_gather output);
 *   weights  [T, H] fp32;  ks, ke [T] int32 (ks NULL means all zero);
 *   logits   [T, logits_row_stride] fp32 out, logits_row_stride >= S.
 *   clean != 0: columns outside [ks, ke) of [0, S) are set to -inf;
 *   clean == 0: they are left untouched.
 * H must be a multiple of 16 in [16, 128]; 0 <= S <= 2^31 - 1025 (columns are
 * int32 in the kernel).  Accumulation is fp32 (exact products, fp32 sums over
 * the 4 blocks and the heads). */
int idx_logits_prefill(const uint8_t* q_values, const uint8_t* q_scales,
                       const uint8_t* k_values, const uint8_t* k_scales,
                       const float* weights, const int32_t* ks, const int32_t* ke,
                       int64_t T, int H, int64_t S,
                       float* logits, int64_t logits_row_stride, int clean,
                       hipStream_t stream);

/* idx_logits_paged -- decode logits read through the block table
 * (paged_mqa_logits, P3 "SparseAttnIndexerKpool"; the paged-decode MQA-logits
 * kernel of P2 "Summary").  Row r = b*next_n + i (the i-th of the last next_n
 * tokens of sequence b, context length L_b = context_lens[b]) scores columns
 * s < L_b - next_n + i + 1, reading token s from page
 * block_table[b, s / page_size].
 *   q_values [B*next_n, H, 64], q_scales [B*next_n, H, 4], weights [B*next_n, H];
 *   cache [num_pages, page_size*68]; block_table [B, bt_row_stride] int32;
 *   context_lens [B] int32, each <= max_context_len;
 *   logits [B*next_n, logits_row_stride] fp32 out, logits_row_stride >= max_context_len.
 *   clean != 0: columns of [0, max_context_len) that a row does not score
 *   are set to -inf; clean == 0: they are left untouched.
 * page_size must be 64; H a multiple of 16 in [16, 128]; next_n in [1, 16];
 * 1 <= B <= IDX_MAX_DECODE_SEQS; num_pages >= 1; B * ceil(max_context_len / 64)
 * < 2^31.  Pages whose block-table entry lies outside [0, num_pages) are
 * skipped (their logits are not written). */
int idx_logits_paged(const uint8_t* q_values, const uint8_t* q_scales,
                     const float* weights, const uint8_t* cache, int64_t num_pages,
                     int page_size, const int32_t* block_table, int64_t bt_row_stride,
                     const int32_t* context_lens, int B, int next_n, int H,
                     int64_t max_context_len, float* logits, int64_t logits_row_stride,
                     int clean, hipStream_t stream);

/* idx_logits_paged_insert -- a decode step's two encodes and its paged logits in
 * one launch: equal, byte for byte and bit for bit, to idx_insert of the new
 * tokens into their block-table slots, idx_quantize of q, then
 * idx_logits_paged (the indexer K quant-and-cache of P1 "Changes", the FP4 q of
 * P3 "forward_cuda" and the paged_mqa_logits of P3 "SparseAttnIndexerKpool").
 * For decode steps bound by launch count.
 *   q:      [B*next_n, H, 128] bf16 (dtype IDX_BF16) or fp32 (IDX_F32),
 *           contiguous, 16-byte aligned: the query rows, encoded in the kernel.
 *   k_new:  [B*next_n, 128] in the same dtype, contiguous, 16-byte aligned:
 *           row b*next_n + i is the K row of sequence b's token at position
 *           context_lens[b] - next_n + i (the sequence's last next_n tokens);
 *           it is written to page block_table[b, pos / 64], offset pos % 64.
 *           Positions < 0, pages whose table entry is outside [0, num_pages)
 *           and pages past max_context_len are not written.
 *   cache:  updated in place (the new tokens' 68 bytes only), and read.
 *   All other arguments, the logits and the error behaviour are those of
 *   idx_logits_paged.  The new tokens' pages must not appear in another
 *   sequence's block table: they are written while the other sequences' pages
 *   are read. */
int idx_logits_paged_insert(const void* q, const void* k_new, int dtype, const float* weights,
                            uint8_t* cache, int64_t num_pages, int page_size,
                            const int32_t* block_table, int64_t bt_row_stride,
                            const int32_t* context_lens, int B, int next_n, int H,
                            int64_t max_context_len, float* logits, int64_t logits_row_stride,
                            int clean, hipStream_t stream);

/* idx_logits_paged_insert_rope -- idx_logits_paged_insert with the query rows
 * rotated (idx_rope) before the in-kernel encode: the decode step of P1
 * "Notes"' fused q-rope-mxfp4 kernel, its K quant-and-cache and its paged
 * logits in one launch.
 *   rope: required.  positions, when given, is [B*next_n] int64 (row
 *         b*next_n + i takes table row positions[b*next_n + i]); NULL puts the
 *         row at its token's position context_lens[b] - next_n + i.  Rows whose
 *         position lies outside [0, table_rows) are not rotated.  Neox pairing
 *         needs rope_dim 0, 64 or 128 here (each lane's partner block is then
 *         one other lane's); interleaved takes any multiple of 16.
 * Equal, byte for byte and bit for bit, to idx_insert of the new tokens,
 * idx_quantize_rope of q with those positions, then idx_logits_paged.  Errors:
 * those of idx_logits_paged_insert, plus IDX_ERR_ARG for a missing or invalid
 * rope block or an unsupported neox rope_dim. */
int idx_logits_paged_insert_rope(const void* q, const void* k_new, int dtype,
                                 const float* weights, uint8_t* cache, int64_t num_pages,
                                 int page_size, const int32_t* block_table, int64_t bt_row_stride,
                                 const int32_t* context_lens, int B, int next_n, int H,
                                 int64_t max_context_len, float* logits,
                                 int64_t logits_row_stride, int clean, const idx_rope* rope,
                                 hipStream_t stream);

/* ---------------------------------------------------------------------------
 * FP8 indexer cache: the format the MXFP4 cache replaces (P1 "Benefit": 132
 * bytes per token per head against 68), with the same calls.
 *
 * FP8 row (132 bytes): 128 OCP E4M3 values (bias 7, largest finite 448, no
 * infinities) and one little-endian fp32 scale.  Encode rule: s = amax / 448
 * rounded to fp32, floored at 2^-126 (IDX_FP8_SCALE_F32), or s = 2^E with E the
 * smallest integer such that amax <= 448 * 2^E, clamped to [-126, 127]
 * (IDX_FP8_SCALE_POW2, the power-of-two "round_scale" of P3
 * "_kpool_compress_insert"); each element is x / s rounded to fp32, then to the
 * nearest E4M3 value, ties to the even code; the sign bit is kept.
 * Page (block-split, as the MXFP4 page copies it; P1 live-validation comment):
 * the page_size value rows (128 B each) in token order, then the page_size
 * scale words (4 B each).  Slot s = page * page_size + offset.
 * FP8 q is a single tensor whose per-row scale is folded into the head weights
 * (P3 "forward_cuda"): the logits take w' = w * s_q.  Logits:
 *   logits[t, s] = s_k[s] * sum_h w'[t,h] * max(0, q8[t,h] . k8[s])
 * with q8, k8 the E4M3 values, fp32 accumulation.
 * ------------------------------------------------------------------------- */
typedef enum { IDX_FP8_SCALE_F32 = 0, IDX_FP8_SCALE_POW2 = 1 } idx_fp8_scale;
#define IDX_FP8_ROW_BYTES 132

/* idx_quantize_fp8 -- FP8-encode `rows` rows of 128 values (the FP8 query).
 *   x, dtype, rows, row_stride: as for idx_quantize.
 *   scale_fmt: IDX_FP8_SCALE_F32 or IDX_FP8_SCALE_POW2.
 *   values: [rows, 128] uint8 out (16-byte aligned);  scales: [rows] fp32 out.
 *   w_in, w_out: both NULL, or both [rows] fp32: w_out[r] = w_in[r] * scales[r]
 *   (one fp32 product), the folded weights for a query whose rows are
 *   [T, H, 128] and weights [T, H] (w_out may alias w_in). */
int idx_quantize_fp8(const void* x, int dtype, int64_t rows, int64_t row_stride, int scale_fmt,
                     uint8_t* values, float* scales, const float* w_in, float* w_out,
                     hipStream_t stream);

/* idx_insert_fp8 -- quantize K rows to FP8 and scatter them into the FP8 paged
 * cache [num_pages, page_size * 132] (the indexer K quant-and-cache of the FP8
 * format); slots as for idx_insert (negative or out-of-range slots write
 * nothing).  page_size must be 64; the cache 16-byte aligned. */
int idx_insert_fp8(const void* k, int dtype, int64_t num_tokens, int64_t k_row_stride,
                   int scale_fmt, const int64_t* slot_mapping, uint8_t* cache, int64_t num_pages,
                   int page_size, hipStream_t stream);

/* idx_gather_fp8 -- FP8 paged cache -> contiguous k_values [total_tokens, 128]
 * uint8 and k_scales [total_tokens] fp32; addressing and skipping as for
 * idx_gather. */
int idx_gather_fp8(const uint8_t* cache, int64_t num_pages, int page_size,
                   const int32_t* block_table, int64_t bt_row_stride, const int32_t* seq_lens,
                   const int64_t* cu_seq_offsets, int batch, int64_t max_seq_len,
                   int64_t total_tokens, uint8_t* k_values, float* k_scales, hipStream_t stream);

/* idx_logits_prefill_fp8 -- dense FP8 logits (mqa_logits on the FP8 format):
 *   q_values [T, H, 128] (idx_quantize_fp8 output), weights [T, H] fp32 holding
 *   w' (the query scales folded in), k_values [S, 128], k_scales [S] fp32;
 *   ks, ke, T, H, S, logits, logits_row_stride, clean: as for idx_logits_prefill. */
int idx_logits_prefill_fp8(const uint8_t* q_values, const float* weights, const uint8_t* k_values,
                           const float* k_scales, const int32_t* ks, const int32_t* ke, int64_t T,
                           int H, int64_t S, float* logits, int64_t logits_row_stride, int clean,
                           hipStream_t stream);

/* idx_logits_paged_fp8 -- paged FP8 decode logits (paged_mqa_logits on the FP8
 * format): q_values [B*next_n, H, 128], weights [B*next_n, H] fp32 (w'), the FP8
 * cache; every other argument, the visibility rule and the error behaviour
 * are those of idx_logits_paged. */
int idx_logits_paged_fp8(const uint8_t* q_values, const float* weights, const uint8_t* cache,
                         int64_t num_pages, int page_size, const int32_t* block_table,
                         int64_t bt_row_stride, const int32_t* context_lens, int B, int next_n,
                         int H, int64_t max_context_len, float* logits, int64_t logits_row_stride,
                         int clean, hipStream_t stream);

/* idx_logits_paged_insert_fp8 -- the FP8 decode step's two encodes and its paged
 * logits in one launch: equal, byte for byte and bit for bit, to idx_insert_fp8
 * of the new tokens into their block-table slots, idx_quantize_fp8 of q with the
 * weights folded (P3 "forward_cuda": FP8 q is a single tensor, its per-token
 * scale folded into the weights), then idx_logits_paged_fp8 with those rows and
 * w'.  For decode steps bound by launch count.
 *   q:         [B*next_n, H, 128] bf16 (IDX_BF16) or fp32 (IDX_F32), contiguous,
 *              16-byte aligned: the query rows, encoded in the kernel.
 *   k_new:     [B*next_n, 128] in the same dtype, contiguous, 16-byte aligned:
 *              row b*next_n + i is the K row of sequence b's token at position
 *              context_lens[b] - next_n + i, written to page
 *              block_table[b, pos / 64], offset pos % 64 (positions < 0, pages
 *              whose table entry is outside [0, num_pages) and pages past
 *              max_context_len are not written).
 *   weights:   [B*next_n, H] fp32, not folded (the kernel folds them).
 *   scale_fmt: IDX_FP8_SCALE_F32 or IDX_FP8_SCALE_POW2, for q and the new K rows.
 *   cache:     the FP8 cache, updated in place (the new tokens' 132 bytes) and read.
 *   All other arguments, the logits and the error behaviour are those of
 *   idx_logits_paged_fp8; the new tokens' pages must not appear in another
 *   sequence's block table. */
int idx_logits_paged_insert_fp8(const void* q, const void* k_new, int dtype, const float* weights,
                                int scale_fmt, uint8_t* cache, int64_t num_pages, int page_size,
                                const int32_t* block_table, int64_t bt_row_stride,
                                const int32_t* context_lens, int B, int next_n, int H,
                                int64_t max_context_len, float* logits,
                                int64_t logits_row_stride, int clean, hipStream_t stream);

/* idx_kpool_insert -- the pooled indexer-K insert of P3
 * "vllm.models.glm5next.nvidia.sparse_indexer", section "_kpool_compress_insert":
 * kpool consecutive tokens pooled into one K row, quantized and written at a
 * pool slot.  As P3 prints it: slot_mapping [n] int64 is pool-granular (only the
 * last token of a complete pool carries a slot >= 0); position i is written iff
 * slot_mapping[i] >= 0 and i >= kpool - 1, from the pool of tokens
 * i - kpool + 1 .. i; with n < kpool nothing is written.  The pooling, which the
 * page does not print, is read here as a per-dimension softmax gate:
 *   pooled[d] = sum_j softmax_j(gate_score[i-kpool+1+j, d] + ape[j, d]) * k[i-kpool+1+j, d]
 * computed in fp32 (maximum subtracted, exp, both sums in token order, one
 * division) -- so the bytes written may differ from an exact computation's in
 * the last place of the pooled value, i.e. by one code step where it lies
 * within that distance of a rounding boundary.
 *   k:            [n, k_row_stride] bf16 or fp32 (as for idx_insert).
 *   gate_score:   [n, 128] fp32, ape: [kpool, 128] fp32, both 16-byte aligned.
 *   kpool:        1 .. IDX_KPOOL_MAX.
 *   cache_format: IDX_CACHE_MXFP4 (68-byte rows, the cache of idx_insert) or
 *                 IDX_CACHE_FP8 (132-byte rows, the cache of idx_insert_fp8, with
 *                 fp8_scale_fmt as there; P3's round_scale = IDX_FP8_SCALE_POW2).
 *                 fp8_scale_fmt must be valid (it is ignored for MXFP4).
 *   cache:        [num_pages, 64 * row bytes], 16-byte aligned; slots outside it
 *                 write nothing.  page_size must be 64.
 *   compressed:   NULL, or [n, 128] fp32 out (16-byte aligned): the pooled rows
 *                 of the written positions (P3's return_compressed); other rows
 *                 are left untouched. */
typedef enum { IDX_CACHE_MXFP4 = 0, IDX_CACHE_FP8 = 1 } idx_cache_format;
#define IDX_KPOOL_MAX 1024
int idx_kpool_insert(const void* k, int dtype, int64_t n, int64_t k_row_stride,
                     const float* gate_score, const float* ape, const int64_t* slot_mapping,
                     int kpool, int cache_format, int fp8_scale_fmt, uint8_t* cache,
                     int64_t num_pages, int page_size, float* compressed, hipStream_t stream);

/* idx_topk -- per-row top-k column indices (top_k_per_row, P3
 * "SparseAttnIndexerKpool"; exact sets as tested in P2 "Validation").
 *   logits [rows, logits_row_stride] fp32 (finite in [ks, ke));
 *   ks [rows] int32 or NULL (= 0); ke [rows] int32;
 *   out_idx [rows, k] int32 out: the columns of the min(k, ke-ks) largest values
 *   in [ks, ke), ranked by value then by lower column (-0.0 == +0.0); the
 *   remaining slots hold -1.  The set is exact; the order of the returned
 *   columns is deterministic but not part of the contract.
 *   1 <= k <= 2048; columns are absolute indices into the row. */
int idx_topk(const float* logits, int64_t rows, int64_t logits_row_stride,
             const int32_t* ks, const int32_t* ke, int k, int32_t* out_idx,
             hipStream_t stream);

/* idx_topk_workspace_bytes -- size of the device workspace idx_topk_ws needs
 * for `rows` rows of a logits matrix with row stride `logits_row_stride`.
 * Non-zero only when idx_topk_ws splits rows over several workgroups: fewer
 * than 512 rows that may hold more than 8,192 columns, with a row stride of at
 * most 64 x 8,192 columns.  For the 64 x 131,072 long-context batch it is
 * about 33.6 MB (64 rows x 16 parts x 4,096 (key, column) pairs, plus a
 * header per part).  0 for invalid sizes. */
size_t idx_topk_workspace_bytes(int64_t rows, int64_t logits_row_stride);

/* idx_topk_ws -- idx_topk with a device workspace: the same exact sets (same
 * arguments, ranking and -1 padding).  When few rows are long it splits each
 * into parts of 8,192 columns, one workgroup per part, each keeping the keys
 * at or above an estimate of the row's top-k threshold in the workspace; a
 * second launch on the same stream selects each row's top-k from its kept
 * keys, or over the whole row when the kept keys cannot be shown to hold it.
 * The order of the returned columns is deterministic but differs from
 * idx_topk's.
 *   workspace: device memory of at least idx_topk_workspace_bytes(rows,
 *   logits_row_stride) bytes, 256-byte aligned, owned by the caller; its
 *   contents need no initialization and are scratch after the call.  Calls
 *   that share a workspace must not run concurrently.  May be NULL when that
 *   size is 0.  IDX_ERR_ARG if it is missing, misaligned or too small. */
int idx_topk_ws(const float* logits, int64_t rows, int64_t logits_row_stride,
                const int32_t* ks, const int32_t* ke, int k, int32_t* out_idx,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* idx_topk_noalloc -- idx_topk_ws for callers that cannot allocate device
 * memory: code under HIP graph capture that may not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation.  The same arguments,
 * kernels and exact sets as idx_topk_ws, the workspace being the library's
 * own static device array of IDX_TOPK_NOALLOC_MAX_WORKSPACE bytes (36 MiB, which
 * holds the workspace of 64 rows of up to 131,072 columns) instead of a
 * caller's buffer.  Each device holds its own copy of that array from the
 * library's load until the process ends; its address is looked up once per
 * device, on the first call there.  Nothing is allocated or freed per call.
 *   Returns IDX_ERR_ARG (before any device work) when the call needs more
 *   workspace than the array holds, i.e. when
 *   idx_topk_workspace_bytes(rows, logits_row_stride) >
 *   IDX_TOPK_NOALLOC_MAX_WORKSPACE.
 *   Every call on a device shares that device's array, which keeps the last
 *   call's contents (no call depends on them: each split call rewrites every
 *   byte it reads).  Calls that may overlap on one device -- on different
 *   streams, or from several host threads without ordering -- race on the
 *   array and must not be issued. */
#define IDX_TOPK_NOALLOC_MAX_WORKSPACE (36ll << 20)
int idx_topk_noalloc(const float* logits, int64_t rows, int64_t logits_row_stride,
                     const int32_t* ks, const int32_t* ke, int k, int32_t* out_idx,
                     hipStream_t stream);

/* idx_topk_merge -- merge per-rank top-k lists into a sequence's top-k: the
 * exchange step of decode with the context split over `world` ranks (P3
 * "SparseAttnIndexerKpool": dcp_rank, dcp_world_size,
 * cp_kv_cache_interleave_size).  Rank s holds the sequence's positions in runs
 * of `interleave` consecutive positions dealt round-robin, so its local
 * position l is global position (l / interleave) * interleave * world +
 * s * interleave + l % interleave.
 *   values  [world, rows, k_in] fp32 (finite): rank s's candidate values for row r;
 *   indices [world, rows, k_in] int32: their local positions, -1 = empty slot;
 *   out_idx [rows, k] int32 out: the global positions of the min(k, valid)
 *   best candidates, ranked by value then by lower global position
 *   (-0.0 == +0.0), then -1.  The set is exact (with each rank's exact
 *   top-k as input it is the unsharded top-k); the order is deterministic but
 *   not part of the contract.
 * 1 <= world, 1 <= k_in, world * k_in <= IDX_MERGE_MAX_CANDIDATES,
 * 1 <= k <= 2048, interleave >= 1; global positions must be < 2^31. */
int idx_topk_merge(const float* values, const int32_t* indices, int world, int64_t rows,
                   int k_in, int interleave, int k, int32_t* out_idx, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXIDX_H */
