"""Plain CPU oracle for the MXFP4 paged indexer-cache path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never routes through it, and this package imports
nothing from the HIP library (``mxfp4_paged_cache_quant_amd``); the two share no
code.  Inputs for both sides come from ``workloads`` (seeded generators that
hold none of the method's arithmetic).

Sources (the three web pages on the subject):

* P1 -- "[Kernel] MXFP4 indexer cache for GLM-5.2 / DSA (glm_moe_dsa)"
  (vLLM pull request 48558): sections "Changes" (E2M1 values + UE8M0 block-32
  scales, written by a K quant-and-cache kernel through an int64 slot mapping),
  "Benefit" (132 -> 68 bytes per token per head) and the live-validation
  comment (block-split value/scale page layout shared with the gather and the
  paged logits reader).
* P2 -- "Enable SM86 MXFP4 sparse-indexer cache" (Whamp/vllm pull request 14):
  "Summary" (software E2M1/UE8M0 query and cache writers, prefill and
  paged-decode MQA-logits kernels) and "Validation" (exact top-k sets,
  ordering margin, poisoned tail, clean_logits=False paged tests).
* P3 -- API page "vllm.models.glm5next.nvidia.sparse_indexer":
  "SparseAttnIndexerKpool" (mqa_logits, paged_mqa_logits, top_k_per_row;
  FP4 q as a (values, scales) pair, forward_cuda) and "_kpool_compress_insert"
  (slot -1 means "no write").
* The OCP Microscaling Formats (MX) v1.0 specification (public), for the
  E2M1 element and E8M0 scale encodings that "MXFP4" names.

Arithmetic: integer bit operations for the codec, float64 for the logits.
Every reading taken where the pages are silent is stated in the function
that takes it.

Parity status: every function here is pinned on the CPU against values fixed
independently of its code.  Function -> pin (test file):

* mxfp4.e2m1_value -- the OCP E2M1 table, all 16 nibbles (test_oracle_codec)
* mxfp4.ue8m0_exponent -- its defining property (smallest E with
  amax <= 6 * 2**E), exhaustively over positive finite bf16 and at fp32
  boundaries (test_oracle_codec)
* mxfp4.e2m1_encode -- brute-force nearest grid point, ties to the even code,
  over every finite bf16 pattern (test_oracle_codec)
* mxfp4.quantize_rows / dequantize_rows -- hand-worked blocks A-G
  (tests/golden/mxfp4_blocks.txt) and the exact round trip (test_oracle_codec)
* paged_cache.insert / write_rows / gather / read_token -- hand-worked byte
  offsets, canaries, slot -1 and the insert/gather round trip (test_oracle_codec)
* logits.mqa_logits / paged_mqa_logits -- exact rational arithmetic, closed
  forms (one head, one-hot weights), 2**m scaling, page-order invariance, paged
  == dense (test_oracle_logits)
* logits.abs_bound and the with_bound outputs -- the exact rational A, and
  equality of the three ways of computing it (test_oracle_tolerance)
* topk.top_k_per_row, merge_shard_topk, shard_to_global / global_to_shard --
  brute-force sorts, hand-worked rows and layouts (test_oracle_topk)
* topk.kth_value -- a plain Python sort (test_oracle_tolerance)
* tolerance.logits_close, tolerance.topk_end_to_end_ok -- exact boundary
  cases and hand-worked rows (test_oracle_tolerance)
* fp8.e4m3_value / e4m3_encode / scale_exponent / row_scales / quantize_rows /
  fold_weights -- the OCP E4M3 table and hand-worked rows
  (tests/golden/fp8_e4m3.txt), brute-force nearest values over every bf16
  pattern and every midpoint, exact rational fp32 rounding (test_oracle_fp8)
* fp8.write_rows / insert / gather -- hand-worked 132-byte offsets, canaries,
  slot -1, round trip; fp8.mqa_logits / paged_mqa_logits -- exact rational
  arithmetic, a closed form, 2**m scaling, paged == dense (test_oracle_fp8)
* rope.apply_rope / quantize_rope -- hand-worked rotations, exact rational
  fp32 rounding of every product and sum (a fused-multiply-add copy must
  fail), identities, the complex-rotation closed form (test_oracle_rope)
* kpool.write_mask / pool_indices / pooled_rows / insert -- P3's printed
  bookkeeping worked by hand, plain-loop brute force, closed forms (mean,
  selection, shift invariance), masked writes only (test_oracle_kpool)

The pins of the comparison rules and of A are also run against copies of the
functions with one planted mistake each, and must reject every copy.  The
byte-layout choices that the pages leave open (page split, nibble order, sign
of zero, scale byte order) are pinned by the hand-worked bytes derived from the
adopted reading.
"""

from . import mxfp4, paged_cache, logits, topk, tolerance, fp8, rope, kpool  # noqa: F401
