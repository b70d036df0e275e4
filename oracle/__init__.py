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

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, exhaustive brute force, hand-worked bytes
(``tests/golden/``) or exact rational arithmetic.  No function is left
"parity unpinned", but the byte-layout choices that the pages leave open
(page split, nibble order, sign of zero, scale byte order) are pinned only by
the hand-worked bytes derived from the adopted reading.
"""

from . import mxfp4, paged_cache, logits, topk, tolerance  # noqa: F401
