"""Paged MXFP4 indexer-K cache: insert (quantize + scatter) and gather (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Layout (P1 live-validation comment: "block-split value/scale layout", shared
by the gather and the paged logits reader; P1 "Benefit": 68 bytes per
token):  a page of P tokens is P*68 bytes.  The first P*64 bytes hold the
tokens' code rows in token order, the last P*4 bytes their scale rows in
token order.  Token ``off`` of page ``p`` therefore has its codes at
``p*P*68 + off*64`` and its scales at ``p*P*68 + P*64 + off*4``.

Slot mapping (P1 live-validation comment: int64 ``slot_mapping`` argument of
the insert kernel; P3 "_kpool_compress_insert": slot -1 means "do not
write"): slot = page * P + offset; a negative slot writes nothing.
Non-negative slots are assumed distinct within one call.
"""

import numpy as np

from .mxfp4 import CODE_BYTES, SCALE_BYTES, ROW_BYTES, quantize_rows

PAGE_SIZE = 64


def page_bytes(page_size=PAGE_SIZE):
    return page_size * ROW_BYTES


def code_offset(page, off, page_size=PAGE_SIZE):
    """Byte offset of token ``off`` of page ``page``'s 64 code bytes in the cache."""
    return page * page_bytes(page_size) + off * CODE_BYTES


def scale_offset(page, off, page_size=PAGE_SIZE):
    """Byte offset of token ``off`` of page ``page``'s 4 scale bytes in the cache."""
    return page * page_bytes(page_size) + page_size * CODE_BYTES + off * SCALE_BYTES


def write_rows(cache, codes, scales, slot_mapping, page_size=PAGE_SIZE):
    """Scatter already-encoded rows into a copy of ``cache`` (flat uint8)."""
    out = np.array(cache, dtype=np.uint8, copy=True).reshape(-1)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for i in np.nonzero(slots >= 0)[0]:
        page, off = divmod(int(slots[i]), page_size)
        c0 = code_offset(page, off, page_size)
        s0 = scale_offset(page, off, page_size)
        out[c0:c0 + CODE_BYTES] = codes[i]
        out[s0:s0 + SCALE_BYTES] = scales[i]
    return out.reshape(np.shape(cache))


def insert(cache, k_values, slot_mapping, page_size=PAGE_SIZE):
    """Quantize K rows (exact float64 values [N, 128]) and scatter them.

    Returns the new cache; bytes of tokens with slot < 0 and of every other
    slot are left as they were.
    """
    codes, scales = quantize_rows(k_values)
    return write_rows(cache, codes, scales, slot_mapping, page_size)


def read_token(cache, page, off, page_size=PAGE_SIZE):
    """(codes[64], scales[4]) of one cached token."""
    flat = np.asarray(cache, dtype=np.uint8).reshape(-1)
    c0 = code_offset(page, off, page_size)
    s0 = scale_offset(page, off, page_size)
    return flat[c0:c0 + CODE_BYTES].copy(), flat[s0:s0 + SCALE_BYTES].copy()


def gather(cache, block_table, seq_lens, cu_seq_offsets, total_tokens,
           page_size=PAGE_SIZE):
    """Paged cache -> contiguous (codes [total, 64], scales [total, 4]).

    Token j of sequence b lives in page ``block_table[b, j // P]`` at offset
    ``j % P`` and lands in output row ``cu_seq_offsets[b] + j``.  Rows not
    covered by any sequence are left zero.
    """
    flat = np.asarray(cache, dtype=np.uint8).reshape(-1)
    codes = np.zeros((total_tokens, CODE_BYTES), dtype=np.uint8)
    scales = np.zeros((total_tokens, SCALE_BYTES), dtype=np.uint8)
    for b in range(len(seq_lens)):
        n = int(seq_lens[b])
        j = np.arange(n)
        page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
        off = j % page_size
        c0 = page * page_bytes(page_size) + off * CODE_BYTES
        s0 = page * page_bytes(page_size) + page_size * CODE_BYTES + off * SCALE_BYTES
        rows = int(cu_seq_offsets[b]) + j
        codes[rows] = flat[c0[:, None] + np.arange(CODE_BYTES)]
        scales[rows] = flat[s0[:, None] + np.arange(SCALE_BYTES)]
    return codes, scales
