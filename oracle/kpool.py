"""Pooled ("kpool") indexer-K insert (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P3 "vllm.models.glm5next.nvidia.sparse_indexer", section
"_kpool_compress_insert", prints the bookkeeping of this insert: ``kpool``
consecutive tokens are pooled into one K row that is quantized and written
at a pool slot; ``slot_mapping`` is pool-granular -- only the last token of a
complete pool carries a slot >= 0, the tokens inside a pool carry -1 -- and
every position is treated as a candidate pool end, with

    write_mask = (slot_mapping >= 0) & (position >= kpool - 1),

the pool of position i being the tokens i - kpool + 1 .. i (gathered to
[n, kpool, head_dim] along with their gate scores; ``ape`` is passed whole);
no pool can complete when n < kpool.  The pooling itself is not printed.
Reading taken here (the compressor form that gate scores plus an absolute
positional embedding suggest): per dimension d, the pooled value is the
softmax-weighted sum over the pool,

    z[j, d] = gate_score[i - kpool + 1 + j, d] + ape[j, d]
    pooled[d] = sum_j softmax_j(z[., d])[j] * k[i - kpool + 1 + j, d],

gate_score [n, 128] and ape [kpool, 128] fp32, k the exact input values.
The pooled row is then encoded by the cache's own rule (MXFP4, or the FP8
row of ``oracle.fp8`` with its optional power-of-two scale, P3's
``round_scale``) and written at the slot; slots outside the cache write
nothing.  Arithmetic here is float64 (the z sums of two fp32 values are
exact; exp and the sums round at ~1e-16).
"""

import numpy as np

from . import fp8 as ofp8
from . import mxfp4, paged_cache

HEAD_DIM = 128


def write_mask(slot_mapping, kpool):
    """Positions that complete a pool and carry a slot (P3's write_mask)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    n = len(slots)
    if n < kpool:
        return np.zeros(n, dtype=bool)
    pos = np.arange(n)
    return (slots >= 0) & (pos >= kpool - 1)


def pool_indices(n, kpool):
    """[n, kpool] token indices of each position's pool, clamped at 0 for the
    leading positions (which the write mask drops)."""
    pos = np.arange(n)
    return np.maximum(pos - (kpool - 1), 0)[:, None] + np.arange(kpool)[None, :]


def pooled_rows(k, gate_score, ape, kpool):
    """float64 [n, 128]: the softmax-weighted pool of every position (rows of
    positions that cannot complete a pool are computed over the clamped
    indices and are never written)."""
    k = np.asarray(k, dtype=np.float64)
    n = k.shape[0]
    idx = pool_indices(n, kpool)
    z = np.asarray(gate_score, dtype=np.float64)[idx] + np.asarray(ape, dtype=np.float64)[None]
    z = z - z.max(axis=1, keepdims=True)                     # [n, kpool, 128]
    e = np.exp(z)
    w = e / e.sum(axis=1, keepdims=True)
    return (w * k[idx]).sum(axis=1)


def insert(cache, k, gate_score, ape, slot_mapping, kpool, fmt="mxfp4", round_scale=False):
    """The new cache after the pooled insert; also returns (mask, pooled rows)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    mask = write_mask(slots, kpool)
    if not mask.any():
        return np.array(cache, copy=True), mask, None
    pooled = pooled_rows(k, gate_score, ape, kpool)
    s = np.where(mask, slots, -1)
    if fmt == "mxfp4":
        codes, scales = mxfp4.quantize_rows(pooled.astype(np.float32).astype(np.float64))
        num_slots = np.asarray(cache).size // mxfp4.ROW_BYTES
        s = np.where(s < num_slots, s, -1)
        out = paged_cache.write_rows(cache, codes, scales, s)
    elif fmt == "fp8":
        codes, scales = ofp8.quantize_rows(pooled.astype(np.float32).astype(np.float64), round_scale)
        out = ofp8.write_rows(cache, codes, scales, s)
    else:
        raise ValueError(fmt)
    return out, mask, pooled
