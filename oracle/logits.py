"""Indexer logits, dense (mqa_logits) and paged (paged_mqa_logits) (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition (the DSA lightning-indexer score computed by the kernels that P3
"SparseAttnIndexerKpool" names mqa_logits and paged_mqa_logits; P2
"Summary" names the prefill and paged-decode MQA-logits kernels):

    logit[t, s] = sum_h w[t, h] * max(0, sum_i qhat[t, h, i] * khat[s, i])

where qhat and khat are the exact values of the MXFP4 rows (both block scales
applied before the ReLU: P3 "forward_cuda" passes FP4 q as a (values, scales)
pair, so the q scale is part of the dot and ``w`` is used as given).

Visibility: column s of row t is computed for ks[t] <= s < ke[t]; every other
column is -inf (the caller compares masked entries only for clean output).
Decode row r = b*next_n + i of sequence b with context length L sees
s < L - next_n + i + 1 (causal over the next_n new tokens, which are the
last next_n tokens of the sequence).

Arithmetic: float64 matrix products over the dequantized values.  Every
product of two MXFP4 values is exact in float64 and each 32-element block dot
has at most 13 significant bits, so the head dot is exact whenever the block
exponents of a (q, k) pair span at most 38 binary orders; ``check_exact``
asserts that.  The result is then the mathematical definition up to the
rounding of the final weighted head sum (~1e-16 relative).
"""

import numpy as np

from .mxfp4 import dequantize_rows, HEAD_DIM, NBLOCKS, BLOCK
from .paged_cache import gather, PAGE_SIZE


def _live_scale_range(codes, scales):
    """(min, max) scale byte over blocks that hold a non-zero element, or None."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, NBLOCKS, BLOCK // 2)
    s = np.asarray(scales, dtype=np.uint8).reshape(-1, NBLOCKS).astype(np.int64)
    live = ((c & 0x77) != 0).any(axis=-1)          # a magnitude bit set in the block
    if not live.any():
        return None
    return int(s[live].min()), int(s[live].max())


def check_exact(q_codes, q_scales, k_codes, k_scales):
    """Assert that the float64 head dots are exact for these rows.

    Blocks whose elements are all zero contribute nothing and are ignored.
    """
    rq = _live_scale_range(q_codes, q_scales)
    rk = _live_scale_range(k_codes, k_scales)
    if rq is None or rk is None:
        return
    spread = (rq[1] + rk[1]) - (rq[0] + rk[0])
    assert spread <= 38, f"block exponent spread {spread} too wide for exact float64 dots"


def _dequant_q(q_codes, q_scales):
    q_codes = np.asarray(q_codes)
    T, H = q_codes.shape[0], q_codes.shape[1]
    return dequantize_rows(q_codes.reshape(-1, 64), np.asarray(q_scales).reshape(-1, 4)).reshape(T, H, HEAD_DIM)


def mqa_logits(q_codes, q_scales, k_codes, k_scales, w, ks, ke, width=None, chunk=64,
               rows=None, with_bound=False):
    """Dense logits, float64 [len(rows), width], -inf outside [ks, ke).

    q_codes [T, H, 64], q_scales [T, H, 4], k_codes [S, 64], k_scales [S, 4],
    w [T, H] (float32 values), ks/ke [T] (ke is clipped to S).  ``rows``
    selects query rows (default all); ``width`` defaults to S.  With
    ``with_bound`` also returns A (see ``abs_bound``) for the same entries
    (0 where masked).
    """
    check_exact(q_codes, q_scales, k_codes, k_scales)
    T = np.asarray(q_codes).shape[0]
    S = np.asarray(k_codes).shape[0]
    width = S if width is None else width
    rows = np.arange(T) if rows is None else np.asarray(rows)
    ks = np.asarray(ks)
    ke = np.minimum(np.asarray(ke), S)
    khat = dequantize_rows(k_codes, k_scales)                    # [S, 128]
    out = np.full((len(rows), width), -np.inf, dtype=np.float64)
    bound = np.zeros((len(rows), width), dtype=np.float64) if with_bound else None
    w = np.asarray(w, dtype=np.float64)
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        qh = _dequant_q(np.asarray(q_codes)[rr], np.asarray(q_scales)[rr])  # [c, H, 128]
        lo = int(np.min(ks[rr]))
        hi = int(np.max(ke[rr]))
        if hi <= lo:
            continue
        d = qh @ khat[lo:hi].T                                   # [c, H, hi-lo]
        score = np.einsum("th,ths->ts", w[rr], np.maximum(d, 0.0))
        if with_bound:
            ab = np.zeros_like(d)
            for b in range(NBLOCKS):
                sl = slice(b * BLOCK, (b + 1) * BLOCK)
                ab += np.abs(qh[:, :, sl] @ khat[lo:hi, sl].T)
            bnd = np.einsum("th,ths->ts", np.abs(w[rr]), ab)
        for j, t in enumerate(rr):
            a, b = int(ks[t]), int(ke[t])
            if b > a:
                out[c0 + j, a:b] = score[j, a - lo:b - lo]
                if with_bound:
                    bound[c0 + j, a:b] = bnd[j, a - lo:b - lo]
    return (out, bound) if with_bound else out


def abs_bound(q_codes, q_scales, k_codes, k_scales, w, rows, cols):
    """A[t, s] = sum_h |w[t,h]| * sum_b |c_{h,b}[t,s]| for the listed (row, col) pairs.

    c_{h,b} is the exact scaled dot of block b.  Used by the logits tolerance
    (it bounds the fp32 rounding of the 4-block and head sums).
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    qh = _dequant_q(np.asarray(q_codes)[rows], np.asarray(q_scales)[rows])      # [n, H, 128]
    kh = dequantize_rows(np.asarray(k_codes)[cols], np.asarray(k_scales)[cols])  # [n, 128]
    qb = qh.reshape(qh.shape[0], qh.shape[1], NBLOCKS, BLOCK)
    kb = kh.reshape(kh.shape[0], 1, NBLOCKS, BLOCK)
    c = np.abs((qb * kb).sum(axis=-1)).sum(axis=-1)                            # [n, H]
    return (np.abs(np.asarray(w, dtype=np.float64)[rows]) * c).sum(axis=-1)


def decode_visible_end(context_lens, next_n):
    """ke for decode rows: row b*next_n + i sees s < L_b - next_n + i + 1."""
    L = np.asarray(context_lens, dtype=np.int64)
    i = np.arange(next_n)
    return (L[:, None] - next_n + i[None, :] + 1).reshape(-1)


def paged_mqa_logits(q_codes, q_scales, w, cache, block_table, context_lens, next_n,
                     width, page_size=PAGE_SIZE, seqs=None, with_bound=False):
    """Paged decode logits, float64 [B*next_n, width] (-inf where not visible).

    q_codes [B*next_n, H, 64], q_scales [B*next_n, H, 4], w [B*next_n, H].
    The K rows of sequence b are read through ``block_table[b]``.  ``seqs``
    restricts the work to some sequences (other rows stay -inf).
    """
    B = len(context_lens)
    out = np.full((B * next_n, width), -np.inf, dtype=np.float64)
    bound = np.zeros((B * next_n, width), dtype=np.float64) if with_bound else None
    ke_all = decode_visible_end(context_lens, next_n)
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        L = int(context_lens[b])
        kc, ksc = gather(cache, np.asarray(block_table)[b:b + 1], [L], [0], L, page_size)
        r = np.arange(b * next_n, (b + 1) * next_n)
        sub = mqa_logits(np.asarray(q_codes)[r], np.asarray(q_scales)[r], kc, ksc,
                         np.asarray(w)[r], np.zeros(next_n, np.int64), np.maximum(ke_all[r], 0),
                         width=L, with_bound=with_bound)
        if with_bound:
            out[r, :L], bound[r, :L] = sub
        else:
            out[r, :L] = sub
    return (out, bound) if with_bound else out
