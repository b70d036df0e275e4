"""FP8 indexer cache: E4M3 codec, per-token scale, 132-byte paged rows and the
FP8 indexer logits (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The FP8 indexer cache is the format the MXFP4 cache replaces: 132 bytes per
token per head (P1 "Benefit": 132 -> 68), i.e. 128 FP8 values and one 4-byte
scale per token; its page keeps the block-split value/scale layout that the
MXFP4 cache copies (P1 live-validation comment).  FP8 q is a single tensor
whose per-token scale the caller folds into the head weights (P3
"forward_cuda"); the insert can round its scale to a power of two
(``round_scale`` of P3 "_kpool_compress_insert").

Readings where the pages are silent (each pinned by a test):

* element format: OCP FP8 E4M3 ("e4m3fn": bias 7, subnormals, no
  infinities, S.1111.111 is NaN, largest finite 448);
* scale: s = amax / 448 rounded to fp32 (so the block maximum maps to 448),
  floored at the smallest normal fp32 2**-126 (an all-zero row, or one so
  small that amax / 448 underflows, keeps a finite divisor); with
  ``round_scale`` s = 2**E, E the smallest integer with amax <= 448 * 2**E,
  clamped to [-126, 127];
* elements: y = x / s rounded to fp32 (one correctly rounded fp32 division,
  the precision the kernel takes the decision in), then the nearest E4M3 value,
  ties to the even code (mantissa bit 0), |y| > 448 saturating to 448
  (unreachable under the scale rule); the sign bit is the sign bit of y;
* the scale is stored as a little-endian fp32 (4 bytes), also when it is a
  power of two;
* page of P tokens: the P value rows (128 B each) in token order, then the P
  scale words (4 B each): 132 * P bytes;
* query: the same row encode; the caller's head weights become
  w' = fl32(w * s_q) (one fp32 product), and the logits use w' as given;
* logits: logit[t, s] = s_k[s] * sum_h w'[t, h] * max(0, sum_i q8[t,h,i] *
  k8[s,i]) with q8, k8 the E4M3 values (unscaled): the dot of the dequantized
  rows, with both positive scales taken out of the ReLU.
"""

import numpy as np

HEAD_DIM = 128
ROW_VALUE_BYTES = 128
ROW_SCALE_BYTES = 4
ROW_BYTES = ROW_VALUE_BYTES + ROW_SCALE_BYTES    # 132
E4M3_MAX = 448.0
SCALE_FLOOR = 2.0 ** -126
PAGE_SIZE = 64


def e4m3_value(code):
    """Real value of an E4M3 byte from its bit fields (NaN for S.1111.111)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def _round_half_even(q):
    """Nearest integer, ties to even (exact for float64 inputs)."""
    f = np.floor(q)
    d = q - f
    up = (d > 0.5) | ((d == 0.5) & (np.fmod(f, 2.0) != 0))
    return f + up


def e4m3_encode(y):
    """E4M3 bytes of fp32 values y (given as float32 or their exact float64).

    Magnitude: normal range (|y| >= 2**-6): exponent e = floor(log2 |y|), the
    mantissa |y| / 2**e - 1 in eighths rounded half to even (a carry moves to
    the next binade); subnormal range: |y| / 2**-9 rounded half to even.
    Above 448 the code saturates to 448.  Sign bit: signbit(y).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    frac, ex = np.frexp(a)                 # a = frac * 2**ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1            # a in [2**e, 2**(e+1))
    normal = a >= 2.0 ** -6
    # normal: mantissa eighths
    mq = _round_half_even((np.ldexp(a, -np.clip(e, -6, 8)) - 1.0) * 8.0)
    e_n = np.clip(e, -6, 8) + (mq >= 8)
    m_n = np.where(mq >= 8, 0, mq)
    field_n = e_n + 7
    # subnormal: multiples of 2**-9
    sq = _round_half_even(np.ldexp(a, 9))
    field_s = np.where(sq >= 8, 1, 0)
    m_s = np.where(sq >= 8, 0, sq)
    field = np.where(normal, field_n, field_s).astype(np.int64)
    mant = np.where(normal, m_n, m_s).astype(np.int64)
    # saturation: beyond 448 (field 15, mantissa 6) -> 448
    over = (field > 15) | ((field == 15) & (mant > 6)) | (a > E4M3_MAX)
    field = np.where(over, 15, field)
    mant = np.where(over, 6, mant)
    sign = np.signbit(y).astype(np.int64)
    return ((sign << 7) | (field << 3) | mant).astype(np.uint8)


def e4m3_decode(codes):
    """float64 values of E4M3 bytes (NaN codes give NaN)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def scale_exponent(amax):
    """Smallest integer E with amax <= 448 * 2**E, clamped to [-126, 127]
    (-126 for amax == 0).  448 = 7 * 2**6 and amax = f * 2**x with f in [0.5, 1):
    E is x - 9 or x - 8; the test amax <= 448 * 2**(x-9) is exact in float64."""
    amax = np.asarray(amax, dtype=np.float64)
    _, x = np.frexp(amax)
    x = x.astype(np.int64)
    E = np.where(amax <= np.ldexp(E4M3_MAX, x - 9), x - 9, x - 8)
    E = np.where(amax == 0.0, -126, E)
    return np.clip(E, -126, 127)


def row_scales(x, round_scale=False):
    """Per-row fp32 scale of rows x [R, 128] (exact float64 values of fp32 inputs)."""
    amax = np.abs(np.asarray(x, dtype=np.float64)).max(axis=-1)
    if round_scale:
        return np.ldexp(np.float32(1.0), scale_exponent(amax)).astype(np.float32)
    s = (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)   # fp32 division
    return np.maximum(s, np.float32(SCALE_FLOOR)).astype(np.float32)


def quantize_rows(x, round_scale=False):
    """FP8-encode rows of 128 values (exact float64 values of bf16 / fp32 inputs).

    Returns (codes uint8 [R, 128], scales float32 [R])."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    s = row_scales(x, round_scale)
    y = (x.astype(np.float32) / s[:, None]).astype(np.float32)               # fp32 division
    return e4m3_encode(y), s


def dequantize_rows(codes, scales):
    """Exact values (float64 [R, 128]) of FP8 rows: e4m3(code) * scale."""
    v = e4m3_decode(np.asarray(codes).reshape(-1, HEAD_DIM))
    return v * np.asarray(scales, dtype=np.float64).reshape(-1, 1)


def fold_weights(w, q_scales):
    """w' = fl32(w * s_q): the query's per-row scale folded into its head weight."""
    return (np.asarray(w, dtype=np.float32) * np.asarray(q_scales, dtype=np.float32)).astype(np.float32)


# --------------------------------------------------------------------------- paged cache

def page_bytes(page_size=PAGE_SIZE):
    return page_size * ROW_BYTES


def value_offset(page, off, page_size=PAGE_SIZE):
    """Byte offset of token ``off`` of page ``page``'s 128 value bytes."""
    return page * page_bytes(page_size) + off * ROW_VALUE_BYTES


def scale_offset(page, off, page_size=PAGE_SIZE):
    """Byte offset of token ``off`` of page ``page``'s 4 scale bytes."""
    return page * page_bytes(page_size) + page_size * ROW_VALUE_BYTES + off * ROW_SCALE_BYTES


def write_rows(cache, codes, scales, slot_mapping, page_size=PAGE_SIZE):
    """Scatter encoded rows into a copy of ``cache`` [num_pages, P * 132]
    (slot = page * P + offset).  Negative slots write nothing (P3
    "_kpool_compress_insert": -1 = no write), and so do slots beyond the cache
    (the safety reading the MXFP4 insert takes too)."""
    out = np.array(cache, dtype=np.uint8, copy=True).reshape(-1)
    num_slots = out.size // ROW_BYTES
    sbytes = np.asarray(scales, dtype="<f4").view(np.uint8).reshape(-1, 4)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for i in np.nonzero((slots >= 0) & (slots < num_slots))[0]:
        page, off = divmod(int(slots[i]), page_size)
        v0 = value_offset(page, off, page_size)
        s0 = scale_offset(page, off, page_size)
        out[v0:v0 + ROW_VALUE_BYTES] = codes[i]
        out[s0:s0 + ROW_SCALE_BYTES] = sbytes[i]
    return out.reshape(np.shape(cache))


def insert(cache, k_values, slot_mapping, round_scale=False, page_size=PAGE_SIZE):
    """Quantize K rows (exact float64 values [N, 128]) and scatter them."""
    codes, scales = quantize_rows(k_values, round_scale)
    return write_rows(cache, codes, scales, slot_mapping, page_size)


def gather(cache, block_table, seq_lens, cu_seq_offsets, total_tokens, page_size=PAGE_SIZE):
    """Paged cache -> contiguous (codes [total, 128] uint8, scales [total] float32);
    token j of sequence b is read from page block_table[b, j // P], offset j % P."""
    flat = np.asarray(cache, dtype=np.uint8).reshape(-1)
    codes = np.zeros((total_tokens, ROW_VALUE_BYTES), dtype=np.uint8)
    sbytes = np.zeros((total_tokens, ROW_SCALE_BYTES), dtype=np.uint8)
    for b in range(len(seq_lens)):
        n = int(seq_lens[b])
        j = np.arange(n)
        page = np.asarray(block_table)[b, j // page_size].astype(np.int64)
        off = j % page_size
        v0 = page * page_bytes(page_size) + off * ROW_VALUE_BYTES
        s0 = page * page_bytes(page_size) + page_size * ROW_VALUE_BYTES + off * ROW_SCALE_BYTES
        rows = int(cu_seq_offsets[b]) + j
        codes[rows] = flat[v0[:, None] + np.arange(ROW_VALUE_BYTES)]
        sbytes[rows] = flat[s0[:, None] + np.arange(ROW_SCALE_BYTES)]
    return codes, sbytes.view("<f4").reshape(-1).astype(np.float32)


# --------------------------------------------------------------------------- logits

def mqa_logits(q_codes, w_folded, k_codes, k_scales, ks, ke, width=None, rows=None, chunk=64,
               with_bound=False):
    """Dense FP8 logits, float64 [len(rows), width], -inf outside [ks, ke).

    q_codes [T, H, 128] E4M3 bytes; w_folded [T, H] float32 (w' = w * s_q);
    k_codes [S, 128], k_scales [S] float32.  Every product of two E4M3 values
    is exact in float64, and a 128-term dot needs at most 8 + 34 bits, so the
    head dots are exact; the result is the definition up to the rounding of
    the final weighted sum (~1e-16 relative).  With ``with_bound`` also returns
    A = s_k * sum_h |w'| * sum_i |q8_i k8_i| (0 where masked), the scale of the
    fp32 rounding error of any summation order of the dot and head sums.
    """
    q_codes = np.asarray(q_codes)
    T, H = q_codes.shape[0], q_codes.shape[1]
    S = np.asarray(k_codes).shape[0]
    width = S if width is None else width
    rows = np.arange(T) if rows is None else np.asarray(rows)
    ks = np.asarray(ks)
    ke = np.minimum(np.asarray(ke), S)
    k8 = e4m3_decode(k_codes)                                   # [S, 128]
    sk = np.asarray(k_scales, dtype=np.float64)
    w = np.asarray(w_folded, dtype=np.float64)
    out = np.full((len(rows), width), -np.inf, dtype=np.float64)
    bound = np.zeros((len(rows), width), dtype=np.float64) if with_bound else None
    for c0 in range(0, len(rows), chunk):
        rr = rows[c0:c0 + chunk]
        q8 = e4m3_decode(q_codes[rr].reshape(-1, HEAD_DIM)).reshape(len(rr), H, HEAD_DIM)
        lo = int(np.min(ks[rr]))
        hi = int(np.max(ke[rr]))
        if hi <= lo:
            continue
        d = q8 @ k8[lo:hi].T                                    # [c, H, hi-lo], exact
        score = np.einsum("th,ths->ts", w[rr], np.maximum(d, 0.0)) * sk[None, lo:hi]
        if with_bound:
            ad = np.abs(q8) @ np.abs(k8[lo:hi]).T
            bnd = np.einsum("th,ths->ts", np.abs(w[rr]), ad) * sk[None, lo:hi]
        for j, t in enumerate(rr):
            a, b = int(ks[t]), int(ke[t])
            if b > a:
                out[c0 + j, a:b] = score[j, a - lo:b - lo]
                if with_bound:
                    bound[c0 + j, a:b] = bnd[j, a - lo:b - lo]
    return (out, bound) if with_bound else out


def paged_mqa_logits(q_codes, w_folded, cache, block_table, context_lens, next_n, width,
                     page_size=PAGE_SIZE, seqs=None, with_bound=False):
    """Paged FP8 decode logits, float64 [B*next_n, width]; row b*next_n + i of
    sequence b (context L_b) sees s < L_b - next_n + i + 1."""
    B = len(context_lens)
    out = np.full((B * next_n, width), -np.inf, dtype=np.float64)
    bound = np.zeros((B * next_n, width), dtype=np.float64) if with_bound else None
    L_all = np.asarray(context_lens, dtype=np.int64)
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        L = int(L_all[b])
        kc, ksc = gather(cache, np.asarray(block_table)[b:b + 1], [L], [0], L, page_size)
        r = np.arange(b * next_n, (b + 1) * next_n)
        ke = np.maximum(L - next_n + np.arange(next_n) + 1, 0)
        sub = mqa_logits(np.asarray(q_codes)[r], np.asarray(w_folded)[r], kc, ksc,
                         np.zeros(next_n, np.int64), ke, width=L, with_bound=with_bound)
        if with_bound:
            out[r, :L], bound[r, :L] = sub
        else:
            out[r, :L] = sub
    return (out, bound) if with_bound else out
