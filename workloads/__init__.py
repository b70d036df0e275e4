"""Seeded synthetic inputs for the MXFP4 indexer-cache path.

This module only draws random numbers and lays out bookkeeping arrays (page
permutations, block tables, slot mappings, visibility ranges).  It holds none
of the method's arithmetic (no quantization, no logits, no selection); both
the HIP path and the oracle take their inputs from here.

Every case is a plain dict of NumPy arrays.  Random streams: one
``numpy.random.SeedSequence(seed)`` is split into independent child streams
for, in order, lengths, K, q, weights, page permutation and sampled rows, so
that changing one size does not reshuffle the other draws.

K and q values are drawn in float32 and, for bf16 cases, rounded to
bfloat16 (round to nearest even) before anything else sees them; the bf16
data are handed over as uint16 bit patterns.  Distributions:

* ``normal``       N(0, 1);
* ``lognormal``    N(0, 1) * 2**u with one u ~ N(0, (8/3)**2) clipped to
                   [-8, 8] per (token, 32-element block), so that block
                   scales span 2**-8 .. 2**8;
* ``student_t3``   Student-t with 3 degrees of freedom (heavy tails).

Weights are U(0, 1) (times ``w_scale``).
"""

import numpy as np

PAGE_SIZE = 64
HEAD_DIM = 128
CANARY = 0xA5


def _streams(seed):
    names = ("lengths", "k", "q", "w", "pages", "samples")
    kids = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.default_rng(s) for n, s in zip(names, kids)}


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def draw_values(rng, shape, dist):
    """float32 draws of the named distribution (see module docstring)."""
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "student_t3":
        return rng.standard_t(3, size=shape).astype(np.float32)
    if dist == "lognormal":
        x = rng.standard_normal(shape, dtype=np.float32)
        lead = shape[:-1] + (shape[-1] // 32, 1)
        u = np.clip(rng.normal(0.0, 8.0 / 3.0, size=lead), -8.0, 8.0)
        return (x.reshape(lead[:-1] + (32,)) * np.exp2(u).astype(np.float32)).reshape(shape)
    raise ValueError(dist)


def _values(rng, shape, dist, dtype):
    x = draw_values(rng, shape, dist)
    return bf16_bits(x) if dtype == "bf16" else x


def allocate_pages(rng, seq_lens, spare_pages, page_size=PAGE_SIZE, min_cols=1):
    """Fragmented page allocation.

    Physical page ids are a random permutation of all pages; sequence b takes
    the next ceil(L_b / P) ids of it.  ``spare_pages`` ids are never used (they
    stay canary-filled).  The table has at least ``min_cols`` columns; unused
    entries point at page 0 (always a valid page), never past the cache.
    Returns (block_table int32 [B, max_pages], slot_mapping int64 [sum L],
    num_pages).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = (seq_lens + page_size - 1) // page_size
    num_pages = int(need.sum()) + int(spare_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(min_cols, int(need.max()) if len(need) else 1)
    bt = np.zeros((len(seq_lens), max_pages), dtype=np.int32)
    slots = []
    pos = 0
    for b, (L, n) in enumerate(zip(seq_lens, need)):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
        j = np.arange(L, dtype=np.int64)
        slots.append(bt[b, j // page_size].astype(np.int64) * page_size + j % page_size)
    slot_mapping = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return bt, slot_mapping, num_pages


def decode_case(seed, seq_lens=None, H=32, next_n=1, dtype="bf16", k_dist="normal",
                q_dist="normal", w_scale=1.0, topk=2048, spare_pages=2, width=None,
                batch=None, len_range=None, name="decode"):
    """Paged decode: every sequence's K is inserted, the last next_n tokens query.

    Either ``seq_lens`` (explicit) or ``batch`` + ``len_range`` (uniform
    integer lengths in [lo, hi]) gives the context lengths.
    """
    st = _streams(seed)
    if seq_lens is None:
        lo, hi = len_range
        seq_lens = st["lengths"].integers(lo, hi + 1, size=batch)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    N = int(seq_lens.sum())
    k = _values(st["k"], (N, HEAD_DIM), k_dist, dtype)
    q = _values(st["q"], (B * next_n, H, HEAD_DIM), q_dist, dtype)
    w = (st["w"].random((B * next_n, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    width = int(seq_lens.max()) if width is None else int(width)
    bt, slots, num_pages = allocate_pages(st["pages"], seq_lens, spare_pages,
                                          min_cols=-(-width // PAGE_SIZE))
    return dict(name=name, kind="decode", dtype=dtype, k=k, q=q, w=w,
                slot_mapping=slots, block_table=bt, context_lens=seq_lens,
                num_pages=num_pages, page_size=PAGE_SIZE, next_n=next_n, H=H,
                topk=topk, width=width, seed=seed)


def prefill_case(seed, T, S, H=32, dtype="bf16", k_dist="normal", q_dist="normal",
                 w_scale=1.0, topk=2048, spare_pages=2, ks=None, ke=None,
                 n_sample_rows=None, name="prefill"):
    """Prefill: one sequence of S cached tokens whose last T tokens are the query chunk.

    Default visibility is causal: query t sits at position S - T + t and sees
    columns [0, S - T + t + 1).  ``ks``/``ke`` override it.
    """
    st = _streams(seed)
    k = _values(st["k"], (S, HEAD_DIM), k_dist, dtype)
    q = _values(st["q"], (T, H, HEAD_DIM), q_dist, dtype)
    w = (st["w"].random((T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    bt, slots, num_pages = allocate_pages(st["pages"], [S], spare_pages)
    if ks is None:
        ks = np.zeros(T, dtype=np.int32)
    if ke is None:
        ke = (S - T + np.arange(T) + 1).astype(np.int32)
    sample_rows = None
    if n_sample_rows is not None and n_sample_rows < T:
        pick = st["samples"].choice(np.arange(1, T - 1), size=n_sample_rows - 2, replace=False)
        sample_rows = np.unique(np.concatenate([[0, T - 1], pick])).astype(np.int64)
    return dict(name=name, kind="prefill", dtype=dtype, k=k, q=q, w=w,
                slot_mapping=slots, block_table=bt, seq_lens=np.array([S], np.int32),
                cu_seq_offsets=np.array([0], np.int64), num_pages=num_pages,
                page_size=PAGE_SIZE, T=T, S=S, H=H, ks=np.asarray(ks, np.int32),
                ke=np.asarray(ke, np.int32), topk=topk, width=S, seed=seed,
                sample_rows=sample_rows, new_token_start=S - T)


# ---------------------------------------------------------------------------
# The five named workloads.  Seeds 0..4.
# ---------------------------------------------------------------------------

def tiny(seed=0):
    """256 fp32 tokens (4 pages + 2 canary pages), 4 queries x 32 heads at positions 252..255, top-64."""
    c = decode_case(seed, seq_lens=[256], H=32, next_n=4, dtype="f32", w_scale=1.0 / 32,
                    topk=64, spare_pages=2, name="tiny")
    return c


def tiny_prefill(seed=0):
    """The tiny workload in prefill form: T=4 queries over S=256 contiguous tokens."""
    return prefill_case(seed, T=4, S=256, H=32, dtype="f32", w_scale=1.0 / 32, topk=64,
                        spare_pages=2, name="tiny_prefill")


def paged_decode(seed=1):
    """Batch 16, 8192-token contexts, 32 heads, next_n 1, top-2048, permuted pages."""
    return decode_case(seed, seq_lens=[8192] * 16, H=32, next_n=1, topk=2048,
                       spare_pages=0, name="paged_decode_16x8192")


def long_decode(seed=2):
    """Batch 64, contexts U[32768, 131072], lognormal block scales, width 131072."""
    return decode_case(seed, batch=64, len_range=(32768, 131072), H=32, next_n=1,
                       k_dist="lognormal", topk=2048, spare_pages=64, width=131072,
                       name="long_decode_64xU32K-128K")


def prefill_chunk(seed=3):
    """8192 new tokens, causal ks=0 / ke=t+1, 32 heads, top-2048."""
    return prefill_case(seed, T=8192, S=8192, H=32, topk=2048, spare_pages=0,
                        name="prefill_chunk_8192")


def long_prefill(seed=4):
    """16384 queries over 122880 cached tokens (chunk = last 16384), 64 heads, Student-t."""
    return prefill_case(seed, T=16384, S=122880, H=64, k_dist="student_t3",
                        q_dist="student_t3", topk=2048, spare_pages=0,
                        n_sample_rows=256, name="long_prefill_16384x122880")


def rope_tables(n_rows, rope_dim, base=10000.0):
    """RoPE angle tables, an input of the RoPE calls: cos / sin of
    pos * base**(-2j/rope_dim) for pos < n_rows, j < rope_dim/2, rounded to fp32."""
    half = rope_dim // 2
    j = np.arange(half)
    inv = base ** (-2.0 * j / max(rope_dim, 1))
    ang = np.arange(n_rows)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
