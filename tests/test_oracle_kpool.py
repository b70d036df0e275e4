"""Pins for the oracle's pooled (kpool) insert (CPU only): the bookkeeping P3
"_kpool_compress_insert" prints (write mask, pool gather, n < kpool), and the
softmax pooling reading (closed forms: equal scores give the mean, a dominant
score selects its token, per-dimension shifts cancel; a plain-loop brute force)."""

import math

import numpy as np
import pytest

from oracle import fp8 as ofp8, kpool, mxfp4, paged_cache


def test_write_mask_hand_worked():
    # kpool 4, n 10: pool ends at 3 and 7 carry slots; position 9 carries one too
    # (the mask takes it, as printed); position 1's slot is dropped (1 < kpool - 1)
    slots = [-1, 5, -1, 7, -1, -1, -1, 12, -1, 30]
    assert kpool.write_mask(slots, 4).tolist() == [False, False, False, True, False, False, False,
                                                   True, False, True]
    assert not kpool.write_mask([3, 4, 5], 4).any()          # n < kpool: nothing completes
    assert kpool.write_mask([9], 1).tolist() == [True]       # kpool 1: every slotted token


def test_pool_indices_hand_worked():
    idx = kpool.pool_indices(7, 4)
    assert idx[5].tolist() == [2, 3, 4, 5]
    assert idx[3].tolist() == [0, 1, 2, 3]
    assert idx[1].tolist() == [0, 1, 2, 3]                   # clamped (never written)


def _brute(k, gate, ape, kp):
    """Plain loops with math.exp."""
    n = len(k)
    out = np.zeros((n, 128))
    for i in range(n):
        toks = [max(i - kp + 1, 0) + j for j in range(kp)]
        for d in range(128):
            z = [float(gate[t, d]) + float(ape[j, d]) for j, t in enumerate(toks)]
            m = max(z)
            e = [math.exp(v - m) for v in z]
            s = sum(e)
            out[i, d] = sum(e[j] / s * float(k[t, d]) for j, t in enumerate(toks))
    return out


@pytest.mark.parametrize("kp", [1, 2, 4, 7])
def test_pooling_against_plain_loops(kp):
    rng = np.random.default_rng(kp)
    n = 12
    k = rng.standard_normal((n, 128)).astype(np.float32)
    gate = rng.standard_normal((n, 128)).astype(np.float32)
    ape = rng.standard_normal((kp, 128)).astype(np.float32)
    got = kpool.pooled_rows(k, gate, ape, kp)
    want = _brute(k, gate, ape, kp)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-14)


def test_pooling_closed_forms():
    rng = np.random.default_rng(9)
    n, kp = 9, 3
    k = rng.standard_normal((n, 128)).astype(np.float32)
    zero_g = np.zeros((n, 128), np.float32)
    zero_a = np.zeros((kp, 128), np.float32)
    got = kpool.pooled_rows(k, zero_g, zero_a, kp)
    for i in range(kp - 1, n):
        assert np.allclose(got[i], k[i - kp + 1:i + 1].astype(np.float64).mean(axis=0), rtol=0, atol=1e-15)
    # a dominant score selects its token (per dimension)
    g = zero_g.copy()
    g[4, :64] = 1000.0
    got = kpool.pooled_rows(k, g, zero_a, kp)
    assert np.array_equal(got[5, :64], k[4, :64].astype(np.float64))     # pool of 5 = tokens 3..5
    assert np.array_equal(got[6, :64], k[4, :64].astype(np.float64))     # pool of 6 = tokens 4..6
    # a shift of a dimension's scores by a constant cancels in the softmax
    a2 = rng.standard_normal((kp, 128)).astype(np.float32)
    shift = np.float32(3.0)
    base = kpool.pooled_rows(k, zero_g, a2, kp)
    moved = kpool.pooled_rows(k, zero_g + shift, a2, kp)
    assert np.allclose(base, moved, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("fmt", ["mxfp4", "fp8"])
def test_insert_writes_only_masked_pools(fmt):
    rng = np.random.default_rng(10)
    n, kp = 20, 4
    k = rng.standard_normal((n, 128)).astype(np.float32)
    gate = rng.standard_normal((n, 128)).astype(np.float32)
    ape = rng.standard_normal((kp, 128)).astype(np.float32)
    slots = np.full(n, -1, np.int64)
    slots[[3, 7, 11, 15, 19]] = [64 + 0, 64 + 1, 2, 64 + 3, 3 * 64 + 9]     # the last is out of range
    slots[1] = 5                                                            # dropped: 1 < kpool - 1
    row = 68 if fmt == "mxfp4" else 132
    cache0 = np.full((3, 64 * row), 0xA5, np.uint8)
    out, mask, pooled = kpool.insert(cache0, k, gate, ape, slots, kp, fmt)
    assert mask.tolist() == [i in (3, 7, 11, 15, 19) for i in range(n)]
    p32 = pooled.astype(np.float32).astype(np.float64)
    if fmt == "mxfp4":
        codes, scales = mxfp4.quantize_rows(p32)
        for i, sl in zip((3, 7, 11, 15), (64, 65, 2, 67)):
            c, s = paged_cache.read_token(out, sl // 64, sl % 64)
            assert np.array_equal(c, codes[i]) and np.array_equal(s, scales[i])
    else:
        codes, scales = ofp8.quantize_rows(p32)
        flat = out.reshape(-1)
        for i, sl in zip((3, 7, 11, 15), (64, 65, 2, 67)):
            v0 = ofp8.value_offset(sl // 64, sl % 64)
            assert np.array_equal(flat[v0:v0 + 128], codes[i])
    # untouched elsewhere: at most the 4 written rows' bytes changed (slot 5 and the
    # out-of-range slot wrote nothing)
    diff_bytes = int(np.sum(out != cache0))
    assert 0 < diff_bytes <= 4 * row
