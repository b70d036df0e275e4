"""Pins for the oracle's indexer logits (CPU only).

The oracle's float64 matrix products are checked against exact rational
arithmetic (fractions.Fraction) written as plain loops, against closed forms
(H = 1, one-hot weights), and against invariants the definition implies
(2**m scaling of a K row, block-table permutation, paged == dense).
"""

from fractions import Fraction

import numpy as np

from oracle import logits, mxfp4, paged_cache


def _quant(rng, shape, scale_spread=0):
    x = rng.standard_normal(shape)
    if scale_spread:
        blk = x.reshape(-1, 4, 32)
        blk *= np.exp2(rng.integers(-scale_spread, scale_spread + 1, size=blk.shape[:2] + (1,)))
        x = blk.reshape(shape)
    c, s = mxfp4.quantize_rows(x)
    return c.reshape(shape[:-1] + (64,)), s.reshape(shape[:-1] + (4,))


def _frac_row(codes, scales):
    """Exact Fraction values of one MXFP4 row, from the bit fields (no numpy math)."""
    out = []
    for i in range(128):
        byte = int(codes[i // 2])
        nib = (byte >> 4) if i % 2 else (byte & 0xF)
        mag = Fraction(mxfp4.e2m1_value(nib & 7))
        e = int(scales[i // 32]) - 127
        val = mag * (Fraction(2) ** e)
        out.append(-val if nib & 8 else val)
    return out


def test_dense_logits_match_exact_rationals():
    rng = np.random.default_rng(0)
    T, H, S = 3, 4, 6
    qc, qs = _quant(rng, (T, H, 128), scale_spread=6)
    kc, kscale = _quant(rng, (S, 128), scale_spread=6)
    w = rng.uniform(-1, 1, size=(T, H)).astype(np.float32)
    ks = np.array([0, 1, 2])
    ke = np.array([6, 4, 3])
    got = logits.mqa_logits(qc, qs, kc, kscale, w, ks, ke)
    kf = [_frac_row(kc[s], kscale[s]) for s in range(S)]
    for t in range(T):
        qf = [_frac_row(qc[t, h], qs[t, h]) for h in range(H)]
        for s in range(S):
            if not (ks[t] <= s < ke[t]):
                assert got[t, s] == -np.inf
                continue
            exact = Fraction(0)
            for h in range(H):
                d = sum(a * b for a, b in zip(qf[h], kf[s]))
                if d > 0:
                    exact += Fraction(float(w[t, h])) * d
            assert abs(Fraction(got[t, s]) - exact) <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_single_head_unit_weight_is_relu_of_dot():
    rng = np.random.default_rng(1)
    qc, qs = _quant(rng, (5, 1, 128))
    kc, kscale = _quant(rng, (7, 128))
    w = np.ones((5, 1), np.float32)
    got = logits.mqa_logits(qc, qs, kc, kscale, w, np.zeros(5, int), np.full(5, 7))
    qh = mxfp4.dequantize_rows(qc.reshape(5, 64), qs.reshape(5, 4))
    kh = mxfp4.dequantize_rows(kc, kscale)
    for t in range(5):
        for s in range(7):
            assert got[t, s] == max(0.0, float(np.dot(qh[t], kh[s])))
    assert np.any(got == 0.0) and np.any(got > 0.0)     # both branches of the ReLU exercised


def test_one_hot_weight_selects_a_head():
    rng = np.random.default_rng(2)
    H = 8
    qc, qs = _quant(rng, (2, H, 128))
    kc, kscale = _quant(rng, (9, 128))
    for h in (0, 5):
        w = np.zeros((2, H), np.float32)
        w[:, h] = 1.0
        got = logits.mqa_logits(qc, qs, kc, kscale, w, np.zeros(2, int), np.full(2, 9))
        single = logits.mqa_logits(qc[:, h:h + 1], qs[:, h:h + 1], kc, kscale, w[:, h:h + 1],
                                   np.zeros(2, int), np.full(2, 9))
        assert np.array_equal(got, single)


def test_hand_worked_logit():
    e0 = np.zeros(128)
    e0[0] = 1.0
    qc, qs = mxfp4.quantize_rows(e0)
    assert qs[0, 0] == 127 - 2 and (qc[0, 0] & 0xF) == 6      # 1.0 = 4 * 2**-2
    w = np.array([[0.5]], np.float32)
    got = logits.mqa_logits(qc.reshape(1, 1, 64), qs.reshape(1, 1, 4), qc, qs, w, [0], [1])
    assert got[0, 0] == 0.5
    kc, ks_ = mxfp4.quantize_rows(-e0)
    got = logits.mqa_logits(qc.reshape(1, 1, 64), qs.reshape(1, 1, 4), kc, ks_, w, [0], [1])
    assert got[0, 0] == 0.0


def test_power_of_two_scaling_of_a_k_row():
    rng = np.random.default_rng(4)
    T, H, S = 3, 16, 10
    x = rng.standard_normal((S, 128))
    q = rng.standard_normal((T, H, 128))
    qc, qs = mxfp4.quantize_rows(q)
    qc, qs = qc.reshape(T, H, 64), qs.reshape(T, H, 4)
    w = rng.random((T, H)).astype(np.float32)
    base = logits.mqa_logits(qc, qs, *mxfp4.quantize_rows(x), w, np.zeros(T, int), np.full(T, S))
    for m in (-7, 3, 9):
        x2 = x.copy()
        x2[4] *= 2.0 ** m
        kc2, ks2 = mxfp4.quantize_rows(x2)
        got = logits.mqa_logits(qc, qs, kc2, ks2, w, np.zeros(T, int), np.full(T, S))
        assert np.array_equal(got[:, 4], base[:, 4] * 2.0 ** m)
        others = np.arange(S) != 4
        assert np.array_equal(got[:, others], base[:, others])


def _paged_setup(rng, lens, H, next_n, perm_seed):
    P = 64
    need = [(L + P - 1) // P for L in lens]
    num_pages = sum(need) + 1
    perm = np.random.default_rng(perm_seed).permutation(num_pages)
    bt = np.zeros((len(lens), max(need)), np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    k = rng.standard_normal((sum(lens), 128))
    slots = np.concatenate([bt[b, np.arange(L) // P] * P + np.arange(L) % P for b, L in enumerate(lens)])
    cache = paged_cache.insert(np.zeros((num_pages, P * 68), np.uint8), k, slots)
    return cache, bt, k


def test_paged_equals_dense_and_ignores_page_order():
    lens = [100, 64, 130]
    H, next_n = 16, 2
    rng = np.random.default_rng(5)
    q = rng.standard_normal((len(lens) * next_n, H, 128))
    qc, qs = mxfp4.quantize_rows(q)
    qc, qs = qc.reshape(-1, H, 64), qs.reshape(-1, H, 4)
    w = rng.random((len(lens) * next_n, H)).astype(np.float32)
    outs = []
    for perm_seed in (10, 11):
        cache, bt, k = _paged_setup(np.random.default_rng(6), lens, H, next_n, perm_seed)
        outs.append(logits.paged_mqa_logits(qc, qs, w, cache, bt, lens, next_n, width=140))
    assert np.array_equal(outs[0], outs[1])
    kc, kscale = mxfp4.quantize_rows(k)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for b, L in enumerate(lens):
        rows = np.arange(b * next_n, (b + 1) * next_n)
        ke = np.array([L - next_n + i + 1 for i in range(next_n)])
        dense = logits.mqa_logits(qc[rows], qs[rows], kc[cu[b]:cu[b + 1]], kscale[cu[b]:cu[b + 1]],
                                  w[rows], np.zeros(next_n, int), ke, width=140)
        assert np.array_equal(outs[0][rows], dense)
        for i in range(next_n):
            assert np.all(np.isneginf(outs[0][rows[i], ke[i]:]))
            assert np.all(np.isfinite(outs[0][rows[i], :ke[i]]))


def test_abs_bound_dominates_and_equals_logit_for_positive_dots():
    rng = np.random.default_rng(8)
    qc, qs = _quant(rng, (2, 4, 128))
    kc, kscale = _quant(rng, (5, 128))
    w = rng.random((2, 4)).astype(np.float32)
    full = logits.mqa_logits(qc, qs, kc, kscale, w, np.zeros(2, int), np.full(2, 5))
    rows = np.repeat(np.arange(2), 5)
    cols = np.tile(np.arange(5), 2)
    A = logits.abs_bound(qc, qs, kc, kscale, w, rows, cols)
    assert np.all(A >= np.abs(full[rows, cols]) - 1e-12)
