"""Pins for the oracle's per-row top-k (CPU only): hand-worked rows and a
brute-force ranking written as a plain Python sort."""

import numpy as np
import pytest

from oracle import topk


def test_hand_worked_rows():
    row = np.array([[0.5, 2.0, 2.0, -np.inf, 1.0]], np.float32)
    assert set(topk.top_k_per_row(row, [0], [5], 2)[0].tolist()) == {1, 2}
    assert set(topk.top_k_per_row(row, [0], [5], 4)[0].tolist()) == {1, 2, 4, 0}
    out = topk.top_k_per_row(row, [0], [2], 3)[0].tolist()
    assert set(out[:2]) == {1, 0} and out[2] == -1


def _brute(row, a, b, k):
    cand = list(range(a, b))
    cand.sort(key=lambda c: (-float(row[c]), c))
    res = cand[:k]
    return res + [-1] * (k - len(res))


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_with_planted_ties(seed):
    rng = np.random.default_rng(seed)
    R, W = 6, int(rng.integers(1, 300))
    x = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0, 3.0], np.float32), size=(R, W))
    x += (rng.random((R, W)) < 0.5) * rng.standard_normal((R, W)).astype(np.float32)
    ks = rng.integers(0, W, size=R)
    ke = np.minimum(W, ks + rng.integers(0, W + 1, size=R))
    k = int(rng.integers(1, 80))
    got = topk.top_k_per_row(x, ks, ke, k)
    for r in range(R):
        assert got[r].tolist() == _brute(x[r], int(ks[r]), int(ke[r]), k)


def test_negative_zero_ties_with_positive_zero():
    row = np.array([[-0.0, 0.0, -0.0, -1.0]], np.float32)
    assert topk.top_k_per_row(row, [0], [4], 2)[0].tolist() == [0, 1]
