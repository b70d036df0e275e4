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


def test_shard_layout_hand_worked():
    # world 2, interleave 3: global 0,1,2 -> rank 0 local 0,1,2; 3,4,5 -> rank 1 local 0,1,2;
    # 6,7,8 -> rank 0 local 3,4,5
    assert topk.shard_to_global([0, 2, 3, 5], 0, 2, 3).tolist() == [0, 2, 6, 8]
    assert topk.shard_to_global([0, 2, 3], 1, 2, 3).tolist() == [3, 5, 9]
    rank, local = topk.global_to_shard(np.arange(12), 2, 3)
    assert rank.tolist() == [0, 0, 0, 1, 1, 1, 0, 0, 0, 1, 1, 1]
    assert local.tolist() == [0, 1, 2, 0, 1, 2, 3, 4, 5, 3, 4, 5]


@pytest.mark.parametrize("world,inter", [(1, 1), (2, 1), (4, 64), (3, 5), (8, 7)])
def test_shard_layout_is_a_bijection(world, inter):
    n = world * inter * 13 + 5
    rank, local = topk.global_to_shard(np.arange(n), world, inter)
    back = np.array([topk.shard_to_global(l, r, world, inter) for r, l in zip(rank, local)])
    assert back.tolist() == list(range(n))


def _brute_merge(values, indices, world_interleave, k):
    R, rows, kin = values.shape
    res = []
    for r in range(rows):
        cand = []
        for s in range(R):
            for j in range(kin):
                li = int(indices[s, r, j])
                if li < 0:
                    continue
                run, off = divmod(li, world_interleave)
                g = (run * R + s) * world_interleave + off
                cand.append((-float(values[s, r, j]), g))
        cand.sort()
        row = [g for _, g in cand[:k]]
        res.append(row + [-1] * (k - len(row)))
    return res


@pytest.mark.parametrize("seed", range(12))
def test_merge_brute_force_with_ties_and_empty_slots(seed):
    rng = np.random.default_rng(100 + seed)
    R, rows, kin = int(rng.integers(1, 5)), 3, int(rng.integers(1, 12))
    inter = int(rng.integers(1, 6))
    vals = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0], np.float32), size=(R, rows, kin))
    idx = np.stack([np.stack([rng.permutation(40)[:kin] for _ in range(rows)]) for _ in range(R)])
    idx[rng.random(idx.shape) < 0.2] = -1
    k = int(rng.integers(1, R * kin + 3))
    got = topk.merge_shard_topk(vals, idx, inter, k)
    assert got.tolist() == _brute_merge(vals, idx, inter, k)


@pytest.mark.parametrize("world,inter,n,k", [(2, 64, 1000, 64), (4, 1, 777, 100), (8, 16, 5000, 256),
                                             (3, 5, 100, 150)])
def test_merge_of_shard_topk_equals_unsharded_topk(world, inter, n, k):
    # each rank selects over its own positions; the merged lists give exactly
    # the top-k of the whole row (ties included: the values carry many repeats)
    rng = np.random.default_rng(world * 1000 + n)
    rows = 4
    x = np.round(rng.standard_normal((rows, n)) * 4).astype(np.float32) / 4
    full = topk.top_k_per_row(x, np.zeros(rows, int), np.full(rows, n), k)
    rank, local = topk.global_to_shard(np.arange(n), world, inter)
    vals = np.zeros((world, rows, k), np.float32)
    idx = np.full((world, rows, k), -1, np.int32)
    for s in range(world):
        pos = np.nonzero(rank == s)[0]                        # global positions of rank s, by local order
        shard = x[:, pos]
        sel = topk.top_k_per_row(shard, np.zeros(rows, int), np.full(rows, len(pos)), k)
        for r in range(rows):
            m = sel[r] >= 0
            idx[s, r, :m.sum()] = local[pos[sel[r][m]]]
            vals[s, r, :m.sum()] = shard[r, sel[r][m]]
    merged = topk.merge_shard_topk(vals, idx, inter, k)
    assert merged.tolist() == full.tolist()
