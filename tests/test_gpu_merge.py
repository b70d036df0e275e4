"""GPU parity: merge of per-rank top-k lists (context-parallel decode) against
the oracle, and against the unsharded top-k of the whole row."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
from oracle import topk as otk
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _same_sets(got, ref):
    for r in range(ref.shape[0]):
        m = int((ref[r] >= 0).sum())
        assert np.all(got[r, m:] == -1), r
        assert sorted(got[r, :m].tolist()) == sorted(ref[r, :m].tolist()), r


def _shard_lists(x, world, inter, k_in, k_rank):
    """Each rank's exact top-k_rank over its own positions, as the merge's input."""
    rows, n = x.shape
    rank, local = otk.global_to_shard(np.arange(n), world, inter)
    vals = np.zeros((world, rows, k_in), np.float32)
    idx = np.full((world, rows, k_in), -1, np.int32)
    for s in range(world):
        pos = np.nonzero(rank == s)[0]
        shard = x[:, pos]
        sel = otk.top_k_per_row(shard, np.zeros(rows, int), np.full(rows, len(pos)), k_rank)
        for r in range(rows):
            m = sel[r] >= 0
            idx[s, r, :m.sum()] = local[pos[sel[r][m]]]
            vals[s, r, :m.sum()] = shard[r, sel[r][m]]
    return vals, idx


@pytest.mark.parametrize("world,inter,n,k", [(4, 64, 131072, 2048), (2, 1, 30000, 2048), (8, 16, 9000, 1024),
                                             (3, 5, 700, 150), (1, 64, 5000, 300)])
def test_merge_equals_unsharded_topk(world, inter, n, k):
    rng = np.random.default_rng(world * 7 + n)
    rows = 5
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[1] = np.round(x[1] * 4) / 4                       # heavy ties across ranks
    x[2, ::3] = 0.0
    x[2, 1::3] = -0.0
    vals, idx = _shard_lists(x, world, inter, k, k)
    got = host(mx.topk_merge(dev(vals), dev(idx), inter, k))
    full = otk.top_k_per_row(x, np.zeros(rows, int), np.full(rows, n), k)
    _same_sets(got, full)
    _same_sets(got, otk.merge_shard_topk(vals, idx, inter, k))


@pytest.mark.parametrize("seed", range(6))
def test_merge_random_lists_with_empty_slots(seed):
    rng = np.random.default_rng(300 + seed)
    world, rows, k_in = int(rng.integers(1, 5)), 7, int(rng.integers(1, 2049))
    world = min(world, 8192 // k_in)
    inter = int(rng.integers(1, 100))
    vals = rng.choice(np.array([-3.0, -0.0, 0.0, 0.5, 1.0, 7.0], np.float32), size=(world, rows, k_in))
    vals += (rng.random(vals.shape) < 0.5) * rng.standard_normal(vals.shape).astype(np.float32)
    idx = np.stack([np.stack([rng.permutation(3 * k_in)[:k_in] for _ in range(rows)]) for _ in range(world)])
    idx = idx.astype(np.int32)
    idx[rng.random(idx.shape) < 0.3] = -1
    idx[:, 3] = -1                                       # a row with no candidates
    k = int(rng.integers(1, 2049))
    got = host(mx.topk_merge(dev(vals), dev(idx), inter, k))
    _same_sets(got, otk.merge_shard_topk(vals, idx, inter, k))


def test_merge_all_equal_values_take_lowest_global_positions():
    world, rows, k_in, inter, k = 4, 3, 2048, 8, 2048
    vals = np.ones((world, rows, k_in), np.float32)
    idx = np.tile(np.arange(k_in, dtype=np.int32), (world, rows, 1))
    got = host(mx.topk_merge(dev(vals), dev(idx), inter, k))
    for r in range(rows):
        assert sorted(got[r].tolist()) == list(range(k))


def test_merge_fewer_valid_than_k():
    world, rows, k_in, inter = 2, 2, 10, 3
    rng = np.random.default_rng(9)
    vals = rng.standard_normal((world, rows, k_in)).astype(np.float32)
    idx = np.tile(np.arange(k_in, dtype=np.int32), (world, rows, 1))
    idx[:, :, 6:] = -1
    got = host(mx.topk_merge(dev(vals), dev(idx), inter, 50))
    _same_sets(got, otk.merge_shard_topk(vals, idx, inter, 50))
    assert np.all(got[:, 12:] == -1)
