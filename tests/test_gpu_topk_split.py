"""GPU parity of the workspace top-k (idx_topk_ws): few long rows split over
workgroups must give the oracle's exact sets -- on random rows with ragged and
unaligned ranges, ties at the threshold, rows whose parts differ (the merge
falls back to the whole-row path), constant rows (a part keeps more pairs than
its region holds), mixes of split and unsplit rows, repeated calls of
different sizes sharing one uninitialized workspace, and graph replays."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
from oracle import topk as otk
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

PART = 8192           # columns per workgroup of a split row


def _check_sets(got, x, ks, ke, k, what=""):
    ref = otk.top_k_per_row(x, ks, ke, k)
    for r in range(x.shape[0]):
        n = max(0, min(int(ke[r]), x.shape[1]) - int(ks[r]))
        m = min(k, n)
        assert np.all(got[r, m:] == -1), (what, r)
        assert sorted(got[r, :m].tolist()) == sorted(ref[r, :m].tolist()), (what, r)


def _run(x, ks, ke, k, ws=None):
    if ws is None:
        ws = mx.topk_workspace(x.shape[0], x.shape[1])
    out = mx.topk_ws(dev(x), dev(ks), dev(ke), k, ws)
    torch.cuda.synchronize()
    return host(out)


def _ragged(rng, rows, n):
    """Visible ranges: mostly long (several parts), some of one part or less,
    one of at most k keys, one empty, some starting at an unaligned column."""
    ks = np.zeros(rows, np.int32)
    ke = rng.integers(PART + 1, n + 1, rows).astype(np.int32)
    ke[0] = n
    ke[1] = PART                                   # exactly one part
    ke[2] = PART + 1                               # a second part of one key
    if rows > 4:
        ke[3] = 2000                               # fewer than k keys
        ks[4], ke[4] = 77, 77                      # empty
    ks[5::3] = rng.integers(1, 4000, len(ks[5::3]))  # unaligned starts
    return ks, np.maximum(ke, ks)


@pytest.mark.parametrize("rows,n,k", [(8, 40000, 2048), (64, 131072, 2048), (6, 3 * PART, 300),
                                      (300, 20000, 2048), (5, 64 * PART, 2048), (7, 70000, 1)])
def test_split_random_rows(rows, n, k):
    rng = np.random.default_rng(rows * 13 + n + k)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    ks, ke = _ragged(rng, rows, n)
    _check_sets(_run(x, ks, ke, k), x, ks, ke, k, "random")


def test_split_ties_and_signed_zeros():
    rng = np.random.default_rng(5)
    rows, n, k = 6, 90000, 2048
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[0] = np.round(x[0] * 4) / 4                 # a few hundred distinct values
    x[1] = np.round(x[1])                         # the threshold value is shared by thousands
    x[2, ::3] = 0.0
    x[2, 1::3] = -0.0                             # +0 / -0 ties across parts
    x[3] = np.abs(x[3])
    ks = np.zeros(rows, np.int32)
    ke = np.full(rows, n, np.int32)
    ks[4] = 1
    ke[5] = n - 3
    _check_sets(_run(x, ks, ke, k), x, ks, ke, k, "ties")


def test_split_unlike_parts_fall_back_to_the_whole_row():
    # increasing rows keep their top keys in the last part, decreasing ones in
    # the first: fewer than k kept keys reach the highest part threshold, and
    # the merge selects over the whole row; constant rows keep every key of a
    # part (more than its region holds)
    rng = np.random.default_rng(6)
    rows, n, k = 6, 100000, 2048
    ramp = np.linspace(0.0, 60.0, n, dtype=np.float32)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[0] += ramp
    x[1] -= ramp
    x[2] = 1.5
    x[3, : n // 2] = -2.0
    x[4] = np.where(np.arange(n) % 5000 < 30, 100.0, 0.0).astype(np.float32)
    ks = np.zeros(rows, np.int32)
    ke = np.full(rows, n, np.int32)
    ks[5] = 12345
    _check_sets(_run(x, ks, ke, k), x, ks, ke, k, "fallback")


def test_split_matches_the_unsplit_top_k():
    rng = np.random.default_rng(7)
    rows, n, k = 16, 131072, 2048
    x = (rng.standard_normal((rows, n)) * np.exp(rng.standard_normal((rows, 1)))).astype(np.float32)
    ks = np.zeros(rows, np.int32)
    ke = rng.integers(32768, n + 1, rows).astype(np.int32)
    got = _run(x, ks, ke, k)
    plain = host(mx.topk(dev(x), dev(ks), dev(ke), k))
    for r in range(rows):
        assert sorted(got[r].tolist()) == sorted(plain[r].tolist()), r


def test_split_workspace_reused_by_calls_of_different_sizes():
    rng = np.random.default_rng(8)
    big = torch.full((mx.topk_workspace_bytes(100, 70000),), 0x5A, dtype=torch.uint8, device="cuda")
    for rows, n, k in [(100, 70000, 2048), (3, 40000, 512), (100, 70000, 2048), (9, 17000, 2048),
                       (64, 50000, 1000)]:
        assert mx.topk_workspace_bytes(rows, n) <= big.numel()
        x = rng.standard_normal((rows, n)).astype(np.float32)
        ks, ke = _ragged(rng, rows, n)
        _check_sets(_run(x, ks, ke, k, ws=big), x, ks, ke, k, f"reuse {rows}x{n}")


def test_split_graph_replays_equal_eager():
    rng = np.random.default_rng(9)
    rows, n, k = 12, 60000, 2048
    x = torch.empty((rows, n), dtype=torch.float32, device="cuda")
    ks_np = np.zeros(rows, np.int32)
    ke_np = rng.integers(20000, n + 1, rows).astype(np.int32)
    ks, ke = dev(ks_np), dev(ke_np)
    ws = mx.topk_workspace(rows, n)
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    x.copy_(dev(rng.standard_normal((rows, n)).astype(np.float32)))
    mx.topk_ws(x, ks, ke, k, ws, out=out)              # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mx.topk_ws(x, ks, ke, k, ws, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        data = rng.standard_normal((rows, n)).astype(np.float32)
        if rep == 2:
            data[1] += np.linspace(0, 40, n, dtype=np.float32)   # a replay on the fallback path
        x.copy_(dev(data))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(out)
        eager = host(mx.topk_ws(x, ks, ke, k, ws))
        for r in range(rows):
            assert sorted(got[r].tolist()) == sorted(eager[r].tolist()), (rep, r)
        _check_sets(got, data, ks_np, ke_np, k, f"replay {rep}")
