"""GPU parity: per-row top-k sets equal the oracle's on identical float32 input."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
from oracle import topk as otk
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


def _check(x, ks, ke, k, use_ks=True):
    out = mx.topk(dev(x), dev(ks) if use_ks else None, dev(ke), k)
    torch.cuda.synchronize()
    got = host(out)
    ref = otk.top_k_per_row(x, ks if use_ks else np.zeros(len(ke), np.int32), ke, k)
    for r in range(x.shape[0]):
        a = int(ks[r]) if use_ks else 0
        n = max(0, min(int(ke[r]), x.shape[1]) - a)
        m = min(k, n)
        assert np.all(got[r, m:] == -1), r
        assert sorted(got[r, :m].tolist()) == sorted(ref[r, :m].tolist()), r


@pytest.mark.parametrize("n,k", [(1, 1), (63, 64), (64, 64), (65, 64), (3000, 2048), (2049, 2048),
                                 (4096, 64), (4096, 2048), (8192, 2048), (16384, 2048),
                                 (16385, 2048), (40000, 2048),
                                 (131072, 2048), (5000, 1), (20000, 7)])
def test_topk_random_rows(n, k):
    rng = np.random.default_rng(n * 31 + k)
    R = 6
    x = rng.standard_normal((R, n)).astype(np.float32)
    x[0, : n // 3] = np.round(x[0, : n // 3] * 4) / 4         # many exact ties
    x[1, ::7] = 0.0
    x[1, 3::7] = -0.0                                          # +0 / -0 ties
    x[2] = np.abs(x[2])
    ks = np.zeros(R, np.int32)
    ke = np.full(R, n, np.int32)
    ks[3] = n // 5
    ke[4] = max(1, n - n // 7)
    ks[5], ke[5] = n // 3, n // 3                               # empty range
    _check(x, ks, ke, k)
    _check(x, ks, ke, k, use_ks=False)


@pytest.mark.parametrize("n", [4096, 8192, 16384])
def test_topk_full_rows_unaligned_start(n):
    # Rows that fill every slot of the workgroup (4096, 8192 and 16384 keys)
    # but start 4 bytes past a 16-byte boundary, so the keys arrive by scalar
    # loads; one row with many ties, one with +0/-0, one all equal.
    rng = np.random.default_rng(n + 3)
    R, k = 4, 2048
    buf = rng.standard_normal(R * n + 1).astype(np.float32)
    x = buf[1:].reshape(R, n)
    x[0] = np.round(x[0] * 8) / 8
    x[1, ::5] = 0.0
    x[1, 2::5] = -0.0
    x[2] = 0.25
    t = dev(buf)[1:].view(R, n)
    assert t.data_ptr() % 16 == 4
    ke = np.full(R, n, np.int32)
    out = host(mx.topk(t, None, dev(ke), k))
    ref = otk.top_k_per_row(x, np.zeros(R, np.int32), ke, k)
    for r in range(R):
        assert sorted(out[r].tolist()) == sorted(ref[r].tolist()), r


def test_topk_all_equal_and_heavy_ties_take_lowest_columns():
    n, k = 50000, 2048
    x = np.ones((3, n), np.float32)
    x[1, :10] = 2.0                                            # 10 winners, then 2038 lowest-index ties
    x[2] = np.float32(1.0) + (np.arange(n) % 3 == 0) * np.float32(2 ** -20)
    ks = np.zeros(3, np.int32)
    ke = np.full(3, n, np.int32)
    out = host(mx.topk(dev(x), dev(ks), dev(ke), k))
    assert sorted(out[0].tolist()) == list(range(k))
    assert sorted(out[1].tolist()) == list(range(k))
    ref = otk.top_k_per_row(x, ks, ke, k)
    for r in range(3):
        assert sorted(out[r].tolist()) == sorted(ref[r].tolist())


def test_topk_wide_threshold_bin_uses_memory_path():
    # > 8192 keys share the level-1 bin of the k-th value (values differ only in
    # low mantissa bits), so the candidate list cannot live in LDS.
    rng = np.random.default_rng(5)
    n, k = 60000, 2048
    base = np.float32(1.5)
    bits = base.view(np.uint32) + rng.integers(0, 1 << 20, size=n).astype(np.uint32)
    x = bits.view(np.float32).reshape(1, n).copy()
    x[0, rng.integers(0, n, 500)] = 3.0
    _check(x, np.zeros(1, np.int32), np.full(1, n, np.int32), k)


def test_topk_row_stride_and_ke_beyond_width():
    rng = np.random.default_rng(9)
    full = rng.standard_normal((4, 9000)).astype(np.float32)
    t = dev(full)[:, :7000]                                    # row stride 9000
    ke = np.array([7000, 6000, 9000, 100], np.int32)          # 9000 > width: clipped to the stride
    out = host(mx.topk(t, None, dev(ke), 300))
    ref = otk.top_k_per_row(full[:, :9000], np.zeros(4, np.int32), ke, 300)
    for r in range(4):
        assert sorted(out[r].tolist()) == sorted(ref[r].tolist())


def test_topk_deterministic_across_runs():
    rng = np.random.default_rng(3)
    x = dev(np.round(rng.standard_normal((8, 30000)).astype(np.float32) * 8) / 8)
    ke = dev(np.full(8, 30000, np.int32))
    a = host(mx.topk(x, None, ke, 2048))
    b = host(mx.topk(x, None, ke, 2048))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("rows,n,k", [(600, 3000, 2048), (520, 20000, 2048), (512, 9000, 100),
                                      # 16 keys per thread (outputs staged in LDS), odd k
                                      (512, 6000, 1), (512, 6000, 7), (512, 6000, 2047)])
def test_topk_many_rows(rows, n, k):
    # 512 or more rows select the many-rows launch shape (512-thread workgroups)
    rng = np.random.default_rng(rows + n)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    x[::3] = np.round(x[::3] * 8) / 8
    ks = rng.integers(0, n // 4, rows).astype(np.int32)
    ke = (n - rng.integers(0, n // 4, rows)).astype(np.int32)
    _check(x, ks, ke, k)


def test_topk_many_rows_wide_threshold_bin():
    rng = np.random.default_rng(6)
    rows, n, k = 512, 40000, 2048
    bits = np.float32(1.5).view(np.uint32) + rng.integers(0, 1 << 20, size=(rows, n)).astype(np.uint32)
    x = bits.view(np.float32).copy()
    _check(x, np.zeros(rows, np.int32), np.full(rows, n, np.int32), k)


@pytest.mark.parametrize("n,k,width", [(8192, 2048, 20), (3000, 700, 5), (16384, 2048, 64), (8192, 1, 3)])
def test_topk_ties_across_the_kth_value(n, k, width):
    # `width` equal values straddle rank k (a small threshold bin whose ties
    # are broken by column), in rows of distinct values otherwise
    rng = np.random.default_rng(n + k + width)
    R = 4
    x = rng.standard_normal((R, n)).astype(np.float32)
    for r in range(R):
        order = np.argsort(-x[r], kind="stable")
        lo_rank = max(0, k - 1 - width // 2)
        x[r, order[lo_rank:lo_rank + width]] = x[r, order[lo_rank]]
    ks = np.zeros(R, np.int32)
    ke = np.full(R, n, np.int32)
    ks[1] = 7
    ke[2] = n - 5
    _check(x, ks, ke, k)


def _trend_rows(rng, rows, n):
    """Rows whose first chunk misrepresents the row: increasing (the estimate from
    the first chunk keeps nearly every key, overflowing the pair buffer),
    decreasing (it keeps fewer than k), and random (the one-read path)."""
    base = rng.standard_normal((rows, n)).astype(np.float32)
    ramp = np.linspace(0.0, 50.0, n, dtype=np.float32)
    x = base.copy()
    x[0::3] += ramp
    x[1::3] -= ramp
    return x


@pytest.mark.parametrize("rows,n,k", [(6, 40000, 2048), (3, 131072, 2048), (512, 20000, 2048),
                                      (520, 9000, 300)])
def test_topk_long_rows_first_chunk_estimate_and_fallback(rows, n, k):
    rng = np.random.default_rng(rows * 7 + n)
    x = _trend_rows(rng, rows, n)
    ks = np.zeros(rows, np.int32)
    ke = np.full(rows, n, np.int32)
    ke[2::5] = n - n // 9
    ks[4::7] = n // 11
    _check(x, ks, ke, k)


def test_topk_long_rows_fallback_reaches_the_memory_path():
    # increasing values that share their top bits: the estimate fails (the pair
    # buffer overflows) and the two-pass path finds > 8192 keys in the threshold
    # bin of the top digit
    n, k = 60000, 2048
    bits = np.float32(1.5).view(np.uint32) + np.sort(
        np.random.default_rng(8).integers(0, 1 << 20, size=n)).astype(np.uint32)
    x = bits.view(np.float32).reshape(1, n).copy()
    _check(x, np.zeros(1, np.int32), np.full(1, n, np.int32), k)
