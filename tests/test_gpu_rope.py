"""GPU parity of the fused query RoPE + MXFP4 encode (idx_quantize_rope) against
the oracle (oracle/rope.py then oracle/mxfp4.py): code and scale bytes bit-exact,
for both pairings, bf16 and fp32 rows, partial and full rotated ranges, table rows
chosen by positions (out-of-range positions encode unrotated), and rope_dim 0
equal to idx_quantize."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import mxfp4 as omx, rope as orope
from tests.gpu_helpers import dev, host, rope_tables

pytestmark = pytest.mark.gpu


def _exact(q, dtype):
    return omx.bf16_bits_to_f64(q) if dtype == "bf16" else omx.f32_to_f64(q)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["neox", "interleaved"])
@pytest.mark.parametrize("rope_dim", [16, 64, 96, 128])
def test_rope_quantize_bit_exact(dtype, mode, rope_dim):
    rng = np.random.default_rng(rope_dim + (mode == "neox"))
    T, H = 300, 32
    x = workloads.draw_values(rng, (T, H, 128), "lognormal")
    q = workloads.bf16_bits(x) if dtype == "bf16" else x
    cos, sin = rope_tables(5000, rope_dim)
    pos = rng.integers(0, 5000, size=T).astype(np.int64)
    vals, scales = mx.quantize_rope(dev(q), dev(cos), dev(sin), rope_dim, mode, positions=dev(pos))
    torch.cuda.synchronize()
    wc, ws = orope.quantize_rope(_exact(q, dtype), cos, sin, rope_dim, mode, positions=pos)
    gv, gs = host(vals), host(scales)
    assert np.array_equal(gs, ws), np.argwhere(gs != ws)[:4].tolist()
    assert np.array_equal(gv, wc), np.argwhere(gv != wc)[:4].tolist()


def test_rope_without_positions_and_out_of_range_positions():
    rng = np.random.default_rng(5)
    T, H = 40, 16
    q = workloads.bf16_bits(rng.standard_normal((T, H, 128), dtype=np.float32))
    cos, sin = rope_tables(64, 64)
    vals, scales = mx.quantize_rope(dev(q), dev(cos), dev(sin), 64, "neox")
    wc, ws = orope.quantize_rope(omx.bf16_bits_to_f64(q), cos, sin, 64, "neox")
    torch.cuda.synchronize()
    assert np.array_equal(host(vals), wc) and np.array_equal(host(scales), ws)
    # positions outside the table: those tokens are encoded unrotated
    pos = np.arange(T, dtype=np.int64)
    pos[[3, 17]] = [-1, 64]
    vals, scales = mx.quantize_rope(dev(q), dev(cos), dev(sin), 64, "neox", positions=dev(pos))
    torch.cuda.synchronize()
    plain_c, plain_s = omx.quantize_rows(omx.bf16_bits_to_f64(q))
    plain_c, plain_s = plain_c.reshape(T, H, 64), plain_s.reshape(T, H, 4)
    gv, gs = host(vals), host(scales)
    for t in range(T):
        if t in (3, 17):
            assert np.array_equal(gv[t], plain_c[t]) and np.array_equal(gs[t], plain_s[t])
        else:
            assert np.array_equal(gv[t], wc[t]) and np.array_equal(gs[t], ws[t])


def test_rope_dim_zero_equals_quantize():
    rng = np.random.default_rng(6)
    q = workloads.bf16_bits(rng.standard_normal((10, 32, 128), dtype=np.float32))
    empty = torch.empty((0, 0), dtype=torch.float32, device="cuda")
    v0, s0 = mx.quantize_rope(dev(q), empty, empty, 0, "neox")
    v1, s1 = mx.quantize(dev(q))
    torch.cuda.synchronize()
    assert torch.equal(v0, v1) and torch.equal(s0, s1)


def test_rope_decode_query_16x32():
    """The decode workload's query (16 tokens x 32 heads, bf16) at positions 8191,
    rotated over its first 64 dims."""
    case = workloads.paged_decode()
    cos, sin = rope_tables(8192, 64)
    pos = (case["context_lens"].astype(np.int64) - 1)
    vals, scales = mx.quantize_rope(dev(case["q"]), dev(cos), dev(sin), 64, "neox", positions=dev(pos))
    torch.cuda.synchronize()
    wc, ws = orope.quantize_rope(omx.bf16_bits_to_f64(case["q"]), cos, sin, 64, "neox", positions=pos)
    assert np.array_equal(host(vals), wc) and np.array_equal(host(scales), ws)
