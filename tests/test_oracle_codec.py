"""Pins for the oracle's MXFP4 codec and page layout (CPU only).

Each test checks the oracle against something other than itself: the OCP
E2M1 value table, the defining property of the scale exponent, an independent
threshold formulation of round-to-nearest-even, hand-worked bytes, and the
byte counts the pages print.
"""

import math

import numpy as np
import pytest

from oracle import mxfp4, paged_cache
from tests.golden_io import read_blocks

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16():
    with np.errstate(invalid="ignore"):
        v = mxfp4.bf16_bits_to_f64(ALL_BF16)
    return ALL_BF16[np.isfinite(v)], v[np.isfinite(v)]


def test_e2m1_decode_matches_ocp_table():
    # OCP MX v1.0 lists the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for
    # codes 0..7; bit 3 is the sign.
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = mxfp4.e2m1_value(c)
        assert abs(v) == table[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_ue8m0_minimal_exponent_exhaustive_bf16():
    _, v = _finite_bf16()
    amax = np.unique(np.abs(v))
    E = mxfp4.ue8m0_exponent(amax)
    pos = amax > 0
    # Defining property: amax <= 6 * 2**E and (minimality) amax > 6 * 2**(E-1),
    # unless E was clamped at -127.
    assert np.all(amax[pos] <= np.ldexp(6.0, E[pos]))
    unclamped = pos & (E > -127)
    assert np.all(amax[unclamped] > np.ldexp(6.0, E[unclamped] - 1))
    assert np.all(E[~pos] == -127)
    assert E.min() >= -127 and E.max() <= 127


@pytest.mark.parametrize("k", [-130, -127, -126, -20, -1, 0, 1, 5, 100, 125])
def test_ue8m0_boundaries(k):
    x = math.ldexp(6.0, k)
    E = int(mxfp4.ue8m0_exponent(x))
    assert E == max(-127, k)
    # one float32 ulp above the boundary needs the next exponent
    up = float(np.nextafter(np.float32(x), np.float32(np.inf)))
    E_up = int(mxfp4.ue8m0_exponent(up))
    assert E_up == max(-127, k + 1) or (k + 1 < -127 and E_up == -127)


def test_ue8m0_float32_extremes():
    fmax = float(np.finfo(np.float32).max)
    assert int(mxfp4.ue8m0_exponent(fmax)) == 126          # 6*2**126 < fmax <= 6*2**127... fmax < 1.5*2**128
    tiny = float(np.finfo(np.float32).smallest_subnormal)
    assert int(mxfp4.ue8m0_exponent(tiny)) == -127


def _threshold_code(mag):
    """Round-to-nearest-even onto the E2M1 grid written as decision thresholds.

    Between grid points a < b the midpoint goes to whichever of the two codes
    is even: <= for a tie that rounds down, < for a tie that rounds up.
    """
    return ((mag > 0.25).astype(int) + (mag >= 0.75) + (mag > 1.25) + (mag >= 1.75)
            + (mag > 2.5) + (mag >= 3.5) + (mag > 5.0))


def test_e2m1_encode_exhaustive_bf16():
    bits, v = _finite_bf16()
    nib = mxfp4.e2m1_encode(v)
    mag = np.abs(v)
    assert np.array_equal(nib & 7, _threshold_code(mag))
    assert np.array_equal((nib >> 3) & 1, (bits >> 15) & 1)   # sign bit copied (incl. -0)


def test_e2m1_encode_ties_go_to_even_code():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(mxfp4.e2m1_encode(ties)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(mxfp4.e2m1_encode(-ties)) == [8, 10, 10, 12, 12, 14, 14]


def test_hand_worked_blocks():
    blocks, _ = read_blocks()
    assert set(blocks) == set("ABCDEFG")
    for name, b in blocks.items():
        row = np.zeros(128)
        row[:32] = b["in"]
        codes, scales = mxfp4.quantize_rows(row)
        assert codes[0, :16].tolist() == b["codes"].tolist(), name
        assert int(scales[0, 0]) == b["scale"], name


def test_hand_worked_token_offsets():
    blocks, extra = read_blocks()
    row = np.concatenate([blocks[n]["in"] for n in "ABCD"])
    cache = np.full((6, paged_cache.page_bytes()), 0x5A, dtype=np.uint8)
    out = paged_cache.insert(cache, row[None, :], np.array([2 * 64 + 5]))
    flat = out.reshape(-1)
    c0 = int(extra["token_codes_at"])
    s0 = int(extra["token_scales_at"])
    expect_codes = np.concatenate([blocks[n]["codes"] for n in "ABCD"])
    assert flat[c0:c0 + 64].tolist() == expect_codes.tolist()
    assert flat[s0:s0 + 4].tolist() == [0x7F, 0x84, 0x80, 0x7D]
    changed = np.nonzero(flat != 0x5A)[0]
    assert set(changed.tolist()) <= set(range(c0, c0 + 64)) | set(range(s0, s0 + 4))


def test_bytes_per_token_match_pages():
    # P1 "Benefit": 132 -> 68 bytes per token per head.  FP8: 128 values + a
    # 4-byte scale; MXFP4: 128 nibbles + 4 one-byte block scales.
    assert mxfp4.ROW_BYTES == 68
    assert 128 * 1 + 4 == 132
    assert paged_cache.page_bytes(64) == 64 * 68 == 4352
    codes, scales = mxfp4.quantize_rows(np.ones((3, 128)))
    assert codes.shape == (3, 64) and scales.shape == (3, 4)


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(7)
    grid = np.concatenate([mxfp4.GRID, -mxfp4.GRID])
    x = rng.choice(grid, size=(50, 128))
    x[:, ::32] = 6.0                      # pin every block's amax to 6 * 2**E
    E = rng.integers(-100, 100, size=(50, 4))
    x = np.ldexp(x.reshape(50, 4, 32), E[..., None]).reshape(50, 128)
    codes, scales = mxfp4.quantize_rows(x)
    assert np.array_equal(scales.astype(int) - 127, E)
    assert np.array_equal(mxfp4.dequantize_rows(codes, scales), x)


def test_quantization_error_bound():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((200, 128)) * np.exp2(rng.integers(-20, 20, size=(200, 1)))
    codes, scales = mxfp4.quantize_rows(x)
    xh = mxfp4.dequantize_rows(codes, scales)
    E = np.repeat(scales.astype(int) - 127, 32, axis=1)
    y = np.abs(x) / np.exp2(E)
    # half the grid spacing around |y|: 0.25 below 2, 0.5 below 4, 1 above.
    half = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, 1.0))
    assert np.all(np.abs(x - xh) <= half * np.exp2(E) + 0.0)
    assert np.all(np.abs(x) / np.exp2(E) <= 6.0)
    assert np.all((np.signbit(xh) == np.signbit(x)) | (xh == 0))


def test_insert_gather_round_trip_and_canaries():
    rng = np.random.default_rng(3)
    P = 64
    lens = [70, 130, 1]
    num_pages = 9
    perm = rng.permutation(num_pages)
    bt = np.zeros((3, 3), dtype=np.int32)
    bt[0, :2] = perm[0:2]
    bt[1, :3] = perm[2:5]
    bt[2, :1] = perm[5:6]
    k = rng.standard_normal((sum(lens), 128))
    slots = []
    for b, L in enumerate(lens):
        j = np.arange(L)
        slots.append(bt[b, j // P] * P + j % P)
    slots = np.concatenate(slots)
    slots_skip = slots.copy()
    slots_skip[5] = -1
    cache = np.full((num_pages, P * 68), 0xA5, dtype=np.uint8)
    out = paged_cache.insert(cache, k, slots_skip)
    codes, scales = mxfp4.quantize_rows(k)
    cu = np.concatenate([[0], np.cumsum(lens)[:-1]])
    gc, gs = paged_cache.gather(out, bt, lens, cu, sum(lens))
    keep = np.ones(sum(lens), bool)
    keep[5] = False
    assert np.array_equal(gc[keep], codes[keep]) and np.array_equal(gs[keep], scales[keep])
    assert np.all(gc[5] == 0xA5) and np.all(gs[5] == 0xA5)   # slot -1 wrote nothing
    # unused pages (perm[6:]) and tail slots of partly filled pages are untouched
    for p in perm[6:]:
        assert np.all(out[p] == 0xA5)
    p_last = bt[0, 1]
    used = 70 - 64
    assert np.all(out[p_last, used * 64:P * 64] == 0xA5)
    assert np.all(out[p_last, P * 64 + used * 4:] == 0xA5)
