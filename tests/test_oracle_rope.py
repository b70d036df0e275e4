"""Pins for the oracle's query RoPE (the step a fused q-rope-mxfp4 kernel folds
into the MXFP4 encode; P1 "Notes").  CPU only.

* hand-worked rotations with exactly representable cos / sin;
* the fp32 arithmetic (each product rounded, then the sum / difference)
  against exact rational arithmetic with explicit fp32 rounding, and a copy
  that fuses the multiply-add must fail that pin;
* identities: rope_dim 0, cos 1 / sin 0, the untouched dims;
* the closed form (complex multiplication) within the fp32 rounding bound;
* positions select table rows; quantize_rope is the MXFP4 encode of the rotated rows.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import mxfp4, rope


def _rnd32(fr):
    """Nearest fp32 of a Fraction (ties to even), as a Fraction (normal and subnormal range)."""
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    step = Fraction(2) ** (max(e, -126) - 23)
    q = a / step
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * n * step


def test_hand_worked_rotations():
    x = np.zeros((1, 1, 128))
    x[0, 0, 0] = 1.0
    c = np.zeros((1, 32), np.float32)
    s = np.ones((1, 32), np.float32)
    got = rope.apply_rope(x, c, s, 64, "neox")
    want = np.zeros(128, np.float32)
    want[32] = 1.0                                  # (1, 0) -> (0, 1) in the pair (0, 32)
    assert np.array_equal(got[0, 0], want)
    got = rope.apply_rope(x, c, s, 64, "interleaved")
    want = np.zeros(128, np.float32)
    want[1] = 1.0                                   # pair (0, 1)
    assert np.array_equal(got[0, 0], want)
    # a = 1, b = 2, cos = 0.75, sin = 0.5 (all exact): a' = 0.75 - 1 = -0.25, b' = 1.5 + 0.5 = 2
    x = np.zeros((1, 1, 128))
    x[0, 0, 3], x[0, 0, 3 + 32] = 1.0, 2.0
    c = np.full((1, 32), 0.75, np.float32)
    s = np.full((1, 32), 0.5, np.float32)
    got = rope.apply_rope(x, c, s, 64, "neox")
    assert got[0, 0, 3] == -0.25 and got[0, 0, 35] == 2.0


def _exact_rot(a, b, c, s):
    ac, bs = _rnd32(Fraction(a) * Fraction(c)), _rnd32(Fraction(b) * Fraction(s))
    bc, as_ = _rnd32(Fraction(b) * Fraction(c)), _rnd32(Fraction(a) * Fraction(s))
    return _rnd32(ac - bs), _rnd32(bc + as_)


def rope_failures(fn, mode):
    rng = np.random.default_rng(11)
    T, H, D = 3, 2, 64
    x = rng.standard_normal((T, H, 128)).astype(np.float32).astype(np.float64)
    ang = rng.uniform(0, 2 * np.pi, size=(T, D // 2))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    got = fn(x, c, s, D, mode)
    ia, ib, jj = rope.rope_pairs(D, mode)
    bad = []
    for t in range(T):
        for h in range(H):
            for a_i, b_i, j in zip(ia, ib, jj):
                ea, eb = _exact_rot(float(x[t, h, a_i]), float(x[t, h, b_i]), float(c[t, j]), float(s[t, j]))
                if Fraction(float(got[t, h, a_i])) != ea or Fraction(float(got[t, h, b_i])) != eb:
                    bad.append((t, h, int(a_i)))
            rest = np.arange(D, 128)
            if not np.array_equal(got[t, h, rest], x[t, h, rest].astype(np.float32)):
                bad.append((t, h, "rest"))
    return bad


@pytest.mark.parametrize("mode", ["neox", "interleaved"])
def test_fp32_arithmetic_against_exact_rounding(mode):
    assert rope_failures(rope.apply_rope, mode) == []


def _fused(x, cos, sin, rope_dim, mode, positions=None):
    """A copy with fused multiply-adds (one rounding per output): must fail the pin."""
    out = np.asarray(x, np.float64).astype(np.float32).copy()
    ia, ib, _ = rope.rope_pairs(rope_dim, mode)
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    a = out[:, :, ia].astype(np.float64)
    b = out[:, :, ib].astype(np.float64)
    out[:, :, ia] = (a * c - (b * s).astype(np.float32)).astype(np.float32)
    out[:, :, ib] = (b * c + (a * s).astype(np.float32)).astype(np.float32)
    return out


def _swapped_sign(x, cos, sin, rope_dim, mode, positions=None):
    return rope.apply_rope(x, cos, -np.asarray(sin, np.float32), rope_dim, mode, positions)


@pytest.mark.parametrize("mutant", [_fused, _swapped_sign])
def test_pins_catch_planted_mistakes(mutant):
    assert rope_failures(mutant, "neox") != []


def test_identities():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 8, 128)).astype(np.float32).astype(np.float64)
    c = rng.random((4, 64), dtype=np.float32)
    s = rng.random((4, 64), dtype=np.float32)
    assert np.array_equal(rope.apply_rope(x, c[:, :0], s[:, :0], 0, "neox"), x.astype(np.float32))
    one, zero = np.ones((4, 64), np.float32), np.zeros((4, 64), np.float32)
    for mode in ("neox", "interleaved"):
        assert np.array_equal(rope.apply_rope(x, one, zero, 128, mode), x.astype(np.float32))
        got = rope.apply_rope(x, c[:, :16], s[:, :16], 32, mode)
        assert np.array_equal(got[:, :, 32:], x[:, :, 32:].astype(np.float32))


def test_closed_form_complex_rotation():
    rng = np.random.default_rng(13)
    T, H, D = 5, 4, 64
    x = rng.standard_normal((T, H, 128)).astype(np.float32).astype(np.float64)
    ang = rng.uniform(0, 2 * np.pi, size=(T, D // 2))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    for mode in ("neox", "interleaved"):
        got = rope.apply_rope(x, c, s, D, mode).astype(np.float64)
        ia, ib, jj = rope.rope_pairs(D, mode)
        z = (x[:, :, ia] + 1j * x[:, :, ib]) * (c.astype(np.float64) + 1j * s.astype(np.float64))[:, None, jj]
        mag = np.abs(x[:, :, ia]) + np.abs(x[:, :, ib])
        assert np.all(np.abs(got[:, :, ia] - z.real) <= 2 * 2.0 ** -24 * mag * 1.0001)
        assert np.all(np.abs(got[:, :, ib] - z.imag) <= 2 * 2.0 ** -24 * mag * 1.0001)


def test_positions_select_table_rows_and_quantize():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 4, 128)).astype(np.float32).astype(np.float64)
    c = rng.random((50, 32), dtype=np.float32)
    s = rng.random((50, 32), dtype=np.float32)
    pos = np.array([49, 0, 7, 7, 30, 2])
    for mode in ("neox", "interleaved"):
        a = rope.apply_rope(x, c, s, 64, mode, positions=pos)
        b = rope.apply_rope(x, c[pos], s[pos], 64, mode)
        assert np.array_equal(a, b)
        codes, scales = rope.quantize_rope(x, c, s, 64, mode, positions=pos)
        wc, ws = mxfp4.quantize_rows(a.astype(np.float64))
        assert np.array_equal(codes.reshape(-1, 64), wc) and np.array_equal(scales.reshape(-1, 4), ws)


def test_positions_outside_the_table_leave_the_token_unrotated():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((5, 3, 128)).astype(np.float32).astype(np.float64)
    c = rng.random((20, 32), dtype=np.float32)
    s = rng.random((20, 32), dtype=np.float32)
    pos = np.array([-1, 4, 20, 19, -7])
    inside = np.array([False, True, False, True, False])
    for mode in ("neox", "interleaved"):
        got = rope.apply_rope(x, c, s, 64, mode, positions=pos)
        assert np.array_equal(got[~inside], x[~inside].astype(np.float32))
        want = rope.apply_rope(x[inside], c, s, 64, mode, positions=pos[inside])
        assert np.array_equal(got[inside], want)
        assert not np.array_equal(got[inside], x[inside].astype(np.float32))
