"""Pins for the oracle's FP8 (E4M3) indexer codec, cache layout and logits (CPU only).

* E4M3 values: the hand-worked table in tests/golden/fp8_e4m3.txt (OCP OFP8), plus
  the format's counts and ordering;
* encode: brute-force nearest grid value (ties to the even code) over every bf16
  pattern of magnitude <= 448 and every midpoint between adjacent E4M3 values with
  its fp32 neighbours;
* the scale rule: the hand-worked rows, exact rational rounding of amax / 448 and
  x / s to fp32 (integer arithmetic, not numpy's float32), and the power-of-two
  exponent's defining property;
* cache: hand-worked byte offsets, canaries, slot -1 and the insert / gather round trip;
* logits: exact rational arithmetic, a closed form, and 2**m scaling of a K row.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8
from tests.golden_io import read_fp8

VALUES, ROWS, LAYOUT = read_fp8()


def test_e4m3_hand_worked_values():
    for code, val in VALUES.items():
        got = fp8.e4m3_value(code)
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_grid_shape():
    vals = [fp8.e4m3_value(c) for c in range(0x7F)]
    assert len(set(vals)) == 127 and vals == sorted(vals)          # 0x00..0x7E ascending
    assert max(vals) == 448.0 and vals[1] == 2.0 ** -9
    nans = [c for c in range(256) if np.isnan(fp8.e4m3_value(c))]
    assert nans == [0x7F, 0xFF]
    for c in range(0x7F):                                          # sign symmetry
        assert fp8.e4m3_value(c | 0x80) == -fp8.e4m3_value(c)


GRID = np.array([fp8.e4m3_value(c) for c in range(0x7F)])


def _brute(y):
    """Nearest E4M3 code of a float, ties to the even code, saturating at 448."""
    a = min(abs(y), 448.0)
    d = np.abs(GRID - a)
    best = np.nonzero(d == d.min())[0]
    c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if np.signbit(y) else 0)


def test_encode_every_bf16_pattern_within_range():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    y = y[np.isfinite(y) & (np.abs(y) <= 448)]
    got = fp8.e4m3_encode(y)
    want = np.array([_brute(float(v)) for v in y], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_encode_midpoints_and_their_neighbours():
    mids = (GRID[1:] + GRID[:-1]) / 2
    cases = []
    for m in mids.astype(np.float32):
        cases += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1000))]
    y = np.array(cases + [-c for c in cases], dtype=np.float32)
    got = fp8.e4m3_encode(y)
    want = np.array([_brute(float(v)) for v in y], dtype=np.uint8)
    assert np.array_equal(got, want)
    # values above 448 saturate (the midpoint 464 and beyond included)
    assert fp8.e4m3_encode(np.float32([464, 500, 1e30, -470])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def _fp32_round(fr):
    """Round a positive Fraction to the nearest fp32 (ties to even), exactly; returns a Fraction."""
    assert fr > 0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    e = max(e, -126)                      # subnormals share the 2**-149 step
    step = Fraction(2) ** (e - 23)
    q = fr / step
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * step


@pytest.mark.parametrize("row", ROWS, ids=[f"{r['name']}{int(r['round_scale'])}" for r in ROWS])
def test_hand_worked_rows(row):
    x = np.zeros(128)
    x[:len(row["in"])] = row["in"]
    codes, scales = fp8.quantize_rows(x[None], round_scale=row["round_scale"])
    n = len(row["codes"])
    assert codes[0, :n].tolist() == row["codes"].tolist()
    assert np.all(codes[0, n:] == 0)
    assert scales.astype("<f4").tobytes() == row["scale"]


def test_scale_and_division_are_correctly_rounded_fp32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((40, 128)) * np.exp2(rng.integers(-20, 20, size=(40, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :] = 0.0
    x[1, 7] = 1e-44                       # amax / 448 underflows: the 2**-126 floor
    codes, scales = fp8.quantize_rows(x.astype(np.float64))
    for r in range(len(x)):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        s = _fp32_round(amax / 448) if amax else Fraction(0)
        s = max(s, Fraction(2) ** -126)
        assert Fraction(float(scales[r])) == s, r
        for i in range(0, 128, 7):
            v = Fraction(float(x[r, i]))
            y = _fp32_round(abs(v) / s) if v else Fraction(0)
            y = -y if x[r, i] < 0 or (x[r, i] == 0 and np.signbit(x[r, i])) else y
            assert codes[r, i] == _brute(float(y) if y else float(x[r, i])), (r, i)


def test_power_of_two_exponent_definition():
    rng = np.random.default_rng(4)
    amax = np.concatenate([np.abs(rng.standard_normal(2000)) * np.exp2(rng.integers(-130, 130, 2000)),
                           448.0 * np.exp2(np.arange(-20, 21.0)), [0.0, 448.0, 448.0 * (1 + 2 ** -52)]])
    E = fp8.scale_exponent(amax)
    for a, e in zip(amax, E):
        if a == 0:
            assert e == -126
            continue
        lo, hi = -126, 127
        want = next((k for k in range(lo, hi + 1) if Fraction(a) <= 448 * Fraction(2) ** k), hi)
        assert e == want, a


def test_fold_weights_is_one_fp32_product():
    w = np.float32([0.3, 1e-3, 7.0])
    s = np.float32([1 / 448, 3.0, 2.0 ** -7])
    got = fp8.fold_weights(w, s)
    for i in range(3):
        assert Fraction(float(got[i])) == _fp32_round(Fraction(float(w[i])) * Fraction(float(s[i])))


def test_cache_layout_offsets_and_round_trip():
    assert fp8.ROW_BYTES == 132 and fp8.page_bytes() == 8448
    v0, s0 = LAYOUT
    assert fp8.value_offset(2, 5) == v0 and fp8.scale_offset(2, 5) == s0
    rng = np.random.default_rng(5)
    k = rng.standard_normal((150, 128)).astype(np.float32).astype(np.float64)
    num_pages = 4
    perm = np.array([2, 0, 3])
    slots = perm[np.arange(150) // 64] * 64 + np.arange(150) % 64
    slots[7] = -1                                             # not written
    slots[8] = num_pages * 64 + 1                             # beyond the cache: not written
    cache = np.full((num_pages, 8448), 0xA5, np.uint8)
    cache = fp8.insert(cache, k, slots)
    codes, scales = fp8.quantize_rows(k)
    flat = cache.reshape(-1)
    for i in (0, 63, 64, 149):
        p, o = divmod(int(slots[i]), 64)
        assert flat[fp8.value_offset(p, o):fp8.value_offset(p, o) + 128].tolist() == codes[i].tolist()
        assert flat[fp8.scale_offset(p, o):fp8.scale_offset(p, o) + 4].tobytes() == \
            scales[i:i + 1].astype("<f4").tobytes()
    p7, o7 = divmod(int(perm[0] * 64 + 7), 64)
    assert np.all(flat[fp8.value_offset(p7, o7):fp8.value_offset(p7, o7) + 128] == 0xA5)
    assert np.all(cache[1] == 0xA5)                          # unused page untouched
    bt = perm[None, :].astype(np.int32)
    gc, gs = fp8.gather(cache, bt, [150], [0], 150)
    keep = (np.arange(150) != 7) & (np.arange(150) != 8)
    assert np.array_equal(gc[keep], codes[keep]) and np.array_equal(gs[keep], scales[keep])


def _frac_row(codes, scale):
    return [Fraction(fp8.e4m3_value(int(c))) * Fraction(float(scale)) for c in codes]


def test_logits_match_exact_rationals():
    rng = np.random.default_rng(6)
    T, H, S = 3, 4, 6
    q = rng.standard_normal((T * H, 128)) * np.exp2(rng.integers(-8, 8, size=(T * H, 1)))
    k = rng.standard_normal((S, 128)) * np.exp2(rng.integers(-8, 8, size=(S, 1)))
    qc, qs = fp8.quantize_rows(q)
    kc, kscale = fp8.quantize_rows(k, round_scale=True)
    w = rng.uniform(-1, 1, size=(T, H)).astype(np.float32)
    wf = fp8.fold_weights(w, qs.reshape(T, H))
    ks, ke = np.array([0, 1, 2]), np.array([6, 4, 3])
    got, A = fp8.mqa_logits(qc.reshape(T, H, 128), wf, kc, kscale, ks, ke, with_bound=True)
    for t in range(T):
        for s in range(S):
            if not ks[t] <= s < ke[t]:
                assert got[t, s] == -np.inf and A[t, s] == 0
                continue
            k8 = [Fraction(fp8.e4m3_value(int(c))) for c in kc[s]]
            exact, bound = Fraction(0), Fraction(0)
            for h in range(H):
                q8 = [Fraction(fp8.e4m3_value(int(c))) for c in qc[t * H + h]]
                d = sum(a * b for a, b in zip(q8, k8))
                exact += Fraction(float(wf[t, h])) * max(d, Fraction(0))
                bound += abs(Fraction(float(wf[t, h]))) * sum(abs(a * b) for a, b in zip(q8, k8))
            exact *= Fraction(float(kscale[s]))
            bound *= Fraction(float(kscale[s]))
            assert abs(Fraction(got[t, s]) - exact) <= abs(exact) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)
            assert abs(Fraction(A[t, s]) - bound) <= bound * Fraction(1, 10 ** 14)
            # the logit is the weighted ReLU of the dequantized dot, scales taken out
            qhat = [_frac_row(qc[t * H + h], qs[t * H + h]) for h in range(H)]
            khat = _frac_row(kc[s], kscale[s])
            direct = sum(Fraction(float(w[t, h])) * max(sum(a * b for a, b in zip(qhat[h], khat)), 0)
                         for h in range(H))
            assert abs(Fraction(got[t, s]) - direct) <= abs(direct) * Fraction(1, 10 ** 6) + Fraction(1, 10 ** 300)


def test_single_head_closed_form_and_row_scaling():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 128))
    k = rng.standard_normal((5, 128))
    qc, qs = fp8.quantize_rows(q, round_scale=True)
    kc, kscale = fp8.quantize_rows(k, round_scale=True)
    w1 = np.ones((2, 1), np.float32)
    got = fp8.mqa_logits(qc.reshape(2, 1, 128), w1, kc, kscale, [0, 0], [5, 5])
    kh = fp8.dequantize_rows(kc, kscale)
    q8 = fp8.e4m3_decode(qc)
    for t in range(2):
        for s in range(5):
            assert got[t, s] == max(0.0, float(np.dot(q8[t], kh[s])))
    # a K row scaled by 2**m: with power-of-two scales its codes are unchanged and
    # its logits scale by exactly 2**m
    for m in (-5, 3):
        k2 = k.copy()
        k2[2] *= 2.0 ** m
        kc2, ks2 = fp8.quantize_rows(k2, round_scale=True)
        assert np.array_equal(kc2, kc) and ks2[2] == kscale[2] * 2.0 ** m
        got2 = fp8.mqa_logits(qc.reshape(2, 1, 128), w1, kc2, ks2, [0, 0], [5, 5])
        assert np.array_equal(got2[:, 2], got[:, 2] * 2.0 ** m)


def test_paged_equals_dense():
    rng = np.random.default_rng(8)
    lens, H, nn = [70, 3, 128], 16, 2
    k = rng.standard_normal((sum(lens), 128))
    q = rng.standard_normal((len(lens) * nn * H, 128))
    qc, qs = fp8.quantize_rows(q)
    w = fp8.fold_weights(rng.random((len(lens) * nn, H)).astype(np.float32), qs.reshape(-1, H))
    need = [(L + 63) // 64 for L in lens]
    perm = rng.permutation(sum(need) + 1)
    bt = np.zeros((len(lens), max(need)), np.int32)
    slots, pos = [], 0
    for b, L in enumerate(lens):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        slots.append(bt[b, np.arange(L) // 64] * 64 + np.arange(L) % 64)
    cache = fp8.insert(np.zeros((sum(need) + 1, 8448), np.uint8), k, np.concatenate(slots))
    got = fp8.paged_mqa_logits(qc.reshape(-1, H, 128), w, cache, bt, lens, nn, 130)
    kc, kscale = fp8.quantize_rows(k)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for b, L in enumerate(lens):
        r = np.arange(b * nn, (b + 1) * nn)
        ke = np.maximum(L - nn + np.arange(nn) + 1, 0)
        dense = fp8.mqa_logits(qc.reshape(-1, H, 128)[r], w[r], kc[cu[b]:cu[b + 1]],
                               kscale[cu[b]:cu[b + 1]], [0] * nn, ke, width=130)
        assert np.array_equal(got[r], dense)
