"""Pins for the oracle's comparison rules and its logits error bound (CPU only).

The GPU parity tests pass or fail through ``oracle.tolerance.logits_close``,
``oracle.tolerance.topk_end_to_end_ok``, ``oracle.topk.kth_value`` and the
bound A returned by ``oracle.logits.abs_bound`` / ``mqa_logits(with_bound=True)``.
Each is pinned here against values fixed independently of its code:

* logits_close: boundary cases whose float64 arithmetic is exact (powers of
  two for the relative term, A = 2**21 * 2**m for the absolute one), so the
  exact tolerance and the first float64 past it are known;
* topk_end_to_end_ok: hand-worked rows whose outcomes follow from the
  ordering-margin rule (P2 "Enable SM86 MXFP4 sparse-indexer cache", section
  "Validation": exact top-k sets with an ordering margin) -- every column
  clearly above the k-th value present, none clearly below it, exact sets only
  when the k / k+1 margin exceeds twice the tolerance;
* kth_value: a plain Python sort;
* the A bound: exact rational arithmetic (fractions.Fraction) over the bit
  fields of the MXFP4 rows.

Each pin is run first on the oracle's function and then on copies with one
planted mistake each (a dropped term, a flipped comparison, an off-by-one);
every copy must be caught by at least one check.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import logits, mxfp4, tolerance, topk

# ---------------------------------------------------------------------------
# logits_close
# ---------------------------------------------------------------------------


def _next_up(x):
    return float(np.nextafter(x, np.inf))


def _next_down(x):
    return float(np.nextafter(x, -np.inf))


def _largest_within(r, t):
    """Largest float64 g >= r with g - r <= t exactly (r a power of two, t < r)."""
    ulp = float(np.spacing(r))
    return r + np.floor(t / ulp) * ulp


def _smallest_within(r, t):
    """Smallest float64 g <= r with r - g <= t exactly (r a power of two, t < r/2)."""
    ulp = float(np.spacing(r)) / 2.0               # spacing just below a power of two
    return r - np.floor(t / ulp) * ulp


def logits_close_failures(fn):
    """Checks of a logits_close implementation; returns the failed ones."""
    bad = []

    def expect(name, gpu, ref, bound, want):
        got = np.asarray(fn(np.array([gpu]), np.array([ref]), np.array([bound])))
        if got.shape != (1,) or bool(got[0]) != want:
            bad.append(name)

    # absolute term alone: ref 0, A = 2**21 -> tolerance exactly 1.0
    A = 2.0 ** 21
    expect("abs: at +tol", 1.0, 0.0, A, True)
    expect("abs: at -tol", -1.0, 0.0, A, True)
    expect("abs: one ulp past +tol", _next_up(1.0), 0.0, A, False)
    expect("abs: one ulp past -tol", -_next_up(1.0), 0.0, A, False)
    expect("abs: A = 2**22 doubles it", 2.0, 0.0, 2 * A, True)
    expect("abs: A = 2**22, past", _next_up(2.0), 0.0, 2 * A, False)
    expect("abs: A = 0 needs equality", 0.0, 0.0, 0.0, True)
    expect("abs: A = 0, smallest difference", 2.0 ** -1074, 0.0, 0.0, False)
    # relative term alone: ref a power of two, A = 0 -> 1e-5 * |ref| exactly
    for r in (2.0 ** 20, 1.0, 2.0 ** -30, -(2.0 ** 7)):
        t = tolerance.REL * abs(r)                  # exact: |r| is a power of two
        s = np.sign(r)
        hi = s * _largest_within(abs(r), t)         # away from zero
        lo = s * _smallest_within(abs(r), t)        # towards zero
        expect(f"rel {r}: edge away from 0", hi, r, 0.0, True)
        expect(f"rel {r}: edge towards 0", lo, r, 0.0, True)
        expect(f"rel {r}: past away from 0", s * (abs(hi) + float(np.spacing(abs(hi)))), r, 0.0, False)
        expect(f"rel {r}: past towards 0", s * _next_down(abs(lo)), r, 0.0, False)
    # both terms: A chosen so that 2**-21 * A == 1e-5 * |ref|; the tolerance is twice
    # either term (exactly), so an implementation that drops one term fails
    r = 2.0 ** 10
    t1 = tolerance.REL * r
    A = t1 * 2.0 ** 21
    edge = _largest_within(r, 2 * t1)
    expect("both: at 2 * term", edge, r, A, True)
    expect("both: past 2 * term", edge + float(np.spacing(edge)), r, A, False)
    expect("both: beyond one term only", _largest_within(r, 1.5 * t1), r, A, True)
    # NaN and inf never pass against a finite reference
    expect("nan", float("nan"), 1.0, 1.0, False)
    expect("inf", float("inf"), 1.0, 2.0 ** 40, False)
    # elementwise: one call over many entries agrees with the scalar outcomes
    g = np.array([1.0, _next_up(1.0), -1.0, 0.5])
    got = np.asarray(fn(g, np.zeros(4), np.full(4, 2.0 ** 21)))
    if got.tolist() != [True, False, True, True]:
        bad.append("elementwise")
    return bad


def _lc_strict(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    tol = tolerance.REL * np.abs(ref) + tolerance.ABS_FACTOR * np.asarray(bound, np.float64)
    return np.abs(gpu - ref) < tol


def _lc_rel_on_gpu(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    tol = tolerance.REL * np.abs(gpu) + tolerance.ABS_FACTOR * np.asarray(bound, np.float64)
    return np.abs(gpu - ref) <= tol


def _lc_no_bound(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    return np.abs(gpu - ref) <= tolerance.REL * np.abs(ref)


def _lc_wide_factor(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    tol = tolerance.REL * np.abs(ref) + 2.0 ** -20 * np.asarray(bound, np.float64)
    return np.abs(gpu - ref) <= tol


def _lc_one_sided(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    tol = tolerance.REL * np.abs(ref) + tolerance.ABS_FACTOR * np.asarray(bound, np.float64)
    return gpu - ref <= tol


def _lc_rel_1e4(gpu, ref, bound):
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    tol = 1e-4 * np.abs(ref) + tolerance.ABS_FACTOR * np.asarray(bound, np.float64)
    return np.abs(gpu - ref) <= tol


def test_logits_close_pins():
    assert tolerance.REL == 1e-5 and tolerance.ABS_FACTOR == 2.0 ** -21
    assert logits_close_failures(tolerance.logits_close) == []


def test_logits_close_fp8_factor():
    # the FP8 rule's factor 2**-15: A = 2**15 gives a tolerance of exactly 1
    assert tolerance.ABS_FACTOR_FP8 == 2.0 ** -15
    f = tolerance.logits_close
    assert f([1.0], [0.0], [2.0 ** 15], abs_factor=tolerance.ABS_FACTOR_FP8)[0]
    assert not f([_next_up(1.0)], [0.0], [2.0 ** 15], abs_factor=tolerance.ABS_FACTOR_FP8)[0]
    # the first-order rounding count of the derivation (127 + 131 + 1 roundings of
    # 2**-24) stays below the factor
    assert (127 + 131 + 1) * 2.0 ** -24 < tolerance.ABS_FACTOR_FP8


@pytest.mark.parametrize("mutant", [_lc_strict, _lc_rel_on_gpu, _lc_no_bound, _lc_wide_factor,
                                    _lc_one_sided, _lc_rel_1e4])
def test_logits_close_pins_catch_planted_mistakes(mutant):
    assert logits_close_failures(mutant) != []


# ---------------------------------------------------------------------------
# topk_end_to_end_ok
# ---------------------------------------------------------------------------

# columns:          0    1    2    3            4    5    6     7
ROW = np.array([5.0, 1.0, 3.0, 3.0 + 1e-9, 0.5, 4.0, -1.0, 2.0])
# descending: 5 (c0), 4 (c5), 3+1e-9 (c3), 3 (c2), 2 (c7), 1 (c1), 0.5 (c4), -1 (c6)
ROW2 = np.array([10.0, 5.0, 4.95, 4.88, 1.0])


def e2e_failures(fn):
    """Hand-worked outcomes for a topk_end_to_end_ok implementation; returns the
    checks it gets wrong.  Each case is (name, idx, ks, ke, k, tol, ok, exact)."""
    cases = [
        # k = 3: v_k = 3+1e-9 (c3), v_k+1 = 3 (c2), margin 1e-9
        ("loose tol, best set", [0, 5, 3], 0, 8, 3, 0.1, True, False),
        ("loose tol, tie choice", [5, 0, 2], 0, 8, 3, 0.1, True, False),
        ("loose tol, column below v_k - tol", [0, 5, 7], 0, 8, 3, 0.1, False, None),
        ("loose tol, must-column 5 missing", [0, 3, 2], 0, 8, 3, 0.1, False, None),
        ("loose tol, must-column 0 missing", [5, 3, 2], 0, 8, 3, 0.1, False, None),
        ("tight tol, exact set", [3, 0, 5], 0, 8, 3, 1e-12, True, True),
        ("tight tol, wrong tie", [0, 5, 2], 0, 8, 3, 1e-12, False, None),
        # margin 1e-9 between tol and 2 tol: a pass, not exact-required; above
        # 2 tol: exact-required (the flag, on a passing set)
        ("margin between tol and 2 tol", [0, 5, 3], 0, 8, 3, 0.75e-9, True, False),
        ("margin just above 2 tol", [0, 5, 3], 0, 8, 3, 0.45e-9, True, True),
        ("margin below tol, tie choice", [0, 5, 2], 0, 8, 3, 1.5e-9, True, False),
        # k = 2: v_k = 4 (c5), v_k+1 = 3+1e-9, margin ~1
        ("k=2 exact", [5, 0], 0, 8, 2, 0.1, True, True),
        ("k=2 wrong", [0, 3], 0, 8, 2, 0.1, False, None),
        ("duplicate column", [0, 5, 5], 0, 8, 3, 0.1, False, None),
        ("column == ke", [0, 5, 8], 0, 8, 3, 10.0, False, None),
        ("column below ks", [0, 5, 3], 1, 8, 3, 10.0, False, None),
        ("negative column in the first m", [0, 5, -1], 0, 8, 3, 10.0, False, None),
        # ks = 1: column 0 (value 5) is not visible; visible descending is
        # 4 (c5), 3+1e-9 (c3), 3 (c2), 2 (c7), ...: k = 3 gives v_k = 3, margin 1
        ("ks=1 exact set", [5, 3, 2], 1, 8, 3, 1e-12, True, True),
        ("ks=1 column below v_k - tol", [5, 3, 7], 1, 8, 3, 1e-12, False, None),
        ("ks=1 high value outside the range", [0, 5, 3], 1, 8, 3, 10.0, False, None),
        # padding: k = 10 over 8 visible columns -> 8 columns then -1, -1
        ("padded", [0, 1, 2, 3, 4, 5, 6, 7, -1, -1], 0, 8, 10, 0.0, True, True),
        ("pad slot holds a column", [0, 1, 2, 3, 4, 5, 6, 7, -1, 7], 0, 8, 10, 0.0, False, None),
        ("pad slot holds 0", [0, 1, 2, 3, 4, 5, 6, 7, 0, -1], 0, 8, 10, 0.0, False, None),
        ("a column missing, -1 instead", [0, 1, 2, 3, 4, 5, 6, -1, -1, -1], 0, 8, 10, 0.0, False, None),
        # k = n exactly: every column, exact by definition
        ("k = n", [7, 6, 5, 4, 3, 2, 1, 0], 0, 8, 8, 0.5, True, True),
        # empty visible range
        ("empty row", [-1, -1, -1], 5, 5, 3, 0.0, True, True),
        ("empty row, a column", [5, -1, -1], 5, 5, 3, 0.0, False, None),
        ("ke < ks", [-1, -1], 6, 2, 2, 0.0, True, True),
    ]
    # ROW2 = [10, 5, 4.95, 4.88, 1], k = 2, tol = 0.1: v_k = 5, v_k+1 = 4.95 (margin
    # 0.05 <= tol); 4.95 lies within tol of v_k, 4.88 does not (but lies within tol
    # of v_k+1, so a rule measured from the k+1-th value would take it)
    cases2 = [
        ("row2 tie within tol", [0, 2], 0, 5, 2, 0.1, True, False),
        ("row2 best set", [1, 0], 0, 5, 2, 0.1, True, False),
        ("row2 below v_k - tol", [0, 3], 0, 5, 2, 0.1, False, None),
    ]
    bad = []
    for row, table in ((ROW, cases), (ROW2, cases2)):
        for name, idx, ks, ke, k, tol, ok, exact in table:
            try:
                got_ok, got_exact = fn(np.array(idx), row, ks, ke, k, tol)
            except Exception:                       # a crash is a wrong outcome too
                bad.append(name)
                continue
            if bool(got_ok) != ok or (exact is not None and bool(got_exact) != exact):
                bad.append(name)
    return bad


def test_hand_worked_rows_by_plain_sort():
    """The outcome table's k-th values, from a plain Python sort of ROW."""
    def ranked(ks, ke):
        return sorted(range(ks, ke), key=lambda c: (-ROW[c], c))
    assert ranked(0, 8)[:4] == [0, 5, 3, 2]
    assert ranked(1, 8)[:4] == [5, 3, 2, 7]


def test_topk_end_to_end_ok_pins():
    assert e2e_failures(tolerance.topk_end_to_end_ok) == []


def _fn_variant(drop_must=False, invert_margin=False, drop_below=False, drop_pad=False,
                drop_dup=False, drop_range=False, margin_factor=2.0, kth_off=0):
    """topk_end_to_end_ok with one planted mistake (a copy of the rule it pins)."""
    def fn(idx, ref_row, ks, ke, k, tol):
        idx = np.asarray(idx, dtype=np.int64)
        n = max(0, ke - ks)
        m = min(k, n)
        valid = idx[:m]
        if not drop_pad and np.any(idx[m:] != -1):
            return False, False
        if not drop_dup and len(set(valid.tolist())) != m:
            return False, False
        if not drop_range and (np.any(valid < ks) or np.any(valid >= ke)):
            return False, False
        if m == 0:
            return True, True
        vals = np.sort(ref_row[ks:ke])[::-1]
        vk = vals[max(0, min(m - 1 + kth_off, len(vals) - 1))]
        chosen = ref_row[valid]
        if not drop_below and np.any(chosen < vk - tol):
            return False, False
        must = np.nonzero(ref_row[ks:ke] > vk + tol)[0] + ks
        if not drop_must and not np.all(np.isin(must, valid)):
            return False, False
        margin_ok = (m == n) or (vals[m - 1] - vals[m] > margin_factor * tol)
        if invert_margin:
            margin_ok = not margin_ok
        if margin_ok:
            exact = np.lexsort((np.arange(ks, ke), -ref_row[ks:ke]))[:m] + ks
            return set(exact.tolist()) == set(valid.tolist()), True
        return True, False
    return fn


@pytest.mark.parametrize("mistake", [
    dict(drop_must=True), dict(invert_margin=True), dict(drop_below=True), dict(drop_pad=True),
    dict(drop_dup=True), dict(drop_range=True), dict(margin_factor=1.0), dict(kth_off=1),
    dict(kth_off=-1),
])
def test_topk_end_to_end_ok_pins_catch_planted_mistakes(mistake):
    assert e2e_failures(_fn_variant(**mistake)) != []


def test_unmutated_copy_passes():
    # the copy used for the planted mistakes is itself the rule the table pins
    assert e2e_failures(_fn_variant()) == []


# ---------------------------------------------------------------------------
# kth_value
# ---------------------------------------------------------------------------


def _kth_plain(row, ks, ke, k):
    vis = sorted((float(row[c]) for c in range(ks, ke)), reverse=True)
    if not vis:
        return None
    return vis[min(k, len(vis)) - 1]


def kth_failures(fn):
    rng = np.random.default_rng(7)
    bad = []
    for trial in range(200):
        W = int(rng.integers(1, 40))
        row = rng.choice(np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 1.0, 3.0]), size=W)
        row = row + (rng.random(W) < 0.5) * rng.standard_normal(W)
        ks = int(rng.integers(0, W + 1))
        ke = int(rng.integers(0, W + 1))
        k = int(rng.integers(1, W + 3))
        want = _kth_plain(row, ks, ke, k)
        got = fn(row, ks, ke, k)
        if (want is None) != (got is None) or (want is not None and got != want):
            bad.append(trial)
    return bad


def _kth_off_by_one(row, ks, ke, k):
    vals = np.sort(np.asarray(row, np.float64)[ks:ke])[::-1]
    return None if len(vals) == 0 else vals[min(k, len(vals) - 1)]


def _kth_ascending(row, ks, ke, k):
    vals = np.sort(np.asarray(row, np.float64)[ks:ke])
    return None if len(vals) == 0 else vals[min(k, len(vals)) - 1]


def _kth_whole_row(row, ks, ke, k):
    vals = np.sort(np.asarray(row, np.float64))[::-1]
    return None if ke <= ks else vals[min(k, len(vals)) - 1]


def test_kth_value_pins():
    assert kth_failures(topk.kth_value) == []


@pytest.mark.parametrize("mutant", [_kth_off_by_one, _kth_ascending, _kth_whole_row])
def test_kth_value_pins_catch_planted_mistakes(mutant):
    assert kth_failures(mutant) != []


# ---------------------------------------------------------------------------
# the A bound of the logits tolerance
# ---------------------------------------------------------------------------


def _frac_row(codes, scales):
    """Exact Fraction values of one MXFP4 row from its bit fields (no numpy math):
    E2M1 magnitudes from the OCP table, scale 2**(byte - 127)."""
    table = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]
    out = []
    for i in range(128):
        byte = int(codes[i // 2])
        nib = (byte >> 4) if i % 2 else (byte & 0xF)
        val = table[nib & 7] * Fraction(2) ** (int(scales[i // 32]) - 127)
        out.append(-val if nib & 8 else val)
    return out


def _exact_bound(qf_heads, kf, w_row):
    """A = sum_h |w_h| * sum_b |sum_{i in block b} q_i k_i|, exactly."""
    A = Fraction(0)
    for h, qf in enumerate(qf_heads):
        blocks = Fraction(0)
        for b in range(4):
            blocks += abs(sum(qf[i] * kf[i] for i in range(32 * b, 32 * b + 32)))
        A += abs(Fraction(float(w_row[h]))) * blocks
    return A


def _case(seed, T=3, H=4, S=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, 128))
    k = rng.standard_normal((S, 128))
    # block scales far apart, so the 4 block dots cancel and A exceeds |logit|
    q *= np.exp2(rng.integers(-5, 6, size=(T, H, 4, 1))).repeat(32, -1).reshape(T, H, 128)
    k *= np.exp2(rng.integers(-5, 6, size=(S, 4, 1))).repeat(32, -1).reshape(S, 128)
    qc, qs = mxfp4.quantize_rows(q)
    kc, kscale = mxfp4.quantize_rows(k)
    w = rng.uniform(-1, 1, size=(T, H)).astype(np.float32)
    return qc.reshape(T, H, 64), qs.reshape(T, H, 4), kc, kscale, w


def bound_failures(abs_bound_fn, seed=21):
    qc, qs, kc, kscale, w = _case(seed)
    T, H = w.shape
    S = kc.shape[0]
    rows = np.repeat(np.arange(T), S)
    cols = np.tile(np.arange(S), T)
    got = abs_bound_fn(qc, qs, kc, kscale, w, rows, cols)
    kf = [_frac_row(kc[s], kscale[s]) for s in range(S)]
    bad = []
    for j, (t, s) in enumerate(zip(rows, cols)):
        exact = _exact_bound([_frac_row(qc[t, h], qs[t, h]) for h in range(H)], kf[s], w[t])
        if abs(Fraction(float(got[j])) - exact) > exact * Fraction(1, 10 ** 14):
            bad.append((int(t), int(s)))
    return bad


def test_abs_bound_equals_exact_rational_value():
    assert bound_failures(logits.abs_bound) == []


def test_with_bound_paths_equal_abs_bound_and_exact_value():
    qc, qs, kc, kscale, w = _case(22)
    T, H = w.shape
    S = kc.shape[0]
    ks = np.array([0, 1, 2])
    ke = np.array([5, 4, 3])
    vals, A = logits.mqa_logits(qc, qs, kc, kscale, w, ks, ke, with_bound=True)
    kf = [_frac_row(kc[s], kscale[s]) for s in range(S)]
    for t in range(T):
        qf = [_frac_row(qc[t, h], qs[t, h]) for h in range(H)]
        for s in range(S):
            if not ks[t] <= s < ke[t]:
                assert A[t, s] == 0.0 and vals[t, s] == -np.inf
                continue
            exact = _exact_bound(qf, kf[s], w[t])
            assert abs(Fraction(float(A[t, s])) - exact) <= exact * Fraction(1, 10 ** 14)
            assert A[t, s] == pytest.approx(
                logits.abs_bound(qc, qs, kc, kscale, w, [t], [s])[0], rel=1e-14, abs=0)
    # the bound is not slack: it exceeds |logit| here (the block dots cancel) but
    # equals it when every weight and block dot is non-negative
    vis = np.isfinite(vals)
    assert np.all(A[vis] >= np.abs(vals[vis]) * (1 - 1e-15))
    assert np.any(A[vis] > 2 * np.abs(vals[vis]))


def test_bound_equals_logit_for_nonnegative_terms():
    # one head, w = 1, q and k non-negative: every block dot >= 0, so A = logit
    rng = np.random.default_rng(23)
    q = np.abs(rng.standard_normal((1, 1, 128)))
    k = np.abs(rng.standard_normal((4, 128)))
    qc, qs = mxfp4.quantize_rows(q)
    kc, kscale = mxfp4.quantize_rows(k)
    w = np.ones((1, 1), np.float32)
    vals, A = logits.mqa_logits(qc.reshape(1, 1, 64), qs.reshape(1, 1, 4), kc, kscale, w,
                                [0], [4], with_bound=True)
    assert np.array_equal(A, vals)


def test_paged_with_bound_equals_dense():
    from oracle import paged_cache
    qc, qs, kc, kscale, w = _case(24, T=2, H=4, S=70)
    # one sequence of 70 tokens in pages 1 and 0 (reversed), next_n = 2
    bt = np.array([[1, 0]], np.int32)
    slots = np.concatenate([64 + np.arange(64), np.arange(6)])
    cache = paged_cache.write_rows(np.zeros((2, 64 * 68), np.uint8), kc, kscale, slots)
    vals, A = logits.paged_mqa_logits(qc, qs, w, cache, bt, [70], 2, 70, with_bound=True)
    dv, dA = logits.mqa_logits(qc, qs, kc, kscale, w, [0, 0], [69, 70], with_bound=True)
    assert np.array_equal(vals, dv) and np.array_equal(A, dA)


def _bound_abs_outside(q_codes, q_scales, k_codes, k_scales, w, rows, cols):
    # |sum_b c_b| instead of sum_b |c_b|
    qh = logits._dequant_q(np.asarray(q_codes)[rows], np.asarray(q_scales)[rows])
    kh = mxfp4.dequantize_rows(np.asarray(k_codes)[cols], np.asarray(k_scales)[cols])
    c = np.abs((qh * kh[:, None, :]).sum(axis=-1))
    return (np.abs(np.asarray(w, np.float64)[rows]) * c).sum(axis=-1)


def _bound_signed_w(q_codes, q_scales, k_codes, k_scales, w, rows, cols):
    qh = logits._dequant_q(np.asarray(q_codes)[rows], np.asarray(q_scales)[rows])
    kh = mxfp4.dequantize_rows(np.asarray(k_codes)[cols], np.asarray(k_scales)[cols])
    qb = qh.reshape(qh.shape[0], qh.shape[1], 4, 32)
    kb = kh.reshape(kh.shape[0], 1, 4, 32)
    c = np.abs((qb * kb).sum(axis=-1)).sum(axis=-1)
    return (np.asarray(w, np.float64)[rows] * c).sum(axis=-1)


def _bound_inflated(*args):
    return 2.0 * logits.abs_bound(*args)


def _bound_one_head(q_codes, q_scales, k_codes, k_scales, w, rows, cols):
    return logits.abs_bound(np.asarray(q_codes)[:, :1], np.asarray(q_scales)[:, :1], k_codes,
                            k_scales, np.asarray(w)[:, :1], rows, cols)


@pytest.mark.parametrize("mutant", [_bound_abs_outside, _bound_signed_w, _bound_inflated,
                                    _bound_one_head])
def test_bound_pins_catch_planted_mistakes(mutant):
    assert bound_failures(mutant) != []
