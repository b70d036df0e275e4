"""Comparison rules between the HIP path and the oracle (test infrastructure only).

* Cache, gathered and q bytes: bit-exact.
* Logits (float32 accumulation on the device, float64 here): pass when

      |g - r| <= 1e-5 * |r| + 2**-21 * A[t, s]

  A = sum_h |w| * sum_b |c_{h,b}| (``oracle.logits.abs_bound``).  The relative
  term is the stated 1e-5 bar; the A term is the unavoidable float32
  rounding of the 4-block and head sums when they cancel.  Both sides must
  agree exactly on which entries are masked.
* FP8 logits (``oracle.fp8``): the same rule with A = s_k * sum_h |w'| *
  sum_i |q8_i k8_i| and the factor 2**-15.  Derivation (first-order bounds,
  unit roundoff u = 2**-24): an fp32 sum of n terms in any order errs by at
  most (n-1) * u * (the sum of their magnitudes); the 128-term dot
  contributes 127 u A, the head sum (at most 128 fused multiply-adds, then
  the three adds across lane groups) 131 u A, and the final scale product u
  |r| <= u A: 259 u < 512 u = 2**-15.  (The MXFP4 block dots are exact in fp32, so
  only their 4-block and head sums round there.)
* Top-k: the exact set on identical float32 input.  Against the oracle's own
  logits (end to end): a row is compared as a set only when its k-th / k+1-th
  margin exceeds twice the logits tolerance; on every row, each column whose
  value exceeds the k-th value by more than the tolerance must be present, no
  returned column may fall below the k-th value by more than the tolerance,
  and the returned columns are distinct, visible and min(k, n) in number.
"""

import numpy as np

REL = 1e-5
ABS_FACTOR = 2.0 ** -21
ABS_FACTOR_FP8 = 2.0 ** -15


def logits_close(gpu, ref, bound, abs_factor=ABS_FACTOR):
    """Elementwise pass mask for finite reference entries."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = REL * np.abs(ref) + abs_factor * np.asarray(bound, dtype=np.float64)
    return np.abs(gpu - ref) <= tol


def topk_end_to_end_ok(idx, ref_row, ks, ke, k, tol):
    """Check one row of GPU top-k indices against exact reference values.

    ``ref_row``: float64 reference logits of the full row; ``tol``: absolute
    tolerance on logits near the k-th value.  Returns (ok, exact_required).
    """
    idx = np.asarray(idx, dtype=np.int64)
    n = max(0, ke - ks)
    m = min(k, n)
    valid = idx[:m]
    if np.any(idx[m:] != -1):
        return False, False
    if len(set(valid.tolist())) != m or np.any(valid < ks) or np.any(valid >= ke):
        return False, False
    if m == 0:
        return True, True
    vals = np.sort(ref_row[ks:ke])[::-1]
    vk = vals[m - 1]
    chosen = ref_row[valid]
    if np.any(chosen < vk - tol):
        return False, False
    must = np.nonzero(ref_row[ks:ke] > vk + tol)[0] + ks
    if not np.all(np.isin(must, valid)):
        return False, False
    margin_ok = (m == n) or (vals[m - 1] - vals[m] > 2 * tol)
    if margin_ok:
        exact = np.lexsort((np.arange(ks, ke), -ref_row[ks:ke]))[:m] + ks
        return set(exact.tolist()) == set(valid.tolist()), True
    return True, False
