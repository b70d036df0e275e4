"""Per-row top-k over a visible column range (top_k_per_row) (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P3 "SparseAttnIndexerKpool" names top_k_per_row and a preallocated
``topk_indices_buffer``; P2 "Validation" tests exact top-k sets.  The pages do
not fix ties, order or padding; the readings taken here:

* candidates of row r are the columns c with ks[r] <= c < ke[r];
* they are ranked by value descending, then column ascending (so among
  equal values the lower column wins); -0.0 and +0.0 are equal values;
* the first min(k, ke-ks) ranked columns are returned, the rest of the k
  output slots hold -1;
* indices are absolute columns of the logits row;
* the order of the returned columns is not part of the contract (sets are
  compared), but this function returns them in rank order.

Input: the float32 logits themselves (the GPU's, for the standalone exact
test, or the oracle's rounded to float32).
"""

import numpy as np


def top_k_per_row(logits, ks, ke, k):
    logits = np.asarray(logits, dtype=np.float32)
    R = logits.shape[0]
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        a, b = int(ks[r]), int(ke[r])
        if b <= a:
            continue
        cols = np.arange(a, b, dtype=np.int64)
        vals = logits[r, a:b].astype(np.float64)
        # lexsort: the last key is the primary one.  -vals ascending == vals
        # descending; equal values (including -0.0 vs +0.0) fall back to the
        # column, ascending.
        order = np.lexsort((cols, -vals))
        n = min(k, b - a)
        out[r, :n] = cols[order[:n]]
    return out


def kth_value(logits_row, ks, ke, k):
    """The k-th largest value among the visible columns (k clipped to their count)."""
    vals = np.sort(np.asarray(logits_row, dtype=np.float64)[ks:ke])[::-1]
    if len(vals) == 0:
        return None
    return vals[min(k, len(vals)) - 1]
