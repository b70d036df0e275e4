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


def shard_to_global(local, rank, world, interleave):
    """Global position of local position ``local`` on context-parallel rank
    ``rank`` of ``world``: the sequence's tokens are dealt to the ranks
    round-robin in runs of ``interleave`` consecutive positions (the
    decode-context-parallel layout named by P3 "SparseAttnIndexerKpool":
    dcp_rank, dcp_world_size, cp_kv_cache_interleave_size; the formula is the
    reading taken here).  Run j of rank r covers global positions
    (j*world + r)*interleave .. +interleave-1."""
    local = np.asarray(local, dtype=np.int64)
    return (local // interleave) * (interleave * world) + rank * interleave + local % interleave


def global_to_shard(pos, world, interleave):
    """Inverse of shard_to_global: (rank, local position) of global positions."""
    pos = np.asarray(pos, dtype=np.int64)
    run = pos // interleave
    return run % world, (run // world) * interleave + pos % interleave


def merge_shard_topk(values, indices, world_interleave, k):
    """Merge per-rank top-k lists into the sequence's top-k (the exchange step
    of context-parallel decode: every rank selects over its own share of the
    positions, the lists are gathered and merged).

    values [R, rows, kin] float32, indices [R, rows, kin] int32: rank s's
    candidates for row r, as local positions (-1 = empty slot).
    world_interleave: the interleave size (R is values.shape[0]).
    Returns [rows, k] int32 global positions of the k best candidates, ranked
    by value descending then global position ascending (-0.0 == +0.0), in
    rank order, then -1 padding."""
    values = np.asarray(values, dtype=np.float32)
    indices = np.asarray(indices, dtype=np.int64)
    R, rows, _ = values.shape
    out = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        v, c = [], []
        for s in range(R):
            ok = indices[s, r] >= 0
            v.append(values[s, r][ok].astype(np.float64))
            c.append(shard_to_global(indices[s, r][ok], s, R, world_interleave))
        v = np.concatenate(v)
        c = np.concatenate(c)
        order = np.lexsort((c, -v))
        n = min(k, len(order))
        out[r, :n] = c[order[:n]]
    return out
