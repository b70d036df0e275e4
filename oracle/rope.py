"""Rotary position embedding of the indexer query before its MXFP4 encode (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

P1 "[Kernel] MXFP4 indexer cache for GLM-5.2 / DSA", section "Notes": the
MXFP4 query quantization runs as a separate step, and a fused
q-rope-mxfp4 kernel could follow.  The pages give neither the rotated
sub-range nor the pairing nor the angle tables, so this module takes the
plainest reading and states it:

* the caller supplies the angle tables: cos[p, j] and sin[p, j] (float32,
  j < rope_dim / 2) for table row p, and optionally positions[t] choosing the
  table row of query token t (default: row t); a token whose table row lies
  outside the table is left unrotated (a safety reading: the pages say
  nothing of it);
* the first ``rope_dim`` of the 128 dims of every head are rotated (0 <=
  rope_dim <= 128, a multiple of 16); the others pass through unchanged;
* pairing: ``neox`` rotates the pairs (j, j + rope_dim/2), ``interleaved``
  the pairs (2j, 2j + 1), j < rope_dim / 2, by the angle of index j:
      a' = a * cos - b * sin,   b' = b * cos + a * sin;
* arithmetic: in fp32 (the precision the encode then takes its decisions
  in), each product rounded, then the sum or difference rounded -- no fused
  multiply-add -- so the rotated values are exactly defined;
* the rotated rows are then MXFP4-encoded by the rule of ``oracle.mxfp4``.
"""

import numpy as np

from . import mxfp4

HEAD_DIM = 128


def rope_pairs(rope_dim, mode):
    """Index arrays (a, b, j): element a[j] pairs with b[j] under angle index j."""
    half = rope_dim // 2
    j = np.arange(half)
    if mode == "neox":
        return j, j + half, j
    if mode == "interleaved":
        return 2 * j, 2 * j + 1, j
    raise ValueError(mode)


def apply_rope(x, cos, sin, rope_dim, mode, positions=None):
    """Rotate the first rope_dim dims of every head of q.

    x: exact values [T, H, 128] (float64 holding bf16 / fp32 values);
    cos, sin: float32 [P, rope_dim / 2]; positions: int [T] or None.
    Returns float32 [T, H, 128].
    """
    x = np.asarray(x, dtype=np.float64).astype(np.float32)     # exact for bf16 / fp32 inputs
    T = x.shape[0]
    assert rope_dim % 16 == 0 and 0 <= rope_dim <= HEAD_DIM
    out = x.copy()
    if rope_dim == 0 or T == 0:
        return out
    pos = np.arange(T) if positions is None else np.asarray(positions, dtype=np.int64)
    cos = np.asarray(cos, dtype=np.float32)
    inside = (pos >= 0) & (pos < cos.shape[0])
    row = np.where(inside, pos, 0)
    c = cos[row][:, None, :]                                     # [T, 1, half]
    s = np.asarray(sin, dtype=np.float32)[row][:, None, :]
    ia, ib, _ = rope_pairs(rope_dim, mode)
    a = x[:, :, ia]
    b = x[:, :, ib]
    # float32 numpy arithmetic: every product and every sum is rounded to fp32
    ac, bs = (a * c).astype(np.float32), (b * s).astype(np.float32)
    bc, as_ = (b * c).astype(np.float32), (a * s).astype(np.float32)
    out[:, :, ia] = (ac - bs).astype(np.float32)
    out[:, :, ib] = (bc + as_).astype(np.float32)
    out[~inside] = x[~inside]                                    # outside the table: unrotated
    return out


def quantize_rope(x, cos, sin, rope_dim, mode, positions=None):
    """RoPE then MXFP4: (codes uint8 [T, H, 64], scales uint8 [T, H, 4])."""
    r = apply_rope(x, cos, sin, rope_dim, mode, positions)
    T, H = r.shape[0], r.shape[1]
    codes, scales = mxfp4.quantize_rows(r.astype(np.float64))
    return codes.reshape(T, H, 64), scales.reshape(T, H, 4)
