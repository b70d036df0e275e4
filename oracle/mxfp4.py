"""MXFP4 codec for one 128-wide indexer row (oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Format (P1 "Changes": E2M1 values + UE8M0 block-32 scales; P1 "Benefit":
68 bytes per token per head): a row of 128 values is cut into 4 blocks of 32.
Each block stores one UE8M0 scale byte (a bare power of two, 2**(byte-127),
OCP MX v1.0 E8M0) and 32 E2M1 elements (OCP MX v1.0: 1 sign bit, 2 exponent
bits with bias 1, 1 mantissa bit).  The row is 64 code bytes + 4 scale bytes.

Readings where the pages are silent (each pinned by a test):

* scale rule: E is the smallest integer with amax <= 6 * 2**E, so no element
  of the block saturates; amax == 0 gives E = -127; E is clamped to
  [-127, 127] and the byte is E + 127 (0xFF is never written);
* element rounding: nearest value of the E2M1 grid, ties to the even code
  (mantissa bit 0); magnitudes above 6 saturate to 6;
* sign of zero: the sign bit is the sign bit of the input, so -0.0 and
  negative values that round to zero encode as 0x8;
* nibble order: element 2j is the low nibble of code byte j, element 2j+1 the
  high nibble;
* scale byte b belongs to block b (elements 32b .. 32b+31).
"""

import numpy as np

HEAD_DIM = 128
BLOCK = 32
NBLOCKS = HEAD_DIM // BLOCK          # 4
CODE_BYTES = HEAD_DIM // 2           # 64
SCALE_BYTES = NBLOCKS                # 4
ROW_BYTES = CODE_BYTES + SCALE_BYTES  # 68
E_MIN, E_MAX = -127, 127


def e2m1_value(nibble):
    """Real value of a 4-bit E2M1 code, from its bit fields (OCP MX v1.0).

    Exponent field 0 is subnormal: value 0.m (times 2**(1-bias) = 1).
    Otherwise 2**(e-1) * (1 + m/2).
    """
    s = (nibble >> 3) & 1
    e = (nibble >> 1) & 3
    m = nibble & 1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -mag if s else mag


# Magnitudes of the 8 non-negative codes 0..7.
GRID = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)


def bf16_bits_to_f64(bits):
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x):
    """Exact value of float32 inputs as float64."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def ue8m0_exponent(amax):
    """Block exponent E: the smallest integer with amax <= 6 * 2**E.

    amax = m * 2**e with m in [0.5, 1) (frexp).  Then 6 * 2**(e-4) < amax
    and 6 * 2**(e-2) > amax, so E is e-3 or e-2; the test
    ``amax <= 6 * 2**(e-3)`` (exact in float64) picks it.  amax == 0 gives
    -127; the result is clamped to [-127, 127].
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    e = e.astype(np.int64)
    E = e - 3
    E = np.where(amax <= np.ldexp(6.0, E), E, E + 1)
    E = np.where(amax == 0.0, E_MIN, E)
    return np.clip(E, E_MIN, E_MAX).astype(np.int64)


def e2m1_encode(y):
    """Nibbles (sign<<3 | code) for already-scaled values y (float64).

    Magnitude: the grid point nearest to |y|; on a tie (|y| exactly between
    two grid points) the even code wins; |y| > 6 saturates to 6.  Sign bit:
    signbit(y).
    """
    y = np.asarray(y, dtype=np.float64)
    # Saturation: a magnitude beyond the largest grid point takes that point.
    mag = np.minimum(np.abs(y), GRID[-1])
    dist = np.abs(mag[..., None] - GRID)                 # [..., 8]
    nearest = dist == dist.min(axis=-1, keepdims=True)   # 1 or 2 candidates
    codes = np.arange(8)
    even_nearest = nearest & (codes % 2 == 0)
    has_even = even_nearest.any(axis=-1)
    code = np.where(has_even, even_nearest.argmax(axis=-1), nearest.argmax(axis=-1))
    sign = np.signbit(y).astype(np.int64)
    return ((sign << 3) | code).astype(np.uint8)


def quantize_rows(x, chunk=8192):
    """MXFP4-encode rows of 128 values.

    x: float64-convertible array [..., 128] holding the exact input values.
    Returns (codes uint8 [R, 64], scales uint8 [R, 4]) with R = x.size // 128.
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1, HEAD_DIM)
    R = x.shape[0]
    codes = np.empty((R, CODE_BYTES), dtype=np.uint8)
    scales = np.empty((R, SCALE_BYTES), dtype=np.uint8)
    for r0 in range(0, R, chunk):
        blk = x[r0:r0 + chunk].reshape(-1, NBLOCKS, BLOCK)
        amax = np.abs(blk).max(axis=-1)                   # [r, 4]
        E = ue8m0_exponent(amax)                          # [r, 4]
        y = np.ldexp(blk, -E[..., None])                  # exact
        nib = e2m1_encode(y).reshape(-1, HEAD_DIM)
        codes[r0:r0 + chunk] = nib[:, 0::2] | (nib[:, 1::2] << 4)
        scales[r0:r0 + chunk] = (E + 127).astype(np.uint8)
    return codes, scales


def dequantize_rows(codes, scales):
    """Exact values (float64 [R, 128]) of MXFP4 rows: (-1)^s * grid[c] * 2**(byte-127)."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, CODE_BYTES)
    scales = np.asarray(scales, dtype=np.uint8).reshape(-1, SCALE_BYTES)
    R = codes.shape[0]
    nib = np.empty((R, HEAD_DIM), dtype=np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    mag = GRID[nib & 7]
    val = np.where(nib & 8, -mag, mag)
    E = scales.astype(np.int64) - 127                     # [R, 4]
    return np.ldexp(val.reshape(R, NBLOCKS, BLOCK), E[..., None]).reshape(R, HEAD_DIM)
