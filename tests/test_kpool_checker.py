"""CPU pins of the GPU kpool test's acceptance rule (tests/test_gpu_kpool.py): the
oracle's own encoding of a pooled row passes it, and encodings with a planted
mistake -- a code two steps off, a flipped sign, a wrong scale -- fail it."""

import numpy as np
import pytest

from oracle import fp8 as ofp8, mxfp4 as omx
from tests.test_gpu_kpool import _check_fp8_row, _check_mxfp4_row


def _row(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(128) * np.exp2(rng.integers(-5, 5, size=(4, 1))).repeat(32, 1).reshape(-1)
    return x.astype(np.float32).astype(np.float64), np.abs(x) * 2.0 ** -20


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("seed", range(5))
def test_mxfp4_rule(seed):
    x, d = _row(seed)
    codes, scales = omx.quantize_rows(x[None])
    codes, scales = codes[0], scales[0]
    _check_mxfp4_row(codes, scales, x, d)                       # the oracle's bytes pass
    big = int(np.argmax(np.abs(x[:32])))                        # a large element of block 0
    bad = codes.copy()
    nib = (bad[big // 2] >> (4 * (big % 2))) & 0xF
    new = (nib & 8) | max((nib & 7) - 2, 0)                     # two magnitude steps down
    bad[big // 2] = (bad[big // 2] & (0xF0 if big % 2 == 0 else 0x0F)) | (new << (4 * (big % 2)))
    assert _fails(_check_mxfp4_row, bad, scales, x, d)
    flip = codes.copy()
    flip[big // 2] ^= 0x08 << (4 * (big % 2))                    # sign of a non-zero element
    assert _fails(_check_mxfp4_row, flip, scales, x, d)
    wrong = scales.copy()
    wrong[1] += 1                                               # block 1 scale one step up
    assert _fails(_check_mxfp4_row, codes, wrong, x, d)


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_rule(round_scale):
    x, d = _row(11)
    codes, scales = ofp8.quantize_rows(x[None], round_scale)
    _check_fp8_row(codes[0], scales[0], x, d, round_scale)
    big = int(np.argmax(np.abs(x)))
    bad = codes[0].copy()
    bad[big] = (bad[big] & 0x80) | max((bad[big] & 0x7F) - 2, 0)
    assert _fails(_check_fp8_row, bad, scales[0], x, d, round_scale)
    assert _fails(_check_fp8_row, codes[0], np.float32(scales[0] * 2), x, d, round_scale)
