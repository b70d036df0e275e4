"""GPU parity of the pooled (kpool) insert (idx_kpool_insert) against the oracle
(oracle/kpool.py): the write mask and every untouched byte exactly; the pooled
fp32 rows (P3's return_compressed) within a derived bound delta of the oracle's
float64 pool; the written bytes equal to the oracle's encoding except where the
exact pooled value lies within delta of a rounding or scale boundary, where the
neighbouring code (scale) is also accepted.  Both cache formats (MXFP4, FP8 with
both scale rules), bf16 and fp32 K.

The bound: the kernel pools in fp32 (z = gate + ape, the maximum subtracted,
exp, two sums over the pool, one division).  With unit roundoff u = 2**-24 and
an exp within 2 u, each weight e_j errs by at most about 4u(1 + max|z|)
relative, the sums by kpool*u, the division by u, so
|pooled_gpu - pooled| <= (2**-21 (1 + max|z|) + (kpool + 2) 2**-23) max_j |k_j|;
delta doubles that."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import fp8 as ofp8, kpool as okp, mxfp4 as omx
from tests.gpu_helpers import CANARY, dev, host

pytestmark = pytest.mark.gpu


def _delta(k, gate, ape, kp):
    n = k.shape[0]
    idx = okp.pool_indices(n, kp)
    z = gate.astype(np.float64)[idx] + ape.astype(np.float64)[None]
    zmax = np.abs(z).max(axis=1)
    kmax = np.abs(k.astype(np.float64)[idx]).max(axis=1)
    return 2 * (2.0 ** -21 * (1 + zmax) + (kp + 2) * 2.0 ** -23) * kmax


def _dec_e2m1(nib):
    return np.where(nib & 8, -1.0, 1.0) * omx.GRID[nib & 7]


def _check_mxfp4_row(codes, scales, x, d):
    """GPU row (64 code bytes, 4 scale bytes) vs the exact pooled row x with bound d."""
    nib = np.empty(128, np.uint8)
    nib[0::2], nib[1::2] = codes & 0xF, codes >> 4
    for b in range(4):
        sl = slice(32 * b, 32 * b + 32)
        xb, db = x[sl], d[sl]
        amax, da = np.abs(xb).max(), db.max()
        e_lo = int(omx.ue8m0_exponent(max(amax - da, 0.0)))
        e_hi = int(omx.ue8m0_exponent(amax + da))
        E = int(scales[b]) - 127
        assert e_lo <= E <= e_hi, f"block {b}: scale {E} outside [{e_lo}, {e_hi}]"
        y, dy = np.ldexp(xb, -E), np.ldexp(db, -E)
        lo = _dec_e2m1(omx.e2m1_encode(y - dy))
        hi = _dec_e2m1(omx.e2m1_encode(y + dy))
        v = _dec_e2m1(nib[sl])
        assert np.all((lo <= v) & (v <= hi)), f"block {b}: a code outside its bound"
        zero = v == 0
        sign_ok = (np.signbit(y - dy) | np.signbit(y + dy)) | ~(nib[sl] >> 3).astype(bool)
        sign_ok &= ~np.signbit(y + dy) | (nib[sl] >> 3).astype(bool) | (y - dy <= 0)
        assert np.all(~zero | sign_ok), f"block {b}: sign of a zero code"


def _check_fp8_row(codes, scale, x, d, round_scale):
    amax, da = np.abs(x).max(), d.max()
    s_lo = ofp8.row_scales(np.array([[max(amax - da, 0.0)]]), round_scale)[0]
    s_hi = ofp8.row_scales(np.array([[amax + da]]), round_scale)[0]
    assert s_lo <= scale <= s_hi, f"scale {scale} outside [{s_lo}, {s_hi}]"
    y = x / np.float64(scale)
    dy = d / np.float64(scale) + np.abs(y) * 2.0 ** -23        # + the fp32 division's rounding
    lo = ofp8.e4m3_decode(ofp8.e4m3_encode(y - dy))
    hi = ofp8.e4m3_decode(ofp8.e4m3_encode(y + dy))
    v = ofp8.e4m3_decode(codes)
    assert np.all((lo <= v) & (v <= hi)), "a code outside its bound"


def _run(dtype, kp, fmt, round_scale, n=2000, seed=0):
    rng = np.random.default_rng(seed + kp)
    x = workloads.draw_values(rng, (n, 128), "lognormal")
    k = workloads.bf16_bits(x) if dtype == "bf16" else x
    kexact = omx.bf16_bits_to_f64(k) if dtype == "bf16" else omx.f32_to_f64(k)
    gate = (3 * rng.standard_normal((n, 128))).astype(np.float32)
    ape = rng.standard_normal((kp, 128)).astype(np.float32)
    num_pages = 3 + n // (64 * kp)
    slots = np.full(n, -1, np.int64)
    ends = np.arange(kp - 1, n, kp)
    slots[ends] = rng.permutation((num_pages - 1) * 64)[:len(ends)]
    slots[rng.choice(n, 5, replace=False)] = num_pages * 64 + 7   # beyond the cache: skipped
    if kp > 1:
        slots[0] = 3                                               # 0 < kpool - 1: dropped
    row = 68 if fmt == "mxfp4" else 132
    cache = torch.full((num_pages, 64 * row), CANARY, dtype=torch.uint8, device="cuda")
    _, comp = mx.kpool_insert(dev(k), dev(gate), dev(ape), dev(slots), cache, kp, fmt=fmt,
                              round_scale=round_scale, return_compressed=True)
    torch.cuda.synchronize()
    ref_cache, mask, pooled = okp.insert(np.full((num_pages, 64 * row), CANARY, np.uint8), kexact,
                                         gate, ape, slots, kp, fmt, round_scale)
    delta = _delta(kexact, gate, ape, kp)
    got, g_comp = host(cache), host(comp)
    written = mask & (slots < num_pages * 64)
    # pooled rows within delta; unwritten rows of the compressed output untouched (zero)
    assert np.all(np.abs(g_comp[written] - pooled[written]) <= delta[written])
    assert np.all(g_comp[~written] == 0)
    # bytes: rows that are not written keep the canary; written rows are valid
    # encodings and almost all elements equal the oracle's
    flat_g, flat_r = got.reshape(-1), ref_cache.reshape(-1)
    touched = np.zeros(flat_g.size, bool)
    exact_elems = total_elems = 0
    for i in np.nonzero(written)[0]:
        p, o = divmod(int(slots[i]), 64)
        if fmt == "mxfp4":
            c0, s0 = p * 4352 + o * 64, p * 4352 + 4096 + o * 4
            codes, scales = flat_g[c0:c0 + 64], flat_g[s0:s0 + 4]
            _check_mxfp4_row(codes, scales, pooled[i], delta[i])
            touched[c0:c0 + 64] = touched[s0:s0 + 4] = True
            exact_elems += int(np.sum(codes == flat_r[c0:c0 + 64]))
            total_elems += 64
        else:
            v0, s0 = ofp8.value_offset(p, o), ofp8.scale_offset(p, o)
            codes = flat_g[v0:v0 + 128]
            scale = flat_g[s0:s0 + 4].view("<f4")[0]
            _check_fp8_row(codes, scale, pooled[i], delta[i], round_scale)
            touched[v0:v0 + 128] = touched[s0:s0 + 4] = True
            exact_elems += int(np.sum(codes == flat_r[v0:v0 + 128]))
            total_elems += 128
    assert np.all(flat_g[~touched] == CANARY), "a byte outside the written rows changed"
    assert exact_elems >= 0.99 * total_elems, f"only {exact_elems}/{total_elems} bytes equal the oracle's"
    return exact_elems, total_elems


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kp", [1, 4, 16])
def test_kpool_mxfp4(dtype, kp):
    _run(dtype, kp, "mxfp4", False)


@pytest.mark.parametrize("round_scale", [False, True])
@pytest.mark.parametrize("kp", [4, 7])
def test_kpool_fp8(round_scale, kp):
    _run("bf16", kp, "fp8", round_scale)


def test_kpool_fewer_tokens_than_a_pool_writes_nothing():
    rng = np.random.default_rng(3)
    k = workloads.bf16_bits(rng.standard_normal((3, 128), dtype=np.float32))
    cache = torch.full((2, 64 * 68), CANARY, dtype=torch.uint8, device="cuda")
    mx.kpool_insert(dev(k), dev(np.zeros((3, 128), np.float32)), dev(np.zeros((4, 128), np.float32)),
                    dev(np.array([0, 1, 2], np.int64)), cache, 4)
    torch.cuda.synchronize()
    assert torch.all(cache == CANARY)


def test_kpool_one_million_tokens_sampled():
    """The bench's size (1,048,576 bf16 tokens, kpool 4, 262,143 pool rows over
    permuted pages, pool ends shifted by two positions from the chunk start), checked
    on 512 sampled pool rows against the oracle's pool of the same four tokens."""
    n, kp = 1 << 20, 4
    rng = np.random.default_rng(404)
    x = workloads.draw_values(rng, (n, 128), "lognormal")
    k = workloads.bf16_bits(x)
    gate = (3 * rng.standard_normal((n, 128))).astype(np.float32)
    ape = rng.standard_normal((kp, 128)).astype(np.float32)
    ends = np.arange(kp + 1, n, kp)                  # positions 5, 9, ...: pools 2..5, 6..9, ...
    num_pages = -(-len(ends) // 64)
    slots = np.full(n, -1, np.int64)
    slots[ends] = rng.permutation(num_pages * 64)[:len(ends)]
    cache = torch.full((num_pages, 64 * 68), CANARY, dtype=torch.uint8, device="cuda")
    mx.kpool_insert(dev(k), dev(gate), dev(ape), dev(slots), cache, kp)
    torch.cuda.synchronize()
    flat = host(cache).reshape(-1)
    for i in np.sort(rng.choice(ends, 512, replace=False)):
        sl = slice(i - kp + 1, i + 1)
        kx = omx.bf16_bits_to_f64(k[sl])
        pooled = okp.pooled_rows(kx, gate[sl], ape, kp)[-1]
        d = _delta(kx, gate[sl], ape, kp)[-1]
        p, o = divmod(int(slots[i]), 64)
        c0, s0 = p * 4352 + o * 64, p * 4352 + 4096 + o * 4
        _check_mxfp4_row(flat[c0:c0 + 64], flat[s0:s0 + 4], pooled, d)
    # the one slot no pool maps to keeps the canary
    unused = np.setdiff1d(np.arange(num_pages * 64), slots[ends])
    for s_ in unused:
        p, o = divmod(int(s_), 64)
        assert np.all(flat[p * 4352 + o * 64:p * 4352 + o * 64 + 64] == CANARY)
        assert np.all(flat[p * 4352 + 4096 + o * 4:p * 4352 + 4096 + o * 4 + 4] == CANARY)
