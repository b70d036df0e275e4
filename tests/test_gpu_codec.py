"""GPU parity: MXFP4 quantize, paged insert and gather, bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import mxfp4 as omx, paged_cache as opc
from tests.gpu_helpers import CANARY, dev, exact, host, new_cache

pytestmark = pytest.mark.gpu


def _bf16_value(v):
    return workloads.bf16_bits(np.array([v], np.float32))[0]


def _patterned_bf16_rows():
    """Every finite bf16 pattern, 31 per block, with a block amax M pinning the scale.

    For each M the block exponent is fixed, so the 65k patterns are encoded at
    that scale (values above M are left out of that group)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = omx.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    Ms = [6.0 * 2.0 ** e for e in (-125, -120, -60, -3, -2, -1, 0, 1, 7, 60, 125)]
    Ms += [1.5 * 2.0 ** -125, 7.0 * 2.0 ** -3, 3.0e38, 9.2e-41, 1.0e-38]
    blocks = []
    for M in Ms:
        mb = _bf16_value(M)
        Mv = float(omx.bf16_bits_to_f64(np.array([mb]))[0])
        sel = bits[finite & (np.abs(vals) <= Mv)]
        nb = -(-len(sel) // 31)
        blk = np.zeros((nb, 32), np.uint16)
        flat = blk[:, :31].reshape(-1)
        flat[:len(sel)] = sel
        blk[:, :31] = flat.reshape(nb, 31)
        blk[:, 31] = mb
        blocks.append(blk)
    blk = np.concatenate(blocks)
    pad = (-len(blk)) % 4
    blk = np.concatenate([blk, np.zeros((pad, 32), np.uint16)])
    # also every pattern as its own block amax (scale chosen by the value itself)
    own = np.zeros((int(finite.sum()), 32), np.uint16)
    own[:, 0] = bits[finite]
    own[:, 5] = bits[finite] ^ 0x8000          # same magnitude, other sign
    pad2 = (-len(own)) % 4
    own = np.concatenate([own, np.zeros((pad2, 32), np.uint16)])
    return np.concatenate([blk, own]).reshape(-1, 128)


def test_quantize_bf16_all_patterns_bit_exact():
    rows = _patterned_bf16_rows()
    v, s = mx.quantize(dev(rows))
    torch.cuda.synchronize()
    rc, rs = omx.quantize_rows(omx.bf16_bits_to_f64(rows))
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(v), rc)


def _tie_rows_f32(rng):
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 6.0], np.float32)
    rows = []
    for E in (-127, -126, -100, -1, 0, 3, 100, 125):
        scale = np.float32(2.0 ** E)
        blk = np.zeros(32, np.float32)
        blk[0] = np.float32(6.0) * scale
        m = ties * scale
        blk[1:12] = m
        blk[12:23] = -m
        blk[23:28] = np.nextafter(m[:5], np.float32(np.inf))
        blk[28:31] = np.nextafter(m[:3], np.float32(0))
        blk[31] = -0.0
        rows.append(blk)
    rows = np.stack(rows)
    rows = rows[: len(rows) // 4 * 4].reshape(-1, 128)
    rnd = (rng.standard_normal((64, 128)) * np.exp2(rng.integers(-40, 40, (64, 1)))).astype(np.float32)
    sub = (rng.standard_normal((8, 128)) * np.float32(1e-40)).astype(np.float32)   # subnormal blocks
    zero = np.zeros((4, 128), np.float32)
    zero[1, ::3] = -0.0
    return np.concatenate([rows, rnd, sub, zero])


def test_quantize_f32_ties_extremes_bit_exact():
    rows = _tie_rows_f32(np.random.default_rng(0))
    v, s = mx.quantize(dev(rows))
    torch.cuda.synchronize()
    rc, rs = omx.quantize_rows(omx.f32_to_f64(rows))
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(v), rc)


def test_quantize_strided_rows_and_empty():
    rng = np.random.default_rng(1)
    base = workloads.bf16_bits(rng.standard_normal((37, 200)).astype(np.float32))
    x = dev(base)[:, 16:144]                       # row stride 200 elements, offset 32 B
    v, s = mx.quantize(x)
    torch.cuda.synchronize()
    rc, rs = omx.quantize_rows(omx.bf16_bits_to_f64(base[:, 16:144]))
    assert np.array_equal(host(v), rc) and np.array_equal(host(s), rs)
    e = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    v0, s0 = mx.quantize(e)
    assert v0.shape == (0, 64) and s0.shape == (0, 4)


def test_insert_tiny_whole_cache_bit_exact_with_canaries():
    case = workloads.tiny()
    slots = case["slot_mapping"].copy()
    slots[[3, 77, 200]] = -1                        # no write
    cache = new_cache(case["num_pages"])
    mx.insert(dev(case["k"]), dev(slots), cache)
    torch.cuda.synchronize()
    ref = opc.insert(np.full((case["num_pages"], 64 * 68), CANARY, np.uint8), exact(case, "k"), slots)
    assert np.array_equal(host(cache), ref)


def test_insert_out_of_range_slots_are_skipped():
    rng = np.random.default_rng(2)
    k = workloads.bf16_bits(rng.standard_normal((40, 128)).astype(np.float32))
    slots = rng.permutation(3 * 64)[:40].astype(np.int64)
    bad = slots.copy()
    bad[[0, 5]] = [3 * 64, 10 ** 9]                 # beyond the 3-page cache
    cache = new_cache(3)
    mx.insert(dev(k), dev(bad), cache)
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[[0, 5]] = -1
    ref = opc.insert(np.full((3, 64 * 68), CANARY, np.uint8), omx.bf16_bits_to_f64(k), ok)
    assert np.array_equal(host(cache), ref)


def test_insert_paged_decode_cache_bit_exact():
    case = workloads.paged_decode()
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    torch.cuda.synchronize()
    ref = opc.insert(np.zeros((case["num_pages"], 64 * 68), np.uint8), exact(case, "k"),
                     case["slot_mapping"])
    assert np.array_equal(host(cache), ref)


def test_gather_ragged_sequences_bit_exact():
    case = workloads.decode_case(7, seq_lens=[70, 130, 1, 64, 200], H=16, spare_pages=3)
    cache = new_cache(case["num_pages"])
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    lens = case["context_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    kv, ksc = mx.gather(cache, dev(case["block_table"]), dev(lens), dev(cu), int(lens.max()), total)
    torch.cuda.synchronize()
    rc, rs = opc.gather(host(cache), case["block_table"], lens, cu, total)
    assert np.array_equal(host(kv), rc) and np.array_equal(host(ksc), rs)
    # and the round trip equals quantizing the K rows directly
    qc, qs = omx.quantize_rows(exact(case, "k"))
    assert np.array_equal(rc, qc) and np.array_equal(rs, qs)


def test_gather_prefill_chunk_bit_exact():
    case = workloads.prefill_chunk()
    cache = new_cache(case["num_pages"])
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                        dev(case["cu_seq_offsets"]), case["S"], case["S"])
    torch.cuda.synchronize()
    qc, qs = omx.quantize_rows(exact(case, "k"))
    assert np.array_equal(host(kv), qc) and np.array_equal(host(ksc), qs)


@pytest.mark.parametrize("k_dtype,q_dtype,n_tok,q_rows", [("bf16", "bf16", 16, 512), ("f32", "bf16", 40, 3),
                                                          ("bf16", "f32", 1, 700), ("f32", "f32", 300, 64),
                                                          ("bf16", "bf16", 0, 33), ("bf16", "bf16", 50, 0)])
def test_insert_quantize_matches_separate_calls_and_oracle(k_dtype, q_dtype, n_tok, q_rows):
    rng = np.random.default_rng(n_tok * 7 + q_rows)

    def draw(rows, dt):
        x = (rng.standard_normal((rows, 128)) * 2.0 ** rng.integers(-20, 20, (rows, 1))).astype(np.float32)
        return workloads.bf16_bits(x) if dt == "bf16" else x

    def f64(a):
        return omx.bf16_bits_to_f64(a) if a.dtype == np.uint16 else omx.f32_to_f64(a)

    k, q = draw(n_tok, k_dtype), draw(q_rows, q_dtype)
    slots = rng.permutation(5 * 64)[:n_tok].astype(np.int64)
    if n_tok > 3:
        slots[[1, 2]] = [-1, 5 * 64 + 9]              # no write; out of range (skipped)
    fused = new_cache(5)
    qv, qs = mx.insert_quantize(dev(k), dev(slots), fused, dev(q))
    sep = new_cache(5)
    mx.insert(dev(k), dev(slots), sep)
    qv2, qs2 = mx.quantize(dev(q))
    torch.cuda.synchronize()
    assert np.array_equal(host(fused), host(sep))
    assert np.array_equal(host(qv), host(qv2)) and np.array_equal(host(qs), host(qs2))
    ok = np.where(slots >= 5 * 64, -1, slots)
    ref = opc.insert(np.full((5, 64 * 68), CANARY, np.uint8), f64(k), ok)
    assert np.array_equal(host(fused), ref)
    rc, rs = omx.quantize_rows(f64(q))
    assert np.array_equal(host(qv), rc) and np.array_equal(host(qs), rs)
