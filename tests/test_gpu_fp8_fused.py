"""GPU parity of the FP8 decode step in one launch (idx_logits_paged_insert_fp8):
the cache bytes and the logits bit-identical to the three separate calls
(idx_insert_fp8 of the new tokens, idx_quantize_fp8 with the weights folded,
idx_logits_paged_fp8) over bf16 / fp32 inputs, 16..128 heads, next_n 1..4, both
scale formats, clean 0 / 1 and sequences shorter than next_n; and the 16 x 8192
bf16 step held to the FP8 oracle directly (cache, sampled logits, top-k)."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import fp8 as of8, logits as olog, tolerance
from tests.gpu_helpers import (CANARY, check_logits, check_topk_end_to_end, check_topk_sets, dev,
                               exact, host, split_new_tokens)

pytestmark = pytest.mark.gpu

F8 = tolerance.ABS_FACTOR_FP8


def _fp8_cache(num_pages):
    return torch.full((num_pages, 64 * 132), CANARY, dtype=torch.uint8, device="cuda")


def _step_pair(case, round_scale=False, clean=True):
    """The one-launch FP8 step and the separate calls on copies of one cache."""
    bt_np = case["block_table"]
    pre_slots, k_new, new_slots = split_new_tokens(case, bt_np)
    bt, ctx = dev(bt_np), dev(case["context_lens"])
    q, w = dev(case["q"]), dev(case["w"])
    cache_a = _fp8_cache(case["num_pages"])
    mx.insert_fp8(dev(case["k"]), dev(pre_slots), cache_a, round_scale=round_scale)
    cache_b = cache_a.clone()
    R, W = case["q"].shape[0], case["width"]
    la = torch.full((R, W), float("nan"), dtype=torch.float32, device="cuda")
    lb = la.clone()
    mx.insert_fp8(dev(k_new), dev(new_slots), cache_a, round_scale=round_scale)
    qv, _, wf = mx.quantize_fp8(q, round_scale=round_scale, weights=w)
    mx.logits_paged_fp8(qv, wf, cache_a, bt, ctx, case["next_n"], W, logits=la, clean=clean)
    mx.logits_paged_insert_fp8(q, dev(k_new), w, cache_b, bt, ctx, case["next_n"], W,
                               round_scale=round_scale, logits=lb, clean=clean)
    torch.cuda.synchronize()
    ca, cb = host(cache_a), host(cache_b)
    assert np.array_equal(ca, cb), f"cache bytes differ at {np.argwhere(ca != cb)[:4].tolist()}"
    a, b = host(la).view(np.uint32), host(lb).view(np.uint32)
    assert np.array_equal(a, b), f"logits differ at {np.argwhere(a != b)[:4].tolist()}"
    return cache_b, lb


@pytest.mark.parametrize("dtype,H,next_n,round_scale,clean", [
    ("bf16", 32, 1, False, True),        # the decode shape
    ("bf16", 32, 1, True, False),
    ("f32", 32, 2, False, True),
    ("bf16", 16, 4, True, True),
    ("f32", 64, 1, True, True),
    ("bf16", 64, 3, False, False),
    ("bf16", 128, 1, False, True),
    ("f32", 128, 2, True, False),
    ("bf16", 48, 2, False, True),
])
def test_fp8_paged_insert_equals_separate_calls(dtype, H, next_n, round_scale, clean):
    lens = [1, 63, 64, 65, 300, 191, 192, 193, 2]
    case = workloads.decode_case(H * 13 + next_n + 7 * round_scale, seq_lens=lens, H=H,
                                 next_n=next_n, dtype=dtype, q_dist="lognormal",
                                 k_dist="lognormal", spare_pages=2, width=max(lens) + 45)
    _step_pair(case, round_scale=round_scale, clean=clean)


def test_fp8_paged_insert_rows_past_the_context_start():
    # sequences shorter than next_n (new-token positions below 0 write nothing)
    case = workloads.decode_case(91, seq_lens=[1, 2, 700, 129], H=32, next_n=3, width=760)
    _step_pair(case, clean=False)


def test_fp8_paged_insert_16x8192_against_oracle():
    """The 16 x 8192 bf16 decode step (H 32, top-2048) in one launch on the FP8
    cache, against the oracle: the whole cache, sampled sequences' logits, top-k."""
    case = workloads.paged_decode()
    cache, logits = _step_pair(case, clean=True)
    ke = olog.decode_visible_end(case["context_lens"], 1).astype(np.int32)
    idx = mx.topk(logits, None, dev(ke), case["topk"])
    torch.cuda.synchronize()
    ref_cache = of8.write_rows(np.full((case["num_pages"], 64 * 132), CANARY, np.uint8),
                               *of8.quantize_rows(exact(case, "k")), case["slot_mapping"])
    assert np.array_equal(host(cache), ref_cache)
    H = case["H"]
    qc, qsc = of8.quantize_rows(exact(case, "q"))
    wref = of8.fold_weights(case["w"].reshape(-1), qsc).reshape(-1, H)
    seqs = [0, 9, 15]
    ref, bound = of8.paged_mqa_logits(qc.reshape(-1, H, 128), wref, ref_cache, case["block_table"],
                                      case["context_lens"], 1, case["width"], seqs=seqs,
                                      with_bound=True)
    g = host(logits)
    check_logits(g[seqs], ref[seqs], bound[seqs], "fp8 one-launch 16x8192", abs_factor=F8)
    zeros = np.zeros(len(ke), np.int32)
    out = host(idx)
    check_topk_sets(g, zeros, ke, case["topk"], out, "fp8 one-launch 16x8192")
    check_topk_end_to_end(ref[seqs], bound[seqs], zeros[seqs], ke[seqs], case["topk"], out[seqs],
                          "fp8 one-launch 16x8192", abs_factor=F8)


def _extreme_rows(rng, n):
    """fp32 rows whose scales and elements reach the ends of the in-wave encode:
    scales on both sides of 2^-64 (reciprocal route / division), at the 2^-126
    floor and near the fp32 maximum; signed zeros, subnormals, E4M3 rounding ties
    and log-uniform magnitudes over the whole exponent range."""
    rows = []
    for amax in (448 * 2.0 ** -64, np.nextafter(np.float32(448 * 2.0 ** -64), np.float32(0)),
                 np.float32(1e-39), 2.0 ** -120, 3.0e38, 448.0, 1.0):
        r = (rng.uniform(-1, 1, 128) * amax).astype(np.float32)
        r[rng.integers(0, 128)] = np.float32(amax)
        rows.append(r)
    # E4M3 ties (nearest-even decides) and tiny quotients at a power-of-two scale
    s = 2.0 ** -3
    t = np.array([2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -12, 1.0625, 1.1875, 17.0,
                  232.0, 0.0, 2.0 ** -9, 5 * 2.0 ** -10, 448.0], np.float64)
    r = np.zeros(128, np.float32)
    r[:len(t)] = t * s
    r[len(t):2 * len(t)] = -t * s
    r[2 * len(t)] = np.float32(-0.0)
    r[2 * len(t) + 1:2 * len(t) + 5] = np.array([1e-45, -1e-45, 1e-40, -3e-39], np.float32)
    rows.append(r)
    while len(rows) < n:
        mag = np.exp2(rng.uniform(-149, 127, 128))
        sign = np.where(rng.random(128) < 0.5, -1.0, 1.0)
        r = (sign * mag).astype(np.float32)
        r[rng.random(128) < 0.05] = np.float32(-0.0)
        rows.append(r)
    out = np.stack(rows[:n])
    assert np.all(np.isfinite(out))
    return out


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_paged_insert_extreme_rows(round_scale):
    """New K rows and query rows at the ends of the encode's range: the one-launch
    step equals the separate calls (cache bytes, logit bits) and its cache equals
    the oracle's for every token."""
    rng = np.random.default_rng(4242 + round_scale)
    lens = [5, 70, 129, 64, 3, 200, 31, 2]
    case = workloads.decode_case(77, seq_lens=lens, H=32, next_n=2, dtype="f32", width=260)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    new = np.concatenate([starts[b] + lens[b] - 2 + np.arange(2) for b in range(len(lens))])
    case["k"][new] = _extreme_rows(rng, len(new))
    R, H = case["q"].shape[:2]
    case["q"] = _extreme_rows(rng, R * H).reshape(R, H, 128)
    cache, _ = _step_pair(case, round_scale=round_scale, clean=True)
    ref_cache = of8.write_rows(np.full((case["num_pages"], 64 * 132), CANARY, np.uint8),
                               *of8.quantize_rows(exact(case, "k"), round_scale=round_scale),
                               case["slot_mapping"])
    assert np.array_equal(host(cache), ref_cache)
