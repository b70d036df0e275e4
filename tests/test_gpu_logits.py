"""GPU parity: paged and dense indexer logits against the float64 oracle, within
the stated tolerance (1e-5 relative plus the fp32 summation floor), with exact
agreement on which entries are masked; plus the invariants of the definition."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import logits as olog, mxfp4 as omx
from tests.gpu_helpers import check_logits, dev, gpu_build_cache, host, oracle_q

pytestmark = pytest.mark.gpu


def _paged_gpu(case, clean=True, logits=None, cache=None):
    cache = gpu_build_cache(case) if cache is None else cache
    qv, qs = mx.quantize(dev(case["q"]))
    out = mx.logits_paged(qv, qs, dev(case["w"]), cache, dev(case["block_table"]),
                          dev(case["context_lens"]), case["next_n"], case["width"], logits=logits,
                          clean=clean)
    torch.cuda.synchronize()
    return out, cache, qv, qs


def _paged_oracle(case, cache_np, seqs=None):
    qc, qs = oracle_q(case)
    return olog.paged_mqa_logits(qc, qs, case["w"], cache_np, case["block_table"],
                                 case["context_lens"], case["next_n"], case["width"], seqs=seqs,
                                 with_bound=True)


def test_paged_tiny():
    case = workloads.tiny()
    out, cache, qv, qs = _paged_gpu(case)
    qc, qsc = oracle_q(case)
    assert np.array_equal(host(qv), qc) and np.array_equal(host(qs), qsc)
    ref, bound = _paged_oracle(case, host(cache))
    check_logits(host(out), ref, bound, "tiny paged")


@pytest.mark.parametrize("H,next_n,lens", [(16, 1, [1, 63, 64, 65, 300]),
                                           (64, 3, [5, 64, 129, 250]),
                                           (128, 2, [100, 17]),
                                           (48, 16, [40, 200]),
                                           (32, 1, [0, 5, 0, 700, 64, 0, 1]),
                                           (32, 2, list(np.random.default_rng(5).integers(0, 1500, 300))),
                                           (16, 3, [3, 64, 130, 1, 2, 700]),
                                           (64, 2, [2, 65, 129, 1000]),
                                           (48, 2, [127, 128, 1]),
                                           (32, 4, [4, 3, 0, 64, 67, 300])])
def test_paged_ragged_heads_and_next_n(H, next_n, lens):
    case = workloads.decode_case(H * 7 + next_n, seq_lens=lens, H=H, next_n=next_n, spare_pages=2,
                                 width=max(lens) + 37)
    out, cache, _, _ = _paged_gpu(case)
    ref, bound = _paged_oracle(case, host(cache))
    check_logits(host(out), ref, bound, f"paged H={H} next_n={next_n}")


def test_paged_clean_false_leaves_poisoned_tail():
    case = workloads.decode_case(11, seq_lens=[90, 130], H=32, next_n=2, width=200)
    poison = torch.full((4, 200), float("nan"), device="cuda")
    out, cache, _, _ = _paged_gpu(case, clean=False, logits=poison)
    ref, bound = _paged_oracle(case, host(cache))
    g = host(out)
    vis = np.isfinite(ref)
    assert np.all(np.isnan(g[~vis]))
    check_logits(np.where(vis, g, -np.inf), ref, bound, "clean=0")


def test_paged_negative_weights():
    case = workloads.decode_case(12, seq_lens=[300], H=32, next_n=1)
    case["w"] = (case["w"] * 2 - 1).astype(np.float32)
    out, cache, _, _ = _paged_gpu(case)
    ref, bound = _paged_oracle(case, host(cache))
    check_logits(host(out), ref, bound, "negative weights")


def test_paged_lognormal_scales():
    case = workloads.decode_case(13, seq_lens=[700, 333], H=32, k_dist="lognormal")
    out, cache, _, _ = _paged_gpu(case)
    ref, bound = _paged_oracle(case, host(cache))
    check_logits(host(out), ref, bound, "lognormal")


def _prefill_gpu(case, clean=True, logits=None):
    cache = gpu_build_cache(case)
    kv, ksc = mx.gather(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                        dev(case["cu_seq_offsets"]), case["S"], case["S"])
    qv, qs = mx.quantize(dev(case["q"]))
    out = mx.logits_prefill(qv, qs, kv, ksc, dev(case["w"]), dev(case["ks"]), dev(case["ke"]),
                            logits=logits, clean=clean)
    torch.cuda.synchronize()
    return out, kv, ksc, qv, qs


def _prefill_oracle(case, rows=None, chunk=16):
    qc, qs = oracle_q(case)
    kc, ksc = omx.quantize_rows(
        omx.bf16_bits_to_f64(case["k"]) if case["dtype"] == "bf16" else omx.f32_to_f64(case["k"]))
    return olog.mqa_logits(qc, qs, kc, ksc, case["w"], case["ks"], case["ke"], rows=rows,
                           chunk=chunk, with_bound=True)


def test_prefill_tiny():
    case = workloads.tiny_prefill()
    out, *_ = _prefill_gpu(case)
    ref, bound = _prefill_oracle(case)
    check_logits(host(out), ref, bound, "tiny prefill")


@pytest.mark.parametrize("T,S,H", [(100, 1500, 32), (37, 2100, 64), (16, 700, 128), (50, 300, 48),
                                   (1, 64, 16)])
def test_prefill_causal_ragged(T, S, H):
    case = workloads.prefill_case(T * 3 + H, T=T, S=S, H=H, spare_pages=1)
    out, *_ = _prefill_gpu(case)
    ref, bound = _prefill_oracle(case)
    check_logits(host(out), ref, bound, f"prefill T={T} S={S} H={H}")


def test_prefill_varlen_ranges_and_clean_false():
    rng = np.random.default_rng(21)
    T, S = 64, 2048
    ks = rng.integers(0, S, T).astype(np.int32)
    ke = np.minimum(S + 50, ks + rng.integers(0, 1500, T)).astype(np.int32)   # some past S: clipped
    ks[0], ke[0] = 10, 10                                                    # empty row
    case = workloads.prefill_case(22, T=T, S=S, H=32, ks=ks, ke=ke)
    poison = torch.full((T, S), float("nan"), device="cuda")
    out, *_ = _prefill_gpu(case, clean=False, logits=poison)
    ref, bound = _prefill_oracle(case)
    g = host(out)
    vis = np.isfinite(ref)
    assert np.all(np.isnan(g[~vis]))
    check_logits(np.where(vis, g, -np.inf), ref, bound, "varlen clean=0")
    out1, *_ = _prefill_gpu(case, clean=True)
    check_logits(host(out1), ref, bound, "varlen clean=1")


@pytest.mark.parametrize("H,clean", [(32, True), (64, False)])
def test_prefill_long_keys_varlen(H, clean):
    """S above 16384 (4096-key workgroups in key-chunk-major order) with windows
    that start and end inside chunks, span several chunks or are empty."""
    rng = np.random.default_rng(H + 5)
    T, S = 24, 20000
    ks = rng.integers(0, S, T).astype(np.int32)
    ke = np.minimum(S, ks + rng.integers(0, 12000, T)).astype(np.int32)
    ks[:4] = [0, 4095, 8192, 100]
    ke[:4] = [S, 4097, 8192, 16390]                                          # row 2 empty
    case = workloads.prefill_case(H * 11 + 3, T=T, S=S, H=H, ks=ks, ke=ke)
    poison = torch.full((T, S), float("nan"), device="cuda")
    out, *_ = _prefill_gpu(case, clean=clean, logits=poison)
    ref, bound = _prefill_oracle(case)
    g = host(out)
    if clean:
        check_logits(g, ref, bound, f"long-key prefill H={H}")
    else:
        vis = np.isfinite(ref)
        assert np.all(np.isnan(g[~vis])), "clean=0 wrote a masked column"
        check_logits(np.where(vis, g, -np.inf), ref, bound, f"long-key prefill H={H} clean=0")


def test_paged_equals_prefill_bitwise_and_page_order_invariant():
    lens = [500]
    a = workloads.decode_case(30, seq_lens=lens, H=32, next_n=4, spare_pages=5)
    out_a, cache_a, qv, qs = _paged_gpu(a)
    # same data, another page permutation
    b = dict(a)
    rng = np.random.default_rng(99)
    perm = rng.permutation(a["num_pages"]).astype(np.int32)
    b["block_table"] = perm[a["block_table"]]
    b["slot_mapping"] = perm[a["slot_mapping"] // 64].astype(np.int64) * 64 + a["slot_mapping"] % 64
    out_b, *_ = _paged_gpu(b)
    assert np.array_equal(host(out_a), host(out_b))
    # dense kernel over the gathered K, same rows and visibility
    kv, ksc = mx.gather(cache_a, dev(a["block_table"]), dev(a["context_lens"]),
                        dev(np.zeros(1, np.int64)), 500, 500)
    ke = olog.decode_visible_end(a["context_lens"], 4).astype(np.int32)
    dense = mx.logits_prefill(qv, qs, kv, ksc, dev(a["w"]), None, dev(ke))
    torch.cuda.synchronize()
    assert np.array_equal(host(dense), host(out_a))


def test_power_of_two_scaling_and_determinism():
    case = workloads.prefill_case(40, T=20, S=400, H=32, dtype="f32")
    out1, *_ = _prefill_gpu(case)
    out2, *_ = _prefill_gpu(case)
    assert np.array_equal(host(out1), host(out2))
    scaled = dict(case)
    k = case["k"].copy()
    k[123] *= np.float32(2.0 ** 5)
    scaled["k"] = k
    out3, *_ = _prefill_gpu(scaled)
    g1, g3 = host(out1), host(out3)
    vis = np.isfinite(g1[:, 123])
    assert np.array_equal(g3[vis, 123], g1[vis, 123] * np.float32(32.0))
    others = np.ones(400, bool)
    others[123] = False
    assert np.array_equal(g3[:, others], g1[:, others])


def test_zero_k_gives_zero_logits():
    case = workloads.prefill_case(41, T=8, S=128, H=16, dtype="f32")
    case["k"] = np.zeros_like(case["k"])
    out, *_ = _prefill_gpu(case)
    g = host(out)
    vis = np.isfinite(g)
    assert vis.sum() == sum(case["ke"] - case["ks"]) and np.all(g[vis] == 0.0)
