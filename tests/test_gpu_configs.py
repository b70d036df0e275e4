"""GPU parity at the full workload sizes, in the launch configuration the bench
times: the whole cache is built on the GPU, logits are computed for every row,
and the oracle checks sampled sequences/rows one by one, plus exact top-k sets
on every row (oracle top-k of the GPU's own logits) and the end-to-end margin
rule on the sampled rows."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import logits as olog, mxfp4 as omx, paged_cache as opc
from tests.gpu_helpers import (check_logits, check_topk_end_to_end, check_topk_sets, dev, exact,  # noqa: F401
                               host, new_cache, oracle_q)

pytestmark = pytest.mark.gpu


def _exact_sets(g_logits, ks, ke, k, out_idx):
    check_topk_sets(g_logits, ks, ke, k, out_idx)


def _end_to_end(ref_rows, bound_rows, ks, ke, k, idx_rows):
    return check_topk_end_to_end(ref_rows, bound_rows, ks, ke, k, idx_rows)


def _decode_case_check(case, sample_seqs, check_bytes_tokens=None, split_topk=False):
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    qv, qs = mx.quantize(dev(case["q"]))
    W = case["width"]
    R = len(case["context_lens"]) * case["next_n"]
    logits = torch.empty((R, W), dtype=torch.float32, device="cuda")
    mx.logits_paged(qv, qs, dev(case["w"]), cache, dev(case["block_table"]),
                    dev(case["context_lens"]), case["next_n"], W, logits=logits, clean=True)
    ke = olog.decode_visible_end(case["context_lens"], case["next_n"]).astype(np.int32)
    idx = mx.topk(logits, None, dev(ke), case["topk"])
    # the workspace top-k the long-context bench times (long rows split over workgroups)
    idx_ws = mx.topk_ws(logits, None, dev(ke), case["topk"], mx.topk_workspace(R, W)) \
        if split_topk else None
    torch.cuda.synchronize()
    cache_np = host(cache)
    if check_bytes_tokens is not None:
        # sampled tokens: cached bytes equal the oracle's encoding of their K rows
        slots = case["slot_mapping"][check_bytes_tokens]
        codes, scales = omx.quantize_rows(exact({"k": case["k"][check_bytes_tokens], "dtype": case["dtype"]}, "k"))
        for i, sl in enumerate(slots):
            c, s = opc.read_token(cache_np, int(sl) // 64, int(sl) % 64)
            assert np.array_equal(c, codes[i]) and np.array_equal(s, scales[i])
    qc, qsc = oracle_q(case)
    assert np.array_equal(host(qv), qc) and np.array_equal(host(qs), qsc)
    ref, bound = olog.paged_mqa_logits(qc, qsc, case["w"], cache_np, case["block_table"],
                                       case["context_lens"], case["next_n"], W, seqs=sample_seqs,
                                       with_bound=True)
    g = host(logits)
    rows = np.concatenate([np.arange(b * case["next_n"], (b + 1) * case["next_n"]) for b in sample_seqs])
    check_logits(g[rows], ref[rows], bound[rows], case["name"])
    out_idx = host(idx)
    _exact_sets(g, np.zeros(R, np.int32), ke, case["topk"], out_idx)
    if idx_ws is not None:
        ws_idx = host(idx_ws)
        _exact_sets(g, np.zeros(R, np.int32), ke, case["topk"], ws_idx)
        _end_to_end(ref[rows], bound[rows], np.zeros(len(rows), np.int32), ke[rows],
                    case["topk"], ws_idx[rows])
    return _end_to_end(ref[rows], bound[rows], np.zeros(len(rows), np.int32), ke[rows],
                       case["topk"], out_idx[rows])


def test_paged_decode_16x8192():
    case = workloads.paged_decode()
    _decode_case_check(case, sample_seqs=[0, 7, 15])


def test_long_context_decode_64_seqs():
    case = workloads.long_decode()
    rng = np.random.default_rng(123)
    toks = rng.choice(len(case["slot_mapping"]), 4096, replace=False)
    _decode_case_check(case, sample_seqs=[int(np.argmax(case["context_lens"])), 5],
                       check_bytes_tokens=toks, split_topk=True)


def test_long_context_decode_next_n2():
    """Two query rows per sequence (multi-token decode) on the long-context batch
    -- the same lengths, pages and K as above, rows seeing L - 1 and L tokens --
    through the kernel the bench times for next_n = 2."""
    case = workloads.decode_case(2, batch=64, len_range=(32768, 131072), H=32, next_n=2,
                                 k_dist="lognormal", topk=2048, spare_pages=64, width=131072,
                                 name="long_decode_64xU32K-128K_next_n2")
    rng = np.random.default_rng(124)
    toks = rng.choice(len(case["slot_mapping"]), 1024, replace=False)
    _decode_case_check(case, sample_seqs=[int(np.argmax(case["context_lens"])), 11],
                       check_bytes_tokens=toks, split_topk=True)


def _prefill_case_check(case, sample_rows):
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                        dev(case["cu_seq_offsets"]), case["S"], case["S"])
    qv, qs = mx.quantize(dev(case["q"]))
    T, S = case["T"], case["S"]
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    mx.logits_prefill(qv, qs, kv, ksc, dev(case["w"]), dev(case["ks"]), dev(case["ke"]),
                      logits=logits, clean=True)
    idx = mx.topk(logits, dev(case["ks"]), dev(case["ke"]), case["topk"])
    torch.cuda.synchronize()
    kc, kscale = omx.quantize_rows(exact(case, "k"))
    assert np.array_equal(host(kv), kc) and np.array_equal(host(ksc), kscale)
    rows = np.asarray(sample_rows)
    H = case["H"]
    qc, qsc = omx.quantize_rows(exact({"q": case["q"][rows], "dtype": case["dtype"]}, "q"))
    qc, qsc = qc.reshape(-1, H, 64), qsc.reshape(-1, H, 4)
    assert np.array_equal(host(qv)[rows], qc) and np.array_equal(host(qs)[rows], qsc)
    ref, bound = olog.mqa_logits(qc, qsc, kc, kscale, case["w"][rows], case["ks"][rows],
                                 case["ke"][rows], chunk=4, with_bound=True)
    g_rows = logits[torch.as_tensor(rows, device="cuda")]
    g = host(g_rows)
    check_logits(g, ref, bound, case["name"])
    # top-k: exact sets for the sampled rows (oracle top-k of the GPU logits),
    # and the end-to-end margin rule against the oracle's logits
    sub_idx = host(idx)[rows]
    _exact_sets(g, case["ks"][rows], case["ke"][rows], case["topk"], sub_idx)
    return _end_to_end(ref, bound, case["ks"][rows], case["ke"][rows], case["topk"], sub_idx)


def test_prefill_chunk_8192():
    case = workloads.prefill_chunk()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 8191], rng.choice(8192, 59, replace=False)]))
    _prefill_case_check(case, rows)


def test_long_prefill_16384x122880_sampled_rows():
    case = workloads.long_prefill()
    rows = case["sample_rows"][::8]          # 32 of the 256 sampled rows, t = 0 and t = T-1 included
    rows = np.unique(np.concatenate([rows, [0, case["T"] - 1]]))
    _prefill_case_check(case, rows)
