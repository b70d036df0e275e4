"""GPU parity of the one-launch decode step (idx_logits_paged_insert): the cache
bytes and logits must equal, bit for bit, those of the separate calls --
idx_insert of the new tokens into their block-table slots, idx_quantize of q,
idx_logits_paged -- and they are also held to the oracle directly: the whole
cache against the oracle's insert of every token, the logits of sampled
sequences at the logits tolerance, and the top-k sets of those rows (the
16 x 8192 bf16 step the bench times, a bf16 next_n = 2 step, and a small fp32
step)."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import logits as olog, paged_cache as opc
from tests.gpu_helpers import (CANARY, check_logits, check_topk_end_to_end, check_topk_sets, dev,
                               exact, host, new_cache, oracle_q, split_new_tokens)

pytestmark = pytest.mark.gpu


def _both(case, clean=True, block_table=None):
    bt_np = case["block_table"] if block_table is None else block_table
    pre_slots, k_new, new_slots = split_new_tokens(case, bt_np)
    bt = dev(bt_np)
    ctx, w, q = dev(case["context_lens"]), dev(case["w"]), dev(case["q"])
    cache_a = new_cache(case["num_pages"])
    mx.insert(dev(case["k"]), dev(pre_slots), cache_a)
    cache_b = cache_a.clone()
    R, W = case["q"].shape[0], case["width"]
    poison = float("nan")
    la = torch.full((R, W), poison, dtype=torch.float32, device="cuda")
    lb = la.clone()
    # separate calls
    mx.insert(dev(k_new), dev(new_slots), cache_a)
    qv, qs = mx.quantize(q)
    mx.logits_paged(qv, qs, w, cache_a, bt, ctx, case["next_n"], W, logits=la, clean=clean)
    # one launch
    mx.logits_paged_insert(q, dev(k_new), w, cache_b, bt, ctx, case["next_n"], W, logits=lb,
                           clean=clean)
    torch.cuda.synchronize()
    return cache_a, cache_b, la, lb


def _assert_same(case, clean=True, block_table=None, what=""):
    cache_a, cache_b, la, lb = _both(case, clean, block_table)
    ca, cb = host(cache_a), host(cache_b)
    assert np.array_equal(ca, cb), f"{what}: cache bytes differ at {np.argwhere(ca != cb)[:4].tolist()}"
    a, b = host(la).view(np.uint32), host(lb).view(np.uint32)
    assert np.array_equal(a, b), f"{what}: logits differ at {np.argwhere(a != b)[:4].tolist()}"
    return cache_b, lb


def test_fused_tiny_against_oracle():
    case = workloads.decode_case(11, seq_lens=[1, 63, 64, 65, 300, 0], H=32, next_n=1,
                                 dtype="f32", width=337)
    cache, logits = _assert_same(case, what="tiny")
    qc, qs = oracle_q(case)
    ref, bound = olog.paged_mqa_logits(qc, qs, case["w"], host(cache), case["block_table"],
                                       case["context_lens"], 1, case["width"], with_bound=True)
    check_logits(host(logits), ref, bound, "fused tiny vs oracle")


@pytest.mark.parametrize("dtype,H,next_n,lens", [
    ("bf16", 32, 1, [1, 63, 64, 65, 300, 0, 191, 192, 193]),
    ("f32", 64, 3, [2, 5, 64, 129, 250, 191, 192, 193]),     # 2 < next_n: position -1 skipped
    ("bf16", 16, 2, [192, 193, 384, 385, 1, 2]),              # new tokens across wave boundaries
    ("bf16", 32, 4, [4, 3, 0, 64, 67, 300]),
    ("bf16", 32, 5, [5, 64, 130, 700, 2]),                     # rows not held in registers
    ("f32", 128, 1, [100, 17, 1000]),
    ("bf16", 48, 2, [127, 128, 1, 640]),
    ("bf16", 64, 16, [40, 200, 16]),
])
def test_fused_equals_separate_calls(dtype, H, next_n, lens):
    case = workloads.decode_case(H * 13 + next_n, seq_lens=lens, H=H, next_n=next_n, dtype=dtype,
                                 spare_pages=3, width=max(lens) + 45)
    _assert_same(case, what=f"{dtype} H={H} next_n={next_n}")


def test_fused_clean_false():
    case = workloads.decode_case(7, seq_lens=[65, 700, 3, 129], H=32, next_n=2, width=800)
    _assert_same(case, clean=False, what="clean=False")


def test_fused_invalid_table_entries_skip_the_page():
    case = workloads.decode_case(8, seq_lens=[130, 300, 64, 65], H=32, next_n=1, width=320)
    bt = case["block_table"].copy()
    bt[0, 2] = -1                          # the page of sequence 0's new token (position 129)
    bt[1, 4] = case["num_pages"] + 5       # the page of sequence 1's new token (position 299)
    _assert_same(case, block_table=bt, what="invalid entries")


def test_fused_paged_decode_16x8192():
    case = workloads.paged_decode()
    _assert_same(case, clean=False, what="16x8192")


def _against_oracle(case, sample_seqs, clean, what):
    """The one-launch step vs the oracle: the whole cache (every token, the new
    ones written by the step itself), the logits of ``sample_seqs`` at the
    logits tolerance, and exact / end-to-end top-k sets of those rows (the GPU
    top-k of the step's logits, as the bench runs it)."""
    cache, logits = _assert_same(case, clean=clean, what=what)
    ke = olog.decode_visible_end(case["context_lens"], case["next_n"]).astype(np.int32)
    R = len(ke)
    idx = mx.topk(logits, None, dev(ke), case["topk"])
    torch.cuda.synchronize()
    ref_cache = opc.insert(np.full((case["num_pages"], 64 * 68), CANARY, np.uint8),
                           exact(case, "k"), case["slot_mapping"])
    got_cache = host(cache)
    assert np.array_equal(got_cache, ref_cache), \
        f"{what}: cache bytes differ from the oracle at {np.argwhere(got_cache != ref_cache)[:4].tolist()}"
    qc, qs = oracle_q(case)
    ref, bound = olog.paged_mqa_logits(qc, qs, case["w"], ref_cache, case["block_table"],
                                       case["context_lens"], case["next_n"], case["width"],
                                       seqs=sample_seqs, with_bound=True)
    nn = case["next_n"]
    rows = np.concatenate([np.arange(b * nn, (b + 1) * nn) for b in sample_seqs])
    g = host(logits)
    if clean:
        check_logits(g[rows], ref[rows], bound[rows], what)
    else:
        # clean = 0 leaves masked columns untouched: compare the visible ones
        for r in rows:
            vis = np.isfinite(ref[r])
            check_logits(g[r][vis][None], ref[r][vis][None], bound[r][vis][None], f"{what} row {r}")
    out = host(idx)
    zeros = np.zeros(R, np.int32)
    gv = np.where(np.arange(g.shape[1])[None, :] < ke[:, None], g, -np.inf).astype(np.float32)
    check_topk_sets(gv[rows], zeros[rows], ke[rows], case["topk"], out[rows], what)
    return check_topk_end_to_end(ref[rows], bound[rows], zeros[rows], ke[rows], case["topk"],
                                 out[rows], what)


def test_fused_paged_decode_16x8192_against_oracle():
    """The bench's timed step (bf16, 16 x 8192, H 32, clean = 0, top-2048)."""
    case = workloads.paged_decode()
    _against_oracle(case, sample_seqs=[0, 5, 11, 15], clean=False, what="16x8192 vs oracle")


def test_fused_bf16_next_n2_against_oracle():
    case = workloads.decode_case(31, seq_lens=[4096, 3001, 8192, 129, 2], H=32, next_n=2,
                                 dtype="bf16", spare_pages=2, width=8192 + 64, topk=2048)
    _against_oracle(case, sample_seqs=[0, 1, 2, 3, 4], clean=True, what="bf16 next_n=2 vs oracle")


def test_fused_f32_next_n4_against_oracle():
    case = workloads.decode_case(32, seq_lens=[700, 64, 65, 3], H=64, next_n=4, dtype="f32",
                                 spare_pages=1, width=768, topk=64)
    _against_oracle(case, sample_seqs=[0, 1, 2, 3], clean=True, what="f32 next_n=4 vs oracle")
