"""HIP graph capture of one decode step (insert -> q quantize -> paged logits ->
top-k, and its one-launch forms for the MXFP4 and FP8 caches) and of the
LDS-staged FP8 prefill: every replay, with eager work and host synchronization
between the replays, must equal the eager result bit for bit (the pages' CUDA
Graph tests, P2 "Validation")."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import logits as olog
from tests.gpu_helpers import dev, host, new_cache

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager():
    case = workloads.decode_case(50, seq_lens=[1000, 4000, 64, 2500], H=32, next_n=1, topk=512)
    B, W = 4, case["width"]
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    last = np.cumsum(case["context_lens"]) - 1                 # the newest token of each sequence
    k_new = dev(case["k"][last])
    slot_new = dev(case["slot_mapping"][last])
    q = dev(case["q"])
    w = dev(case["w"])
    bt = dev(case["block_table"])
    ctx = dev(case["context_lens"])
    ke = dev(olog.decode_visible_end(case["context_lens"], 1).astype(np.int32))
    qv = torch.empty((B, 32, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, 32, 4), dtype=torch.uint8, device="cuda")
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")

    def step():
        mx.insert(k_new, slot_new, cache)
        mx.quantize(q, qv, qs)
        mx.logits_paged(qv, qs, w, cache, bt, ctx, 1, W, logits=logits, clean=True)
        mx.topk(logits, None, ke, 512, out=idx)

    step()                                                     # warm-up (and gate) outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(1)
    for rep in range(3):
        newq = workloads.bf16_bits(rng.standard_normal(case["q"].shape).astype(np.float32))
        q.copy_(dev(newq))
        g.replay()
        torch.cuda.synchronize()
        got_logits, got_idx, got_cache = host(logits).copy(), host(idx).copy(), host(cache).copy()
        _ = torch.randn(1000, device="cuda").sum().item()       # unrelated eager work in between
        step()                                                 # eager reference, same inputs
        torch.cuda.synchronize()
        assert np.array_equal(got_logits, host(logits)), rep
        assert np.array_equal(got_idx, host(idx)), rep
        assert np.array_equal(got_cache, host(cache)), rep


def test_fused_step_and_merge_graph_replays_match_eager():
    # the decode step as the bench runs it (one-launch insert + quantize,
    # next_n 2), followed by a context-parallel merge of two lists
    case = workloads.decode_case(51, seq_lens=[3000, 700, 2100], H=32, next_n=2, topk=256)
    B, W = 3, case["width"]
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    last = np.cumsum(case["context_lens"]) - 1
    k_new, slot_new = dev(case["k"][last]), dev(case["slot_mapping"][last])
    q, w = dev(case["q"]), dev(case["w"])
    bt, ctx = dev(case["block_table"]), dev(case["context_lens"])
    ke = dev(olog.decode_visible_end(case["context_lens"], 2).astype(np.int32))
    qv = torch.empty((2 * B, 32, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((2 * B, 32, 4), dtype=torch.uint8, device="cuda")
    logits = torch.empty((2 * B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((2 * B, 256), dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(4)
    mv = dev(rng.standard_normal((2, 2 * B, 256)).astype(np.float32))
    mi = dev(np.stack([np.stack([rng.permutation(4000)[:256] for _ in range(2 * B)]) for _ in range(2)])
             .astype(np.int32))
    mout = torch.empty((2 * B, 256), dtype=torch.int32, device="cuda")

    def step():
        mx.insert_quantize(k_new, slot_new, cache, q, qv, qs)
        mx.logits_paged(qv, qs, w, cache, bt, ctx, 2, W, logits=logits, clean=False)
        mx.topk(logits, None, ke, 256, out=idx)
        mx.topk_merge(mv, mi, 16, 256, out=mout)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        q.copy_(dev(workloads.bf16_bits(rng.standard_normal(case["q"].shape).astype(np.float32))))
        mv.copy_(dev(rng.standard_normal((2, 2 * B, 256)).astype(np.float32)))
        g.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in (idx, cache, mout)]
        got_vis = [host(logits)[r, :int(host(ke)[r])].copy() for r in range(2 * B)]
        _ = torch.randn(1000, device="cuda").sum().item()
        step()
        torch.cuda.synchronize()
        for a, t in zip(got, (idx, cache, mout)):
            assert np.array_equal(a, host(t)), rep
        for r in range(2 * B):
            assert np.array_equal(got_vis[r], host(logits)[r, :int(host(ke)[r])]), (rep, r)


def test_one_launch_decode_step_graph_replays_match_eager():
    # idx_logits_paged_insert + idx_topk captured; new K rows and queries change between replays
    case = workloads.decode_case(52, seq_lens=[1000, 4000, 64, 2500, 193], H=32, next_n=1, topk=512)
    B, W = 5, case["width"]
    cache = new_cache(case["num_pages"], fill=0)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    last = np.cumsum(case["context_lens"]) - 1
    k_new = dev(case["k"][last])
    q = dev(case["q"])
    w = dev(case["w"])
    bt = dev(case["block_table"])
    ctx = dev(case["context_lens"])
    ke = dev(olog.decode_visible_end(case["context_lens"], 1).astype(np.int32))
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")

    def step():
        mx.logits_paged_insert(q, k_new, w, cache, bt, ctx, 1, W, logits=logits, clean=True)
        mx.topk(logits, None, ke, 512, out=idx)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(3)
    for rep in range(3):
        q.copy_(dev(workloads.bf16_bits(rng.standard_normal(case["q"].shape).astype(np.float32))))
        k_new.copy_(dev(workloads.bf16_bits(rng.standard_normal((B, 128)).astype(np.float32))))
        g.replay()
        torch.cuda.synchronize()
        got_logits, got_idx, got_cache = host(logits).copy(), host(idx).copy(), host(cache).copy()
        _ = torch.randn(1000, device="cuda").sum().item()
        step()
        torch.cuda.synchronize()
        assert np.array_equal(got_logits, host(logits)), rep
        assert np.array_equal(got_idx, host(idx)), rep
        assert np.array_equal(got_cache, host(cache)), rep


def test_fp8_one_launch_step_graph_replays_match_eager():
    # idx_logits_paged_insert_fp8 + idx_topk captured; queries and new K rows change
    case = workloads.decode_case(53, seq_lens=[700, 3000, 65, 1800], H=32, next_n=1, topk=256)
    B, W = 4, case["width"]
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    last = np.cumsum(case["context_lens"]) - 1
    k_new = dev(case["k"][last])
    q, w = dev(case["q"]), dev(case["w"])
    bt, ctx = dev(case["block_table"]), dev(case["context_lens"])
    ke = dev(olog.decode_visible_end(case["context_lens"], 1).astype(np.int32))
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, 256), dtype=torch.int32, device="cuda")

    def step():
        mx.logits_paged_insert_fp8(q, k_new, w, cache, bt, ctx, 1, W, logits=logits, clean=True)
        mx.topk(logits, None, ke, 256, out=idx)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(5)
    for rep in range(3):
        q.copy_(dev(workloads.bf16_bits(rng.standard_normal(case["q"].shape).astype(np.float32))))
        k_new.copy_(dev(workloads.bf16_bits(rng.standard_normal((B, 128)).astype(np.float32))))
        g.replay()
        torch.cuda.synchronize()
        got = host(logits).copy(), host(idx).copy(), host(cache).copy()
        _ = torch.randn(1000, device="cuda").sum().item()
        step()
        torch.cuda.synchronize()
        for a, b in zip(got, (host(logits), host(idx), host(cache))):
            assert np.array_equal(a, b), rep


def test_fp8_prefill_graph_replays_match_eager():
    # the LDS-staged FP8 prefill (barriers, buffer-to-LDS copies) captured, queries change
    T, S, H = 40, 17000, 64
    case = workloads.prefill_case(54, T=T, S=S, H=H)
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                            dev(case["cu_seq_offsets"]), S, S)
    q, w = dev(case["q"]), dev(case["w"])
    ks, ke = dev(case["ks"]), dev(case["ke"])
    qv, _, wf = mx.quantize_fp8(q, weights=w)
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")

    def step():
        mx.logits_prefill_fp8(qv, wf, kv, ksc, ks, ke, logits=logits, clean=True)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(6)
    for rep in range(3):
        qn = dev(workloads.bf16_bits(rng.standard_normal(case["q"].shape).astype(np.float32)))
        qv2, _, wf2 = mx.quantize_fp8(qn, weights=w)
        qv.copy_(qv2)
        wf.copy_(wf2)
        g.replay()
        torch.cuda.synchronize()
        got = host(logits).copy()
        _ = torch.randn(1000, device="cuda").sum().item()
        step()
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), host(logits).view(np.uint32)), rep
