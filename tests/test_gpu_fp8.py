"""GPU parity of the FP8 (E4M3) indexer cache, the format the MXFP4 cache replaces
(P1 "Benefit": 132 bytes per token), against the FP8 oracle (oracle/fp8.py):
codes, scales, folded weights, cache and gathered bytes bit-exact; logits within
the FP8 rule of the logits tolerance; top-k exact on identical input and by the
margin rule end to end.  Inputs are the seeded workloads of the MXFP4 tests."""

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import fp8 as of8, logits as olog, tolerance
from tests.gpu_helpers import (CANARY, check_logits, check_topk_end_to_end, check_topk_sets, dev,
                               exact, host)

pytestmark = pytest.mark.gpu

F8 = tolerance.ABS_FACTOR_FP8


def _rows_with_amax_448(vals):
    """Rows of 128: element 0 is 448 (so s = 1 exactly), the rest are `vals`."""
    n = -(-len(vals) // 127)
    rows = np.zeros((n, 128), np.float32)
    rows[:, 0] = 448.0
    flat = np.zeros(n * 127, np.float32)
    flat[:len(vals)] = vals
    rows[:, 1:] = flat.reshape(n, 127)
    return rows


def _gpu_quant(x_np, dtype, round_scale, w=None):
    if dtype == "bf16":
        bits = workloads.bf16_bits(x_np)
        xt = dev(bits)
        xe = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        xt = dev(np.ascontiguousarray(x_np, dtype=np.float32))
        xe = np.asarray(x_np, np.float32).astype(np.float64)
    res = mx.quantize_fp8(xt, round_scale=round_scale, weights=None if w is None else dev(w))
    torch.cuda.synchronize()
    return [host(t) for t in res], xe


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_every_bf16_pattern_bit_exact(dtype):
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    vals = bits[np.isfinite(bits) & (np.abs(bits) <= 448)]
    rows = _rows_with_amax_448(vals)
    (codes, scales), xe = _gpu_quant(rows, dtype, False)
    want_c, want_s = of8.quantize_rows(xe)
    assert np.all(scales == 1.0)
    bad = np.argwhere(codes != want_c)
    assert len(bad) == 0, f"{len(bad)} codes differ, e.g. x={xe[tuple(bad[0])]} gpu {codes[tuple(bad[0])]:#x} oracle {want_c[tuple(bad[0])]:#x}"
    assert np.array_equal(scales, want_s)


def test_fp8_midpoints_and_neighbours_bit_exact():
    grid = np.array([of8.e4m3_value(c) for c in range(0x7F)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(999))])
    vals = np.concatenate([vals, -vals, np.float32([0.0, -0.0, 1e-30, -1e-30, 2 ** -10])])
    rows = _rows_with_amax_448(vals)
    (codes, scales), xe = _gpu_quant(rows, "f32", False)
    want_c, _ = of8.quantize_rows(xe)
    assert np.array_equal(codes, want_c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_random_rows_scales_and_folded_weights(dtype, round_scale):
    rng = np.random.default_rng(40 + round_scale)
    x = workloads.draw_values(rng, (3000, 128), "lognormal")
    x *= np.exp2(rng.integers(-30, 30, size=(3000, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] = 0.0
    x[2, 5] = 1e-44                       # amax / 448 underflows: the floor
    x[3, :] = 448.0 * 2.0 ** 40
    w = rng.random(3000, dtype=np.float32)
    (codes, scales, wout), xe = _gpu_quant(x, dtype, round_scale, w)
    want_c, want_s = of8.quantize_rows(xe, round_scale=round_scale)
    assert np.array_equal(scales.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(codes, want_c), np.argwhere(codes != want_c)[:4].tolist()
    assert np.array_equal(wout.view(np.uint32), of8.fold_weights(w, want_s).view(np.uint32))


def _fp8_decode(case, round_scale=False, bt=None, slots=None):
    """Insert the case's K into an FP8 cache (canary-filled) on the GPU and return
    (cache, oracle cache)."""
    num_pages = case["num_pages"]
    cache = torch.full((num_pages, 64 * 132), CANARY, dtype=torch.uint8, device="cuda")
    sm = case["slot_mapping"] if slots is None else slots
    mx.insert_fp8(dev(case["k"]), dev(sm), cache, round_scale=round_scale)
    torch.cuda.synchronize()
    ref = of8.insert(np.full((num_pages, 64 * 132), CANARY, np.uint8), exact(case, "k"), sm,
                     round_scale=round_scale)
    return cache, ref


@pytest.mark.parametrize("round_scale", [False, True])
def test_fp8_insert_whole_cache_and_gather(round_scale):
    case = workloads.decode_case(41, seq_lens=[1, 63, 64, 65, 300, 0, 130], H=16, dtype="bf16",
                                 spare_pages=3, width=320)
    slots = case["slot_mapping"].copy()
    slots[5] = -1                                        # written by nobody
    slots[9] = case["num_pages"] * 64 + 3                # beyond the cache: skipped
    cache, ref = _fp8_decode(case, round_scale, slots=slots)
    got = host(cache)
    assert np.array_equal(got, ref), np.argwhere(got != ref)[:4].tolist()
    lens = case["context_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    total = int(lens.sum())
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(lens), dev(cu), int(lens.max()), total)
    torch.cuda.synchronize()
    rc, rs = of8.gather(ref, case["block_table"], lens, cu, total)
    assert np.array_equal(host(kv), rc) and np.array_equal(host(ksc).view(np.uint32), rs.view(np.uint32))


def _fp8_query(case, round_scale=False):
    """GPU FP8 query (values + folded weights) and the oracle's."""
    H = case["q"].shape[1]
    qv, qs, wf = mx.quantize_fp8(dev(case["q"]), round_scale=round_scale, weights=dev(case["w"]))
    torch.cuda.synchronize()
    qc, qsc = of8.quantize_rows(exact(case, "q"), round_scale=round_scale)
    wref = of8.fold_weights(case["w"].reshape(-1), qsc).reshape(-1, H)
    assert np.array_equal(host(qv).reshape(-1, 128), qc)
    assert np.array_equal(host(wf).view(np.uint32), wref.view(np.uint32))
    return qv, wf, qc.reshape(-1, H, 128), wref


@pytest.mark.parametrize("H,next_n,lens,clean", [
    (32, 1, [1, 63, 64, 65, 300, 0, 191, 192, 193], True),
    (16, 2, [2, 5, 64, 129, 250], False),
    (64, 3, [700, 3, 129], True),
    (128, 1, [100, 1000], True),
    (48, 4, [67, 4, 256], False),
])
def test_fp8_paged_logits(H, next_n, lens, clean):
    case = workloads.decode_case(H + next_n, seq_lens=lens, H=H, next_n=next_n, dtype="bf16",
                                 spare_pages=2, width=max(lens) + 40)
    cache, ref_cache = _fp8_decode(case)
    qv, wf, qc, wref = _fp8_query(case)
    R, W = qv.shape[0], case["width"]
    logits = torch.full((R, W), float("nan"), dtype=torch.float32, device="cuda")
    mx.logits_paged_fp8(qv, wf, cache, dev(case["block_table"]), dev(case["context_lens"]), next_n,
                        W, logits=logits, clean=clean)
    torch.cuda.synchronize()
    ref, bound = of8.paged_mqa_logits(qc, wref, ref_cache, case["block_table"],
                                      case["context_lens"], next_n, W, with_bound=True)
    g = host(logits)
    if clean:
        check_logits(g, ref, bound, f"fp8 paged H={H}", abs_factor=F8)
    else:
        for r in range(R):
            vis = np.isfinite(ref[r])
            check_logits(g[r][vis][None], ref[r][vis][None], bound[r][vis][None], f"row {r}", F8)
            assert np.all(np.isnan(g[r][~vis])), "clean=0 wrote a masked column"


@pytest.mark.parametrize("H,T,S,clean", [(32, 200, 700, True), (64, 70, 1300, False),
                                          (16, 40, 100, True), (128, 30, 300, True),
                                          (48, 50, 900, False), (64, 24, 17000, True),
                                          (32, 20, 20000, False)])
def test_fp8_prefill_logits_and_paged_bitwise(H, T, S, clean):
    rng = np.random.default_rng(H + T)
    case = workloads.prefill_case(H * 7 + S, T=T, S=S, H=H, dtype="bf16")
    ks = rng.integers(0, S // 2, size=T).astype(np.int32)
    ke = np.minimum(S, ks + rng.integers(0, S, size=T)).astype(np.int32)
    ke[0], ks[0] = S, 0
    cache, ref_cache = _fp8_decode(case)
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                            dev(case["cu_seq_offsets"]), S, S)
    qv, wf, qc, wref = _fp8_query(case)
    logits = torch.full((T, S + 3), float("nan"), dtype=torch.float32, device="cuda")
    mx.logits_prefill_fp8(qv, wf, kv, ksc, dev(ks), dev(ke), logits=logits, clean=clean)
    torch.cuda.synchronize()
    kc, kscale = of8.quantize_rows(exact(case, "k"))
    ref, bound = of8.mqa_logits(qc, wref, kc, kscale, ks, ke, width=S, with_bound=True)
    g = host(logits)[:, :S]
    if clean:
        check_logits(g, ref, bound, f"fp8 prefill H={H}", abs_factor=F8)
    else:
        for t in range(T):
            vis = np.isfinite(ref[t])
            check_logits(g[t][vis][None], ref[t][vis][None], bound[t][vis][None], f"row {t}", F8)
    assert np.all(np.isnan(host(logits)[:, S:])), "a column past S was written"


def test_fp8_paged_equals_prefill_bitwise():
    """One sequence of 900 tokens, next_n = 4: the paged rows equal the dense rows
    over the gathered K, bit for bit (same operands, same summation order)."""
    case = workloads.decode_case(44, seq_lens=[900], H=32, next_n=4, dtype="bf16", width=900)
    cache, _ = _fp8_decode(case)
    qv, wf, _, _ = _fp8_query(case)
    paged = mx.logits_paged_fp8(qv, wf, cache, dev(case["block_table"]), dev(case["context_lens"]),
                                4, 900, clean=True)
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(case["context_lens"]),
                            dev(np.zeros(1, np.int64)), 900, 900)
    ke = olog.decode_visible_end(case["context_lens"], 4).astype(np.int32)
    dense = mx.logits_prefill_fp8(qv, wf, kv, ksc, None, dev(ke), clean=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(paged).view(np.uint32), host(dense).view(np.uint32))


def test_fp8_paged_decode_16x8192_end_to_end():
    """The paged-decode workload on the FP8 cache: logits of sampled sequences vs
    the oracle, exact top-k sets on every row, the margin rule on sampled rows."""
    case = workloads.paged_decode()
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    qv, wf, qc, wref = _fp8_query(case)
    W = case["width"]
    logits = mx.logits_paged_fp8(qv, wf, cache, dev(case["block_table"]),
                                 dev(case["context_lens"]), 1, W, clean=True)
    ke = olog.decode_visible_end(case["context_lens"], 1).astype(np.int32)
    idx = mx.topk(logits, None, dev(ke), case["topk"])
    torch.cuda.synchronize()
    seqs = [0, 9, 15]
    ref_cache = of8.write_rows(np.zeros((case["num_pages"], 64 * 132), np.uint8),
                               *of8.quantize_rows(exact(case, "k")), case["slot_mapping"])
    assert np.array_equal(host(cache), ref_cache)
    ref, bound = of8.paged_mqa_logits(qc, wref, ref_cache, case["block_table"],
                                      case["context_lens"], 1, W, seqs=seqs, with_bound=True)
    g = host(logits)
    check_logits(g[seqs], ref[seqs], bound[seqs], "fp8 16x8192", abs_factor=F8)
    out = host(idx)
    zeros = np.zeros(len(ke), np.int32)
    check_topk_sets(g, zeros, ke, case["topk"], out, "fp8 16x8192")
    check_topk_end_to_end(ref[seqs], bound[seqs], zeros[seqs], ke[seqs], case["topk"], out[seqs],
                          "fp8 16x8192", abs_factor=F8)


def test_fp8_prefill_chunk_8192_sampled_rows():
    case = workloads.prefill_chunk()
    T, S, H = case["T"], case["S"], case["H"]
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                            dev(case["cu_seq_offsets"]), S, S)
    qv, _, wf = mx.quantize_fp8(dev(case["q"]), weights=dev(case["w"]))
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    mx.logits_prefill_fp8(qv, wf, kv, ksc, dev(case["ks"]), dev(case["ke"]), logits=logits,
                          clean=True)
    idx = mx.topk(logits, dev(case["ks"]), dev(case["ke"]), case["topk"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 2048, 5000, 8191])
    kc, kscale = of8.quantize_rows(exact(case, "k"))
    assert np.array_equal(host(kv), kc) and np.array_equal(host(ksc), kscale)
    qc, qsc = of8.quantize_rows(exact({"q": case["q"][rows], "dtype": case["dtype"]}, "q"))
    wref = of8.fold_weights(case["w"][rows].reshape(-1), qsc).reshape(-1, H)
    ref, bound = of8.mqa_logits(qc.reshape(-1, H, 128), wref, kc, kscale, case["ks"][rows],
                                case["ke"][rows], with_bound=True)
    g = host(logits[torch.as_tensor(rows, device="cuda")])
    check_logits(g, ref, bound, "fp8 prefill chunk", abs_factor=F8)
    sub = host(idx)[rows]
    check_topk_sets(g, case["ks"][rows], case["ke"][rows], case["topk"], sub, "fp8 chunk")
    check_topk_end_to_end(ref, bound, case["ks"][rows], case["ke"][rows], case["topk"], sub,
                          "fp8 chunk", abs_factor=F8)


def test_fp8_long_context_decode_sampled():
    """The long-context batch (64 x U[32K, 128K], lognormal K block scales) on the
    FP8 cache in the launch configuration the bench times (clean = 0, the split
    top-k): the cached bytes of 4096 sampled tokens against the oracle's encoding,
    the logits of the longest sequence and one more against the oracle (over the
    GPU's cache bytes), columns past each context untouched, and the top-k sets
    of those rows exact and by the margin rule."""
    case = workloads.long_decode()
    B, W = len(case["context_lens"]), case["width"]
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    qv, wf, qc, wref = _fp8_query(case)
    logits = torch.full((B, W), float("nan"), dtype=torch.float32, device="cuda")
    mx.logits_paged_fp8(qv, wf, cache, dev(case["block_table"]), dev(case["context_lens"]), 1, W,
                        logits=logits, clean=False)
    ke = case["context_lens"].astype(np.int32)
    idx = mx.topk_ws(logits, None, dev(ke), case["topk"], mx.topk_workspace(B, W))
    torch.cuda.synchronize()
    cache_np = host(cache)
    flat = cache_np.reshape(-1)
    toks = np.random.default_rng(321).choice(len(case["slot_mapping"]), 4096, replace=False)
    codes, scales = of8.quantize_rows(exact({"k": case["k"][toks], "dtype": case["dtype"]}, "k"))
    sbytes = scales.astype("<f4").view(np.uint8).reshape(-1, 4)
    for i, sl in enumerate(case["slot_mapping"][toks]):
        page, off = divmod(int(sl), 64)
        v0, s0 = of8.value_offset(page, off), of8.scale_offset(page, off)
        assert np.array_equal(flat[v0:v0 + 128], codes[i]), f"token {toks[i]} values"
        assert np.array_equal(flat[s0:s0 + 4], sbytes[i]), f"token {toks[i]} scale"
    seqs = [int(np.argmax(case["context_lens"])), 5]
    ref, bound = of8.paged_mqa_logits(qc, wref, cache_np, case["block_table"],
                                      case["context_lens"], 1, W, seqs=seqs, with_bound=True)
    g = host(logits)
    for b in seqs:
        L = int(case["context_lens"][b])
        assert np.all(np.isnan(g[b, L:])), f"sequence {b}: columns past the context written"
    check_logits(np.where(np.isnan(g[seqs]), -np.inf, g[seqs]), ref[seqs], bound[seqs],
                 "fp8 long-context decode", abs_factor=F8)
    out = host(idx)[seqs]
    zeros = np.zeros(len(seqs), np.int32)
    check_topk_sets(g[seqs], zeros, ke[seqs], case["topk"], out, "fp8 long-context")
    check_topk_end_to_end(ref[seqs], bound[seqs], zeros, ke[seqs], case["topk"], out,
                          "fp8 long-context", abs_factor=F8)


def test_fp8_long_prefill_sampled_rows():
    """The long prefill (16,384 queries over 122,880 cached tokens, 64 heads,
    Student-t inputs) on the FP8 cache in the bench's launch configuration
    (clean = 0): gathered K bytes against the oracle's encoding, the folded
    weights of 34 sampled rows, their logits within [ks, ke) and their top-k."""
    case = workloads.long_prefill()
    T, S, H = case["T"], case["S"], case["H"]
    cache = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather_fp8(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                            dev(case["cu_seq_offsets"]), S, S)
    del cache
    qv, _, wf = mx.quantize_fp8(dev(case["q"]), weights=dev(case["w"]))
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    mx.logits_prefill_fp8(qv, wf, kv, ksc, dev(case["ks"]), dev(case["ke"]), logits=logits,
                          clean=False)
    idx = mx.topk(logits, dev(case["ks"]), dev(case["ke"]), case["topk"])
    torch.cuda.synchronize()
    kc, kscale = of8.quantize_rows(exact(case, "k"))
    assert np.array_equal(host(kv), kc) and np.array_equal(host(ksc).view(np.uint32),
                                                           kscale.view(np.uint32))
    rows = np.unique(np.concatenate([case["sample_rows"][::8], [0, T - 1]]))
    qc, qsc = of8.quantize_rows(exact({"q": case["q"][rows], "dtype": case["dtype"]}, "q"))
    wref = of8.fold_weights(case["w"][rows].reshape(-1), qsc).reshape(-1, H)
    rt = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(host(qv[rt]).reshape(-1, 128), qc)
    assert np.array_equal(host(wf[rt]).view(np.uint32), wref.view(np.uint32))
    ref, bound = of8.mqa_logits(qc.reshape(-1, H, 128), wref, kc, kscale, case["ks"][rows],
                                case["ke"][rows], chunk=4, with_bound=True)
    g = host(logits[rt])
    ks_r, ke_r = case["ks"][rows], case["ke"][rows]
    cols = np.arange(S)[None, :]
    inside = (cols >= ks_r[:, None]) & (cols < ke_r[:, None])
    check_logits(np.where(inside, g, -np.inf), ref, bound, "fp8 long prefill", abs_factor=F8)
    sub = host(idx)[rows]
    check_topk_sets(np.where(inside, g, -np.inf), ks_r, ke_r, case["topk"], sub, "fp8 long prefill")
    check_topk_end_to_end(ref, bound, ks_r, ke_r, case["topk"], sub, "fp8 long prefill",
                          abs_factor=F8)
