#!/usr/bin/env python3
"""Benchmark of the MXFP4 paged indexer-cache hot path on one MI355X.

Decode step (the headline): batch 16, one query token each, 8192-token
contexts, 32 index heads, head_dim 128, MXFP4 cache (page 64, permuted block
table), top-2048.  One step = one launch of idx_logits_paged_insert (insert of
the 16 new tokens' K -- quantize + scatter --, MXFP4 quantization of the 16x32
query rows, paged logits over all 131072 cached tokens) -> top-2048 per row.
Metric: scored cache tokens per second = sum over rows of the visible context /
step time.  The same step as three calls (idx_insert_quantize, idx_logits_paged,
idx_topk) is timed beside it, and so is the step with the query RoPE fused into
its encode (idx_logits_paged_insert_rope: first 64 dims, neox pairs, each row
at its token's position).

Timing: the step is captured in HIP graphs; W untimed warm-up steps, then
exactly K steps between two device synchronizations.  The steps rotate over
`--sets` independent copies of the inputs (caches included) so that the 8.9 MB
cache is read from HBM rather than from the 256 MB Infinity Cache.

Also reported: per-kernel average durations (HIP events around graphs of
back-to-back launches of one kernel over the rotating sets, on the stream the
kernels run on), the roofline of the dominant kernel, the prefill-chunk
logits throughput (8192 x 8192 causal, 32 heads) against the FP4 MFMA peak,
and the CPU oracle timed on a bounded sample of the decode step.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=960)
    ap.add_argument("--warmup", type=int, default=96)
    ap.add_argument("--sets", type=int, default=96, help="rotating input sets (defeats the MALL)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="graph replays per kernel timing")
    ap.add_argument("--prefill", choices=["chunk", "none"], default="chunk")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context decode and long prefill measurements")
    ap.add_argument("--only", choices=["decode", "prefill", "long_decode", "long_prefill", "copy",
                                       "fp8", "kpool"],
                    help="run one section only and print its result (for profiler runs)")
    ap.add_argument("--eager", action="store_true",
                    help="launch kernels directly instead of replaying HIP graphs")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("PMC_DIR", "SECTION"),
                    help="write profiles/pmc_bytes_SECTION.json from rocprofv3 counter runs")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 indexer-cache measurements")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class DecodeSet:
    """One independent copy of every input and output of the decode step."""

    def __init__(self, base, case):
        import torch
        B, H = len(case["context_lens"]), case["H"]
        self.cache = base["cache"].clone()
        self.k_new = base["k_new"].clone()
        self.slot_new = base["slot_new"].clone()
        self.q = base["q"].clone()
        self.w = base["w"].clone()
        self.bt = base["bt"].clone()
        self.ctx = base["ctx"].clone()
        self.ke = base["ke"].clone()
        self.qv = torch.empty((B, H, 64), dtype=torch.uint8, device="cuda")
        self.qs = torch.empty((B, H, 4), dtype=torch.uint8, device="cuda")
        self.logits = torch.empty((B, case["width"]), dtype=torch.float32, device="cuda")
        self.idx = torch.empty((B, case["topk"]), dtype=torch.int32, device="cuda")
        self.cos, self.sin = base["cos"], base["sin"]      # read-only angle tables, shared


ROPE_DIM = 64          # decode step with the query RoPE fused: first 64 dims, neox pairs


def build_decode_sets(case, n_sets):
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads
    cache = torch.zeros((case["num_pages"], 64 * 68), dtype=torch.uint8, device="cuda")
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    last = np.cumsum(case["context_lens"]) - 1
    L = case["context_lens"].astype(np.int64)
    ke = (L - case["next_n"] + 1).astype(np.int32)           # next_n == 1: the row sees L tokens
    base = dict(cache=cache, k_new=dev(case["k"][last]), slot_new=dev(case["slot_mapping"][last]),
                q=dev(case["q"]), w=dev(case["w"]), bt=dev(case["block_table"]),
                ctx=dev(case["context_lens"]), ke=dev(ke))
    cos, sin = workloads.rope_tables(int(case["width"]), ROPE_DIM)
    base["cos"], base["sin"] = dev(cos), dev(sin)
    sets = [DecodeSet(base, case) for _ in range(n_sets)]
    torch.cuda.synchronize()
    return sets


def decode_ops(case):
    """The calls of a decode step, each as f(set)."""
    import mxfp4_paged_cache_quant_amd as mx
    W, K = case["width"], case["topk"]
    return {
        # the new tokens' K into the cache, the query rows to MXFP4 and the paged
        # logits, one launch
        "logits_paged_insert": lambda s: mx.logits_paged_insert(s.q, s.k_new, s.w, s.cache, s.bt,
                                                                s.ctx, 1, W, logits=s.logits,
                                                                clean=False),
        # the same with the query rotated first (RoPE over its first ROPE_DIM dims, each
        # row at its token's position)
        "logits_paged_insert_rope": lambda s: mx.logits_paged_insert_rope(
            s.q, s.k_new, s.w, s.cache, s.bt, s.ctx, 1, W, s.cos, s.sin, ROPE_DIM, "neox",
            logits=s.logits, clean=False),
        # the same as two launches: the encodes, then the logits
        "insert_quantize": lambda s: mx.insert_quantize(s.k_new, s.slot_new, s.cache, s.q, s.qv, s.qs),
        # clean=False: the top-k reads each row only up to its visible end
        "logits_paged": lambda s: mx.logits_paged(s.qv, s.qs, s.w, s.cache, s.bt, s.ctx, 1, W,
                                                  logits=s.logits, clean=False),
        "topk": lambda s: mx.topk(s.logits, None, s.ke, K, out=s.idx),
    }


EAGER = False          # --eager: launch directly instead of through HIP graphs (profiler runs)


class _Eager:
    def __init__(self, fns):
        self.fns = list(fns)

    def replay(self):
        for fn in self.fns:
            fn()


def capture(fn_list):
    import torch
    if EAGER:
        return _Eager(fn_list)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fn_list:
            fn()
    return g


def time_graph(g, reps, batches=9, warm_ms=25.0, spread=None):
    """ms per replay: the median over `batches` batches of `reps` replays, timed with
    HIP events on the current stream, after untimed replays for at least warm_ms
    (the clocks settle after a light section; a single warm-up replay left the
    first batches of a heavy kernel up to 20% slow).  With a dict `spread`, the
    10th and 90th percentiles of the batch times are stored there."""
    import numpy as np
    import statistics
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0, n = time.perf_counter(), 0
    while n < 2 or (time.perf_counter() - t0) * 1e3 < warm_ms:
        g.replay()
        torch.cuda.synchronize()
        n += 1
    times = []
    for _ in range(batches):
        start.record()
        for _ in range(reps):
            g.replay()
        stop.record()
        stop.synchronize()
        times.append(start.elapsed_time(stop) / reps)
    if spread is not None:
        spread["p10"], spread["p90"] = (float(v) for v in np.percentile(times, [10, 90]))
    return statistics.median(times)


def bench_decode(args, case, sets, order):
    import torch
    ops = decode_ops(case)

    G = len(sets)
    wfull, wrem = divmod(args.warmup, G)
    # the timed steps start at the set after the warm-up's last one, so that no
    # timed set has been touched since the others evicted it from the MALL
    # (with fewer steps than sets, every timed set is one the warm-up skipped)
    timed = sets[wrem:] + sets[:wrem]

    def step_fns(pool, lo, hi):
        return [(lambda s=s, name=name: ops[name](s)) for s in pool[lo:hi] for name in order]

    # eager warm-up of every call (also runs the architecture gate outside capture)
    # on the set the warm-up replays end with
    for fn in step_fns(sets, max(wrem - 1, 0), max(wrem, 1)):
        fn()
    torch.cuda.synchronize()
    g_full = capture(step_fns(timed, 0, G))
    rem = args.steps % G
    g_rem = capture(step_fns(timed, 0, rem)) if rem else None
    g_wrem = capture(step_fns(sets, 0, wrem)) if wrem else None
    g_wfull = capture(step_fns(sets, 0, G)) if wfull else None
    for _ in range(wfull):
        g_wfull.replay()
    if g_wrem is not None:
        g_wrem.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps // G):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel average durations: a graph of G back-to-back launches of one kernel
    per_kernel, spread = {}, {}
    for name in order:
        g = capture([(lambda s=s: ops[name](s)) for s in sets])
        sp = {}
        per_kernel[name] = time_graph(g, args.kernel_reps, spread=sp) / G * 1e3     # us per launch
        spread[name] = {k: round(v / G * 1e3, 3) for k, v in sp.items()}
        del g
    return elapsed, per_kernel, spread


CASES = {}            # workloads built by the GPU sections, reused by the oracle's legs


def bench_prefill(args):
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads
    case = workloads.prefill_chunk()
    CASES["prefill_chunk"] = case
    T, S, H = case["T"], case["S"], case["H"]
    cache = torch.zeros((case["num_pages"], 64 * 68), dtype=torch.uint8, device="cuda")
    k, slots, q, w = dev(case["k"]), dev(case["slot_mapping"]), dev(case["q"]), dev(case["w"])
    bt, sl, cu = dev(case["block_table"]), dev(case["seq_lens"]), dev(case["cu_seq_offsets"])
    ks, ke = dev(case["ks"]), dev(case["ke"])
    kv = torch.empty((S, 64), dtype=torch.uint8, device="cuda")
    ksc = torch.empty((S, 4), dtype=torch.uint8, device="cuda")
    qv = torch.empty((T, H, 64), dtype=torch.uint8, device="cuda")
    qs = torch.empty((T, H, 4), dtype=torch.uint8, device="cuda")
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, case["topk"]), dtype=torch.int32, device="cuda")
    ops = {
        "insert": lambda: mx.insert(k, slots, cache),
        "quantize": lambda: mx.quantize(q, qv, qs),
        "gather": lambda: mx.gather(cache, bt, sl, cu, S, S, k_values=kv, k_scales=ksc),
        "logits_prefill": lambda: mx.logits_prefill(qv, qs, kv, ksc, w, ks, ke, logits=logits,
                                                    clean=False),
        "topk": lambda: mx.topk(logits, ks, ke, case["topk"], out=idx),
    }
    for fn in ops.values():
        fn()
    torch.cuda.synchronize()
    per, spread = {}, {}
    for name, fn in ops.items():
        per[name] = time_fn(fn, 10, 4, spread, name)
    step_us = sum(per.values())
    # the same logits with clean = 1 (columns outside [ks, ke) written as -inf); not in the step
    t_clean = time_fn(lambda: mx.logits_prefill(qv, qs, kv, ksc, w, ks, ke, logits=logits,
                                                clean=True), 10, 4)
    pairs = int(np.sum(case["ke"].astype(np.int64) - case["ks"]))
    flops = 2.0 * H * 128 * pairs
    tflops = flops / (per["logits_prefill"] * 1e-6) / 1e12
    return {
        "workload": case["name"], "T": T, "S": S, "heads": H, "causal_pairs": pairs,
        "logits_flop": flops, "logits_us": round(per["logits_prefill"], 2),
        "logits_tflops": round(tflops, 1),
        "logits_frac_fp4_peak": round(tflops / FP4_PEAK_TFLOPS, 4),
        "logits_clean1_us": round(t_clean, 2),
        "step_us": round(step_us, 2),
        "kernels_us": {k2: round(v, 2) for k2, v in per.items()},
        "kernels_p10_p90_us": spread,
    }


def time_fn(fn, reps, per_graph=4, spread=None, key=None):
    """Average us per call of fn, from a graph of per_graph back-to-back calls;
    with a dict `spread`, its p10/p90 (us) go there under `key`."""
    g = capture([fn] * per_graph)
    sp = {}
    t = time_graph(g, reps, spread=sp) / per_graph * 1e3
    if spread is not None:
        spread[key] = [round(sp["p10"] / per_graph * 1e3, 2), round(sp["p90"] / per_graph * 1e3, 2)]
    del g
    return t


def bench_long_decode():
    """64 sequences of 32K..128K tokens: cache build (insert), paged logits, top-k."""
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads
    case = workloads.long_decode()
    CASES["long_decode"] = case
    B, H, W = len(case["context_lens"]), case["H"], case["width"]
    N = int(np.sum(case["context_lens"]))
    k, slots = dev(case["k"]), dev(case["slot_mapping"])
    cache = torch.zeros((case["num_pages"], 64 * 68), dtype=torch.uint8, device="cuda")
    qv, qs = mx.quantize(dev(case["q"]))
    w, bt, ctx = dev(case["w"]), dev(case["block_table"]), dev(case["context_lens"])
    ke = dev(case["context_lens"].astype(np.int32))
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, case["topk"]), dtype=torch.int32, device="cuda")
    ins = lambda: mx.insert(k, slots, cache)  # noqa: E731
    # clean=False: the top-k reads each row only up to its visible end; the
    # -inf fill of the columns past it (clean=True) is timed beside it
    lg = lambda: mx.logits_paged(qv, qs, w, cache, bt, ctx, 1, W, logits=logits, clean=False)  # noqa: E731
    lg_clean = lambda: mx.logits_paged(qv, qs, w, cache, bt, ctx, 1, W, logits=logits, clean=True)  # noqa: E731
    # the step's top-k splits each long row over workgroups (workspace from
    # topk_workspace, allocated once); the one-workgroup-per-row call is timed beside it
    ws = mx.topk_workspace(B, W)
    tk = lambda: mx.topk_ws(logits, None, ke, case["topk"], ws, out=idx)  # noqa: E731
    tk_row = lambda: mx.topk(logits, None, ke, case["topk"], out=idx)  # noqa: E731
    # profiler (--eager) runs launch only the calls of the step, so that
    # per-kernel counters are not averaged over the two clean variants
    extra = () if EAGER else (lg_clean,)
    for fn in (ins, *extra, lg, tk):
        fn()
    torch.cuda.synchronize()
    spread = {}
    t_ins = time_fn(ins, 5, 2, spread, "insert")
    t_lgc = None if EAGER else time_fn(lg_clean, 10, 4)
    t_lg = time_fn(lg, 10, 4, spread, "logits_paged")
    t_tk = time_fn(tk, 10, 4, spread, "topk")
    t_tk_row = None if EAGER else time_fn(tk_row, 10, 4)
    # multi-token decode (next_n = 2): the same cache, two query rows per sequence
    # (seeded N(0,1) bf16 q drawn on the device); rows see L-1 and L tokens
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20)
    q2 = torch.randn((2 * B, H, 128), generator=gen, device="cuda").to(torch.bfloat16)
    w2 = torch.rand((2 * B, H), generator=gen, device="cuda")
    qv2, qs2 = mx.quantize(q2)
    logits2 = torch.empty((2 * B, W), dtype=torch.float32, device="cuda")
    lg2 = lambda: mx.logits_paged(qv2, qs2, w2, cache, bt, ctx, 2, W, logits=logits2, clean=False)  # noqa: E731
    lg2()
    torch.cuda.synchronize()
    t_lg2 = None if EAGER else time_fn(lg2, 10, 4)
    # context-parallel merge: 4 ranks' top-2048 lists per sequence -> global top-2048
    # (seeded candidates on the device; local positions distinct per rank)
    world = 4
    mvals = torch.randn((world, B, case["topk"]), generator=gen, device="cuda")
    mpos = torch.argsort(torch.rand((world, B, 32768), generator=gen, device="cuda"), dim=-1)
    midx = mpos[:, :, :case["topk"]].to(torch.int32).contiguous()
    mout = torch.empty((B, case["topk"]), dtype=torch.int32, device="cuda")
    mg = lambda: mx.topk_merge(mvals, midx, 64, case["topk"], out=mout)  # noqa: E731
    mg()
    torch.cuda.synchronize()
    t_mg = None if EAGER else time_fn(mg, 10, 4)
    b_ins = N * (256 + 8 + 68)
    b_lg = N * 72 + B * H * 72
    b_tk = N * 4 + B * case["topk"] * 4
    return {
        "workload": case["name"], "tokens": N, "cache_bytes": case["num_pages"] * 64 * 68,
        "insert_us": round(t_ins, 1), "insert_gbs": round(b_ins / t_ins / 1e3, 1),
        "logits_paged_us": round(t_lg, 1), "logits_paged_gbs": round(b_lg / t_lg / 1e3, 1),
        "logits_paged_frac_hbm": round(b_lg / t_lg / 1e3 / HBM_PEAK_GBS, 4),
        "logits_paged_clean_us": None if t_lgc is None else round(t_lgc, 1),
        "mtp2_logits_paged_us": None if t_lg2 is None else round(t_lg2, 1),
        "mtp2_scored_pairs_per_s": None if t_lg2 is None else round((2 * N - B) / (t_lg2 * 1e-6), 1),
        "dcp4_merge_us": None if t_mg is None else round(t_mg, 1),
        "topk_us": round(t_tk, 1), "topk_gbs": round(b_tk / t_tk / 1e3, 1),
        "topk_one_workgroup_per_row_us": None if t_tk_row is None else round(t_tk_row, 1),
        "decode_step_frac_hbm": round((N * 76 + B * H * 72 + B * case["topk"] * 4)
                                      / ((t_lg + t_tk) * 1e3) / HBM_PEAK_GBS, 4),
        "decode_step_us": round(t_lg + t_tk, 1),
        "scored_tokens_per_s": round(N / ((t_lg + t_tk) * 1e-6), 1),
        "p10_p90_us": spread,
    }


def gather_bytes(tokens):
    """Algorithmic bytes of a gather: 68 B read and 68 B written per token, plus
    the block-table entries (4 B per page)."""
    return tokens * 136 + (tokens + 63) // 64 * 4


def row_rooflines(case, alg_bytes, per_kernel, rope_kernel, prefill, long_decode, long_prefill,
                  kpool, fp8):
    """One roofline entry per hot-path row, on the workload that represents it:
    algorithmic bytes (or FLOP) per launch from the path's per-unit figures, over
    the bench's own average launch time."""
    def hbm(workload, kernel, nbytes, us):
        if us is None:
            return None
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"workload": workload, "kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "alg_bytes": int(nbytes), "us": round(us, 3)}

    def mfma(workload, kernel, flop, us, peak):
        tfs = flop / (us * 1e-6) / 1e12
        return {"workload": workload, "kernel": kernel, "bound": "mfma", "achieved": round(tfs, 1),
                "peak": peak, "unit": "TFLOP/s", "frac": round(tfs / peak, 4), "flop": flop,
                "us": round(us, 3)}

    B, H = len(case["context_lens"]), case["H"]
    scored = int(case["context_lens"].sum())
    out = {"a7_topk_decode": hbm(case["name"], "topk", alg_bytes["topk"], per_kernel["topk"]),
           "a6_logits_paged_decode_step": hbm(case["name"], "logits_paged_insert",
                                              alg_bytes["logits_paged_insert"],
                                              per_kernel["logits_paged_insert"])}
    rope_us = rope_kernel.get("logits_paged_insert_rope")
    # the fused step's bytes plus each row's table row of rope_dim/2 cosines and sines
    out["next2_rope_decode_step"] = hbm(case["name"], "logits_paged_insert_rope",
                                        alg_bytes["logits_paged_insert"] + B * ROPE_DIM * 4,
                                        rope_us)
    if prefill is not None:
        T, Hp = prefill["T"], prefill["heads"]
        out["a3_q_quantize"] = hbm(prefill["workload"], "quantize", T * Hp * (256 + 68),
                                   prefill["kernels_us"]["quantize"])
        out["a5_logits_prefill_chunk"] = mfma(prefill["workload"], "logits_prefill",
                                              prefill["logits_flop"], prefill["logits_us"],
                                              FP4_PEAK_TFLOPS)
    if long_decode is not None:
        lc = CASES["long_decode"]
        N, Bl, H = long_decode["tokens"], len(lc["context_lens"]), lc["H"]
        out["a1_a2_insert"] = hbm(long_decode["workload"], "insert", N * (256 + 8 + 68),
                                  long_decode["insert_us"])
        out["a6_logits_paged"] = hbm(long_decode["workload"], "logits_paged",
                                     N * 72 + Bl * H * 72, long_decode["logits_paged_us"])
        out["a7_topk_long_rows"] = hbm(long_decode["workload"], "topk_ws",
                                       N * 4 + Bl * 2048 * 4, long_decode["topk_us"])
        if long_decode["mtp2_logits_paged_us"] is not None:
            # each page read once for both rows; two rows of logits and queries
            out["next3_logits_paged_next_n2"] = hbm(long_decode["workload"], "logits_paged",
                                                    N * 68 + (2 * N - Bl) * 4 + 2 * Bl * H * 72,
                                                    long_decode["mtp2_logits_paged_us"])
    if long_prefill is not None:
        out["a5_logits_prefill"] = mfma(long_prefill["workload"], "logits_prefill",
                                        long_prefill["logits_flop"], long_prefill["logits_us"],
                                        FP4_PEAK_TFLOPS)
        lp = CASES["long_prefill"]
        out["a7_topk_prefill_rows"] = hbm(long_prefill["workload"], "topk",
                                          long_prefill["causal_pairs"] * 4 + lp["T"] * lp["topk"] * 4,
                                          long_prefill["topk_us"])
        if long_prefill.get("gather_us") is not None:
            out["a4_gather"] = hbm(long_prefill["workload"], "gather",
                                   gather_bytes(CASES["long_prefill"]["S"]), long_prefill["gather_us"])
    if kpool is not None:
        kp = kpool["mxfp4"]
        out["next4_kpool_insert"] = {"workload": kpool["workload"], "kernel": "kpool_insert",
                                     "bound": "hbm", "achieved": kp["gbs"], "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": kp["frac_hbm"],
                                     "alg_bytes": kp["alg_bytes"], "us": kp["us"]}
    if fp8 is not None:
        fl = fp8["long_decode"]
        out["next1_fp8_logits_paged"] = {"workload": "long_decode_64xU32K-128K (FP8 cache)",
                                         "kernel": "logits_paged_fp8", "bound": "hbm",
                                         "achieved": fl["logits_paged_gbs"], "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": fl["logits_paged_frac_hbm"],
                                         "us": fl["logits_paged_us"]}
        fp_ = fp8["long_prefill"]
        out["next1_fp8_logits_prefill"] = {"workload": "long_prefill_16384x122880 (FP8)",
                                           "kernel": "logits_prefill_fp8", "bound": "mfma",
                                           "achieved": fp_["logits_tflops"],
                                           "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                           "frac": fp_["logits_frac_fp8_peak"],
                                           "us": fp_["logits_us"]}
    return out


def bench_long_prefill():
    """16384 queries over 122880 cached tokens, 64 heads: logits and top-k."""
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads
    case = workloads.long_prefill()
    CASES["long_prefill"] = case
    T, S, H = case["T"], case["S"], case["H"]
    cache = torch.zeros((case["num_pages"], 64 * 68), dtype=torch.uint8, device="cuda")
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    kv, ksc = mx.gather(cache, dev(case["block_table"]), dev(case["seq_lens"]),
                        dev(case["cu_seq_offsets"]), S, S)
    qv, qs = mx.quantize(dev(case["q"]))
    w, ks, ke = dev(case["w"]), dev(case["ks"]), dev(case["ke"])
    logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, case["topk"]), dtype=torch.int32, device="cuda")
    lg = lambda: mx.logits_prefill(qv, qs, kv, ksc, w, ks, ke, logits=logits, clean=False)  # noqa: E731
    tk = lambda: mx.topk(logits, ks, ke, case["topk"], out=idx)  # noqa: E731
    bt, sl, cu = dev(case["block_table"]), dev(case["seq_lens"]), dev(case["cu_seq_offsets"])
    ga = lambda: mx.gather(cache, bt, sl, cu, S, S, k_values=kv, k_scales=ksc)  # noqa: E731
    lg()
    tk()
    ga()
    torch.cuda.synchronize()
    spread = {}
    t_lg = time_fn(lg, 3, 2, spread, "logits_prefill")
    t_tk = time_fn(tk, 3, 2, spread, "topk")
    t_ga = None if EAGER else time_fn(ga, 10, 4)
    pairs = int(np.sum(case["ke"].astype(np.int64) - case["ks"]))
    flops = 2.0 * H * 128 * pairs
    tflops = flops / (t_lg * 1e-6) / 1e12
    return {
        "workload": case["name"], "causal_pairs": pairs, "logits_flop": flops,
        "logits_us": round(t_lg, 1), "logits_tflops": round(tflops, 1),
        "logits_frac_fp4_peak": round(tflops / FP4_PEAK_TFLOPS, 4),
        "topk_us": round(t_tk, 1), "topk_gbs": round((pairs * 4 + T * case["topk"] * 4) / t_tk / 1e3, 1),
        "gather_us": None if t_ga is None else round(t_ga, 2),
        "gather_gbs": None if t_ga is None else round(gather_bytes(S) / t_ga / 1e3, 1),
        "p10_p90_us": spread,
    }


def bench_fp8(decode_case):
    """The FP8 (E4M3, 132 B/token) indexer cache that MXFP4 replaces, on the same
    workloads: the decode step (16 x 8192: new tokens' insert, q quantize with the
    weight fold, paged logits, top-k; as four calls and with the encodes and the
    logits in one launch) over rotating caches, the long-context paged logits and
    top-k, and the prefill-chunk and long-prefill logits."""
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads
    out = {"bytes_per_token_per_head": {"fp8": 132, "mxfp4": 68},
           "tokens_per_gib_per_head": {"fp8": round(2 ** 30 / 132), "mxfp4": round(2 ** 30 / 68)}}
    # --- decode step, 48 rotating FP8 caches (830 MB, > 3x the MALL)
    case = decode_case
    B, H, W, K = len(case["context_lens"]), case["H"], case["width"], case["topk"]
    base = torch.zeros((case["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    mx.insert_fp8(dev(case["k"]), dev(case["slot_mapping"]), base)
    last = np.cumsum(case["context_lens"]) - 1
    k_new, slot_new = dev(case["k"][last]), dev(case["slot_mapping"][last])
    q, w, bt, ctx = dev(case["q"]), dev(case["w"]), dev(case["block_table"]), dev(case["context_lens"])
    ke = dev(case["context_lens"].astype(np.int32))
    n_sets = 48
    caches = [base.clone() for _ in range(n_sets)]
    del base
    qv = torch.empty((B, H, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, H), dtype=torch.float32, device="cuda")
    wf = torch.empty((B, H), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ops = {
        "insert_fp8": lambda c: mx.insert_fp8(k_new, slot_new, c),
        "quantize_fp8": lambda c: mx.quantize_fp8(q, weights=w, values=qv, scales=qs, weights_out=wf),
        "logits_paged_fp8": lambda c: mx.logits_paged_fp8(qv, wf, c, bt, ctx, 1, W, logits=logits,
                                                          clean=False),
        "topk": lambda c: mx.topk(logits, None, ke, K, out=idx),
    }
    for fn in ops.values():
        fn(caches[0])
    torch.cuda.synchronize()
    g_step = capture([(lambda c=c, f=f: f(c)) for c in caches for f in ops.values()])
    step_us = time_graph(g_step, 5) / n_sets * 1e3
    del g_step
    per = {}
    for name, f in ops.items():
        g = capture([(lambda c=c, f=f: f(c)) for c in caches])
        per[name] = round(time_graph(g, 10) / n_sets * 1e3, 3)
        del g
    # the same step with the two encodes and the logits in one launch
    ops1 = {
        "logits_paged_insert_fp8": lambda c: mx.logits_paged_insert_fp8(
            q, k_new, w, c, bt, ctx, 1, W, logits=logits, clean=False),
        "topk": ops["topk"],
    }
    for fn in ops1.values():
        fn(caches[0])
    torch.cuda.synchronize()
    g_step = capture([(lambda c=c, f=f: f(c)) for c in caches for f in ops1.values()])
    step1_us = time_graph(g_step, 5) / n_sets * 1e3
    del g_step
    g = capture([(lambda c=c: ops1["logits_paged_insert_fp8"](c)) for c in caches])
    fused_us = round(time_graph(g, 10) / n_sets * 1e3, 3)
    del g
    scored = int(np.sum(case["context_lens"]))
    out["decode_16x8192"] = {
        "step_us": round(step_us, 3), "kernels_us": per,
        "scored_tokens_per_s": round(scored / (step_us * 1e-6), 1),
        "logits_paged_gbs": round((scored * 136 + B * H * 132) / per["logits_paged_fp8"] / 1e3, 1),
        "one_launch": {"step": "logits_paged_insert_fp8+topk", "step_us": round(step1_us, 3),
                       "kernels_us": {"logits_paged_insert_fp8": fused_us, "topk": per["topk"]},
                       "scored_tokens_per_s": round(scored / (step1_us * 1e-6), 1)},
    }
    del caches
    torch.cuda.empty_cache()
    # --- long-context decode (64 x U[32K, 128K])
    lc = CASES.get("long_decode") or workloads.long_decode()
    B, H, W = len(lc["context_lens"]), lc["H"], lc["width"]
    N = int(np.sum(lc["context_lens"]))
    cache = torch.zeros((lc["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
    k, slots = dev(lc["k"]), dev(lc["slot_mapping"])
    ins = lambda: mx.insert_fp8(k, slots, cache)  # noqa: E731
    ins()
    del k
    qv, _, wf = mx.quantize_fp8(dev(lc["q"]), weights=dev(lc["w"]))
    bt, ctx = dev(lc["block_table"]), dev(lc["context_lens"])
    ke = dev(lc["context_lens"].astype(np.int32))
    logits = torch.empty((B, W), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, lc["topk"]), dtype=torch.int32, device="cuda")
    ws = mx.topk_workspace(B, W)
    lg = lambda: mx.logits_paged_fp8(qv, wf, cache, bt, ctx, 1, W, logits=logits, clean=False)  # noqa: E731
    tk = lambda: mx.topk_ws(logits, None, ke, lc["topk"], ws, out=idx)  # noqa: E731
    lg()
    tk()
    torch.cuda.synchronize()
    t_lg, t_tk = time_fn(lg, 10, 4), time_fn(tk, 10, 4)
    b_lg = N * 136 + B * H * 132
    out["long_decode"] = {
        "cache_bytes": lc["num_pages"] * 64 * 132,
        "logits_paged_us": round(t_lg, 1), "logits_paged_gbs": round(b_lg / t_lg / 1e3, 1),
        "logits_paged_frac_hbm": round(b_lg / t_lg / 1e3 / HBM_PEAK_GBS, 4),
        "topk_us": round(t_tk, 1), "decode_step_us": round(t_lg + t_tk, 1),
        "decode_step_frac_hbm": round((N * 140 + B * H * 132 + B * lc["topk"] * 4)
                                      / ((t_lg + t_tk) * 1e3) / HBM_PEAK_GBS, 4),
        "scored_tokens_per_s": round(N / ((t_lg + t_tk) * 1e-6), 1),
    }
    del cache, logits, ws
    torch.cuda.empty_cache()
    # --- prefill logits: the 8192 chunk and the long prefill
    for key, getter in (("prefill_chunk", workloads.prefill_chunk),
                        ("long_prefill", workloads.long_prefill)):
        pc = CASES.get(key) or getter()
        T, S, H = pc["T"], pc["S"], pc["H"]
        cache = torch.zeros((pc["num_pages"], 64 * 132), dtype=torch.uint8, device="cuda")
        mx.insert_fp8(dev(pc["k"]), dev(pc["slot_mapping"]), cache)
        kv, ksc = mx.gather_fp8(cache, dev(pc["block_table"]), dev(pc["seq_lens"]),
                                dev(pc["cu_seq_offsets"]), S, S)
        qv, _, wf = mx.quantize_fp8(dev(pc["q"]), weights=dev(pc["w"]))
        ks_, ke_ = dev(pc["ks"]), dev(pc["ke"])
        logits = torch.empty((T, S), dtype=torch.float32, device="cuda")
        lgp = lambda: mx.logits_prefill_fp8(qv, wf, kv, ksc, ks_, ke_, logits=logits, clean=False)  # noqa: E731
        lgp()
        torch.cuda.synchronize()
        reps = 10 if key == "prefill_chunk" else 3
        t = time_fn(lgp, reps, 4 if key == "prefill_chunk" else 2)
        pairs = int(np.sum(pc["ke"].astype(np.int64) - pc["ks"]))
        tflops = 2.0 * H * 128 * pairs / (t * 1e-6) / 1e12
        out[key] = {"logits_us": round(t, 1), "logits_tflops": round(tflops, 1),
                    "logits_frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4)}
        del cache, kv, ksc, qv, wf, logits
        torch.cuda.empty_cache()
    return out


KPOOL = 4                  # tokens pooled per K row (the calls' index_kpool; the pages fix no value)
KPOOL_TOKENS = 1 << 20


def bench_kpool():
    """Pooled K insert (idx_kpool_insert): 1,048,576 bf16 tokens with fp32 gate scores,
    kpool 4, i.e. 262,144 pool rows written through a permuted page order, as MXFP4
    and as FP8 rows.  HBM-bound: every token's K (256 B) and gate row (512 B) and
    slot (8 B) are read once, each pool row is written once."""
    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    n, kp = KPOOL_TOKENS, KPOOL
    gen = torch.Generator(device="cuda").manual_seed(2026)
    k = torch.randn((n, 128), generator=gen, device="cuda").to(torch.bfloat16)
    gate = torch.randn((n, 128), generator=gen, device="cuda")
    ape = torch.randn((kp, 128), generator=gen, device="cuda") * 0.1
    rows = n // kp
    pages = rows // 64
    # pool-granular slots: the last token of pool j carries its slot, the others -1
    perm = np.random.default_rng(7).permutation(pages)
    pool = np.arange(rows)
    slots_np = np.full(n, -1, np.int64)
    slots_np[pool * kp + kp - 1] = perm[pool // 64] * 64 + pool % 64
    slots = dev(slots_np)
    out = {"workload": f"kpool_insert_{n}_tokens_kpool{kp}", "tokens": n, "kpool": kp,
           "pool_rows": rows}
    for fmt, row in (("mxfp4", 68), ("fp8", 132)):
        cache = torch.zeros((pages, 64 * row), dtype=torch.uint8, device="cuda")
        f = lambda cache=cache, fmt=fmt: mx.kpool_insert(k, gate, ape, slots, cache, kp, fmt)
        f()
        torch.cuda.synchronize()
        sp = {}
        t = time_fn(f, 10, 2, sp, fmt)
        alg = n * (256 + 512 + 8) + rows * row + kp * 512
        gbs = alg / (t * 1e-6) / 1e9
        out[fmt] = {"us": round(t, 1), "p10_p90_us": sp[fmt], "alg_bytes": alg,
                    "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del cache
    return out


def bench_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size: the HBM rate torch's copy kernel reaches,
    and the reference for scaling the profiler's byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    stop.record()
    stop.synchronize()
    us = start.elapsed_time(stop) / reps * 1e3
    # read-only reference: a torch reduction over the same bytes
    src.sum()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        src.sum()
    stop.record()
    stop.synchronize()
    us_r = start.elapsed_time(stop) / reps * 1e3
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(us, 1),
            "gbs": round(2 * nbytes / us / 1e3, 1),
            "read_only_sum_us": round(us_r, 1), "read_only_gbs": round(nbytes / us_r / 1e3, 1)}


def host_info():
    """The host CPU the oracle runs on: model, logical CPUs this process may use,
    physical cores, and the BLAS threads the oracle's matrix products use."""
    model, phys = None, set()
    try:
        cur = {}
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if cur:
                    phys.add((cur.get("physical id"), cur.get("core id")))
                cur = {}
                continue
            key, val = (x.strip() for x in line.split(":", 1))
            cur[key] = val
            if key == "model name" and model is None:
                model = val
        if cur:
            phys.add((cur.get("physical id"), cur.get("core id")))
    except OSError:  # pragma: no cover
        pass
    try:
        logical = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        logical = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = logical
    return {"cpu_model": model, "logical_cpus_available": logical,
            "physical_cores_on_host": len(phys) or None, "blas_threads": int(threads)}


def cpu_baseline(case, seconds, prefill_case=None, long_prefill_case=None):
    """The oracle (never tuned for this) on bounded samples: decode steps of the
    16 x 8192 workload (the headline metric), the whole tiny workload, three
    sequences of the long-context batch, sampled query rows of the 8192 prefill
    chunk and the 256 sampled rows of the long prefill (throughput and
    extrapolated totals, labelled as such)."""
    import numpy as np
    from oracle import logits as olog, mxfp4 as omx, paged_cache as opc, topk as otk
    host = host_info()
    B = len(case["context_lens"])
    H = case["H"]
    cache = np.zeros((case["num_pages"], 64 * 68), np.uint8)
    cache = opc.insert(cache, omx.bf16_bits_to_f64(case["k"]), case["slot_mapping"])
    last = np.cumsum(case["context_lens"]) - 1
    scored, t_total, seqs_done = 0, 0.0, 0
    b = 0
    while t_total < seconds:
        t0 = time.perf_counter()
        cache = opc.insert(cache, omx.bf16_bits_to_f64(case["k"][last[b:b + 1]]),
                           case["slot_mapping"][last[b:b + 1]])
        qc, qsc = omx.quantize_rows(omx.bf16_bits_to_f64(case["q"][b:b + 1]))
        qc, qsc = qc.reshape(1, H, 64), qsc.reshape(1, H, 4)
        L = int(case["context_lens"][b])
        ref = olog.paged_mqa_logits(qc, qsc, case["w"][b:b + 1], cache, case["block_table"][b:b + 1],
                                    case["context_lens"][b:b + 1], 1, L)
        otk.top_k_per_row(ref.astype(np.float32), [0], [L], case["topk"])
        t_total += time.perf_counter() - t0
        scored += L
        seqs_done += 1
        b = (b + 1) % B
    out = {"value": scored / t_total, "unit": "scored cache tokens/s", "cores": host["blas_threads"],
           "kind": "oracle",
           "sample": f"{seqs_done} single-sequence decode steps (new-token insert, q quantize, "
                     f"paged logits over 8192 tokens, top-2048) of the 16x8192 workload, "
                     f"{t_total:.1f} s of CPU time; the oracle's insert returns a new copy of the "
                     f"8.9 MB cache at every step (its plain form), which is included",
           "host": host}

    def prefill_leg(pc, rows, label):
        # K side in full (insert + gather of every token), query side on `rows`
        t0 = time.perf_counter()
        c = opc.insert(np.zeros((pc["num_pages"], 64 * 68), np.uint8),
                       omx.bf16_bits_to_f64(pc["k"]), pc["slot_mapping"])
        kc, kscale = opc.gather(c, pc["block_table"], pc["seq_lens"], pc["cu_seq_offsets"], pc["S"])
        t_k = time.perf_counter() - t0
        t0 = time.perf_counter()
        Hp = pc["H"]
        qc, qsc = omx.quantize_rows(omx.bf16_bits_to_f64(pc["q"][rows]))
        ref = olog.mqa_logits(qc.reshape(-1, Hp, 64), qsc.reshape(-1, Hp, 4), kc, kscale,
                              pc["w"][rows], pc["ks"][rows], pc["ke"][rows], chunk=16)
        otk.top_k_per_row(ref.astype(np.float32), pc["ks"][rows], pc["ke"][rows], pc["topk"])
        t_q = time.perf_counter() - t0
        pairs_s = int(np.sum(pc["ke"][rows].astype(np.int64) - pc["ks"][rows]))
        pairs = int(np.sum(pc["ke"].astype(np.int64) - pc["ks"]))
        est = t_k + t_q * pairs / pairs_s
        return {"sample": label, "k_side_s": round(t_k, 2), "sampled_rows_s": round(t_q, 2),
                "sampled_pairs": pairs_s, "pairs_per_s": round(pairs_s / t_q, 1),
                "logits_tflops": round(2.0 * Hp * 128 * pairs_s / t_q / 1e12, 4),
                "extrapolated_full_s": round(est, 1), "extrapolated": True}

    # config 0: the tiny workload's whole path (insert, q quantize, paged logits of its
    # 4 query rows, top-64), repeated for about a second
    import workloads
    tc = workloads.tiny()
    t0, reps = time.perf_counter(), 0
    while time.perf_counter() - t0 < 1.0:
        c = opc.insert(np.zeros((tc["num_pages"], 64 * 68), np.uint8), omx.f32_to_f64(tc["k"]),
                       tc["slot_mapping"])
        qc, qsc = omx.quantize_rows(omx.f32_to_f64(tc["q"]))
        Ht = tc["H"]
        ref = olog.paged_mqa_logits(qc.reshape(-1, Ht, 64), qsc.reshape(-1, Ht, 4), tc["w"], c,
                                    tc["block_table"], tc["context_lens"], tc["next_n"],
                                    tc["width"])
        ke_t = olog.decode_visible_end(tc["context_lens"], tc["next_n"])
        otk.top_k_per_row(ref.astype(np.float32), np.zeros_like(ke_t), ke_t, tc["topk"])
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    out["tiny"] = {"sample": "the whole tiny path (256 fp32 tokens inserted, 4 query rows x 32 "
                             "heads quantized, paged logits, top-64), repeated",
                   "ms_per_step": round(dt * 1e3, 2),
                   "scored_tokens_per_s": round(float(np.sum(ke_t)) / dt, 1)}
    long_decode_case = CASES.get("long_decode")
    if long_decode_case is not None:
        # config 2: a few sequences of the long-context batch, each with a cache of its own
        # tokens only (the oracle's insert), its paged logits and top-2048; the batch's time
        # extrapolated by scored tokens
        lc = long_decode_case
        lens = lc["context_lens"].astype(np.int64)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        Hl = lc["H"]
        picks = [int(np.argmin(lens)), int(np.argmax(lens)), len(lens) // 2]
        t_l, tok_l = 0.0, 0
        for b in picks:
            L = int(lens[b])
            t0 = time.perf_counter()
            c = opc.insert(np.zeros((lc["num_pages"], 64 * 68), np.uint8),
                           omx.bf16_bits_to_f64(lc["k"][starts[b]:starts[b] + L]),
                           lc["slot_mapping"][starts[b]:starts[b] + L])
            qc, qsc = omx.quantize_rows(omx.bf16_bits_to_f64(lc["q"][b:b + 1]))
            ref = olog.paged_mqa_logits(qc.reshape(1, Hl, 64), qsc.reshape(1, Hl, 4),
                                        lc["w"][b:b + 1], c, lc["block_table"][b:b + 1],
                                        lc["context_lens"][b:b + 1], 1, L)
            otk.top_k_per_row(ref.astype(np.float32), [0], [L], lc["topk"])
            t_l += time.perf_counter() - t0
            tok_l += L
            del c
        rate = tok_l / t_l
        out["long_decode"] = {
            "sample": f"sequences {picks} of the 64 x U[32K, 128K] batch ({tok_l} scored tokens): "
                      f"insert of each sequence's own tokens, q quantize, paged logits, top-2048",
            "sampled_s": round(t_l, 2), "scored_tokens_per_s": round(rate, 1),
            "extrapolated_full_s": round(float(np.sum(lens)) / rate, 1), "extrapolated": True}
    if prefill_case is not None:
        rows = np.arange(0, prefill_case["T"], 16)
        out["prefill_chunk"] = prefill_leg(
            prefill_case, rows, f"insert + gather of all 8192 tokens, then q quantize, logits and "
                                f"top-2048 of {len(rows)} query rows (every 16th) of the 8192 causal "
                                f"chunk; the full chunk's time extrapolated by causal pairs")
    if long_prefill_case is not None:
        rows = np.asarray(long_prefill_case["sample_rows"])
        out["long_prefill"] = prefill_leg(
            long_prefill_case, rows, f"insert + gather of all 122880 tokens, then q quantize, logits "
                                     f"and top-2048 of the {len(rows)} sampled query rows; the full "
                                     f"16384-row time extrapolated by causal pairs")
    return out


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 byte counters
# ---------------------------------------------------------------------------

PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {          # kernel-name prefix -> the source it is compiled from
    "logits_paged_kernel": "logits_paged.hip",
    "logits_prefill_kernel": "logits_prefill.hip",
    "topk_kernel": "topk.hip",
    "topk_part": "topk.hip",
    "mxfp4_rows_kernel": "insert.hip",
    "insert_quantize_kernel": "insert.hip",
    "gather_kernel": "gather.hip",
}


def _source_hash(kernel):
    """16 hex digits of the sha256 of the kernel's source file and of the local
    headers it includes, recursively; launch.hpp (host-side launcher
    declarations, no device code) is left out."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "mxfp4_paged_cache_quant_amd", "csrc")
    for prefix, src in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            seen, todo = set(), [src]
            while todo:
                name = todo.pop(0)
                path = os.path.join(csrc, name)
                if name in seen or name == "launch.hpp" or not os.path.exists(path):
                    continue
                seen.add(name)
                text = open(path, "rb").read()
                h.update(text)
                todo += re.findall(r'#include "([^"]+)"', text.decode())
            return h.hexdigest()[:16]
    return None


def _short(name):
    name = name.replace("mxidx::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def _mean_counter(csv_path):
    import csv
    import collections
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        agg[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


# bench.py arguments of the counter runs, per section (eager launches: the
# counters are collected per dispatch)
PMC_ARGS = {"copy": "--eager", "decode": "--eager --steps 96 --warmup 16 --sets 32 --kernel-reps 2",
            "long_decode": "--eager", "long_prefill": "--eager"}


def pmc_summarize(root, section):
    """Turn the FETCH_SIZE / WRITE_SIZE runs of `section` (and of the plain copy)
    into profiles/pmc_bytes_<section>.json: bytes per dispatch per kernel,
    scaled by what the counters read for a copy of known size."""
    def run(sec, ctr):
        return _mean_counter(os.path.join(root, f"{sec}_{ctr}", "run_counter_collection.csv"))
    copy_f = run("copy", "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    copy_w = run("copy", "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    nbytes = 1 << 30
    f_scale = nbytes / (copy_f * 1024.0)           # bytes per counted KiB, reads
    w_scale = nbytes / (copy_w * 1024.0)
    fetch, write = run(section, "FETCH_SIZE"), run(section, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        src = _source_hash(k)
        if src is None:
            continue
        kernels[k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                      "read_bytes": round(fetch[k] * 1024 * f_scale),
                      "write_bytes": round(write[k] * 1024 * w_scale),
                      "traffic_bytes": round(fetch[k] * 1024 * f_scale + write[k] * 1024 * w_scale),
                      "source_sha256_16": src}
    out = {"section": section,
           "commands": [f"cd /tmp && export TMPDIR=/tmp && timeout -s KILL 180 rocprofv3 --pmc {c} "
                        f"-f csv -d <dir>/{sec}_{c} -o run -- python3 <repo>/bench.py --only {sec} "
                        f"{PMC_ARGS.get(sec, '--eager')}" for sec in ("copy", section)
                        for c in ("FETCH_SIZE", "WRITE_SIZE")],
           "calibration": {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
                           "read_bytes_per_counted_kib": f_scale * 1024,
                           "write_bytes_per_counted_kib": w_scale * 1024},
           "kernels": kernels}
    path = os.path.join(PROFILES, f"pmc_bytes_{section}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return path


def measured_traffic(section, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel's source changed since."""
    path = os.path.join(PROFILES, f"pmc_bytes_{section}.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    for k, v in data["kernels"].items():
        if k.startswith(kernel) and v["source_sha256_16"] == _source_hash(k):
            return v["traffic_bytes"]
    return None


def main():
    args = parse()
    if args.pmc_summarize:
        print(pmc_summarize(*args.pmc_summarize))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MXFP4 indexer path runs on a single GPU and has "
              "no multi-GPU mode (it would shard by sequence, with no exchange between GPUs). "
              "Run with --gpus 1.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import mxfp4_paged_cache_quant_amd as mx
    import workloads

    torch.cuda.set_device(0)
    mx.init(0)
    global EAGER
    EAGER = args.eager
    if args.only is not None:
        section = {"prefill": lambda: bench_prefill(args), "long_decode": bench_long_decode,
                   "long_prefill": bench_long_prefill, "copy": bench_copy, "kpool": bench_kpool,
                   "fp8": lambda: bench_fp8(workloads.paged_decode())}
        if args.only in section:
            print(json.dumps({"section": args.only, "result": section[args.only]()}), flush=True)
            return
    case = workloads.paged_decode()
    log(f"[bench] decode workload {case['name']}: building {args.sets} rotating sets")
    sets = build_decode_sets(case, args.sets)
    elapsed, per_kernel, per_spread = bench_decode(args, case, sets, ["logits_paged_insert", "topk"])
    sep_elapsed, sep_kernel, _ = bench_decode(args, case, sets,
                                              ["insert_quantize", "logits_paged", "topk"])
    rope_elapsed, rope_kernel, _ = bench_decode(args, case, sets,
                                                ["logits_paged_insert_rope", "topk"])
    del sets
    ms_per_step = elapsed / args.steps * 1e3
    scored = int(np.sum(case["context_lens"]))
    value = scored * args.steps / elapsed
    log(f"[bench] decode: {ms_per_step * 1e3:.2f} us/step, kernels {per_kernel}")

    B, H, L = len(case["context_lens"]), case["H"], int(case["context_lens"][0])
    alg_bytes = {
        # cache read + logits written, bf16 q and fp32 weights read, new K read + written
        "logits_paged_insert": scored * (68 + 4) + B * H * (256 + 4) + B * (256 + 68),
        "insert_quantize": B * (256 + 8 + 68) + B * H * (256 + 68),
        "logits_paged": scored * (68 + 4) + B * H * (68 + 4),
        "topk": scored * 4 + B * case["topk"] * 4,
    }
    dominant = max(per_kernel, key=per_kernel.get)
    achieved = alg_bytes[dominant] / (per_kernel[dominant] * 1e-6) / 1e9
    dom_kernel = {"logits_paged_insert": "logits_paged_kernel",
                  "insert_quantize": "insert_quantize_kernel", "logits_paged": "logits_paged_kernel",
                  "topk": "topk_kernel"}[dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("decode", dom_kernel),
                "alg_bytes_per_launch": alg_bytes[dominant],
                "avg_launch_us": round(per_kernel[dominant], 3)}
    kernels = {k: {"avg_us": round(v, 3), "p10_us": per_spread[k]["p10"], "p90_us": per_spread[k]["p90"],
                   "alg_bytes": alg_bytes[k],
                   "gbs": round(alg_bytes[k] / (v * 1e-6) / 1e9, 1)} for k, v in per_kernel.items()}
    separate = {"step": "insert_quantize+logits_paged+topk",
                "us_per_step": round(sep_elapsed / args.steps * 1e6, 3),
                "kernels_us": {k: round(v, 3) for k, v in sep_kernel.items()}}
    log(f"[bench] decode as three calls: {separate}")
    with_rope = {"step": "logits_paged_insert_rope+topk", "rope_dim": ROPE_DIM, "pairing": "neox",
                 "us_per_step": round(rope_elapsed / args.steps * 1e6, 3),
                 "kernels_us": {k: round(v, 3) for k, v in rope_kernel.items()}}
    log(f"[bench] decode with the query RoPE fused: {with_rope}")

    if args.only == "decode":
        print(json.dumps({"section": "decode", "us_per_step": round(ms_per_step * 1e3, 3),
                          "kernels_us": per_kernel, "separate": separate,
                          "with_rope": with_rope}), flush=True)
        return

    prefill = None
    if args.prefill == "chunk":
        log("[bench] prefill chunk 8192x8192")
        prefill = bench_prefill(args)
        log(f"[bench] prefill: {prefill}")

    long_decode = long_prefill = None
    if not args.no_long:
        log("[bench] long-context decode 64 x U[32K,128K]")
        long_decode = bench_long_decode()
        log(f"[bench] long decode: {long_decode}")
        torch.cuda.empty_cache()
        log("[bench] long prefill 16384 x 122880")
        long_prefill = bench_long_prefill()
        log(f"[bench] long prefill: {long_prefill}")
        torch.cuda.empty_cache()

    kpool = None
    if not args.no_long:
        log("[bench] kpool insert, 1M tokens, kpool 4")
        kpool = bench_kpool()
        log(f"[bench] kpool: {kpool}")
        torch.cuda.empty_cache()

    fp8 = None
    if not args.no_fp8:
        log("[bench] FP8 indexer cache (132 B/token) on the same workloads")
        fp8 = bench_fp8(case)
        log(f"[bench] fp8: {fp8}")
        torch.cuda.empty_cache()

    copy = bench_copy()
    log(f"[bench] device copy: {copy}")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(case, args.cpu_seconds, CASES.get("prefill_chunk"),
                           CASES.get("long_prefill"))

    out = {
        "metric": "scored cache tokens/sec (paged decode) + prefill logits TFLOP/s, % of roofline",
        "value": round(value, 1),
        "unit": "scored cache tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": case["name"], "batch": B, "context": L, "heads": H,
                   "head_dim": 128, "page_size": 64, "next_n": 1, "topk": case["topk"],
                   "step": "logits_paged_insert(16 new tokens' K, 512 q rows, paged logits; one launch)+topk",
                   "rotating_sets": args.sets, "hip_graph": True, "parallelism": "none"},
        "roofline": roofline,
        "rooflines": row_rooflines(case, alg_bytes, per_kernel, rope_kernel, prefill, long_decode,
                                   long_prefill, kpool, fp8),
        "kernels": kernels,
        "decode_separate_calls": separate,
        "decode_with_rope": with_rope,
        "prefill": prefill,
        "long_decode": long_decode,
        "long_prefill": long_prefill,
        "kpool_insert": kpool,
        "fp8": fp8,
        "device_copy": copy,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
