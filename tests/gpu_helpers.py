"""Helpers shared by the GPU parity tests: moving seeded workload arrays to the
device, running the HIP path through the C ABI binding, and computing the
oracle's view of the same inputs."""

import numpy as np
import torch

import mxfp4_paged_cache_quant_amd as mx
import workloads
from oracle import mxfp4 as omx

CANARY = 0xA5


def dev(a):
    """numpy array -> device tensor (uint16 arrays are bf16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def exact(case, key):
    """The exact float64 values of a bf16 / fp32 input array of a case."""
    a = case[key]
    return omx.bf16_bits_to_f64(a) if case["dtype"] == "bf16" else omx.f32_to_f64(a)


def new_cache(num_pages, fill=CANARY):
    return torch.full((num_pages, mx.PAGE_SIZE * mx.ROW_BYTES), fill, dtype=torch.uint8, device="cuda")


def gpu_build_cache(case, fill=CANARY):
    cache = new_cache(case["num_pages"], fill)
    mx.insert(dev(case["k"]), dev(case["slot_mapping"]), cache)
    return cache


def gpu_quantize_q(case):
    return mx.quantize(dev(case["q"]))


def oracle_q(case):
    H = case["q"].shape[1]
    c, s = omx.quantize_rows(exact(case, "q"))
    return c.reshape(-1, H, 64), s.reshape(-1, H, 4)


def check_logits(gpu, ref, bound, what="", abs_factor=None):
    """Masked entries must agree exactly (-inf / -inf); visible ones within tolerance
    (the MXFP4 rule, or the FP8 one with abs_factor=tolerance.ABS_FACTOR_FP8)."""
    from oracle import tolerance
    gpu = np.asarray(gpu, dtype=np.float64)
    vis = np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu) & ~vis, ~vis), f"{what}: mask mismatch"
    factor = tolerance.ABS_FACTOR if abs_factor is None else abs_factor
    ok = tolerance.logits_close(gpu[vis], ref[vis], bound[vis], abs_factor=factor)
    if not ok.all():
        bad = np.argwhere(vis)[~ok][:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} logits out of tolerance, e.g. at "
                             f"{bad.tolist()}: gpu {gpu[tuple(bad[0])]} ref {ref[tuple(bad[0])]}")


def check_topk_sets(g_logits, ks, ke, k, out_idx, what=""):
    """Exact top-k sets vs the oracle's top-k of the same (GPU) fp32 logits."""
    from oracle import topk as otk
    ref_sets = otk.top_k_per_row(g_logits, ks, ke, k)
    for r in range(g_logits.shape[0]):
        assert sorted(out_idx[r].tolist()) == sorted(ref_sets[r].tolist()), f"{what} top-k row {r}"


def check_topk_end_to_end(ref_rows, bound_rows, ks, ke, k, idx_rows, what="", abs_factor=None):
    """End-to-end margin rule of GPU top-k rows against the oracle's float64
    logits of the same rows; returns how many rows needed the exact set."""
    from oracle import tolerance, topk as otk
    exact_rows = 0
    for j in range(len(ref_rows)):
        vis = np.isfinite(ref_rows[j])
        vk = otk.kth_value(ref_rows[j], int(ks[j]), int(ke[j]), k)
        if vk is None:
            assert np.all(np.asarray(idx_rows[j]) == -1), f"{what}: empty row {j} returned columns"
            exact_rows += 1
            continue
        factor = tolerance.ABS_FACTOR if abs_factor is None else abs_factor
        tol = tolerance.REL * abs(vk) + factor * float(bound_rows[j][vis].max())
        ok, exact_req = tolerance.topk_end_to_end_ok(idx_rows[j], ref_rows[j], int(ks[j]),
                                                     int(ke[j]), k, tol)
        assert ok, f"{what}: end-to-end top-k, row {j}"
        exact_rows += exact_req
    return exact_rows


def split_new_tokens(case, bt):
    """The cache before the step (every token but the last next_n of each sequence)
    and the step's new K rows with their slots through block table ``bt`` (-1
    where the position is < 0 or the table entry is not a page)."""
    lens = case["context_lens"].astype(np.int64)
    nn = case["next_n"]
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    pre_slots = case["slot_mapping"].copy()
    B = len(lens)
    k = case["k"]
    filler = k[0] if len(k) else np.zeros(128, k.dtype)
    k_new = np.empty((B * nn, 128), dtype=k.dtype)
    new_slots = np.full(B * nn, -1, np.int64)
    for b in range(B):
        for i in range(nn):
            pos = lens[b] - nn + i
            if pos >= 0:
                k_new[b * nn + i] = k[starts[b] + pos]
                page = int(bt[b, pos // 64])
                if 0 <= page < case["num_pages"]:
                    new_slots[b * nn + i] = page * 64 + pos % 64
                pre_slots[starts[b] + pos] = -1
            else:
                k_new[b * nn + i] = filler
    return pre_slots, k_new, new_slots


rope_tables = workloads.rope_tables
