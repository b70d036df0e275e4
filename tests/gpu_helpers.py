"""Helpers shared by the GPU parity tests: moving seeded workload arrays to the
device, running the HIP path through the C ABI binding, and computing the
oracle's view of the same inputs."""

import numpy as np
import torch

import mxfp4_paged_cache_quant_amd as mx
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


def check_logits(gpu, ref, bound, what=""):
    """Masked entries must agree exactly (-inf / -inf); visible ones within tolerance."""
    from oracle import tolerance
    gpu = np.asarray(gpu, dtype=np.float64)
    vis = np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu) & ~vis, ~vis), f"{what}: mask mismatch"
    ok = tolerance.logits_close(gpu[vis], ref[vis], bound[vis])
    if not ok.all():
        bad = np.argwhere(vis)[~ok][:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} logits out of tolerance, e.g. at "
                             f"{bad.tolist()}: gpu {gpu[tuple(bad[0])]} ref {ref[tuple(bad[0])]}")
