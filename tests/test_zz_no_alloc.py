"""GPU parity of the allocation-free top-k entry point (idx_topk_noalloc): its
output must equal, element for element, that of idx_topk_ws -- the same
kernels with a caller-provided workspace -- on two calls in a row through the
C ABI, the second with a smaller input (the static scratch then still holds the
first call's bytes), and a call that needs more scratch than the library holds
is rejected before any device work."""

import ctypes

import numpy as np
import pytest
import torch

import mxfp4_paged_cache_quant_amd as mx
from tests.gpu_helpers import check_topk_sets, host

pytestmark = pytest.mark.gpu


def _rows(rows, width, seed, ragged):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    logits = torch.randn((rows, width), generator=gen, device="cuda")
    # a band of planted ties at a typical threshold value
    logits[:, ::97] = 0.75
    if ragged:
        lens = torch.randint(width // 4, width + 1, (rows,), generator=gen, device="cuda")
        lens[0] = width
        ks = torch.randint(0, 3000, (rows,), generator=gen, device="cuda").to(torch.int32)
        ke = lens.to(torch.int32)
    else:
        ks = None
        ke = torch.full((rows,), width, dtype=torch.int32, device="cuda")
    return logits, ks, ke


def _both(logits, ks, ke, k):
    rows, width = logits.shape
    ws = mx.topk_workspace(rows, width)
    ref = mx.topk_ws(logits, ks, ke, k, ws)
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    mx.topk_noalloc(logits, ks, ke, k, out=out)
    torch.cuda.synchronize()
    return host(ref), host(out)


def test_noalloc_equals_workspace_call_on_two_calls_in_a_row():
    # first call: the long-context decode shape (64 rows of 131,072 columns, the
    # largest the scratch holds); second: fewer, shorter rows, fewer parts each
    cases = [(64, 131072, 2048, 5, False), (9, 40000, 300, 6, True)]
    for rows, width, k, seed, ragged in cases:
        need = mx.topk_workspace_bytes(rows, width)
        assert 0 < need <= mx.TOPK_NOALLOC_MAX_WORKSPACE
        logits, ks, ke = _rows(rows, width, seed, ragged)
        ref, got = _both(logits, ks, ke, k)
        assert np.array_equal(ref, got), f"{rows}x{width}: differs at {np.argwhere(ref != got)[:4].tolist()}"
        # and the sets are the exact top-k of these logits (oracle top-k, a few rows)
        pick = [0, rows // 2, rows - 1]
        ks_np = np.zeros(rows, np.int32) if ks is None else host(ks)
        check_topk_sets(host(logits)[pick], ks_np[pick], host(ke)[pick], k, got[pick],
                        f"{rows}x{width}")


def test_noalloc_short_rows_need_no_scratch():
    # rows of one part: no split, no scratch, the one-workgroup path
    logits, ks, ke = _rows(16, 8192, 7, False)
    assert mx.topk_workspace_bytes(16, 8192) == 0
    ref, got = _both(logits, ks, ke, 2048)
    assert np.array_equal(ref, got)


def test_noalloc_rejects_more_than_its_scratch():
    rows, width = 64, 8192 * 64                 # 64 parts per row: 134 MB of workspace
    assert mx.topk_workspace_bytes(rows, width) > mx.TOPK_NOALLOC_MAX_WORKSPACE
    L = mx.lib()
    fake = ctypes.c_void_p(0x10000)             # never dereferenced: rejected on the host
    st = L.idx_topk_noalloc(fake, rows, width, None, fake, 2048, fake, None)
    assert st == 1                               # IDX_ERR_ARG
