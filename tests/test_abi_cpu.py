"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects host-checkable bad arguments with IDX_ERR_ARG before
touching a device, treats empty work as a no-op, and fails closed
(IDX_ERR_NO_DEVICE) when no device is present."""

import ctypes
import os
import re

import pytest

import mxfp4_paged_cache_quant_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxidx.h")

OK, ERR_ARG, ERR_NO_DEVICE, ERR_ARCH, ERR_LAUNCH = 0, 1, 2, 3, 4

# Fake, suitably aligned "device" addresses: never dereferenced, because every
# call below either fails validation or stops at the device gate.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10001)      # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.lib_path):
        from mxfp4_paged_cache_quant_amd import build
        build.build()
    return mx.lib()


def _has_gpu():
    import torch
    return torch.cuda.is_available()


def test_header_declarations_are_exported(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(idx_[a-z0-9_]+)\s*\(", text))
    assert declared == set(mx.EXPORTS), declared ^ set(mx.EXPORTS)
    for name in declared:
        assert hasattr(L, name)


def test_version_and_strerror(L):
    assert L.idx_version() == 107
    for st in range(5):
        assert L.idx_strerror(st)
    assert L.idx_strerror(99) == b"unknown status"


def test_quantize_argument_validation(L):
    assert L.idx_quantize(P, 2, 4, 128, P, P2, None) == ERR_ARG           # bad dtype
    assert L.idx_quantize(P, 0, -1, 128, P, P2, None) == ERR_ARG          # negative rows
    assert L.idx_quantize(P, 0, 4, 100, P, P2, None) == ERR_ARG           # stride < 128
    assert L.idx_quantize(P, 0, 4, 132, P, P2, None) == ERR_ARG           # bf16 stride % 8
    assert L.idx_quantize(P, 1, 4, 130, P, P2, None) == ERR_ARG           # f32 stride % 4
    assert L.idx_quantize(MIS, 0, 4, 128, P, P2, None) == ERR_ARG         # misaligned input
    assert L.idx_quantize(None, 0, 4, 128, P, P2, None) == ERR_ARG        # null input
    assert L.idx_quantize(P, 0, 4, 128, None, P2, None) == ERR_ARG        # null output
    assert L.idx_quantize(None, 0, 0, 128, None, None, None) == OK        # empty: no-op


def test_insert_argument_validation(L):
    assert L.idx_insert(P, 0, 4, 128, P, P2, 4, 32, None) == ERR_ARG      # page size != 64
    assert L.idx_insert(P, 0, 4, 128, None, P2, 4, 64, None) == ERR_ARG   # null slot mapping
    assert L.idx_insert(P, 0, 4, 128, P, None, 4, 64, None) == ERR_ARG    # null cache
    assert L.idx_insert(P, 0, 4, 128, P, P2, -1, 64, None) == ERR_ARG     # negative pages
    assert L.idx_insert(None, 0, 0, 128, None, None, 0, 64, None) == OK


def test_insert_quantize_argument_validation(L):
    f = L.idx_insert_quantize
    assert f(P, 0, 4, 128, P, P2, 4, 32, P, 0, 8, 128, P, P2, None) == ERR_ARG   # page size != 64
    assert f(P, 2, 4, 128, P, P2, 4, 64, P, 0, 8, 128, P, P2, None) == ERR_ARG   # bad K dtype
    assert f(P, 0, 4, 128, P, P2, 4, 64, P, 2, 8, 128, P, P2, None) == ERR_ARG   # bad q dtype
    assert f(P, 0, 4, 128, None, P2, 4, 64, P, 0, 8, 128, P, P2, None) == ERR_ARG  # null slots
    assert f(P, 0, 4, 128, P, P2, 4, 64, P, 0, 8, 100, P, P2, None) == ERR_ARG   # q stride < 128
    assert f(P, 0, 4, 128, P, P2, 4, 64, MIS, 0, 8, 128, P, P2, None) == ERR_ARG  # misaligned q
    assert f(P, 0, 4, 128, P, P2, 4, 64, P, 0, 8, 128, None, P2, None) == ERR_ARG  # null q out
    assert f(P, 0, 4, 128, P, P2, -1, 64, P, 0, 8, 128, P, P2, None) == ERR_ARG  # negative pages
    assert f(None, 0, 0, 128, None, None, 0, 64, None, 0, 0, 128, None, None, None) == OK  # empty


def test_topk_merge_argument_validation(L):
    f = L.idx_topk_merge
    assert f(P, P2, 0, 4, 64, 1, 16, P, None) == ERR_ARG          # world < 1
    assert f(P, P2, 2, 4, 0, 1, 16, P, None) == ERR_ARG           # k_in < 1
    assert f(P, P2, 2, 4, 64, 0, 16, P, None) == ERR_ARG          # interleave < 1
    assert f(P, P2, 2, 4, 64, 1, 0, P, None) == ERR_ARG           # k < 1
    assert f(P, P2, 2, 4, 64, 1, 2049, P, None) == ERR_ARG        # k > 2048
    assert f(P, P2, 5, 4, 2048, 1, 16, P, None) == ERR_ARG        # more than 8192 candidates
    assert f(P, P2, 2, -1, 64, 1, 16, P, None) == ERR_ARG         # negative rows
    assert f(MIS, P2, 2, 4, 64, 1, 16, P, None) == ERR_ARG        # misaligned values
    assert f(P, None, 2, 4, 64, 1, 16, P, None) == ERR_ARG        # null indices
    assert f(P, P2, 2, 4, 64, 1, 16, None, None) == ERR_ARG       # null output
    assert f(None, None, 2, 0, 64, 1, 16, None, None) == OK       # no rows


def test_gather_argument_validation(L):
    assert L.idx_gather(P, 4, 64, P, 1, P, P, 2, 128, 256, P, P2, None) == ERR_ARG  # bt stride < 2 pages
    assert L.idx_gather(MIS, 4, 64, P, 2, P, P, 2, 128, 256, P, P2, None) == ERR_ARG
    assert L.idx_gather(P, 4, 64, P, 2, P, P, 2, 128, 256, MIS, P2, None) == ERR_ARG
    assert L.idx_gather(P, 4, 64, P, 2, P, P, 0, 128, 256, P, P2, None) == OK        # no sequences


def test_logits_argument_validation(L):
    # H must be a multiple of 16 in [16, 128]
    for H in (0, 8, 24, 144):
        assert L.idx_logits_prefill(P, P, P, P, P, None, P, 4, H, 64, P, 64, 1, None) == ERR_ARG
        assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 1, H, 64, P, 64, 1, None) == ERR_ARG
    assert L.idx_logits_prefill(P, P, P, P, P, None, P, 4, 32, 64, P, 63, 1, None) == ERR_ARG   # ld < S
    assert L.idx_logits_prefill(P, P, P, P, P, None, None, 4, 32, 64, P, 64, 1, None) == ERR_ARG  # null ke
    assert L.idx_logits_prefill(P, P, P, P, MIS, None, P, 4, 32, 64, P, 64, 1, None) == ERR_ARG
    assert L.idx_logits_prefill(P, P, P, P, P, None, P, 0, 32, 64, P, 64, 1, None) == OK
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 0, 32, 64, P, 64, 1, None) == ERR_ARG   # next_n 0
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 17, 32, 64, P, 64, 1, None) == ERR_ARG  # next_n 17
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 1, 32, 65, P, 65, 1, None) == ERR_ARG   # bt stride
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 1, 32, 64, P, 63, 1, None) == ERR_ARG   # ld
    assert L.idx_logits_paged(P, P, P, P, 4, 48, P, 1, P, 1, 1, 32, 64, P, 64, 1, None) == ERR_ARG   # page
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 0, 1, 32, 64, P, 64, 1, None) == OK


def test_logits_paged_insert_argument_validation(L):
    # idx_logits_paged_insert(q, k_new, dtype, w, cache, num_pages, page, bt, bt_stride, ctx,
    #                         B, next_n, H, max_len, logits, ld, clean, stream)
    def call(q=P, k=P, dtype=0, H=32, next_n=1, max_len=64, bt_stride=1, ld=64, page=64, B=1):
        return L.idx_logits_paged_insert(q, k, dtype, P, P, 4, page, P, bt_stride, P, B, next_n, H,
                                         max_len, P, ld, 1, None)
    for dtype in (-1, 2):
        assert call(dtype=dtype) == ERR_ARG
    for H in (0, 8, 24, 144):
        assert call(H=H) == ERR_ARG
    assert call(q=None) == ERR_ARG
    assert call(k=None) == ERR_ARG
    assert call(q=MIS) == ERR_ARG
    assert call(k=MIS) == ERR_ARG
    assert call(next_n=0) == ERR_ARG
    assert call(next_n=17) == ERR_ARG
    assert call(max_len=65, ld=65) == ERR_ARG     # block-table stride below the pages needed
    assert call(ld=63) == ERR_ARG
    assert call(page=48) == ERR_ARG
    assert call(B=0) == OK
    assert call(max_len=0) == OK


def test_logits_paged_insert_fp8_argument_validation(L):
    # idx_logits_paged_insert_fp8(q, k_new, dtype, w, scale_fmt, cache, num_pages, page, bt,
    #                             bt_stride, ctx, B, next_n, H, max_len, logits, ld, clean, stream)
    def call(q=P, k=P, dtype=0, fmt=0, H=32, next_n=1, max_len=64, bt_stride=1, ld=64, page=64,
             B=1):
        return L.idx_logits_paged_insert_fp8(q, k, dtype, P, fmt, P, 4, page, P, bt_stride, P, B,
                                             next_n, H, max_len, P, ld, 1, None)
    for dtype in (-1, 2):
        assert call(dtype=dtype) == ERR_ARG
    for fmt in (-1, 2):
        assert call(fmt=fmt) == ERR_ARG
    for H in (0, 8, 24, 144):
        assert call(H=H) == ERR_ARG
    assert call(q=None) == ERR_ARG
    assert call(k=MIS) == ERR_ARG
    assert call(next_n=0) == ERR_ARG
    assert call(next_n=17) == ERR_ARG
    assert call(max_len=65, ld=65) == ERR_ARG     # block-table stride below the pages needed
    assert call(ld=63) == ERR_ARG
    assert call(page=48) == ERR_ARG
    assert call(B=0) == OK
    assert call(max_len=0) == OK


def test_topk_argument_validation(L):
    for k in (0, -3, 2049):
        assert L.idx_topk(P, 4, 64, None, P, k, P, None) == ERR_ARG
    assert L.idx_topk(P, 4, 64, None, None, 8, P, None) == ERR_ARG   # null ke
    assert L.idx_topk(MIS, 4, 64, None, P, 8, P, None) == ERR_ARG
    assert L.idx_topk(P, 0, 64, None, P, 8, P, None) == OK


def test_topk_workspace_sizes(L):
    f = L.idx_topk_workspace_bytes
    # 64 rows x 16 parts of 8192 columns: 16-byte part headers, then 4096 pairs per part
    assert f(64, 131072) == 64 * 16 * 16 + 64 * 16 * 4096 * 8
    assert f(3, 8193) == 256 + 3 * 2 * 4096 * 8
    assert f(64, 8192) == 0             # one workgroup holds a row
    assert f(512, 131072) == 0          # many rows fill the GPU unsplit
    assert f(8, 64 * 8192) > 0 and f(8, 64 * 8192 + 1) == 0     # at most 64 parts
    assert f(0, 131072) == 0 and f(-1, 131072) == 0 and f(4, -5) == 0


def test_topk_ws_argument_validation(L):
    f = L.idx_topk_ws
    need = L.idx_topk_workspace_bytes(4, 40000)
    assert need > 0
    assert f(P, 4, 40000, None, P, 0, P, P2, need, None) == ERR_ARG        # k < 1
    assert f(P, 4, 40000, None, None, 8, P, P2, need, None) == ERR_ARG     # null ke
    assert f(P, 4, 40000, None, P, 8, P, None, need, None) == ERR_ARG      # no workspace
    assert f(P, 4, 40000, None, P, 8, P, P2, need - 1, None) == ERR_ARG    # too small
    assert f(P, 4, 40000, None, P, 8, P, ctypes.c_void_p(0x20080), need, None) == ERR_ARG  # misaligned
    assert f(P, 0, 40000, None, P, 8, P, None, 0, None) == OK              # empty: no-op


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_fails_closed_without_device(L):
    assert L.idx_init(0) == ERR_NO_DEVICE
    assert L.idx_quantize(P, 0, 4, 128, P, P2, None) == ERR_NO_DEVICE
    assert L.idx_topk(P, 4, 64, None, P, 8, P, None) == ERR_NO_DEVICE
    assert L.idx_topk_ws(P, 4, 64, None, P, 8, P, None, 0, None) == ERR_NO_DEVICE   # no split: no workspace
    assert L.idx_topk_ws(P, 4, 40000, None, P, 8, P, P2, 1 << 24, None) == ERR_NO_DEVICE
    assert L.idx_logits_paged(P, P, P, P, 4, 64, P, 1, P, 1, 1, 32, 64, P, 64, 1, None) == ERR_NO_DEVICE
    assert L.idx_logits_paged_insert(P, P, 0, P, P, 4, 64, P, 1, P, 1, 1, 32, 64, P, 64, 1,
                                     None) == ERR_NO_DEVICE
    assert L.idx_logits_paged_insert_fp8(P, P, 0, P, 1, P, 4, 64, P, 1, P, 1, 1, 32, 64, P, 64, 1,
                                         None) == ERR_NO_DEVICE


def test_python_wrapper_raises_on_error(L):
    with pytest.raises(mx.MxidxError):
        mx._check(ERR_ARG, "probe")


def test_arch_rule_fails_closed(L):
    """The gate's architecture rule (P2 "Summary": fail-closed capability gates):
    only gfx950, bare or with target features, is accepted."""
    for name in (b"gfx950", b"gfx950:sramecc+:xnack-", b"gfx950:xnack+"):
        assert L.idx_arch_supported(name) == OK, name
    for name in (b"gfx942", b"gfx942:sramecc+:xnack-", b"gfx9500", b"gfx95", b"gfx90a", b"gfx1100",
                 b"", b"sm_100", b" gfx950", b"GFX950"):
        assert L.idx_arch_supported(name) == ERR_ARCH, name
    assert L.idx_arch_supported(None) == ERR_ARCH


def test_prefill_key_count_limit(L):
    """S up to 2^31 - 1025 is accepted (here with no query rows: a no-op), one
    more is rejected before any device work."""
    lim = 0x7fffffff - 1024
    assert L.idx_logits_prefill(P, P, P, P, P, P, P, 0, 32, lim, P, lim, 1, None) == OK
    assert L.idx_logits_prefill(P, P, P, P, P, P, P, 0, 32, lim + 1, P, lim + 1, 1, None) == ERR_ARG
    assert L.idx_logits_prefill(P, P, P, P, P, P, P, 4, 32, lim + 1, P, lim + 1, 1, None) == ERR_ARG


def test_topk_noalloc_argument_validation(L):
    f = L.idx_topk_noalloc
    assert f(P, 4, 64, None, P, 0, P2, None) == ERR_ARG                 # k = 0
    assert f(P, 4, 64, None, P, 2049, P2, None) == ERR_ARG              # k > 2048
    assert f(MIS, 4, 64, None, P, 8, P2, None) == ERR_ARG               # misaligned logits
    assert f(P, 4, 64, None, None, 8, P2, None) == ERR_ARG              # null ke
    assert f(None, 0, 64, None, None, 8, None, None) == OK              # no rows: no-op
    # more workspace than the library's scratch holds: rejected on the host
    assert L.idx_topk_workspace_bytes(64, 8192 * 64) > mx.TOPK_NOALLOC_MAX_WORKSPACE
    assert f(P, 64, 8192 * 64, None, P, 2048, P2, None) == ERR_ARG
    # the long-context decode shape fits (it stops at the device gate here)
    assert 0 < L.idx_topk_workspace_bytes(64, 131072) <= mx.TOPK_NOALLOC_MAX_WORKSPACE
    if not _has_gpu():
        assert f(P, 64, 131072, None, P, 2048, P2, None) == ERR_NO_DEVICE


def test_fp8_argument_validation(L):
    q = L.idx_quantize_fp8
    assert q(P, 0, 4, 128, 2, P, P2, None, None, None) == ERR_ARG         # bad scale format
    assert q(P, 0, 4, 128, 0, P, P2, P, None, None) == ERR_ARG            # w_in without w_out
    assert q(P, 0, 4, 128, 0, MIS, P2, None, None, None) == ERR_ARG       # misaligned values
    assert q(P, 2, 4, 128, 0, P, P2, None, None, None) == ERR_ARG         # bad dtype
    assert q(None, 0, 0, 128, 1, None, None, None, None, None) == OK      # no rows
    ins = L.idx_insert_fp8
    assert ins(P, 0, 4, 128, 0, P, P2, 4, 32, None) == ERR_ARG            # page size
    assert ins(P, 0, 4, 128, 3, P, P2, 4, 64, None) == ERR_ARG            # scale format
    assert ins(P, 0, 4, 128, 0, None, P2, 4, 64, None) == ERR_ARG         # null slots
    assert ins(None, 0, 0, 128, 0, None, None, 0, 64, None) == OK
    g = L.idx_gather_fp8
    assert g(P, 4, 64, P, 1, P, P, 1, 65, 65, P, P2, None) == ERR_ARG     # bt stride < pages
    assert g(P, 4, 64, P, 2, P, P, 1, 65, 65, P, MIS, None) == ERR_ARG    # misaligned scales
    assert g(P, 4, 64, P, 2, P, P, 0, 65, 65, P, P2, None) == OK          # no sequences
    pf = L.idx_logits_prefill_fp8
    for H in (0, 8, 24, 144):
        assert pf(P, P, P, P, None, P, 4, H, 64, P, 64, 1, None) == ERR_ARG
    assert pf(P, MIS, P, P, None, P, 4, 32, 64, P, 64, 1, None) == ERR_ARG  # misaligned weights
    assert pf(P, P, P, P, None, P, 4, 32, 64, P, 63, 1, None) == ERR_ARG    # ld < S
    assert pf(P, P, P, P, None, P, 0, 32, 64, P, 64, 1, None) == OK
    pg = L.idx_logits_paged_fp8
    assert pg(P, P, P, 4, 64, P, 1, P, 1, 0, 32, 64, P, 64, 1, None) == ERR_ARG   # next_n 0
    assert pg(P, P, P, 4, 64, P, 1, P, 1, 1, 32, 65, P, 65, 1, None) == ERR_ARG   # bt stride
    assert pg(P, P, P, 4, 48, P, 1, P, 1, 1, 32, 64, P, 64, 1, None) == ERR_ARG   # page size
    assert pg(P, P, P, 4, 64, P, 1, P, 0, 1, 32, 64, P, 64, 1, None) == OK        # no sequences
    if not _has_gpu():
        assert pg(P, P, P, 4, 64, P, 1, P, 1, 1, 32, 64, P, 64, 1, None) == ERR_NO_DEVICE


def test_quantize_rope_argument_validation(L):
    f = L.idx_quantize_rope
    assert f(P, 0, 4, 8, 128, P, P2, 4, None, 24, 0, P, P2, None) == ERR_ARG     # rope_dim % 16
    assert f(P, 0, 4, 8, 128, P, P2, 4, None, 144, 0, P, P2, None) == ERR_ARG    # rope_dim > 128
    assert f(P, 0, 4, 8, 128, P, P2, 4, None, 64, 2, P, P2, None) == ERR_ARG     # mode
    assert f(P, 0, 4, 8, 128, P, P2, 3, None, 64, 0, P, P2, None) == ERR_ARG     # table < T, no positions
    assert f(P, 0, 4, 8, 128, MIS, P2, 4, None, 64, 0, P, P2, None) == ERR_ARG   # misaligned cos
    assert f(P, 0, 4, 8, 128, None, None, 0, None, 64, 0, P, P2, None) == ERR_ARG  # no tables
    assert f(P, 0, 4, 0, 128, P, P2, 4, None, 64, 0, P, P2, None) == ERR_ARG     # H = 0
    assert f(None, 0, 0, 8, 128, None, None, 0, None, 64, 0, None, None, None) == OK   # T = 0
    if not _has_gpu():
        assert f(P, 0, 4, 8, 128, None, None, 0, None, 0, 0, P, P2, None) == ERR_NO_DEVICE  # rope_dim 0
        assert f(P, 0, 4, 8, 128, P, P2, 1, P, 64, 1, P, P2, None) == ERR_NO_DEVICE       # positions


def test_kpool_insert_argument_validation(L):
    f = L.idx_kpool_insert
    assert f(P, 0, 8, 128, P, P2, P, 0, 0, 0, P2, 4, 64, None, None) == ERR_ARG      # kpool 0
    assert f(P, 0, 8, 128, P, P2, P, 2000, 0, 0, P2, 4, 64, None, None) == ERR_ARG   # kpool too big
    assert f(P, 0, 8, 128, P, P2, P, 4, 2, 0, P2, 4, 64, None, None) == ERR_ARG      # format
    assert f(P, 0, 8, 128, P, P2, P, 4, 1, 5, P2, 4, 64, None, None) == ERR_ARG      # fp8 scale format
    assert f(P, 0, 8, 128, MIS, P2, P, 4, 0, 0, P2, 4, 64, None, None) == ERR_ARG    # misaligned gate
    assert f(P, 0, 8, 128, P, P2, P, 4, 0, 0, P2, 4, 32, None, None) == ERR_ARG     # page size
    assert f(P, 0, 8, 128, P, P2, P, 4, 0, 0, P2, 4, 64, MIS, None) == ERR_ARG      # misaligned out
    assert f(P, 0, 3, 128, None, None, None, 4, 0, 0, None, 4, 64, None, None) == OK  # n < kpool
    if not _has_gpu():
        assert f(P, 0, 8, 128, P, P2, P, 4, 1, 1, P2, 4, 64, None, None) == ERR_NO_DEVICE


def _rope(rope_dim=64, mode=0, cos=P, sin=P2, table_rows=8, positions=None):
    return mx._Rope(cos, sin, table_rows, positions, rope_dim, mode)


def test_insert_quantize_rope_argument_validation(L):
    # idx_insert_quantize_rope(k, k_dtype, n, k_stride, slots, cache, num_pages, page, q, q_dtype,
    #                          q_rows, q_stride, q_heads, rope, q_values, q_scales, stream)
    def call(rope, q_rows=16, q_heads=8, n=4):
        r = rope
        return L.idx_insert_quantize_rope(P, 0, n, 128, P, P2, 4, 64, P, 0, q_rows, 128, q_heads,
                                          None if r is None else ctypes.addressof(r), P, P2, None)
    assert call(None) == ERR_ARG                                 # no rope block
    assert call(_rope(rope_dim=24)) == ERR_ARG                   # rope_dim % 16
    assert call(_rope(rope_dim=144)) == ERR_ARG                  # rope_dim > 128
    assert call(_rope(mode=2)) == ERR_ARG                        # pairing
    assert call(_rope(cos=MIS)) == ERR_ARG                       # misaligned table
    assert call(_rope(cos=None)) == ERR_ARG                      # missing table
    assert call(_rope(positions=MIS)) == ERR_ARG                 # misaligned positions
    assert call(_rope(table_rows=-1)) == ERR_ARG
    assert call(_rope(table_rows=1)) == ERR_ARG                  # 2 tokens, 1 table row, no positions
    assert call(_rope(), q_heads=0) == ERR_ARG
    assert call(_rope(), q_rows=12, q_heads=8) == ERR_ARG        # rows not a multiple of heads
    assert call(_rope(), q_rows=0, n=0) == OK                    # nothing to do
    if not _has_gpu():
        assert call(_rope()) == ERR_NO_DEVICE
        assert call(_rope(rope_dim=0, cos=None, sin=None)) == ERR_NO_DEVICE
        assert call(_rope(table_rows=1, positions=P)) == ERR_NO_DEVICE


def test_logits_paged_insert_rope_argument_validation(L):
    def call(rope, H=32, next_n=1, max_len=64, B=1, dtype=0):
        return L.idx_logits_paged_insert_rope(P, P, dtype, P, P, 4, 64, P, 1, P, B, next_n, H,
                                              max_len, P, 64, 1,
                                              None if rope is None else ctypes.addressof(rope),
                                              None)
    assert call(None) == ERR_ARG
    for dim in (16, 32, 48, 96, 112):                            # neox: 64 or 128 only
        assert call(_rope(rope_dim=dim, mode=0)) == ERR_ARG
    assert call(_rope(rope_dim=24, mode=1)) == ERR_ARG
    assert call(_rope(mode=3)) == ERR_ARG
    assert call(_rope(sin=MIS)) == ERR_ARG
    assert call(_rope(positions=MIS)) == ERR_ARG
    assert call(_rope(), H=24) == ERR_ARG
    assert call(_rope(), next_n=17) == ERR_ARG
    assert call(_rope(), dtype=2) == ERR_ARG
    assert call(_rope(), B=0) == OK
    if not _has_gpu():
        for dim, mode in ((64, 0), (128, 0), (0, 0), (48, 1), (16, 1)):
            assert call(_rope(rope_dim=dim, mode=mode)) == ERR_NO_DEVICE
