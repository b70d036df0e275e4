"""MXFP4 paged indexer cache for MI355X (gfx950): Python binding of libmxidx.so.

Thin ctypes layer over the C ABI in ``include/mxidx.h``: it checks tensor
dtypes/devices/shapes, allocates outputs with torch when the caller passes
none, and hands raw device pointers and the current HIP stream to the
library.  Every step of the path runs in the HIP kernels; there is no CPU or
PyTorch fallback, and a missing library raises ``MxidxError``.

Build the library with ``python -m mxfp4_paged_cache_quant_amd.build``.
"""

import ctypes
import os

__all__ = [
    "MxidxError", "lib", "lib_path", "version", "init",
    "quantize", "insert", "insert_quantize", "gather", "logits_prefill", "logits_paged",
    "logits_paged_insert", "topk", "topk_workspace_bytes", "topk_workspace", "topk_ws",
    "topk_noalloc", "topk_merge", "TOPK_NOALLOC_MAX_WORKSPACE",
    "quantize_rope", "insert_quantize_rope", "logits_paged_insert_rope", "ROPE_NEOX",
    "ROPE_INTERLEAVED", "kpool_insert",
    "quantize_fp8", "insert_fp8", "gather_fp8", "logits_prefill_fp8", "logits_paged_fp8",
    "logits_paged_insert_fp8",
    "FP8_ROW_BYTES", "FP8_SCALE_F32", "FP8_SCALE_POW2",
    "HEAD_DIM", "ROW_BYTES", "PAGE_SIZE", "TOPK_MAX", "EXPORTS",
]

HEAD_DIM = 128
CODE_BYTES = 64
SCALE_BYTES = 4
ROW_BYTES = 68
PAGE_SIZE = 64
TOPK_MAX = 2048
MAX_HEADS = 128
TOPK_NOALLOC_MAX_WORKSPACE = 36 << 20
FP8_ROW_BYTES = 132
FP8_SCALE_F32, FP8_SCALE_POW2 = 0, 1
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1

IDX_BF16, IDX_F32 = 0, 1


class _Rope(ctypes.Structure):
    """The C ABI's idx_rope block (include/mxidx.h)."""
    _fields_ = [("cos_table", ctypes.c_void_p), ("sin_table", ctypes.c_void_p),
                ("table_rows", ctypes.c_int64), ("positions", ctypes.c_void_p),
                ("rope_dim", ctypes.c_int), ("rope_mode", ctypes.c_int)]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmxidx.so")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

# name -> (restype, argtypes); must match include/mxidx.h
EXPORTS = {
    "idx_version": (_int, []),
    "idx_strerror": (ctypes.c_char_p, [_int]),
    "idx_init": (_int, [_int]),
    "idx_arch_supported": (_int, [ctypes.c_char_p]),
    "idx_quantize": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "idx_quantize_rope": (_int, [_c_void_p, _int, _i64, _int, _i64, _c_void_p, _c_void_p, _i64,
                                 _c_void_p, _int, _int, _c_void_p, _c_void_p, _c_void_p]),
    "idx_insert": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _i64, _int, _c_void_p]),
    "idx_insert_quantize": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _i64, _int,
                                   _c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "idx_insert_quantize_rope": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _i64,
                                        _int, _c_void_p, _int, _i64, _i64, _int, _c_void_p,
                                        _c_void_p, _c_void_p, _c_void_p]),
    "idx_gather": (_int, [_c_void_p, _i64, _int, _c_void_p, _i64, _c_void_p, _c_void_p, _int, _i64,
                          _i64, _c_void_p, _c_void_p, _c_void_p]),
    "idx_logits_prefill": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _i64, _int, _i64, _c_void_p, _i64, _int, _c_void_p]),
    "idx_logits_paged": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _int, _c_void_p,
                                _i64, _c_void_p, _int, _int, _int, _i64, _c_void_p, _i64, _int,
                                _c_void_p]),
    "idx_logits_paged_insert": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _i64, _int,
                                       _c_void_p, _i64, _c_void_p, _int, _int, _int, _i64,
                                       _c_void_p, _i64, _int, _c_void_p]),
    "idx_logits_paged_insert_rope": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _c_void_p, _i64,
                                            _int, _c_void_p, _i64, _c_void_p, _int, _int, _int,
                                            _i64, _c_void_p, _i64, _int, _c_void_p, _c_void_p]),
    "idx_quantize_fp8": (_int, [_c_void_p, _int, _i64, _i64, _int, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p]),
    "idx_insert_fp8": (_int, [_c_void_p, _int, _i64, _i64, _int, _c_void_p, _c_void_p, _i64, _int,
                              _c_void_p]),
    "idx_gather_fp8": (_int, [_c_void_p, _i64, _int, _c_void_p, _i64, _c_void_p, _c_void_p, _int,
                              _i64, _i64, _c_void_p, _c_void_p, _c_void_p]),
    "idx_logits_prefill_fp8": (_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                      _c_void_p, _i64, _int, _i64, _c_void_p, _i64, _int,
                                      _c_void_p]),
    "idx_logits_paged_fp8": (_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _int, _c_void_p, _i64,
                                    _c_void_p, _int, _int, _int, _i64, _c_void_p, _i64, _int,
                                    _c_void_p]),
    "idx_logits_paged_insert_fp8": (_int, [_c_void_p, _c_void_p, _int, _c_void_p, _int, _c_void_p,
                                           _i64, _int, _c_void_p, _i64, _c_void_p, _int, _int, _int,
                                           _i64, _c_void_p, _i64, _int, _c_void_p]),
    "idx_kpool_insert": (_int, [_c_void_p, _int, _i64, _i64, _c_void_p, _c_void_p, _c_void_p, _int,
                                _int, _int, _c_void_p, _i64, _int, _c_void_p, _c_void_p]),
    "idx_topk": (_int, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p]),
    "idx_topk_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "idx_topk_ws": (_int, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _int, _c_void_p, _c_void_p,
                           ctypes.c_size_t, _c_void_p]),
    "idx_topk_noalloc": (_int, [_c_void_p, _i64, _i64, _c_void_p, _c_void_p, _int, _c_void_p,
                                _c_void_p]),
    "idx_topk_merge": (_int, [_c_void_p, _c_void_p, _int, _i64, _int, _int, _int, _c_void_p,
                              _c_void_p]),
}


class MxidxError(RuntimeError):
    def __init__(self, what, status=None):
        self.status = status
        super().__init__(what)


_LIB = None


def lib():
    """The loaded ctypes library (raises MxidxError when it is not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise MxidxError(f"{lib_path} is not built: run python -m mxfp4_paged_cache_quant_amd.build")
        handle = ctypes.CDLL(lib_path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status, call):
    if status != 0:
        msg = lib().idx_strerror(status).decode()
        raise MxidxError(f"{call}: {msg} (status {status})", status)


def version():
    return lib().idx_version()


def init(device=0):
    _check(lib().idx_init(device), "idx_init")


# ---------------------------------------------------------------------------
# torch-facing wrappers (torch supplies device memory and the stream only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise MxidxError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise MxidxError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _rows_view(x, name):
    """[..., 128] tensor with unit inner stride -> (rows, row_stride, dtype code)."""
    torch = _torch()
    _dev(x, name)
    if x.dtype == torch.bfloat16:
        code = IDX_BF16
    elif x.dtype == torch.float32:
        code = IDX_F32
    else:
        raise MxidxError(f"{name} must be bfloat16 or float32")
    if x.dim() >= 1 and x.shape[-1] == HEAD_DIM and x.numel() == 0:
        return 0, HEAD_DIM, code                   # no rows: strides are irrelevant
    if x.shape[-1] != HEAD_DIM or x.stride(-1) != 1:
        raise MxidxError(f"{name} must be [..., 128] with a contiguous last dim")
    rows = x.numel() // HEAD_DIM
    if x.dim() == 1:
        stride = HEAD_DIM
    else:
        x2 = x.reshape(-1, HEAD_DIM) if x.dim() > 2 else x
        if x2.data_ptr() != x.data_ptr():
            raise MxidxError(f"{name} rows must be addressable with one row stride")
        stride = x2.stride(0) if rows > 1 else HEAD_DIM
    return rows, stride, code


def quantize(x, values=None, scales=None, stream=None):
    """MXFP4-encode rows of 128 values: returns (values u8 [..., 64], scales u8 [..., 4])."""
    torch = _torch()
    rows, stride, code = _rows_view(x, "x")
    lead = tuple(x.shape[:-1])
    if values is None:
        values = torch.empty(lead + (CODE_BYTES,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (SCALE_BYTES,), dtype=torch.uint8, device=x.device)
    _dev(values, "values", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    if values.numel() != rows * CODE_BYTES or scales.numel() != rows * SCALE_BYTES or \
            not values.is_contiguous() or not scales.is_contiguous():
        raise MxidxError("values/scales must be contiguous [rows, 64] / [rows, 4]")
    _check(lib().idx_quantize(_ptr(x), code, rows, stride, _ptr(values), _ptr(scales), _stream(stream)),
           "idx_quantize")
    return values, scales


def _check_rope_tables(cos, sin, rope_dim, positions, tokens):
    torch = _torch()
    for name, t in (("cos", cos), ("sin", sin)):
        _dev(t, name, torch.float32)
        if not t.is_contiguous() or t.dim() != 2 or t.shape[1] != rope_dim // 2:
            raise MxidxError(f"{name} must be a contiguous fp32 [table_rows, rope_dim/2]")
    if cos.shape != sin.shape:
        raise MxidxError("cos and sin tables must have the same shape")
    if positions is not None:
        _dev(positions, "positions", torch.int64)
        if positions.numel() != tokens or not positions.is_contiguous():
            raise MxidxError(f"positions must be a contiguous int64 [{tokens}]")


def _rope_block(cos, sin, rope_dim, mode, positions):
    """The idx_rope block of a fused call (the tensors must outlive the call)."""
    return _Rope(_ptr(cos), _ptr(sin), cos.shape[0], _ptr(positions), rope_dim,
                 {"neox": ROPE_NEOX, "interleaved": ROPE_INTERLEAVED}[mode])


def quantize_rope(q, cos, sin, rope_dim, mode="neox", positions=None, values=None, scales=None,
                  stream=None):
    """RoPE on the first ``rope_dim`` dims of each head of q [T, H, 128] (cos / sin
    fp32 [table_rows, rope_dim/2], table row positions[t] or t; ``mode`` "neox" or
    "interleaved"), then MXFP4: returns (values u8 [T, H, 64], scales u8 [T, H, 4])."""
    torch = _torch()
    if q.dim() != 3:
        raise MxidxError("q must be [T, H, 128]")
    T, H = q.shape[0], q.shape[1]
    rows, stride, code = _rows_view(q, "q")
    _check_rope_tables(cos, sin, rope_dim, positions, T)
    if values is None:
        values = torch.empty((T, H, CODE_BYTES), dtype=torch.uint8, device=q.device)
    if scales is None:
        scales = torch.empty((T, H, SCALE_BYTES), dtype=torch.uint8, device=q.device)
    _dev(values, "values", torch.uint8)
    _dev(scales, "scales", torch.uint8)
    if values.numel() != rows * CODE_BYTES or scales.numel() != rows * SCALE_BYTES or \
            not values.is_contiguous() or not scales.is_contiguous():
        raise MxidxError("values/scales must be contiguous [T, H, 64] / [T, H, 4]")
    mode_code = {"neox": ROPE_NEOX, "interleaved": ROPE_INTERLEAVED}[mode]
    _check(lib().idx_quantize_rope(_ptr(q), code, T, H, stride, _ptr(cos), _ptr(sin), cos.shape[0],
                                   _ptr(positions), rope_dim, mode_code, _ptr(values), _ptr(scales),
                                   _stream(stream)), "idx_quantize_rope")
    return values, scales


def insert(k, slot_mapping, cache, stream=None):
    """Quantize K rows [N, 128] and scatter them into ``cache`` [num_pages, 64*68] (in place)."""
    torch = _torch()
    rows, stride, code = _rows_view(k, "k")
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(cache, "cache", torch.uint8)
    if slot_mapping.numel() != rows or not slot_mapping.is_contiguous():
        raise MxidxError("slot_mapping must be a contiguous int64 [N]")
    if not cache.is_contiguous() or cache.numel() % (PAGE_SIZE * ROW_BYTES) != 0:
        raise MxidxError("cache must be a contiguous uint8 [num_pages, 64*68]")
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    _check(lib().idx_insert(_ptr(k), code, rows, stride, _ptr(slot_mapping), _ptr(cache), num_pages,
                            PAGE_SIZE, _stream(stream)), "idx_insert")
    return cache


def insert_quantize(k, slot_mapping, cache, q, q_values=None, q_scales=None, stream=None):
    """insert(k, slot_mapping, cache) and quantize(q) in one launch; returns (q_values, q_scales)."""
    torch = _torch()
    rows, stride, code = _rows_view(k, "k")
    q_rows, q_stride, q_code = _rows_view(q, "q")
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(cache, "cache", torch.uint8)
    if slot_mapping.numel() != rows or not slot_mapping.is_contiguous():
        raise MxidxError("slot_mapping must be a contiguous int64 [N]")
    if not cache.is_contiguous() or cache.numel() % (PAGE_SIZE * ROW_BYTES) != 0:
        raise MxidxError("cache must be a contiguous uint8 [num_pages, 64*68]")
    lead = tuple(q.shape[:-1])
    if q_values is None:
        q_values = torch.empty(lead + (CODE_BYTES,), dtype=torch.uint8, device=q.device)
    if q_scales is None:
        q_scales = torch.empty(lead + (SCALE_BYTES,), dtype=torch.uint8, device=q.device)
    _dev(q_values, "q_values", torch.uint8)
    _dev(q_scales, "q_scales", torch.uint8)
    if q_values.numel() != q_rows * CODE_BYTES or q_scales.numel() != q_rows * SCALE_BYTES or \
            not q_values.is_contiguous() or not q_scales.is_contiguous():
        raise MxidxError("q_values/q_scales must be contiguous [rows, 64] / [rows, 4]")
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    _check(lib().idx_insert_quantize(_ptr(k), code, rows, stride, _ptr(slot_mapping), _ptr(cache),
                                     num_pages, PAGE_SIZE, _ptr(q), q_code, q_rows, q_stride,
                                     _ptr(q_values), _ptr(q_scales), _stream(stream)),
           "idx_insert_quantize")
    return q_values, q_scales


def insert_quantize_rope(k, slot_mapping, cache, q, cos, sin, rope_dim, mode="neox",
                         positions=None, q_values=None, q_scales=None, stream=None):
    """insert(k, slot_mapping, cache) and quantize_rope(q [T, H, 128], ...) in one
    launch; returns (q_values [T, H, 64], q_scales [T, H, 4])."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise MxidxError("q must be [T, H, 128]")
    T, H = q.shape[0], q.shape[1]
    rows, stride, code = _rows_view(k, "k")
    q_rows, q_stride, q_code = _rows_view(q, "q")
    _check_rope_tables(cos, sin, rope_dim, positions, T)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(cache, "cache", torch.uint8)
    if slot_mapping.numel() != rows or not slot_mapping.is_contiguous():
        raise MxidxError("slot_mapping must be a contiguous int64 [N]")
    if not cache.is_contiguous() or cache.numel() % (PAGE_SIZE * ROW_BYTES) != 0:
        raise MxidxError("cache must be a contiguous uint8 [num_pages, 64*68]")
    if q_values is None:
        q_values = torch.empty((T, H, CODE_BYTES), dtype=torch.uint8, device=q.device)
    if q_scales is None:
        q_scales = torch.empty((T, H, SCALE_BYTES), dtype=torch.uint8, device=q.device)
    _dev(q_values, "q_values", torch.uint8)
    _dev(q_scales, "q_scales", torch.uint8)
    if q_values.numel() != q_rows * CODE_BYTES or q_scales.numel() != q_rows * SCALE_BYTES or \
            not q_values.is_contiguous() or not q_scales.is_contiguous():
        raise MxidxError("q_values/q_scales must be contiguous [T, H, 64] / [T, H, 4]")
    rope = _rope_block(cos, sin, rope_dim, mode, positions)
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    _check(lib().idx_insert_quantize_rope(_ptr(k), code, rows, stride, _ptr(slot_mapping),
                                          _ptr(cache), num_pages, PAGE_SIZE, _ptr(q), q_code,
                                          q_rows, q_stride, H, ctypes.addressof(rope),
                                          _ptr(q_values), _ptr(q_scales), _stream(stream)),
           "idx_insert_quantize_rope")
    return q_values, q_scales


def gather(cache, block_table, seq_lens, cu_seq_offsets, max_seq_len, total_tokens,
           k_values=None, k_scales=None, stream=None):
    """Paged cache -> contiguous (k_values u8 [total, 64], k_scales u8 [total, 4])."""
    torch = _torch()
    _dev(cache, "cache", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(cu_seq_offsets, "cu_seq_offsets", torch.int64)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise MxidxError("block_table must be [batch, pages] with unit inner stride")
    batch = block_table.shape[0]
    if seq_lens.numel() != batch or cu_seq_offsets.numel() != batch:
        raise MxidxError("seq_lens / cu_seq_offsets must have one entry per sequence")
    if block_table.shape[1] * PAGE_SIZE < max_seq_len or not cache.is_contiguous():
        raise MxidxError("block_table has fewer pages than max_seq_len needs")
    if k_values is None:
        k_values = torch.zeros((total_tokens, CODE_BYTES), dtype=torch.uint8, device=cache.device)
    if k_scales is None:
        k_scales = torch.zeros((total_tokens, SCALE_BYTES), dtype=torch.uint8, device=cache.device)
    for name, t, cols in (("k_values", k_values, CODE_BYTES), ("k_scales", k_scales, SCALE_BYTES)):
        _dev(t, name, torch.uint8)
        if not t.is_contiguous() or t.numel() < total_tokens * cols:
            raise MxidxError(f"{name} must be a contiguous uint8 [total_tokens, {cols}]")
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    _check(lib().idx_gather(_ptr(cache), num_pages, PAGE_SIZE, _ptr(block_table), block_table.stride(0),
                            _ptr(seq_lens), _ptr(cu_seq_offsets), batch, int(max_seq_len),
                            int(total_tokens), _ptr(k_values), _ptr(k_scales), _stream(stream)),
           "idx_gather")
    return k_values, k_scales


def logits_prefill(q_values, q_scales, k_values, k_scales, weights, ks, ke, logits=None,
                   clean=True, stream=None):
    """Dense logits [T, S] (fp32) for rows t over columns [ks[t], ke[t])."""
    torch = _torch()
    T, H = q_values.shape[0], q_values.shape[1]
    S = k_values.shape[0]
    for name, t, dt in (("q_values", q_values, torch.uint8), ("q_scales", q_scales, torch.uint8),
                        ("k_values", k_values, torch.uint8), ("k_scales", k_scales, torch.uint8),
                        ("weights", weights, torch.float32), ("ke", ke, torch.int32)):
        _dev(t, name, dt)
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if ks is not None:
        _dev(ks, "ks", torch.int32)
    if tuple(q_values.shape) != (T, H, CODE_BYTES) or tuple(q_scales.shape) != (T, H, SCALE_BYTES) \
            or tuple(k_values.shape) != (S, CODE_BYTES) or tuple(k_scales.shape) != (S, SCALE_BYTES) \
            or tuple(weights.shape) != (T, H):
        raise MxidxError("shape mismatch among q/k/weights")
    if ke.numel() != T or (ks is not None and (ks.numel() != T or not ks.is_contiguous())):
        raise MxidxError("ks / ke must hold one entry per query row")
    if logits is None:
        fill = float("-inf") if clean else 0.0
        logits = torch.full((T, S), fill, dtype=torch.float32, device=q_values.device)
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < T or logits.shape[1] < S:
        raise MxidxError("logits must be [>=T, >=S] with contiguous rows")
    _check(lib().idx_logits_prefill(_ptr(q_values), _ptr(q_scales), _ptr(k_values), _ptr(k_scales),
                                    _ptr(weights), _ptr(ks), _ptr(ke), T, H, S, _ptr(logits),
                                    logits.stride(0), 1 if clean else 0, _stream(stream)),
           "idx_logits_prefill")
    return logits


def logits_paged(q_values, q_scales, weights, cache, block_table, context_lens, next_n,
                 max_context_len, logits=None, clean=True, stream=None):
    """Decode logits [B*next_n, max_context_len] (fp32) read through the block table."""
    torch = _torch()
    R, H = q_values.shape[0], q_values.shape[1]
    B = context_lens.numel()
    for name, t, dt in (("q_values", q_values, torch.uint8), ("q_scales", q_scales, torch.uint8),
                        ("weights", weights, torch.float32), ("cache", cache, torch.uint8),
                        ("block_table", block_table, torch.int32),
                        ("context_lens", context_lens, torch.int32)):
        _dev(t, name, dt)
    if R != B * next_n:
        raise MxidxError("q rows must be batch * next_n")
    for name, t in (("q_values", q_values), ("q_scales", q_scales), ("weights", weights),
                    ("cache", cache), ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if tuple(q_values.shape) != (R, H, CODE_BYTES) or tuple(q_scales.shape) != (R, H, SCALE_BYTES) \
            or tuple(weights.shape) != (R, H):
        raise MxidxError("shape mismatch among q/weights")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.shape[0] != B:
        raise MxidxError("block_table must be [batch, pages] with unit inner stride")
    if block_table.shape[1] * PAGE_SIZE < max_context_len:
        raise MxidxError("block_table has fewer pages than max_context_len needs")
    if logits is None:
        fill = float("-inf") if clean else 0.0
        logits = torch.full((R, max_context_len), fill, dtype=torch.float32, device=q_values.device)
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < R or \
            logits.shape[1] < max_context_len:
        raise MxidxError("logits must be [>=rows, >=max_context_len] with contiguous rows")
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    _check(lib().idx_logits_paged(_ptr(q_values), _ptr(q_scales), _ptr(weights), _ptr(cache), num_pages,
                                  PAGE_SIZE, _ptr(block_table), block_table.stride(0),
                                  _ptr(context_lens), B, next_n, H, int(max_context_len),
                                  _ptr(logits), logits.stride(0), 1 if clean else 0, _stream(stream)),
           "idx_logits_paged")
    return logits


def _paged_insert_args(q, k_new, weights, cache, block_table, context_lens, next_n,
                       max_context_len, logits, clean):
    """Checks of the one-launch decode step; returns (dtype code, rows, heads,
    batch, logits, num_pages)."""
    torch = _torch()
    for name, t in (("q", q), ("k_new", k_new)):
        _dev(t, name)
        if t.dtype not in (torch.bfloat16, torch.float32):
            raise MxidxError(f"{name} must be bfloat16 or float32")
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if k_new.dtype != q.dtype:
        raise MxidxError("q and k_new must have one dtype")
    code = IDX_BF16 if q.dtype == torch.bfloat16 else IDX_F32
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise MxidxError("q must be [rows, heads, 128]")
    R, H = q.shape[0], q.shape[1]
    B = context_lens.numel()
    if R != B * next_n:
        raise MxidxError("q rows must be batch * next_n")
    if tuple(k_new.shape) != (R, HEAD_DIM):
        raise MxidxError("k_new must be [batch * next_n, 128]")
    for name, t, dt in (("weights", weights, torch.float32), ("cache", cache, torch.uint8),
                        ("block_table", block_table, torch.int32),
                        ("context_lens", context_lens, torch.int32)):
        _dev(t, name, dt)
    for name, t in (("weights", weights), ("cache", cache), ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if tuple(weights.shape) != (R, H):
        raise MxidxError("weights must be [rows, heads]")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.shape[0] != B:
        raise MxidxError("block_table must be [batch, pages] with unit inner stride")
    if block_table.shape[1] * PAGE_SIZE < max_context_len:
        raise MxidxError("block_table has fewer pages than max_context_len needs")
    if logits is None:
        fill = float("-inf") if clean else 0.0
        logits = torch.full((R, max_context_len), fill, dtype=torch.float32, device=q.device)
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < R or \
            logits.shape[1] < max_context_len:
        raise MxidxError("logits must be [>=rows, >=max_context_len] with contiguous rows")
    num_pages = cache.numel() // (PAGE_SIZE * ROW_BYTES)
    return code, R, H, B, logits, num_pages


def logits_paged_insert(q, k_new, weights, cache, block_table, context_lens, next_n,
                        max_context_len, logits=None, clean=True, stream=None):
    """One decode step in one launch: the new tokens' K (k_new [B*next_n, 128], the
    last next_n positions of each sequence) into their block-table slots, q
    [B*next_n, H, 128] encoded to MXFP4, and the decode logits [B*next_n,
    max_context_len] of the updated cache (as insert + quantize + logits_paged)."""
    code, R, H, B, logits, num_pages = _paged_insert_args(
        q, k_new, weights, cache, block_table, context_lens, next_n, max_context_len, logits,
        clean)
    _check(lib().idx_logits_paged_insert(_ptr(q), _ptr(k_new), code, _ptr(weights), _ptr(cache),
                                         num_pages, PAGE_SIZE, _ptr(block_table),
                                         block_table.stride(0), _ptr(context_lens), B, next_n, H,
                                         int(max_context_len), _ptr(logits), logits.stride(0),
                                         1 if clean else 0, _stream(stream)),
           "idx_logits_paged_insert")
    return logits


def logits_paged_insert_rope(q, k_new, weights, cache, block_table, context_lens, next_n,
                             max_context_len, cos, sin, rope_dim, mode="neox", positions=None,
                             logits=None, clean=True, stream=None):
    """logits_paged_insert with q rotated first (as quantize_rope; positions
    [B*next_n] int64, or None: each row at its token's position
    context_lens[b] - next_n + i).  Neox pairing takes rope_dim 64 or 128 here."""
    code, R, H, B, logits, num_pages = _paged_insert_args(
        q, k_new, weights, cache, block_table, context_lens, next_n, max_context_len, logits,
        clean)
    _check_rope_tables(cos, sin, rope_dim, positions, R)
    rope = _rope_block(cos, sin, rope_dim, mode, positions)
    _check(lib().idx_logits_paged_insert_rope(_ptr(q), _ptr(k_new), code, _ptr(weights),
                                              _ptr(cache), num_pages, PAGE_SIZE,
                                              _ptr(block_table), block_table.stride(0),
                                              _ptr(context_lens), B, next_n, H,
                                              int(max_context_len), _ptr(logits),
                                              logits.stride(0), 1 if clean else 0,
                                              ctypes.addressof(rope), _stream(stream)),
           "idx_logits_paged_insert_rope")
    return logits


def topk(logits, ks, ke, k, out=None, stream=None):
    """Per-row top-k column indices (int32 [rows, k], -1 padded)."""
    torch = _torch()
    _dev(logits, "logits", torch.float32)
    _dev(ke, "ke", torch.int32)
    if ks is not None:
        _dev(ks, "ks", torch.int32)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise MxidxError("logits must be 2-D with contiguous rows")
    rows = logits.shape[0]
    if ke.numel() != rows or not ke.is_contiguous() or \
            (ks is not None and (ks.numel() != rows or not ks.is_contiguous())):
        raise MxidxError("ks / ke must hold one entry per row")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    _dev(out, "out", torch.int32)
    if not out.is_contiguous() or tuple(out.shape) != (rows, k):
        raise MxidxError("out must be a contiguous int32 [rows, k]")
    _check(lib().idx_topk(_ptr(logits), rows, logits.stride(0), _ptr(ks), _ptr(ke), k, _ptr(out),
                          _stream(stream)), "idx_topk")
    return out


def topk_workspace_bytes(rows, row_stride):
    """Bytes of device workspace topk_ws needs for `rows` rows of stride `row_stride`
    (0 when it does not split rows)."""
    return int(lib().idx_topk_workspace_bytes(rows, row_stride))


def topk_workspace(rows, row_stride, device=None):
    """A uint8 workspace for topk_ws (uninitialized; reusable across calls in stream order)."""
    torch = _torch()
    n = topk_workspace_bytes(rows, row_stride)
    return torch.empty(max(n, 1), dtype=torch.uint8,
                       device=device if device is not None else torch.cuda.current_device())


def topk_ws(logits, ks, ke, k, workspace, out=None, stream=None):
    """topk with a device workspace (from topk_workspace): the same sets; few long rows
    are split over workgroups."""
    torch = _torch()
    _dev(logits, "logits", torch.float32)
    _dev(ke, "ke", torch.int32)
    _dev(workspace, "workspace", torch.uint8)
    if ks is not None:
        _dev(ks, "ks", torch.int32)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise MxidxError("logits must be 2-D with contiguous rows")
    rows = logits.shape[0]
    if ke.numel() != rows or not ke.is_contiguous() or \
            (ks is not None and (ks.numel() != rows or not ks.is_contiguous())):
        raise MxidxError("ks / ke must hold one entry per row")
    if not workspace.is_contiguous():
        raise MxidxError("workspace must be contiguous")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    _dev(out, "out", torch.int32)
    if not out.is_contiguous() or tuple(out.shape) != (rows, k):
        raise MxidxError("out must be a contiguous int32 [rows, k]")
    _check(lib().idx_topk_ws(_ptr(logits), rows, logits.stride(0), _ptr(ks), _ptr(ke), k, _ptr(out),
                             _ptr(workspace), workspace.numel(), _stream(stream)), "idx_topk_ws")
    return out


# ---------------------------------------------------------------------------
# FP8 (E4M3) indexer cache: 128 E4M3 values + an fp32 scale per row
# ---------------------------------------------------------------------------

def _fp8_cache_pages(cache):
    torch = _torch()
    _dev(cache, "cache", torch.uint8)
    if not cache.is_contiguous() or cache.numel() % (PAGE_SIZE * FP8_ROW_BYTES) != 0:
        raise MxidxError("cache must be a contiguous uint8 [num_pages, 64*132]")
    return cache.numel() // (PAGE_SIZE * FP8_ROW_BYTES)


def quantize_fp8(x, round_scale=False, weights=None, values=None, scales=None, weights_out=None,
                 stream=None):
    """FP8-encode rows of 128 values: returns (values u8 [..., 128], scales f32 [...]) and,
    with ``weights`` (one fp32 per row, e.g. [T, H] for q [T, H, 128]), also the folded
    weights w' = weights * scales as a third result."""
    torch = _torch()
    rows, stride, code = _rows_view(x, "x")
    lead = tuple(x.shape[:-1])
    if values is None:
        values = torch.empty(lead + (HEAD_DIM,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead, dtype=torch.float32, device=x.device)
    _dev(values, "values", torch.uint8)
    _dev(scales, "scales", torch.float32)
    if values.numel() != rows * HEAD_DIM or scales.numel() != rows or \
            not values.is_contiguous() or not scales.is_contiguous():
        raise MxidxError("values/scales must be contiguous [rows, 128] / [rows]")
    if weights is not None:
        _dev(weights, "weights", torch.float32)
        if weights.numel() != rows or not weights.is_contiguous():
            raise MxidxError("weights must be a contiguous fp32 tensor with one entry per row")
        if weights_out is None:
            weights_out = torch.empty_like(weights)
        _dev(weights_out, "weights_out", torch.float32)
        if weights_out.numel() != rows or not weights_out.is_contiguous():
            raise MxidxError("weights_out must be a contiguous fp32 tensor with one entry per row")
    fmt = FP8_SCALE_POW2 if round_scale else FP8_SCALE_F32
    _check(lib().idx_quantize_fp8(_ptr(x), code, rows, stride, fmt, _ptr(values), _ptr(scales),
                                  _ptr(weights), _ptr(weights_out), _stream(stream)),
           "idx_quantize_fp8")
    return (values, scales) if weights is None else (values, scales, weights_out)


def insert_fp8(k, slot_mapping, cache, round_scale=False, stream=None):
    """FP8-encode K rows [N, 128] into ``cache`` [num_pages, 64*132] (in place)."""
    torch = _torch()
    rows, stride, code = _rows_view(k, "k")
    _dev(slot_mapping, "slot_mapping", torch.int64)
    if slot_mapping.numel() != rows or not slot_mapping.is_contiguous():
        raise MxidxError("slot_mapping must be a contiguous int64 [N]")
    num_pages = _fp8_cache_pages(cache)
    fmt = FP8_SCALE_POW2 if round_scale else FP8_SCALE_F32
    _check(lib().idx_insert_fp8(_ptr(k), code, rows, stride, fmt, _ptr(slot_mapping), _ptr(cache),
                                num_pages, PAGE_SIZE, _stream(stream)), "idx_insert_fp8")
    return cache


def gather_fp8(cache, block_table, seq_lens, cu_seq_offsets, max_seq_len, total_tokens,
               k_values=None, k_scales=None, stream=None):
    """FP8 paged cache -> contiguous (k_values u8 [total, 128], k_scales f32 [total])."""
    torch = _torch()
    num_pages = _fp8_cache_pages(cache)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(cu_seq_offsets, "cu_seq_offsets", torch.int64)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise MxidxError("block_table must be [batch, pages] with unit inner stride")
    batch = block_table.shape[0]
    if seq_lens.numel() != batch or cu_seq_offsets.numel() != batch:
        raise MxidxError("seq_lens / cu_seq_offsets must have one entry per sequence")
    if block_table.shape[1] * PAGE_SIZE < max_seq_len:
        raise MxidxError("block_table has fewer pages than max_seq_len needs")
    if k_values is None:
        k_values = torch.zeros((total_tokens, HEAD_DIM), dtype=torch.uint8, device=cache.device)
    if k_scales is None:
        k_scales = torch.zeros((total_tokens,), dtype=torch.float32, device=cache.device)
    _dev(k_values, "k_values", torch.uint8)
    _dev(k_scales, "k_scales", torch.float32)
    if not k_values.is_contiguous() or k_values.numel() < total_tokens * HEAD_DIM or \
            not k_scales.is_contiguous() or k_scales.numel() < total_tokens:
        raise MxidxError("k_values / k_scales must be contiguous [total, 128] uint8 / [total] fp32")
    _check(lib().idx_gather_fp8(_ptr(cache), num_pages, PAGE_SIZE, _ptr(block_table),
                                block_table.stride(0), _ptr(seq_lens), _ptr(cu_seq_offsets), batch,
                                int(max_seq_len), int(total_tokens), _ptr(k_values), _ptr(k_scales),
                                _stream(stream)), "idx_gather_fp8")
    return k_values, k_scales


def logits_prefill_fp8(q_values, weights, k_values, k_scales, ks, ke, logits=None, clean=True,
                       stream=None):
    """Dense FP8 logits [T, S]: q_values u8 [T, H, 128], weights f32 [T, H] (the folded w'),
    k_values u8 [S, 128], k_scales f32 [S]."""
    torch = _torch()
    T, H = q_values.shape[0], q_values.shape[1]
    S = k_values.shape[0]
    for name, t, dt in (("q_values", q_values, torch.uint8), ("weights", weights, torch.float32),
                        ("k_values", k_values, torch.uint8), ("k_scales", k_scales, torch.float32),
                        ("ke", ke, torch.int32)):
        _dev(t, name, dt)
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if ks is not None:
        _dev(ks, "ks", torch.int32)
    if tuple(q_values.shape) != (T, H, HEAD_DIM) or tuple(weights.shape) != (T, H) or \
            tuple(k_values.shape) != (S, HEAD_DIM) or tuple(k_scales.shape) != (S,):
        raise MxidxError("shape mismatch among q/k/weights")
    if ke.numel() != T or (ks is not None and (ks.numel() != T or not ks.is_contiguous())):
        raise MxidxError("ks / ke must hold one entry per query row")
    if logits is None:
        fill = float("-inf") if clean else 0.0
        logits = torch.full((T, S), fill, dtype=torch.float32, device=q_values.device)
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < T or logits.shape[1] < S:
        raise MxidxError("logits must be [>=T, >=S] with contiguous rows")
    _check(lib().idx_logits_prefill_fp8(_ptr(q_values), _ptr(weights), _ptr(k_values),
                                        _ptr(k_scales), _ptr(ks), _ptr(ke), T, H, S, _ptr(logits),
                                        logits.stride(0), 1 if clean else 0, _stream(stream)),
           "idx_logits_prefill_fp8")
    return logits


def logits_paged_fp8(q_values, weights, cache, block_table, context_lens, next_n,
                     max_context_len, logits=None, clean=True, stream=None):
    """Paged FP8 decode logits [B*next_n, max_context_len]: q_values u8 [B*next_n, H, 128],
    weights f32 [B*next_n, H] (the folded w')."""
    torch = _torch()
    R, H = q_values.shape[0], q_values.shape[1]
    B = context_lens.numel()
    num_pages = _fp8_cache_pages(cache)
    for name, t, dt in (("q_values", q_values, torch.uint8), ("weights", weights, torch.float32),
                        ("block_table", block_table, torch.int32),
                        ("context_lens", context_lens, torch.int32)):
        _dev(t, name, dt)
    if R != B * next_n:
        raise MxidxError("q rows must be batch * next_n")
    for name, t in (("q_values", q_values), ("weights", weights), ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise MxidxError(f"{name} must be contiguous")
    if tuple(q_values.shape) != (R, H, HEAD_DIM) or tuple(weights.shape) != (R, H):
        raise MxidxError("shape mismatch among q/weights")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.shape[0] != B:
        raise MxidxError("block_table must be [batch, pages] with unit inner stride")
    if block_table.shape[1] * PAGE_SIZE < max_context_len:
        raise MxidxError("block_table has fewer pages than max_context_len needs")
    if logits is None:
        fill = float("-inf") if clean else 0.0
        logits = torch.full((R, max_context_len), fill, dtype=torch.float32, device=q_values.device)
    _dev(logits, "logits", torch.float32)
    if logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < R or \
            logits.shape[1] < max_context_len:
        raise MxidxError("logits must be [>=rows, >=max_context_len] with contiguous rows")
    _check(lib().idx_logits_paged_fp8(_ptr(q_values), _ptr(weights), _ptr(cache), num_pages,
                                      PAGE_SIZE, _ptr(block_table), block_table.stride(0),
                                      _ptr(context_lens), B, next_n, H, int(max_context_len),
                                      _ptr(logits), logits.stride(0), 1 if clean else 0,
                                      _stream(stream)), "idx_logits_paged_fp8")
    return logits


def logits_paged_insert_fp8(q, k_new, weights, cache, block_table, context_lens, next_n,
                            max_context_len, round_scale=False, logits=None, clean=True,
                            stream=None):
    """The FP8 decode step in one launch: the new tokens' K (k_new [B*next_n, 128])
    into their block-table slots of the FP8 cache, q [B*next_n, H, 128] encoded to
    E4M3 with its scales folded into the weights (weights [B*next_n, H], not
    folded), and the decode logits (as insert_fp8 + quantize_fp8 + logits_paged_fp8)."""
    code, R, H, B, logits, _ = _paged_insert_args(
        q, k_new, weights, cache, block_table, context_lens, next_n, max_context_len, logits,
        clean)
    num_pages = _fp8_cache_pages(cache)
    fmt = FP8_SCALE_POW2 if round_scale else FP8_SCALE_F32
    _check(lib().idx_logits_paged_insert_fp8(_ptr(q), _ptr(k_new), code, _ptr(weights), fmt,
                                             _ptr(cache), num_pages, PAGE_SIZE,
                                             _ptr(block_table), block_table.stride(0),
                                             _ptr(context_lens), B, next_n, H,
                                             int(max_context_len), _ptr(logits),
                                             logits.stride(0), 1 if clean else 0,
                                             _stream(stream)), "idx_logits_paged_insert_fp8")
    return logits


def kpool_insert(k, gate_score, ape, slot_mapping, cache, kpool, fmt="mxfp4", round_scale=False,
                 return_compressed=False, stream=None):
    """Pool kpool consecutive tokens of k [n, 128] (softmax over gate_score [n, 128] +
    ape [kpool, 128] per dimension) and write the pooled rows of the pool-end
    positions (slot >= 0, position >= kpool - 1) into ``cache`` (MXFP4
    [pages, 64*68] or, with fmt="fp8", [pages, 64*132]).  With
    return_compressed, also returns the fp32 pooled rows [n, 128] (rows of
    unwritten positions are zero)."""
    torch = _torch()
    n, stride, code = _rows_view(k, "k")
    _dev(gate_score, "gate_score", torch.float32)
    _dev(ape, "ape", torch.float32)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(cache, "cache", torch.uint8)
    if gate_score.shape != (n, HEAD_DIM) or not gate_score.is_contiguous():
        raise MxidxError("gate_score must be a contiguous fp32 [n, 128]")
    if ape.shape != (kpool, HEAD_DIM) or not ape.is_contiguous():
        raise MxidxError("ape must be a contiguous fp32 [kpool, 128]")
    if slot_mapping.numel() != n or not slot_mapping.is_contiguous():
        raise MxidxError("slot_mapping must be a contiguous int64 [n]")
    row = {"mxfp4": ROW_BYTES, "fp8": FP8_ROW_BYTES}[fmt]
    if not cache.is_contiguous() or cache.numel() % (PAGE_SIZE * row) != 0:
        raise MxidxError(f"cache must be a contiguous uint8 [num_pages, 64*{row}]")
    comp = torch.zeros((n, HEAD_DIM), dtype=torch.float32, device=k.device) if return_compressed else None
    _check(lib().idx_kpool_insert(_ptr(k), code, n, stride, _ptr(gate_score), _ptr(ape),
                                  _ptr(slot_mapping), kpool, 0 if fmt == "mxfp4" else 1,
                                  FP8_SCALE_POW2 if round_scale else FP8_SCALE_F32, _ptr(cache),
                                  cache.numel() // (PAGE_SIZE * row), PAGE_SIZE, _ptr(comp),
                                  _stream(stream)), "idx_kpool_insert")
    return (cache, comp) if return_compressed else cache


def topk_noalloc(logits, ks, ke, k, out=None, stream=None):
    """topk_ws with the library's static device scratch instead of a caller's
    workspace (no device allocation by the library; `out` is allocated here only
    when it is not given).  Raises when the call needs more than
    TOPK_NOALLOC_MAX_WORKSPACE bytes of workspace."""
    torch = _torch()
    _dev(logits, "logits", torch.float32)
    _dev(ke, "ke", torch.int32)
    if ks is not None:
        _dev(ks, "ks", torch.int32)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise MxidxError("logits must be 2-D with contiguous rows")
    rows = logits.shape[0]
    if ke.numel() != rows or not ke.is_contiguous() or \
            (ks is not None and (ks.numel() != rows or not ks.is_contiguous())):
        raise MxidxError("ks / ke must hold one entry per row")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    _dev(out, "out", torch.int32)
    if not out.is_contiguous() or tuple(out.shape) != (rows, k):
        raise MxidxError("out must be a contiguous int32 [rows, k]")
    _check(lib().idx_topk_noalloc(_ptr(logits), rows, logits.stride(0), _ptr(ks), _ptr(ke), k,
                                  _ptr(out), _stream(stream)), "idx_topk_noalloc")
    return out


def topk_merge(values, indices, interleave, k, out=None, stream=None):
    """Merge per-rank top-k lists (values f32 / indices i32 [world, rows, k_in], local
    positions, -1 empty) into global top-k positions [rows, k] (-1 padded)."""
    torch = _torch()
    _dev(values, "values", torch.float32)
    _dev(indices, "indices", torch.int32)
    if values.dim() != 3 or values.shape != indices.shape:
        raise MxidxError("values and indices must both be [world, rows, k_in]")
    if not values.is_contiguous() or not indices.is_contiguous():
        raise MxidxError("values and indices must be contiguous")
    world, rows, k_in = values.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=values.device)
    _dev(out, "out", torch.int32)
    if out.shape != (rows, k) or not out.is_contiguous():
        raise MxidxError("out must be a contiguous int32 [rows, k]")
    _check(lib().idx_topk_merge(_ptr(values), _ptr(indices), world, rows, k_in, interleave, k,
                                _ptr(out), _stream(stream)), "idx_topk_merge")
    return out
