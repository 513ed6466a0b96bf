"""Paged decode attention over an FP8 e4m3 KV cache with page-tag checks, for
AMD Instinct MI355X (gfx950).

This package is a thin binding over the C ABI in ``include/fp8kv.h``
(``libfp8kv.so``, built in-tree by ``decode_attention_fp8_kv_amd.build``).
The functions below only marshal torch tensors into pointers and sizes;
every step of the computation runs in the library's HIP kernels.  If the
library is missing, every call raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "KV_FP8_E4M3", "KV_BF16", "ABORT_TAG_MISMATCH", "ABORT_BAD_METADATA", "Fp8KvError",
    "lib_path", "load_library", "abi_version", "kv_quant_append", "paged_decode_attn", "paged_decode_step",
    "paged_decode_attn_noalloc",
    "paged_decode_attn_workspace_size", "paged_decode_attn_path", "alloc_workspace",
    "kv_quant_append_checked", "page_pool_init", "page_alloc", "page_free", "kv_absmax_scale",
    "kv_absmax_scale_kv",
    "kv_quant_append_dscale", "int4_gemv", "int4_pack_weights", "int4_tile_shapes",
]

KV_FP8_E4M3 = 0
KV_BF16 = 1
ABORT_TAG_MISMATCH = 1
ABORT_BAD_METADATA = 2
AMAX_WORK_FLOATS = 512  # kv_absmax_scale's work buffer, in floats
INT4_GROUP = 128        # int4_gemv: weights per scale along K
INT4_MAX_M = 64         # int4_gemv: largest number of activation rows
NOALLOC_SCRATCH_BYTES = 32 << 20  # paged_decode_attn_noalloc's fixed device scratch
ERR_SCRATCH = -9        # paged_decode_attn_noalloc: sizes need more than the scratch holds

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libfp8kv.so")
_lib = None


class Fp8KvError(RuntimeError):
    """A negative status from the library."""

    def __init__(self, fn: str, status: int, text: str, hip: str):
        msg = f"{fn} failed with status {status}: {text}"
        if hip:
            msg += f" ({hip})"
        super().__init__(msg)
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load ``libfp8kv.so`` once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(
            f"{lib_path} is missing: build it with `python -m decode_attention_fp8_kv_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(lib_path)
    c = ctypes
    vp, i32, f32, sz = c.c_void_p, c.c_int32, c.c_float, c.c_size_t
    lib.fp8kv_abi_version.restype = c.c_int
    lib.fp8kv_abi_version.argtypes = []
    lib.fp8kv_status_string.restype = c.c_char_p
    lib.fp8kv_status_string.argtypes = [c.c_int]
    lib.fp8kv_last_hip_error.restype = c.c_char_p
    lib.fp8kv_last_hip_error.argtypes = []
    lib.kv_quant_append.restype = c.c_int
    lib.kv_quant_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, f32, f32, vp, vp, i32, i32, i32, i32, i32,
                                    i32, vp]
    lib.paged_decode_attn_workspace_size.restype = sz
    lib.paged_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_decode_attn_path.restype = c.c_int
    lib.paged_decode_attn_path.argtypes = [i32, i32]
    lib.paged_decode_attn.restype = c.c_int
    lib.paged_decode_attn.argtypes = [vp, vp, vp, i32, f32, f32, vp, i32, vp, vp, vp, vp, vp, vp, sz, i32, i32,
                                      i32, i32, i32, i32, f32, i32, vp]
    lib.paged_decode_attn_noalloc.restype = c.c_int
    lib.paged_decode_attn_noalloc.argtypes = [vp, vp, vp, i32, f32, f32, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                              i32, i32, i32, f32, i32, vp]
    lib.paged_decode_step.restype = c.c_int
    lib.paged_decode_step.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, f32, f32, vp, i32, vp, vp, vp, vp, vp,
                                      vp, sz, i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp]
    lib.kv_quant_append_checked.restype = c.c_int
    lib.kv_quant_append_checked.argtypes = [vp, vp, vp, vp, vp, i32, i32, f32, f32, vp, vp, i32, i32, i32, i32,
                                            i32, i32, vp, vp, vp, vp]
    lib.kv_absmax_scale.restype = c.c_int
    lib.kv_absmax_scale.argtypes = [vp, c.c_int64, vp, vp, vp]
    lib.kv_absmax_scale_kv.restype = c.c_int
    lib.kv_absmax_scale_kv.argtypes = [vp, vp, c.c_int64, vp, vp, vp]
    lib.kv_quant_append_dscale.restype = c.c_int
    lib.kv_quant_append_dscale.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           vp]
    lib.page_pool_init.restype = c.c_int
    lib.page_pool_init.argtypes = [vp, vp, i32, vp]
    lib.page_alloc.restype = c.c_int
    lib.page_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.page_free.restype = c.c_int
    lib.page_free.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.int4_gemv.restype = c.c_int
    lib.int4_gemv.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
    lib.int4_pack_weights.restype = c.c_int
    lib.int4_pack_weights.argtypes = [vp, vp, vp, vp, i32, i32, vp]
    _lib = lib
    return lib


def abi_version() -> int:
    return load_library().fp8kv_abi_version()


def _check(fn: str, status: int) -> None:
    if status != 0:
        lib = load_library()
        raise Fp8KvError(fn, status, lib.fp8kv_status_string(status).decode(),
                         lib.fp8kv_last_hip_error().decode())


def _ptr(t, dtypes, name, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _stream_handle(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_U32 = (torch.int32, torch.uint32)
_CACHE = {KV_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn), KV_BF16: (torch.bfloat16,)}


def kv_quant_append(k_new, v_new, row_seq, row_pos, page_table, k_scale, v_scale, k_cache, v_cache,
                    kv_dtype=KV_FP8_E4M3, stream=None):
    """Write rows ``k_new/v_new [n_rows, Hkv, D]`` into the paged caches.

    See ``kv_quant_append`` in ``include/fp8kv.h`` for the exact semantics.
    ``k_cache/v_cache``: ``[num_pages, Hkv, page_size, D]`` uint8 (FP8) or bf16.
    """
    dev = k_cache.device
    n_rows, hkv, d = k_new.shape
    num_pages, hkv_c, page_size, d_c = k_cache.shape
    if (hkv, d) != (hkv_c, d_c) or v_cache.shape != k_cache.shape or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch between rows and caches")
    if row_seq.numel() != n_rows or row_pos.numel() != n_rows:
        raise ValueError("row_seq/row_pos must have n_rows entries")
    batch, max_pages = page_table.shape
    status = load_library().kv_quant_append(
        _ptr(k_new, _BF16, "k_new", dev), _ptr(v_new, _BF16, "v_new", dev),
        _ptr(row_seq, _I32, "row_seq", dev), _ptr(row_pos, _I32, "row_pos", dev),
        _ptr(page_table, _I32, "page_table", dev), batch, max_pages, float(k_scale), float(v_scale),
        _ptr(k_cache, _CACHE[kv_dtype], "k_cache", dev), _ptr(v_cache, _CACHE[kv_dtype], "v_cache", dev),
        num_pages, n_rows, hkv, d, page_size, kv_dtype, _stream_handle(dev, stream))
    _check("kv_quant_append", status)


def paged_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages,
                                     num_blocks=0) -> int:
    return int(load_library().paged_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                               page_size, max_pages, num_blocks))


def paged_decode_attn_path(num_q_heads, num_kv_heads) -> int:
    return int(load_library().paged_decode_attn_path(num_q_heads, num_kv_heads))


def alloc_workspace(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages, num_blocks=0,
                    device="cuda"):
    """A workspace of the size the library asks for (allocated by torch; needs no initialization)."""
    n = paged_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages,
                                         num_blocks)
    if n == 0:
        raise ValueError("invalid sizes for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


def paged_decode_attn(q, k_cache, v_cache, page_table, seq_lens, out, abort_flags, workspace, *,
                      kv_dtype=KV_FP8_E4M3, k_scale=1.0, v_scale=1.0, page_tags=None, expected_tags=None,
                      softmax_scale=None, num_blocks=0, stream=None):
    """One decode step of attention; writes ``out`` (bf16) and ``abort_flags`` (uint8).

    See ``paged_decode_attn`` in ``include/fp8kv.h`` for the exact semantics.
    """
    dev = q.device
    batch, hq, d = q.shape
    num_pages, hkv, page_size, _ = k_cache.shape
    max_pages = page_table.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out.shape != q.shape or abort_flags.numel() != batch or page_table.shape[0] != batch:
        raise ValueError("shape mismatch")
    status = load_library().paged_decode_attn(
        _ptr(q, _BF16, "q", dev), _ptr(k_cache, _CACHE[kv_dtype], "k_cache", dev),
        _ptr(v_cache, _CACHE[kv_dtype], "v_cache", dev), kv_dtype, float(k_scale), float(v_scale),
        _ptr(page_table, _I32, "page_table", dev), max_pages, _ptr(seq_lens, _I32, "seq_lens", dev),
        _ptr(page_tags, _U32, "page_tags", dev), _ptr(expected_tags, _U32, "expected_tags", dev),
        _ptr(out, _BF16, "out", dev), _ptr(abort_flags, (torch.uint8,), "abort_flags", dev),
        _ptr(workspace, (torch.uint8,), "workspace", dev), workspace.numel(),
        batch, hq, hkv, d, page_size, num_pages, float(softmax_scale), int(num_blocks),
        _stream_handle(dev, stream))
    _check("paged_decode_attn", status)


def paged_decode_attn_noalloc(q, k_cache, v_cache, page_table, seq_lens, out, abort_flags, *,
                              kv_dtype=KV_FP8_E4M3, k_scale=1.0, v_scale=1.0, page_tags=None, expected_tags=None,
                              softmax_scale=None, num_blocks=0, stream=None):
    """paged_decode_attn with the library's fixed device scratch as its workspace (nothing is
    allocated; calls that overlap on one device race).  See ``paged_decode_attn_noalloc`` in
    ``include/fp8kv.h``."""
    dev = q.device
    batch, hq, d = q.shape
    num_pages, hkv, page_size, _ = k_cache.shape
    max_pages = page_table.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out.shape != q.shape or abort_flags.numel() != batch or page_table.shape[0] != batch:
        raise ValueError("shape mismatch")
    status = load_library().paged_decode_attn_noalloc(
        _ptr(q, _BF16, "q", dev), _ptr(k_cache, _CACHE[kv_dtype], "k_cache", dev),
        _ptr(v_cache, _CACHE[kv_dtype], "v_cache", dev), kv_dtype, float(k_scale), float(v_scale),
        _ptr(page_table, _I32, "page_table", dev), max_pages, _ptr(seq_lens, _I32, "seq_lens", dev),
        _ptr(page_tags, _U32, "page_tags", dev), _ptr(expected_tags, _U32, "expected_tags", dev),
        _ptr(out, _BF16, "out", dev), _ptr(abort_flags, (torch.uint8,), "abort_flags", dev),
        batch, hq, hkv, d, page_size, num_pages, float(softmax_scale), int(num_blocks),
        _stream_handle(dev, stream))
    _check("paged_decode_attn_noalloc", status)


def _event_handle(ev):
    """The hipEvent_t of a torch.cuda.Event (created by recording it once if needed), or None."""
    if ev is None:
        return None
    if not ev.cuda_event:
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def paged_decode_step(k_new, v_new, row_seq, row_pos, q, k_cache, v_cache, page_table, seq_lens, out, abort_flags,
                      workspace, *, kv_dtype=KV_FP8_E4M3, k_scale=1.0, v_scale=1.0, page_tags=None,
                      expected_tags=None, softmax_scale=None, num_blocks=0, decode_events=None, stream=None):
    """One decode step: kv_quant_append of the new rows ``k_new/v_new [n_rows, Hkv, D]``, then
    paged_decode_attn, with the page check (tags on) run inside the append's launch.  Results are
    bit-identical to the two calls.  ``decode_events``: optional pair of torch.cuda.Event recorded
    right before and right after the decode kernel.  See ``paged_decode_step`` in ``include/fp8kv.h``."""
    dev = q.device
    batch, hq, d = q.shape
    num_pages, hkv, page_size, _ = k_cache.shape
    max_pages = page_table.shape[1]
    n_rows = k_new.shape[0]
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out.shape != q.shape or abort_flags.numel() != batch or page_table.shape[0] != batch:
        raise ValueError("shape mismatch")
    if tuple(k_new.shape[1:]) != (hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between rows and caches")
    if row_seq.numel() != n_rows or row_pos.numel() != n_rows:
        raise ValueError("row_seq/row_pos must have n_rows entries")
    ev0, ev1 = (None, None) if decode_events is None else decode_events
    status = load_library().paged_decode_step(
        _ptr(k_new, _BF16, "k_new", dev), _ptr(v_new, _BF16, "v_new", dev), _ptr(row_seq, _I32, "row_seq", dev),
        _ptr(row_pos, _I32, "row_pos", dev), n_rows,
        _ptr(q, _BF16, "q", dev), _ptr(k_cache, _CACHE[kv_dtype], "k_cache", dev),
        _ptr(v_cache, _CACHE[kv_dtype], "v_cache", dev), kv_dtype, float(k_scale), float(v_scale),
        _ptr(page_table, _I32, "page_table", dev), max_pages, _ptr(seq_lens, _I32, "seq_lens", dev),
        _ptr(page_tags, _U32, "page_tags", dev), _ptr(expected_tags, _U32, "expected_tags", dev),
        _ptr(out, _BF16, "out", dev), _ptr(abort_flags, (torch.uint8,), "abort_flags", dev),
        _ptr(workspace, (torch.uint8,), "workspace", dev), workspace.numel(),
        batch, hq, hkv, d, page_size, num_pages, float(softmax_scale), int(num_blocks),
        _event_handle(ev0), _event_handle(ev1), _stream_handle(dev, stream))
    _check("paged_decode_step", status)


def kv_quant_append_checked(k_new, v_new, row_seq, row_pos, page_table, k_scale, v_scale, k_cache, v_cache,
                            page_tags, expected_tags, row_status, kv_dtype=KV_FP8_E4M3, stream=None):
    """kv_quant_append that writes a row only if its page's tag still equals the
    sequence's expected tag; ``row_status [n_rows]`` uint8 receives 0 written,
    1 tag mismatch, 2 bad destination.  See ``kv_quant_append_checked`` in
    ``include/fp8kv.h``."""
    dev = k_cache.device
    n_rows, hkv, d = k_new.shape
    num_pages, hkv_c, page_size, d_c = k_cache.shape
    if (hkv, d) != (hkv_c, d_c) or v_cache.shape != k_cache.shape or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch between rows and caches")
    if row_seq.numel() != n_rows or row_pos.numel() != n_rows or row_status.numel() != n_rows:
        raise ValueError("row_seq/row_pos/row_status must have n_rows entries")
    batch, max_pages = page_table.shape
    if page_tags.numel() != num_pages or tuple(expected_tags.shape) != (batch, max_pages):
        raise ValueError("page_tags must be [num_pages] and expected_tags [batch, max_pages]")
    status = load_library().kv_quant_append_checked(
        _ptr(k_new, _BF16, "k_new", dev), _ptr(v_new, _BF16, "v_new", dev),
        _ptr(row_seq, _I32, "row_seq", dev), _ptr(row_pos, _I32, "row_pos", dev),
        _ptr(page_table, _I32, "page_table", dev), batch, max_pages, float(k_scale), float(v_scale),
        _ptr(k_cache, _CACHE[kv_dtype], "k_cache", dev), _ptr(v_cache, _CACHE[kv_dtype], "v_cache", dev),
        num_pages, n_rows, hkv, d, page_size, kv_dtype, _ptr(page_tags, _U32, "page_tags", dev),
        _ptr(expected_tags, _U32, "expected_tags", dev), _ptr(row_status, (torch.uint8,), "row_status", dev),
        _stream_handle(dev, stream))
    _check("kv_quant_append_checked", status)


def page_pool_init(free_pages, free_count, stream=None):
    """Every page free: ``free_pages [num_pages]`` int32 stacked so pops return
    0, 1, 2, ...; ``free_count [1]`` int32 = num_pages."""
    dev = free_pages.device
    status = load_library().page_pool_init(_ptr(free_pages, _I32, "free_pages", dev),
                                           _ptr(free_count, _I32, "free_count", dev), free_pages.numel(),
                                           _stream_handle(dev, stream))
    _check("page_pool_init", status)


def page_alloc(n_new, page_counts, page_table, expected_tags, page_tags, free_pages, free_count, status,
               stream=None):
    """Hand out pages (see ``page_alloc`` in ``include/fp8kv.h``); every argument
    is a device tensor, updated in place."""
    dev = page_table.device
    batch, max_pages = page_table.shape
    st = load_library().page_alloc(
        _ptr(n_new, _I32, "n_new", dev), _ptr(page_counts, _I32, "page_counts", dev),
        _ptr(page_table, _I32, "page_table", dev), _ptr(expected_tags, _U32, "expected_tags", dev),
        _ptr(page_tags, _U32, "page_tags", dev), _ptr(free_pages, _I32, "free_pages", dev),
        _ptr(free_count, _I32, "free_count", dev), _ptr(status, (torch.uint8,), "status", dev),
        batch, max_pages, free_pages.numel(), _stream_handle(dev, stream))
    _check("page_alloc", st)


def page_free(release, page_counts, page_table, free_pages, free_count, status, stream=None):
    """Return the pages of released sequences (see ``page_free`` in
    ``include/fp8kv.h``)."""
    dev = page_table.device
    batch, max_pages = page_table.shape
    st = load_library().page_free(
        _ptr(release, (torch.uint8,), "release", dev), _ptr(page_counts, _I32, "page_counts", dev),
        _ptr(page_table, _I32, "page_table", dev), _ptr(free_pages, _I32, "free_pages", dev),
        _ptr(free_count, _I32, "free_count", dev), _ptr(status, (torch.uint8,), "status", dev),
        batch, max_pages, free_pages.numel(), _stream_handle(dev, stream))
    _check("page_free", st)


def kv_absmax_scale(x, out, work=None, stream=None):
    """``out[0]`` = max |x| over the finite elements of the bf16 tensor ``x``,
    ``out[1]`` = out[0] / 448 (1 if out[0] is 0); ``out`` is a float32 device
    tensor of at least 2 elements.  ``work`` is float32 device scratch of at
    least AMAX_WORK_FLOATS elements (any contents; one is allocated when
    None).  See ``kv_absmax_scale`` in ``include/fp8kv.h``."""
    dev = x.device
    if out.dtype != torch.float32 or out.numel() < 2:
        raise ValueError("out must be a float32 tensor with at least 2 elements")
    if work is None:
        work = torch.empty(AMAX_WORK_FLOATS, dtype=torch.float32, device=dev)
    if work.dtype != torch.float32 or work.numel() < AMAX_WORK_FLOATS:
        raise ValueError(f"work must be a float32 tensor with at least {AMAX_WORK_FLOATS} elements")
    st = load_library().kv_absmax_scale(_ptr(x, _BF16, "x", dev), x.numel(),
                                        _ptr(out, (torch.float32,), "out", dev),
                                        _ptr(work, (torch.float32,), "work", dev), _stream_handle(dev, stream))
    _check("kv_absmax_scale", st)


def kv_absmax_scale_kv(k, v, out, work=None, stream=None):
    """kv_absmax_scale of ``k`` and ``v`` (bf16, the same number of elements)
    in one call: ``out[0:2]`` for k, ``out[2:4]`` for v (float32 device
    tensor of at least 4 elements); ``work`` is float32 device scratch of at
    least 2 * AMAX_WORK_FLOATS elements (allocated when None).  See
    ``kv_absmax_scale_kv`` in ``include/fp8kv.h``."""
    dev = k.device
    if k.numel() != v.numel():
        raise ValueError("k and v must have the same number of elements")
    if out.dtype != torch.float32 or out.numel() < 4:
        raise ValueError("out must be a float32 tensor with at least 4 elements")
    if work is None:
        work = torch.empty(2 * AMAX_WORK_FLOATS, dtype=torch.float32, device=dev)
    if work.dtype != torch.float32 or work.numel() < 2 * AMAX_WORK_FLOATS:
        raise ValueError(f"work must be a float32 tensor with at least {2 * AMAX_WORK_FLOATS} elements")
    st = load_library().kv_absmax_scale_kv(_ptr(k, _BF16, "k", dev), _ptr(v, _BF16, "v", dev), k.numel(),
                                           _ptr(out, (torch.float32,), "out", dev),
                                           _ptr(work, (torch.float32,), "work", dev), _stream_handle(dev, stream))
    _check("kv_absmax_scale_kv", st)


def kv_quant_append_dscale(k_new, v_new, row_seq, row_pos, page_table, k_scale_dev, v_scale_dev, k_cache,
                           v_cache, stream=None):
    """kv_quant_append into an FP8 cache with the scales read from device
    memory: ``k_scale_dev`` / ``v_scale_dev`` are float32 device tensors whose
    first element is the scale (e.g. ``out[1:]`` of kv_absmax_scale)."""
    dev = k_cache.device
    n_rows, hkv, d = k_new.shape
    num_pages, hkv_c, page_size, d_c = k_cache.shape
    if (hkv, d) != (hkv_c, d_c) or v_cache.shape != k_cache.shape or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch between rows and caches")
    batch, max_pages = page_table.shape
    st = load_library().kv_quant_append_dscale(
        _ptr(k_new, _BF16, "k_new", dev), _ptr(v_new, _BF16, "v_new", dev),
        _ptr(row_seq, _I32, "row_seq", dev), _ptr(row_pos, _I32, "row_pos", dev),
        _ptr(page_table, _I32, "page_table", dev), batch, max_pages,
        k_scale_dev.data_ptr(), v_scale_dev.data_ptr(),
        _ptr(k_cache, _CACHE[KV_FP8_E4M3], "k_cache", dev), _ptr(v_cache, _CACHE[KV_FP8_E4M3], "v_cache", dev),
        num_pages, n_rows, hkv, d, page_size, _stream_handle(dev, stream))
    _check("kv_quant_append_dscale", st)


def int4_tile_shapes(n, k):
    """Shapes of the tile-layout codes (int32) and scales (bf16) for an
    [n][k] weight matrix: ((Np/16, k/128, 16, 16), (Np/16, k/128, 16))."""
    t, g = -(-n // 16), k // INT4_GROUP
    return (t, g, 16, 16), (t, g, 16)


def int4_pack_weights(w_rows, s_rows, w_tiles, s_tiles, stream=None):
    """Row layout (``w_rows`` int32 [N][K/8], ``s_rows`` bf16 [N][K/128]) ->
    tile layout (``w_tiles`` int32, ``s_tiles`` bf16, shapes from
    ``int4_tile_shapes``).  See ``int4_pack_weights`` in ``include/fp8kv.h``."""
    dev = w_rows.device
    n, kw = w_rows.shape
    k = kw * 8
    ws, ss = int4_tile_shapes(n, k)
    if tuple(s_rows.shape) != (n, k // INT4_GROUP) or w_tiles.numel() != math.prod(ws) or \
            s_tiles.numel() != math.prod(ss):
        raise ValueError("shape mismatch between row and tile layouts")
    st = load_library().int4_pack_weights(_ptr(w_rows, _I32, "w_rows", dev), _ptr(s_rows, _BF16, "s_rows", dev),
                                          _ptr(w_tiles, _I32, "w_tiles", dev), _ptr(s_tiles, _BF16, "s_tiles", dev),
                                          n, k, _stream_handle(dev, stream))
    _check("int4_pack_weights", st)


def int4_gemv(x, w_tiles, s_tiles, y, stream=None):
    """y = x @ (q * s)^T for INT4 weights in the tile layout: ``x`` bf16
    [M][K], ``w_tiles`` int32 and ``s_tiles`` bf16 with the shapes of
    ``int4_tile_shapes(N, K)``, ``y`` bf16 [M][N] (written; N is taken from
    it).  See ``int4_gemv`` in ``include/fp8kv.h``."""
    dev = x.device
    if x.dim() != 2 or y.dim() != 2:
        raise ValueError("x and y must be 2-D")
    m, k = x.shape
    n = y.shape[1]
    ws, ss = int4_tile_shapes(n, k)
    if y.shape[0] != m or w_tiles.numel() != math.prod(ws) or s_tiles.numel() != math.prod(ss):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, w_tiles {tuple(w_tiles.shape)}, "
                         f"s_tiles {tuple(s_tiles.shape)}, y {tuple(y.shape)}")
    st = load_library().int4_gemv(_ptr(x, _BF16, "x", dev), _ptr(w_tiles, _I32, "w_tiles", dev),
                                  _ptr(s_tiles, _BF16, "s_tiles", dev), _ptr(y, _BF16, "y", dev), m, n, k,
                                  _stream_handle(dev, stream))
    _check("int4_gemv", st)
