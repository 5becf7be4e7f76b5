"""Python binding of libpa.so: the MI355X paged KV-cache write and PagedAttention decode.

Argument marshalling only: each function checks torch tensors (device, dtype,
shape, contiguity), passes their data pointers and the current HIP stream to
the C ABI declared in include/pa.h, and raises on a non-zero status.  Every
step of the computation runs in the library's HIP kernels or its C++ block
manager.  If libpa.so is missing, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "lib", "PAError", "cache_write", "copy_blocks", "decode", "decode_partitions",
    "decode_reduce", "decode_plan", "decode_workspace_size", "decode_schedule",
    "decode_scheduled", "decode_schedule_shared", "decode_scheduled_shared", "stream_read",
    "decode_contiguous", "copy_blocks_between", "prefill",
    "debug_status", "use_debug_library", "PA_DEBUG_TABLE", "PA_DEBUG_SLOT", "PA_DEBUG_PAIR",
    "PA_DEBUG_ITEM",
    "BlockManager",
    "DTYPE_CODES", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
# the same library built with PA_DEBUG (device checks of slots, block ids, copy pairs)
LIB_DEBUG_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_debug.so")
_LIB = None
_LIB_DEBUG = None
_USE_DEBUG = False

PA_DEBUG_TABLE = 1
PA_DEBUG_SLOT = 2
PA_DEBUG_PAIR = 4
PA_DEBUG_ITEM = 8

PA_OK = 0
PA_ERR_NO_BLOCKS = -4
_c = ctypes
_vp, _i32, _i64, _f32, _sz = _c.c_void_p, _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t
_pi32, _pi64 = _c.POINTER(_c.c_int32), _c.POINTER(_c.c_int64)

_DECODE_ARGS = [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _i32,
                _vp, _vp, _sz, _i32, _vp]

_SIGNATURES = {
    "pa_status_string": (_c.c_char_p, [_c.c_int]),
    "pa_version": (_c.c_int, []),
    "pa_debug_status": (_c.c_int, [_vp]),
    "pa_debug_enabled": (_c.c_int, []),
    "pa_cache_write": (_c.c_int, [_vp, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp]),
    "pa_copy_blocks": (_c.c_int, [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp]),
    "pa_decode": (_c.c_int, _DECODE_ARGS),
    "pa_decode_partitions": (_c.c_int, _DECODE_ARGS),
    "pa_decode_reduce": (_c.c_int, _DECODE_ARGS),
    "pa_decode_noalloc": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i64,
                                     _f32, _i32, _i32, _vp, _i32, _vp]),
    "pa_decode_scheduled": (_c.c_int, _DECODE_ARGS + [_vp, _i32]),
    "pa_decode_scheduled_shared": (_c.c_int, _DECODE_ARGS + [_vp, _i32, _vp, _i32, _vp]),
    "pa_decode_schedule_shared": (_c.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                             _vp, _i32, _pi32, _vp, _i32, _pi32, _vp, _i32,
                                             _pi32, _pi32, _pi32, _c.POINTER(_sz)]),
    "pa_decode_schedule": (_c.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _pi32,
                                      _pi32, _pi32]),
    "pa_decode_plan": (_c.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32,
                                  _c.POINTER(_sz)]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_bm_create": (_c.c_int, [_i64, _i32, _vp, _i64, _c.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_seq": (_c.c_int, [_vp, _i64, _i64]),
    "pa_bm_fork": (_c.c_int, [_vp, _i64, _i64]),
    "pa_bm_append_slot": (_c.c_int, [_vp, _i64, _pi64, _pi32, _pi32]),
    "pa_bm_append_slots": (_c.c_int, [_vp, _vp, _i32, _vp, _vp, _pi32, _pi32]),
    "pa_bm_step": (_c.c_int, [_vp, _vp, _i32, _vp, _vp, _pi32, _vp, _i32, _i32, _vp]),
    "pa_bm_free_seq": (_c.c_int, [_vp, _i64]),
    "pa_bm_select": (_c.c_int, [_vp, _vp, _vp, _i32, _vp, _i32]),
    "pa_bm_set_host_pool": (_c.c_int, [_vp, _i64, _vp, _i64]),
    "pa_bm_swap_out": (_c.c_int, [_vp, _vp, _i32, _vp, _i32, _pi32]),
    "pa_bm_swap_in": (_c.c_int, [_vp, _vp, _i32, _vp, _i32, _pi32]),
    "pa_bm_is_swapped": (_c.c_int, [_vp, _i64]),
    "pa_bm_num_free_host": (_i64, [_vp]),
    "pa_bm_host_free_list": (_i64, [_vp, _vp, _i64]),
    "pa_bm_host_refcount": (_i32, [_vp, _i32]),
    "pa_bm_blocks_needed": (_i64, [_vp, _vp, _i32]),
    "pa_prefill": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i64,
                              _f32, _i32, _i32, _vp, _vp]),
    "pa_copy_blocks_between": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i32, _i32,
                                          _i32, _i32, _vp]),
    "pa_bm_slots": (_c.c_int, [_vp, _i64, _i64, _i64, _vp]),
    "pa_bm_block_table": (_c.c_int, [_vp, _i64, _vp, _i32, _pi32]),
    "pa_bm_block_tables": (_c.c_int, [_vp, _vp, _i32, _vp, _i32, _i32, _vp]),
    "pa_bm_seq_len": (_i64, [_vp, _i64]),
    "pa_bm_refcount": (_i32, [_vp, _i32]),
    "pa_bm_num_free": (_i64, [_vp]),
    "pa_bm_num_seqs": (_i64, [_vp]),
    "pa_bm_free_list": (_i64, [_vp, _vp, _i64]),
    "pa_engine_staging_bytes": (_sz, [_i32, _i32, _i32]),
    "pa_engine_create": (_c.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _vp, _i32, _vp, _c.POINTER(_vp)]),
    "pa_engine_destroy": (None, [_vp]),
    "pa_engine_workspace_bytes": (_sz, [_vp, _i32]),
    "pa_engine_step": (_c.c_int, [_vp, _vp, _i32, _vp, _vp, _vp, _f32, _vp, _vp, _sz, _i32, _vp,
                                  _vp]),
    "pa_engine_last_step": (_c.c_int, [_vp, _i32, _vp, _vp, _vp, _i32]),
    "pa_engine_set_decode_events": (_c.c_int, [_vp, _vp, _vp]),
    "pa_engine_set_sharing": (_c.c_int, [_vp, _i32]),
    "pa_engine_set_mapped_staging": (_c.c_int, [_vp, _i32]),
    "pa_engine_has_mapped_staging": (_i32, [_vp]),
    "pa_stream_read": (_c.c_int, [_vp, _i64, _vp, _i32, _vp]),
    "pa_tile_read": (_c.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _vp]),
    "pa_decode_contiguous": (_c.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _i64, _i64,
                                        _i64, _f32, _i32, _i32, _vp, _vp, _sz, _i32, _vp, _vp,
                                        _i32]),
}


class StepInfo(_c.Structure):
    _fields_ = [("num_cow", _c.c_int32), ("max_context_len", _c.c_int32),
                ("partition_tokens", _c.c_int32), ("num_items", _c.c_int32),
                ("num_group_items", _c.c_int32), ("sum_context_len", _c.c_int64)]


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().pa_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status})")


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_cache_write_amd.build`")
    import torch  # noqa: F401  (loads torch's libamdhip64 first)
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """Load libpa.so (after torch, so that both use torch's HIP runtime), or
    libpa_debug.so while use_debug_library(True) is in effect."""
    global _LIB, _LIB_DEBUG
    if _USE_DEBUG:
        if _LIB_DEBUG is None:
            _LIB_DEBUG = _load(LIB_DEBUG_PATH)
        return _LIB_DEBUG
    if _LIB is None:
        _LIB = _load(LIB_PATH)
    return _LIB


def use_debug_library(on: bool = True) -> bool:
    """Route the following calls to libpa_debug.so (on) or libpa.so (off);
    returns the previous setting.  Objects keep the library they were made
    with (a BlockManager holds its handle's library)."""
    global _USE_DEBUG
    prev, _USE_DEBUG = _USE_DEBUG, bool(on)
    return prev


def debug_status(stream=None) -> int:
    """pa_debug_status: wait for the stream, return and clear the device error
    bits (PA_DEBUG_* ; always 0 from the release library)."""
    rc = lib().pa_debug_status(_stream(stream, None))
    if rc < 0:
        raise PAError(rc, "pa_debug_status")
    return rc


def _check(status: int, where: str):
    if status != PA_OK:
        raise PAError(status, where)


# ----------------------------------------------------------------- device
def _torch():
    import torch
    return torch


def DTYPE_CODES():
    torch = _torch()
    return {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def _dt(t) -> int:
    code = DTYPE_CODES().get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _dev(t, name, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None):
    """k_cache[s//bs, :, s%bs, :] = k[n] (and v) for every slot s = slot_mapping[n] >= 0."""
    torch = _torch()
    N, H, D = k.shape
    NB, Hc, bs, Dc = k_cache.shape
    if (Hc, Dc) != (H, D) or v.shape != k.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if slot_mapping.shape != (N,):
        raise ValueError("slot_mapping must be [N]")
    for t in (v, k_cache, v_cache):
        if t.dtype != k.dtype:
            raise TypeError("k, v and the caches must share a dtype")
    rc = lib().pa_cache_write(
        _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int64), N,
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), NB, H, D, bs, _dt(k),
        _stream(stream, k.device))
    _check(rc, "pa_cache_write")


def copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """k_cache[dst] = k_cache[src] (and v) for each (src, dst) row of block_pairs [n, 2]."""
    torch = _torch()
    NB, H, bs, D = k_cache.shape
    n = int(block_pairs.shape[0])
    if n and tuple(block_pairs.shape) != (n, 2):
        raise ValueError("block_pairs must be [n, 2]")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("cache mismatch")
    if n == 0:
        return
    rc = lib().pa_copy_blocks(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_pairs, "block_pairs", torch.int32), n, NB, H, D, bs, _dt(k_cache),
        _stream(stream, k_cache.device))
    _check(rc, "pa_copy_blocks")


def prefill(q, k_cache, v_cache, block_tables, cu_q, context_lens, scale, max_q_len, out=None,
            stream=None):
    """pa_prefill: causal attention of the packed new tokens ``q`` [T, H, D] over the
    paged cache; ``cu_q`` int32 [S+1] query offsets, ``context_lens`` int32 [S]
    (new tokens included, already written)."""
    torch = _torch()
    T, H, D = q.shape
    NB, Hc, bs, Dc = k_cache.shape
    S = int(context_lens.shape[0])
    if (Hc, Dc) != (H, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or cu_q.shape != (S + 1,):
        raise ValueError("block_tables must be [S, maxB] and cu_q [S + 1]")
    if out is None:
        out = torch.empty_like(q)
    rc = lib().pa_prefill(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(cu_q, "cu_q", torch.int32), _dev(context_lens, "context_lens", torch.int32), S, H,
        D, bs, NB, float(scale), int(max_q_len), _dt(q), _dev(out, "out"),
        _stream(stream, q.device))
    _check(rc, "pa_prefill")
    return out


def copy_blocks_between(src_k, src_v, dst_k, dst_v, block_pairs, stream=None):
    """dst[pairs[i,1]] = src[pairs[i,0]] for K and V between two pools of blocks
    [NB, H, bs, D] (device memory or pinned host memory): swapping."""
    torch = _torch()
    _, H, bs, D = src_k.shape
    n = int(block_pairs.shape[0])
    for t in (src_v, dst_k, dst_v):
        if tuple(t.shape[1:]) != (H, bs, D) or t.dtype != src_k.dtype:
            raise ValueError("pools must share [H, bs, D] and dtype")
    if not all(t.is_contiguous() for t in (src_k, src_v, dst_k, dst_v)):
        raise ValueError("pools must be contiguous")
    if n == 0:
        return
    if tuple(block_pairs.shape) != (n, 2) or block_pairs.dtype != torch.int32:
        raise ValueError("block_pairs must be int32 [n, 2]")
    if not (block_pairs.is_cuda or block_pairs.is_pinned()):
        raise ValueError("block_pairs must be device or pinned host memory")
    dev = src_k.device if src_k.is_cuda else dst_k.device
    rc = lib().pa_copy_blocks_between(src_k.data_ptr(), src_v.data_ptr(), dst_k.data_ptr(),
                                      dst_v.data_ptr(), block_pairs.data_ptr(), n,
                                      int(src_k.shape[0]), int(dst_k.shape[0]), H, D, bs,
                                      _dt(src_k), _stream(stream, dev))
    _check(rc, "pa_copy_blocks_between")


def decode_plan(num_seqs, num_heads, head_dim, block_size, max_context_len, dtype_code,
                partition_tokens=0):
    """(tokens per partition, partitions of the longest context, workspace bytes)."""
    pt, nparts, ws = _c.c_int32(), _c.c_int32(), _c.c_size_t()
    rc = lib().pa_decode_plan(num_seqs, num_heads, head_dim, block_size, max_context_len,
                              dtype_code, partition_tokens, _c.byref(pt), _c.byref(nparts),
                              _c.byref(ws))
    _check(rc, "pa_decode_plan")
    return pt.value, nparts.value, ws.value


def decode_workspace_size(num_seqs, num_heads, head_dim, block_size, max_context_len,
                          dtype_code, partition_tokens=0):
    return decode_plan(num_seqs, num_heads, head_dim, block_size, max_context_len, dtype_code,
                       partition_tokens)[2]


def _decode_call(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale,
                 max_context_len, out, workspace, partition_tokens, stream, extra=(),
                 ws_min_part=0):
    torch = _torch()
    S, H, D = q.shape
    NB, Hc, bs, Dc = k_cache.shape
    if (Hc, Dc) != (H, D) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, max_blocks]")
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [S]")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    for t in (k_cache, v_cache):
        if t.dtype != q.dtype:
            raise TypeError("q and the caches must share a dtype")
    dt = _dt(q)
    ws_need = decode_workspace_size(S, H, D, bs, int(max_context_len), dt, partition_tokens)
    if ws_min_part:  # shared-prefix launches also use partitions of ws_min_part tokens
        ws_need = max(ws_need, decode_workspace_size(S, H, D, bs, int(max_context_len), dt,
                                                     ws_min_part))
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = getattr(lib(), fn_name)(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables", torch.int32), int(block_tables.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), S, H, D, bs, NB, float(scale),
        int(max_context_len), dt, _dev(out, "out"), ws_ptr, ws_bytes, int(partition_tokens),
        _stream(stream, q.device), *extra)
    _check(rc, fn_name)
    return out


def decode_schedule(context_lens_host, num_heads, head_dim, block_size, dtype_code,
                    partition_tokens=0):
    """Host work list for pa_decode_scheduled: (items int32 [n, 5], partition_tokens,
    max_context_len)."""
    ctx = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    n, pt, mx = _c.c_int32(), _c.c_int32(), _c.c_int32()
    rc = lib().pa_decode_schedule(_ptr(ctx), ctx.size, num_heads, head_dim, block_size,
                                  dtype_code, partition_tokens, None, 0, _c.byref(n),
                                  _c.byref(pt), _c.byref(mx))
    if rc not in (PA_OK, -8):
        _check(rc, "pa_decode_schedule")
    items = np.empty((max(n.value, 1), 5), dtype=np.int32)
    rc = lib().pa_decode_schedule(_ptr(ctx), ctx.size, num_heads, head_dim, block_size,
                                  dtype_code, partition_tokens, _ptr(items), n.value,
                                  _c.byref(n), _c.byref(pt), _c.byref(mx))
    _check(rc, "pa_decode_schedule")
    return items[:n.value], pt.value, mx.value


def decode_contiguous(q, k, v, context_lens, scale, max_context_len, layout="SLHD", out=None,
                      workspace=None, partition_tokens=0, items=None, stream=None):
    """pa_decode_contiguous over non-paged K/V: ``layout`` "SLHD" ([S, L, H, D]) or
    "SHLD" ([S, H, L, D]); ``items`` an optional device work list from
    decode_schedule(..., block_size=16, ...)."""
    torch = _torch()
    S, H, D = q.shape
    if k.shape != v.shape or k.dim() != 4 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k, v must be 4-d tensors of q's dtype with equal shapes")
    if layout == "SLHD":
        if (k.shape[0], k.shape[2], k.shape[3]) != (S, H, D):
            raise ValueError("k must be [S, L, H, D]")
        L = int(k.shape[1])
        strides = (L * H * D, H * D, D)
    elif layout == "SHLD":
        if (k.shape[0], k.shape[1], k.shape[3]) != (S, H, D):
            raise ValueError("k must be [S, H, L, D]")
        L = int(k.shape[2])
        strides = (H * L * D, D, L * D)
    else:
        raise ValueError(layout)
    if context_lens.shape != (S,):
        raise ValueError("context_lens must be [S]")
    if out is None:
        out = torch.empty_like(q)
    dt = _dt(q)
    ws_need = decode_workspace_size(S, H, D, 16, int(max_context_len), dt, partition_tokens)
    if ws_need and (workspace is None or workspace.numel() * workspace.element_size() < ws_need):
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    n = int(items.shape[0]) if items is not None else 0
    rc = lib().pa_decode_contiguous(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(context_lens, "context_lens", torch.int32),
        S, H, D, strides[0], strides[1], strides[2], L, float(scale), int(max_context_len), dt,
        _dev(out, "out"), ws_ptr, ws_bytes, int(partition_tokens), _stream(stream, q.device),
        _dev(items, "items", torch.int32) if items is not None else None, n)
    _check(rc, "pa_decode_contiguous")
    return out


def stream_read(buf, sink, waves=0, stream=None):
    """pa_stream_read over the bytes of device tensor ``buf`` (plain streaming read;
    the achievable-bandwidth reference).  ``sink``: device int32 tensor of >= 1."""
    torch = _torch()
    nbytes = buf.numel() * buf.element_size()
    _check(lib().pa_stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink", torch.int32), waves,
                                _stream(stream, buf.device)), "pa_stream_read")


def tile_read(a, b, tile_bytes, offsets, ids, sink, stream=None):
    """pa_tile_read: unit u reads tiles ``ids[offsets[u]:offsets[u + 1]]`` of device
    tensors ``a`` and ``b`` (same size, ``tile_bytes`` per tile; the decode's
    gathered-read reference).  ``offsets``, ``ids``: device int32; ``sink``:
    device int32 tensor of >= 1."""
    torch = _torch()
    nbytes = a.numel() * a.element_size()
    if b.numel() * b.element_size() != nbytes:
        raise ValueError("tile_read: a and b differ in size")
    units = offsets.numel() - 1
    if units < 0:
        raise ValueError("tile_read: offsets needs units + 1 entries")
    _check(lib().pa_tile_read(_dev(a, "a"), _dev(b, "b"), int(tile_bytes),
                              nbytes // int(tile_bytes), _dev(offsets, "offsets", torch.int32),
                              _dev(ids, "ids", torch.int32), units,
                              _dev(sink, "sink", torch.int32), _stream(stream, a.device)),
           "pa_tile_read")


def decode_schedule_shared(context_lens_host, block_tables_host, num_heads, head_dim,
                           block_size, dtype_code, partition_tokens=0):
    """Host work lists with shared-prefix groups: dict(items [n,5], groups [g,5],
    members [m,2], partition_tokens, max_context_len, workspace_bytes)."""
    ctx = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    tab = np.ascontiguousarray(block_tables_host, dtype=np.int32)
    S, W = tab.shape
    cap = S * (-(-int(W) * block_size // 32) + 1)
    items = np.empty((cap, 5), np.int32)
    groups = np.empty((cap, 5), np.int32)
    members = np.empty((max(S, 1), 2), np.int32)
    n, ng, nm, pt, mx = (_c.c_int32() for _ in range(5))
    ws = _c.c_size_t()
    rc = lib().pa_decode_schedule_shared(
        _ptr(ctx), _ptr(tab), W, S, num_heads, head_dim, block_size, dtype_code,
        partition_tokens, _ptr(items), cap, _c.byref(n), _ptr(groups), cap, _c.byref(ng),
        _ptr(members), members.shape[0], _c.byref(nm), _c.byref(pt), _c.byref(mx),
        _c.byref(ws))
    _check(rc, "pa_decode_schedule_shared")
    return dict(items=items[:n.value].copy(), groups=groups[:ng.value].copy(),
                members=members[:nm.value].copy(), partition_tokens=pt.value,
                max_context_len=mx.value, workspace_bytes=ws.value)


def decode_scheduled_shared(q, k_cache, v_cache, block_tables, context_lens, scale,
                            max_context_len, items, groups, members, partition_tokens,
                            out=None, workspace=None, stream=None):
    """pa_decode over device work lists from decode_schedule_shared."""
    torch = _torch()
    n, ng = int(items.shape[0]), int(groups.shape[0])
    return _decode_call("pa_decode_scheduled_shared", q, k_cache, v_cache, block_tables,
                        context_lens, scale, max_context_len, out, workspace, partition_tokens,
                        stream,
                        extra=(_dev(items, "items", torch.int32) if n else None, n,
                               _dev(groups, "groups", torch.int32) if ng else None, ng,
                               _dev(members, "members", torch.int32) if ng else None),
                        ws_min_part=256 if ng else 0)


def decode_scheduled(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                     items, partition_tokens, out=None, workspace=None, stream=None):
    """pa_decode over a device work list ``items`` [n, 5] int32 from decode_schedule."""
    torch = _torch()
    n = int(items.shape[0])
    return _decode_call("pa_decode_scheduled", q, k_cache, v_cache, block_tables, context_lens,
                        scale, max_context_len, out, workspace, partition_tokens, stream,
                        extra=(_dev(items, "items", torch.int32), n))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out=None,
           workspace=None, partition_tokens=0, stream=None):
    """PagedAttention decode of one query token per sequence; returns out [S, H, D]."""
    return _decode_call("pa_decode", q, k_cache, v_cache, block_tables, context_lens, scale,
                        max_context_len, out, workspace, partition_tokens, stream)


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                      out, workspace=None, partition_tokens=0, stream=None):
    """First launch of decode (per-partition attention); see pa_decode_partitions."""
    return _decode_call("pa_decode_partitions", q, k_cache, v_cache, block_tables, context_lens,
                        scale, max_context_len, out, workspace, partition_tokens, stream)


def decode_reduce(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                  out, workspace=None, partition_tokens=0, stream=None):
    """Second launch of decode (log-sum-exp merge of partitions); see pa_decode_reduce."""
    return _decode_call("pa_decode_reduce", q, k_cache, v_cache, block_tables, context_lens,
                        scale, max_context_len, out, workspace, partition_tokens, stream)


# ---------------------------------------------------------- block manager
def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp) if a.size else None


class BlockManager:
    """Host block manager (C++): FIFO free list, refcounts, block tables, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self._lib = lib()  # the library that owns the handle
        h = _vp()
        if free_order is None:
            rc = self._lib.pa_bm_create(num_blocks, block_size, None, 0, _c.byref(h))
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            rc = self._lib.pa_bm_create(num_blocks, block_size, _ptr(fo), fo.size, _c.byref(h))
        _check(rc, "pa_bm_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        L = getattr(self, "_lib", None)
        if h is not None and L is not None:
            L.pa_bm_destroy(h)
            self._h = None

    def add_seq(self, seq: int, num_tokens: int):
        _check(self._lib.pa_bm_add_seq(self._h, seq, num_tokens), "pa_bm_add_seq")

    def fork(self, parent: int, child: int):
        _check(self._lib.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def append_slot(self, seq: int):
        """Returns (slot, cow) with cow None or (src, dst)."""
        slot, src, dst = _c.c_int64(), _c.c_int32(), _c.c_int32()
        rc = self._lib.pa_bm_append_slot(self._h, seq, _c.byref(slot), _c.byref(src), _c.byref(dst))
        if rc < 0:
            _check(rc, "pa_bm_append_slot")
        return slot.value, ((src.value, dst.value) if rc == 1 else None)

    def append_slots(self, seqs):
        """Append one token to each listed sequence in order: (slots int64 [n], cow int32 [k, 2])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        n = seqs.size
        slots = np.empty(n, dtype=np.int64)
        cows = np.empty(2 * max(n, 1), dtype=np.int32)
        ncow, done = _c.c_int32(), _c.c_int32()
        rc = self._lib.pa_bm_append_slots(self._h, _ptr(seqs), n, _ptr(slots), _ptr(cows),
                                      _c.byref(ncow), _c.byref(done))
        _check(rc, "pa_bm_append_slots")
        return slots, cows[:2 * ncow.value].reshape(-1, 2).copy()

    def step_into(self, seqs: np.ndarray, slots: np.ndarray, cows: np.ndarray,
                  tables: np.ndarray, pad: int, context_lens: np.ndarray) -> int:
        """pa_bm_step into caller arrays (views of pinned memory); returns the CoW count."""
        ncow = _c.c_int32()
        rc = self._lib.pa_bm_step(self._h, _ptr(seqs), seqs.size, _ptr(slots), _ptr(cows),
                              _c.byref(ncow), _ptr(tables), tables.shape[1], pad,
                              _ptr(context_lens))
        _check(rc, "pa_bm_step")
        return ncow.value

    def free_seq(self, seq: int):
        _check(self._lib.pa_bm_free_seq(self._h, seq), "pa_bm_free_seq")

    def select(self, pairs, retire):
        """Beam selection: fork child from parent for each (parent, child), then free
        every sequence in ``retire`` (one call, checked before any change)."""
        pr = np.ascontiguousarray([p for p, _ in pairs], dtype=np.int64)
        ch = np.ascontiguousarray([c for _, c in pairs], dtype=np.int64)
        rt = np.ascontiguousarray(list(retire), dtype=np.int64)
        _check(self._lib.pa_bm_select(self._h, _ptr(pr) if pr.size else None,
                                  _ptr(ch) if ch.size else None, int(pr.size),
                                  _ptr(rt) if rt.size else None, int(rt.size)), "pa_bm_select")

    def slots(self, seq: int, start: int, n: int) -> np.ndarray:
        out = np.empty(n, dtype=np.int64)
        _check(self._lib.pa_bm_slots(self._h, seq, start, n, _ptr(out)), "pa_bm_slots")
        return out

    def block_table(self, seq: int) -> list:
        n = _c.c_int32()
        rc = self._lib.pa_bm_block_table(self._h, seq, None, 0, _c.byref(n))
        if rc not in (PA_OK, -8):
            _check(rc, "pa_bm_block_table")
        out = np.empty(n.value, dtype=np.int32)
        _check(self._lib.pa_bm_block_table(self._h, seq, _ptr(out), n.value, _c.byref(n)),
               "pa_bm_block_table")
        return out.tolist()

    def block_tables(self, seqs, max_blocks: int, pad: int):
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.empty((seqs.size, max_blocks), dtype=np.int32)
        ctx = np.empty(seqs.size, dtype=np.int32)
        _check(self._lib.pa_bm_block_tables(self._h, _ptr(seqs), seqs.size, _ptr(tables), max_blocks,
                                        pad, _ptr(ctx)), "pa_bm_block_tables")
        return tables, ctx

    def seq_len(self, seq: int) -> int:
        n = self._lib.pa_bm_seq_len(self._h, seq)
        if n < 0:
            _check(int(n), "pa_bm_seq_len")
        return int(n)

    def refcount(self, block: int) -> int:
        r = self._lib.pa_bm_refcount(self._h, block)
        if r < 0:
            _check(int(r), "pa_bm_refcount")
        return int(r)

    @property
    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    @property
    def num_seqs(self) -> int:
        return int(self._lib.pa_bm_num_seqs(self._h))

    def free_list(self) -> list:
        n = int(self._lib.pa_bm_free_list(self._h, None, 0))
        out = np.empty(n, dtype=np.int32)
        self._lib.pa_bm_free_list(self._h, _ptr(out), n)
        return out.tolist()

    def refcounts(self) -> list:
        return [self.refcount(b) for b in range(self.num_blocks)]

    # ------------------------------------------------ preemption by swapping
    def set_host_pool(self, num_host_blocks: int, free_order=None):
        self.num_host_blocks = int(num_host_blocks)
        if free_order is None:
            rc = self._lib.pa_bm_set_host_pool(self._h, num_host_blocks, None, 0)
        else:
            fo = np.ascontiguousarray(free_order, dtype=np.int32)
            rc = self._lib.pa_bm_set_host_pool(self._h, num_host_blocks, _ptr(fo), fo.size)
        _check(rc, "pa_bm_set_host_pool")

    def _move(self, fn, seqs):
        arr = np.ascontiguousarray(seqs, dtype=np.int64)
        cap = 0
        while True:
            pairs = np.empty((max(cap, 1), 2), dtype=np.int32)
            n = _c.c_int32()
            rc = getattr(lib(), fn)(self._h, _ptr(arr), arr.size, _ptr(pairs), cap, _c.byref(n))
            if rc == -8 and n.value > cap:      # PA_ERR_CAPACITY: retry with room
                cap = n.value
                continue
            _check(rc, fn)
            return pairs[:n.value].copy()

    def swap_out(self, seqs) -> np.ndarray:
        """Move seqs (a group holding its blocks alone) to host blocks; returns the
        (device block, host block) pairs to copy."""
        return self._move("pa_bm_swap_out", seqs)

    def swap_in(self, seqs) -> np.ndarray:
        """Move swapped-out seqs back to device blocks; returns (host block, device
        block) pairs to copy."""
        return self._move("pa_bm_swap_in", seqs)

    def is_swapped(self, seq: int) -> bool:
        rc = self._lib.pa_bm_is_swapped(self._h, seq)
        _check(min(rc, 0), "pa_bm_is_swapped")
        return rc == 1

    @property
    def num_free_host(self) -> int:
        return int(self._lib.pa_bm_num_free_host(self._h))

    def host_free_list(self) -> list:
        n = int(self._lib.pa_bm_host_free_list(self._h, None, 0))
        out = np.empty(n, dtype=np.int32)
        self._lib.pa_bm_host_free_list(self._h, _ptr(out), n)
        return out.tolist()

    def host_refcounts(self) -> list:
        return [int(self._lib.pa_bm_host_refcount(self._h, b))
                for b in range(getattr(self, "num_host_blocks", 0))]

    def blocks_needed(self, seqs) -> int:
        """Device blocks the next append of each of seqs would take (no change)."""
        arr = np.ascontiguousarray(seqs, dtype=np.int64)
        n = int(self._lib.pa_bm_blocks_needed(self._h, _ptr(arr) if arr.size else None, arr.size))
        _check(min(n, 0), "pa_bm_blocks_needed")
        return n
