"""Python binding of libsfi, the SFI decode-attention path for MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libsfi.so`` behind the C ABI declared in ``include/sfi.h``.  PyTorch supplies
device memory and streams.  There is no fallback: if the library is missing or
a call fails, an exception is raised.

Names follow that header:
    dense_attn_with_stats  slow step (t_q = 1) / causal verification (t_q > 1)
    select_topk            the Selector
    pack_compact           gather-pack of sink + selected rows
    sparse_decode_attn     fast step over compact + recent
    mixed_attn             drafting and verifying requests in one launch
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional, Sequence

import torch

__all__ = [
    "LIB_PATH", "SfiError", "load", "bind", "BoundCall", "dense_attn_with_stats",
    "select_topk", "pack_compact", "dense_attn_with_stats_deferred",
    "sparse_decode_indexed_attn_merge",
    "sparse_decode_attn", "sparse_decode_attn_static", "mixed_attn", "plan_splits", "stream_copy", "stream_read", "workspace_size",
    "SFI_OK", "SFI_ERR_INVALID_ARG", "SFI_ERR_UNSUPPORTED", "SFI_ERR_WORKSPACE", "SFI_ERR_HIP",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsfi.so")

SFI_OK, SFI_ERR_INVALID_ARG, SFI_ERR_UNSUPPORTED, SFI_ERR_WORKSPACE, SFI_ERR_HIP = 0, 1, 2, 3, 4
SFI_F32, SFI_BF16 = 0, 1
PAGE_SIZE = 16


class SfiShape(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("num_q_heads", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("dtype", c_int32), ("scale", c_float)]


class SfiPagedKV(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("block_table", c_void_p), ("max_pages", c_int32),
                ("page_size", c_int32), ("num_pages", c_int32), ("max_seq_len", c_int32)]


class SfiError(RuntimeError):
    def __init__(self, status: int, call: str, message: str):
        super().__init__(f"{call} failed with status {status}: {message}")
        self.status = status


_SHAPE_P, _KV_P = POINTER(SfiShape), POINTER(SfiPagedKV)
_SIGS = {
    "sfi_dense_attn_with_stats": [_SHAPE_P, _KV_P, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                  c_void_p, c_void_p, c_int64, c_void_p, c_size_t, c_void_p],
    "sfi_dense_attn_workspace_size": [_SHAPE_P, _KV_P, c_int32, POINTER(c_size_t)],
    "sfi_select_topk": [c_void_p, c_int32, c_int32, c_int64, c_void_p, c_int32, c_int32, c_int32, c_int32,
                        c_void_p, c_void_p, c_size_t, c_void_p],
    "sfi_select_topk_workspace_size": [c_int32, c_int32, c_int64, c_int32, c_int32, POINTER(c_size_t)],
    "sfi_dense_attn_with_stats_deferred": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                           c_void_p, c_void_p, c_int64, c_void_p, c_size_t, c_void_p],
    "sfi_sparse_decode_indexed_attn_merge": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                             c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_size_t, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "sfi_pack_compact": [_SHAPE_P, _KV_P, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                         c_void_p, c_void_p],
    "sfi_sparse_decode_attn": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                               c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "sfi_sparse_decode_workspace_size": [_SHAPE_P, _KV_P, c_int32, c_int32, POINTER(c_size_t)],
    "sfi_sparse_decode_attn_static": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                      c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
    "sfi_static_scratch_bytes": [],
    "sfi_sparse_decode_append_attn": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                      c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_size_t, c_void_p],
    "sfi_sparse_decode_indexed_attn": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                       c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p],
    "sfi_dense_attn_with_head_stats": [_SHAPE_P, _KV_P, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_int64, c_void_p, c_size_t, c_void_p],
    "sfi_mixed_attn": [_SHAPE_P, _KV_P, c_void_p, POINTER(c_int32), POINTER(c_int32), c_void_p, c_int32,
                       c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                       c_void_p, c_size_t, c_void_p],
    "sfi_mixed_attn_workspace_size": [_SHAPE_P, _KV_P, POINTER(c_int32), POINTER(c_int32), c_int32, c_int32,
                                      POINTER(c_size_t)],
    "sfi_plan_splits": [c_int32, _SHAPE_P, _KV_P, c_int32, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32)],
    "sfi_stream_copy": [c_void_p, c_void_p, c_size_t, c_void_p],
    "sfi_stream_read": [c_void_p, c_size_t, c_void_p, c_void_p],
    "sfi_status_string": [c_int32],
    "sfi_last_error": [],
    "sfi_version": [],
}
_RES = {"sfi_status_string": c_char_p, "sfi_last_error": c_char_p, "sfi_static_scratch_bytes": c_size_t}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libsfi.so from this package directory (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_kv_cache_sfi_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RES.get(name, c_int32)
        _lib = lib
    return _lib


_binding: Optional[dict] = None
_HOST_ONLY = ("_workspace_size", "sfi_plan_splits")


def _call(name: str, *args) -> None:
    lib = load()
    if _binding is not None and not name.endswith(_HOST_ONLY):
        _binding["calls"].append((name, args))   # bind(): record the launch instead of making it
        return
    st = getattr(lib, name)(*args)
    if st != SFI_OK:
        raise SfiError(st, name, lib.sfi_last_error().decode())


class BoundCall:
    """One library launch with its arguments marshalled once (see bind()).  ``outputs``
    is what the entry point returned; the object keeps every tensor it was given and
    every buffer it allocated alive, since the launch holds their device addresses."""

    def __init__(self, name: str, args: tuple, outputs, keep: list):
        self.name = name
        self.outputs = outputs
        self._fn = getattr(load(), name)
        self._args = args
        self._keep = keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != SFI_OK:
            raise SfiError(st, self.name, load().sfi_last_error().decode())


def bind(op, *args, **kwargs) -> BoundCall:
    """Marshal one entry-point call (e.g. ``bind(sparse_decode_attn, q, ...)``) without making
    it.  Calling the result makes that launch on the same tensors and stream with only the C
    call's own cost on the host; host-side size queries run once, here.  The bound call
    holds a reference to every tensor passed in and every buffer the entry point
    allocates, so none of them is freed while it exists."""
    global _binding
    _binding = {"calls": [], "keep": []}
    try:
        outputs = op(*args, **kwargs)
        rec = _binding
    finally:
        _binding = None
    if len(rec["calls"]) != 1:
        raise ValueError(f"{getattr(op, '__name__', op)} does not make exactly one launch")
    name, cargs = rec["calls"][0]
    given = [a for a in list(args) + list(kwargs.values()) if isinstance(a, torch.Tensor)]
    return BoundCall(name, cargs, outputs, rec["keep"] + given)


# --------------------------------------------------------------------------- marshalling helpers

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SFI_BF16
    if t.dtype == torch.float32:
        return SFI_F32
    raise TypeError(f"inputs must be bfloat16 or float32 (got {t.dtype})")


def _stream(stream, device) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _shape(B: int, Hq: int, Hkv: int, d: int, dtype: int, scale: Optional[float]) -> SfiShape:
    return SfiShape(B, Hq, Hkv, d, dtype, float(scale if scale is not None else 1.0 / math.sqrt(d)))


def _kv(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor, max_seq_len: int) -> SfiPagedKV:
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool"), (block_table, "block_table")):
        _dev(t, n)
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype:
        raise ValueError("k_pool and v_pool must have the same shape and dtype")
    return SfiPagedKV(k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(), block_table.shape[1],
                      k_pool.shape[2], k_pool.shape[0], int(max_seq_len))


def _check_pool(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor, B: int, d: int) -> int:
    """The pools' layout against the call's batch and head size; returns the pools' KV heads.
    The library takes every size from the descriptors it is given, so a tensor that disagrees
    with the pools would make it address memory outside them."""
    if k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.shape[2] != PAGE_SIZE:
        raise ValueError("k_pool and v_pool must both be [num_pages, Hkv, 16, d]")
    if v_pool.dtype != k_pool.dtype:
        raise TypeError("k_pool and v_pool must share a dtype")
    if k_pool.shape[3] != d:
        raise ValueError(f"head size {d} does not match the pools' {k_pool.shape[3]}")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages]")
    return k_pool.shape[1]


def _f32_out(t: Optional[torch.Tensor], shape: tuple, name: str) -> None:
    if t is None:
        return
    _dev(t, name)
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be float32 {tuple(shape)}")


def _i32(t: torch.Tensor, name: str) -> None:
    _dev(t, name)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def _workspace(nbytes: int, workspace: Optional[torch.Tensor], device, stream=None,
               zero: bool = True) -> Optional[torch.Tensor]:
    if workspace is not None:
        _dev(workspace, "workspace")
        return workspace
    if nbytes == 0:
        return None
    # Zero-filled (unless the call needs no zeros): the split-K arrival counters at its start
    # must read zero on first use.  The fill runs on the stream the call is made on, and the
    # allocator is told that stream uses the block, so neither the fill nor a reuse of the
    # block can overtake the launch.
    s = stream if stream is not None else torch.cuda.current_stream(device)
    with torch.cuda.stream(s):
        ws = (torch.zeros if zero else torch.empty)(nbytes, dtype=torch.uint8, device=device)
    ws.record_stream(s)
    if _binding is not None:
        _binding["keep"].append(ws)
    return ws


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# --------------------------------------------------------------------------- entry points

def workspace_size(op: str, *, k_pool, block_table, Hq: int, dtype: torch.dtype, max_seq_len: int,
                   t_q: int = 1, cap: int = 0, n_recent: int = 0, modes=None, t_q_per_req=None) -> int:
    """Bytes of workspace the named call needs ('dense', 'sparse', 'select' or 'mixed')."""
    B = block_table.shape[0]
    num_pages, Hkv, P, d = k_pool.shape
    shape = _shape(B, Hq, Hkv, d, SFI_BF16 if dtype == torch.bfloat16 else SFI_F32, None)
    kv = SfiPagedKV(k_pool.data_ptr(), k_pool.data_ptr(), block_table.data_ptr(), block_table.shape[1], P,
                    num_pages, int(max_seq_len))
    out = c_size_t(0)
    if op == "dense":
        _call("sfi_dense_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), t_q, ctypes.byref(out))
    elif op == "sparse":
        _call("sfi_sparse_decode_workspace_size", ctypes.byref(shape), ctypes.byref(kv), cap, n_recent,
              ctypes.byref(out))
    elif op == "mixed":
        m = (c_int32 * B)(*[int(x) for x in modes])
        t = (c_int32 * B)(*[int(x) for x in t_q_per_req])
        _call("sfi_mixed_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), m, t, cap, n_recent,
              ctypes.byref(out))
    else:
        raise ValueError(op)
    return int(out.value)


def dense_attn_with_stats(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, *, max_seq_len: int, n_sink: int = 0, n_recent: int = 0,
                          scale: Optional[float] = None, with_scores: bool = True, score_stride: Optional[int] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    """Slow step / verification: q [B, t_q, Hq, d] -> (out [B, t_q, Hq, d] fp32, lse [B, t_q, Hq], scores
    [B, Hkv, score_stride] or None)."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    if q.dim() != 4:
        raise ValueError("q must be [B, t_q, Hq, d]")
    B, t_q, Hq, d = q.shape
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    Hkv = _check_pool(k_pool, v_pool, block_table, B, d)
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens must be [B]")
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, t_q, Hq, d), "out")
    _f32_out(lse, (B, t_q, Hq), "lse")
    if out is None:
        out = torch.empty((B, t_q, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, t_q, Hq), dtype=torch.float32, device=dev)
    if with_scores and scores is None:
        stride = int(score_stride if score_stride is not None else max_seq_len)
        scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=dev)
    if scores is not None:
        _f32_out(scores, (B, Hkv, scores.shape[-1]), "scores")
    stride = scores.shape[-1] if scores is not None else 0
    need = c_size_t(0)
    _call("sfi_dense_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), t_q, ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_dense_attn_with_stats", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(), t_q,
          seq_lens.data_ptr(), n_sink, n_recent, out.data_ptr(), _ptr(lse), _ptr(scores), stride, _ptr(ws),
          _nbytes(ws), _stream(stream, dev))
    return out, lse, scores


def dense_attn_with_stats_deferred(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                   block_table: torch.Tensor, seq_lens: torch.Tensor, *, max_seq_len: int,
                                   n_sink: int = 0, n_recent: int = 0, scale: Optional[float] = None,
                                   score_stride: Optional[int] = None, out: Optional[torch.Tensor] = None,
                                   lse: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Slow step whose split-K combine is left to sparse_decode_indexed_attn_merge: q [B, 1, Hq, d] ->
    (out, lse, scores, workspace).  out and lse are complete only once that call has run with them and the
    returned workspace as slow_out, slow_lse and slow_workspace."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [B, 1, Hq, d]")
    B, _, Hq, d = q.shape
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    Hkv = _check_pool(k_pool, v_pool, block_table, B, d)
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens must be [B]")
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, 1, Hq, d), "out")
    _f32_out(lse, (B, 1, Hq), "lse")
    if out is None:
        out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        stride = int(score_stride if score_stride is not None else max_seq_len)
        scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=dev)
    _f32_out(scores, (B, Hkv, scores.shape[-1]), "scores")
    need = c_size_t(0)
    _call("sfi_dense_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), 1, ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_dense_attn_with_stats_deferred", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(),
          seq_lens.data_ptr(), n_sink, n_recent, out.data_ptr(), _ptr(lse), scores.data_ptr(), scores.shape[-1],
          _ptr(ws), _nbytes(ws), _stream(stream, dev))
    return out, lse, scores, ws


def select_topk(scores: torch.Tensor, seq_lens: torch.Tensor, *, k: int, n_sink: int, n_recent: int,
                t_q: int = 1, sel_idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """Selector: scores [B, Hkv, stride] fp32 -> sel_idx [B, Hkv, k] int32 (ascending, -1 padded)."""
    _dev(scores, "scores")
    _i32(seq_lens, "seq_lens")
    B, Hkv, stride = scores.shape
    if sel_idx is None:
        sel_idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=scores.device)
    need = c_size_t(0)
    _call("sfi_select_topk_workspace_size", B, Hkv, stride, n_sink, k, ctypes.byref(need))
    ws = _workspace(need.value, workspace, scores.device, stream, zero=False)   # candidates: no zeros needed
    _call("sfi_select_topk", scores.data_ptr(), B, Hkv, stride, seq_lens.data_ptr(), t_q, n_sink, n_recent, k,
          sel_idx.data_ptr(), _ptr(ws), _nbytes(ws), _stream(stream, scores.device))
    return sel_idx


def pack_compact(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 sel_idx: torch.Tensor, *, n_sink: int, cap: int, max_seq_len: int,
                 compact_k: Optional[torch.Tensor] = None, compact_v: Optional[torch.Tensor] = None,
                 n_compact: Optional[torch.Tensor] = None, stream=None):
    """Gather-pack: -> (compact_k, compact_v [B, Hkv, cap, d], n_compact [B] int32)."""
    _i32(sel_idx, "sel_idx")
    _i32(seq_lens, "seq_lens")
    if sel_idx.dim() != 3:
        raise ValueError("sel_idx must be [B, Hkv, k]")
    B, Hkv, k = sel_idx.shape
    d = k_pool.shape[3]
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    if _check_pool(k_pool, v_pool, block_table, B, d) != Hkv:
        raise ValueError(f"sel_idx has {Hkv} rows per request; the pools hold {k_pool.shape[1]} KV heads")
    shape = _shape(B, Hkv, Hkv, d, _dtype_code(k_pool), None)
    dev = k_pool.device
    if compact_k is None:
        compact_k = torch.empty((B, Hkv, cap, d), dtype=k_pool.dtype, device=dev)
    if compact_v is None:
        compact_v = torch.empty((B, Hkv, cap, d), dtype=k_pool.dtype, device=dev)
    if n_compact is None:
        n_compact = torch.empty((B,), dtype=torch.int32, device=dev)
    for t, n in ((compact_k, "compact_k"), (compact_v, "compact_v")):
        _dev(t, n)
        if t.dtype != k_pool.dtype or tuple(t.shape) != (B, Hkv, cap, d):
            raise ValueError(f"{n} must be [B, Hkv, cap, d] = {(B, Hkv, cap, d)} in the pool dtype")
    _i32(n_compact, "n_compact")
    if tuple(seq_lens.shape) != (B,) or tuple(n_compact.shape) != (B,):
        raise ValueError("seq_lens and n_compact must be [B]")
    _call("sfi_pack_compact", ctypes.byref(shape), ctypes.byref(kv), seq_lens.data_ptr(), n_sink,
          sel_idx.data_ptr(), k, compact_k.data_ptr(), compact_v.data_ptr(), cap, n_compact.data_ptr(),
          _stream(stream, dev))
    return compact_k, compact_v, n_compact


def sparse_decode_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                       seq_lens: torch.Tensor, compact_k: torch.Tensor, compact_v: torch.Tensor,
                       n_compact: torch.Tensor, *, n_sink: int, n_recent: int, max_seq_len: int,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                       k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                       _static: bool = False):
    """Fast step: q [B, Hq, d] -> (out [B, Hq, d] fp32, lse [B, Hq]).  With k_new / v_new
    [B, Hkv, d] (the decoded token's K/V) the launch also stores them into the pools at
    position seq_lens[b] - 1 (sfi_sparse_decode_append_attn)."""
    _dev(q, "q")
    if _static and (workspace is not None or k_new is not None):
        raise ValueError("the static-scratch fast step takes no workspace and no appended token")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _dev(t, n)
            if t.dtype != k_pool.dtype or tuple(t.shape) != (q.shape[0], k_pool.shape[1], q.shape[2]):
                raise ValueError(f"{n} must be [B, Hkv, d] in the pool dtype")
    _dev(compact_k, "compact_k")
    _dev(compact_v, "compact_v")
    _i32(seq_lens, "seq_lens")
    _i32(n_compact, "n_compact")
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv, cap = compact_k.shape[1], compact_k.shape[2]
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    if _check_pool(k_pool, v_pool, block_table, B, d) != Hkv:
        raise ValueError(f"compact_k has {Hkv} KV heads; the pools hold {k_pool.shape[1]}")
    for t, n in ((compact_k, "compact_k"), (compact_v, "compact_v")):
        if t.dtype != k_pool.dtype or tuple(t.shape) != (B, Hkv, cap, d):
            raise ValueError(f"{n} must be [B, Hkv, cap, d] in the pool dtype")
    if q.dtype != k_pool.dtype or tuple(n_compact.shape) != (B,) or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens and n_compact must be [B]")
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, Hq, d), "out")
    _f32_out(lse, (B, Hq), "lse")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if _static:
        _call("sfi_sparse_decode_attn_static", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(),
              seq_lens.data_ptr(), n_sink, n_recent, compact_k.data_ptr(), compact_v.data_ptr(), cap,
              n_compact.data_ptr(), out.data_ptr(), _ptr(lse), _stream(stream, dev))
        return out, lse
    need = c_size_t(0)
    _call("sfi_sparse_decode_workspace_size", ctypes.byref(shape), ctypes.byref(kv), cap, n_recent,
          ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    if k_new is None:
        _call("sfi_sparse_decode_attn", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(), seq_lens.data_ptr(),
              n_sink, n_recent, compact_k.data_ptr(), compact_v.data_ptr(), cap, n_compact.data_ptr(),
              out.data_ptr(), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream, dev))
    else:
        _call("sfi_sparse_decode_append_attn", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(),
              k_new.data_ptr(), v_new.data_ptr(), seq_lens.data_ptr(), n_sink, n_recent, compact_k.data_ptr(),
              compact_v.data_ptr(), cap, n_compact.data_ptr(), out.data_ptr(), _ptr(lse), _ptr(ws), _nbytes(ws),
              _stream(stream, dev))
    return out, lse


def sparse_decode_attn_static(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor, compact_k: torch.Tensor,
                              compact_v: torch.Tensor, n_compact: torch.Tensor, *, n_sink: int, n_recent: int,
                              max_seq_len: int, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, stream=None):
    """The fast step for callers that cannot allocate (sfi_sparse_decode_attn_static): its split-K
    scratch is the library's static device array; pass out (and lse) to allocate nothing here either."""
    return sparse_decode_attn(q, k_pool, v_pool, block_table, seq_lens, compact_k, compact_v, n_compact,
                              n_sink=n_sink, n_recent=n_recent, max_seq_len=max_seq_len, scale=scale, out=out,
                              lse=lse, stream=stream, _static=True)


def sparse_decode_indexed_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                               block_table: torch.Tensor, seq_lens: torch.Tensor, sel_idx: torch.Tensor, *,
                               n_sink: int, n_recent: int, max_seq_len: int, scale: Optional[float] = None,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None,
                               k_new: Optional[torch.Tensor] = None, v_new: Optional[torch.Tensor] = None,
                               per_head: bool = False, compact_k: Optional[torch.Tensor] = None,
                               compact_v: Optional[torch.Tensor] = None, n_compact: Optional[torch.Tensor] = None):
    """Fast step over the positions sel_idx [B, Hkv, k] lists (plus sink and recent), every row
    read in place from paged KV: q [B, Hq, d] -> (out [B, Hq, d] fp32, lse [B, Hq])
    (sfi_sparse_decode_indexed_attn).  With per_head, sel_idx is [B, Hq, k], one set per
    query head.  k_new / v_new as in sparse_decode_attn.  With compact_k / compact_v
    [B, units, cap, d] and n_compact [B], the launch also packs them as pack_compact would."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    _i32(sel_idx, "sel_idx")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _dev(t, n)
            if t.dtype != k_pool.dtype or tuple(t.shape) != (q.shape[0], k_pool.shape[1], q.shape[2]):
                raise ValueError(f"{n} must be [B, Hkv, d] in the pool dtype")
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv = _check_pool(k_pool, v_pool, block_table, B, d)
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens must be [B]")
    rows = Hq if per_head else Hkv
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (B, rows):
        raise ValueError(f"sel_idx must be [B, {'Hq' if per_head else 'Hkv'}, k]")
    k = sel_idx.shape[2]
    packing = (compact_k, compact_v, n_compact)
    if any(t is not None for t in packing) and not all(t is not None for t in packing):
        raise ValueError("compact_k, compact_v and n_compact go together")
    cap = 0
    if compact_k is not None:
        for t, n in ((compact_k, "compact_k"), (compact_v, "compact_v")):
            _dev(t, n)
            if t.dtype != k_pool.dtype or t.dim() != 4 or tuple(t.shape[:2]) != (B, rows) or t.shape[3] != d:
                raise ValueError(f"{n} must be [B, units, cap, d] in the pool dtype")
        if compact_v.shape != compact_k.shape:
            raise ValueError("compact_v must match compact_k")
        _i32(n_compact, "n_compact")
        cap = compact_k.shape[2]
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    unit_shape = _shape(B, Hq, rows, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, Hq, d), "out")
    _f32_out(lse, (B, Hq), "lse")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = c_size_t(0)
    _call("sfi_sparse_decode_workspace_size", ctypes.byref(unit_shape), ctypes.byref(kv), n_sink + k, n_recent,
          ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_sparse_decode_indexed_attn", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(), _ptr(k_new),
          _ptr(v_new), seq_lens.data_ptr(), n_sink, n_recent, sel_idx.data_ptr(), k, int(per_head),
          _ptr(compact_k), _ptr(compact_v), cap, _ptr(n_compact), out.data_ptr(), _ptr(lse), _ptr(ws), _nbytes(ws),
          _stream(stream, dev))
    return out, lse


def sparse_decode_indexed_attn_merge(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                     block_table: torch.Tensor, seq_lens: torch.Tensor, sel_idx: torch.Tensor, *,
                                     n_sink: int, n_recent: int, max_seq_len: int, slow_out: torch.Tensor,
                                     slow_lse: Optional[torch.Tensor], slow_workspace: Optional[torch.Tensor],
                                     compact_k: torch.Tensor, compact_v: torch.Tensor, n_compact: torch.Tensor,
                                     scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                     stream=None):
    """The rest of a slow step in one launch (sfi_sparse_decode_indexed_attn_merge): the fast step over
    sel_idx [B, Hkv, k] read in place, q [B, Hq, d] -> (out [B, Hq, d], lse [B, Hq]), which also packs
    compact_k / compact_v [B, Hkv, cap, d] and n_compact [B], and merges the split partials that
    dense_attn_with_stats_deferred left in slow_workspace into slow_out [B, 1, Hq, d] and slow_lse."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    _i32(sel_idx, "sel_idx")
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    Hkv = _check_pool(k_pool, v_pool, block_table, B, d)
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens must be [B]")
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (B, Hkv):
        raise ValueError("sel_idx must be [B, Hkv, k]")
    k = sel_idx.shape[2]
    for t, n in ((compact_k, "compact_k"), (compact_v, "compact_v")):
        _dev(t, n)
        if t.dtype != k_pool.dtype or t.dim() != 4 or tuple(t.shape[:2]) != (B, Hkv) or t.shape[3] != d:
            raise ValueError(f"{n} must be [B, Hkv, cap, d] in the pool dtype")
    if compact_v.shape != compact_k.shape:
        raise ValueError("compact_v must match compact_k")
    _i32(n_compact, "n_compact")
    if tuple(n_compact.shape) != (B,):
        raise ValueError("n_compact must be [B]")
    cap = compact_k.shape[2]
    _f32_out(slow_out, (B, 1, Hq, d), "slow_out")
    _f32_out(slow_lse, (B, 1, Hq), "slow_lse")
    if slow_workspace is not None:
        _dev(slow_workspace, "slow_workspace")
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, Hq, d), "out")
    _f32_out(lse, (B, Hq), "lse")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = c_size_t(0)
    _call("sfi_sparse_decode_workspace_size", ctypes.byref(shape), ctypes.byref(kv), n_sink + k, n_recent,
          ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_sparse_decode_indexed_attn_merge", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(),
          seq_lens.data_ptr(), n_sink, n_recent, sel_idx.data_ptr(), k, compact_k.data_ptr(), compact_v.data_ptr(),
          cap, n_compact.data_ptr(), out.data_ptr(), _ptr(lse), _ptr(ws), _nbytes(ws), slow_out.data_ptr(),
          _ptr(slow_lse), _ptr(slow_workspace), _nbytes(slow_workspace), _stream(stream, dev))
    return out, lse


def dense_attn_with_head_stats(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                               block_table: torch.Tensor, seq_lens: torch.Tensor, *, max_seq_len: int,
                               n_sink: int = 0, n_recent: int = 0, scale: Optional[float] = None,
                               score_stride: Optional[int] = None, out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None, stream=None):
    """Slow step with one logit row per query head: q [B, Hq, d] -> (out [B, Hq, d] fp32,
    lse [B, Hq], scores [B, Hq, score_stride]) (sfi_dense_attn_with_head_stats)."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, d]")
    B, Hq, d = q.shape
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    Hkv = _check_pool(k_pool, v_pool, block_table, B, d)
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens must be [B]")
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (B, Hq, d), "out")
    _f32_out(lse, (B, Hq), "lse")
    stride = int(score_stride if score_stride is not None else max_seq_len)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((B, Hq, stride), dtype=torch.float32, device=dev)
    _dev(scores, "scores")
    if scores.dtype != torch.float32 or tuple(scores.shape) != (B, Hq, stride):
        raise ValueError("scores must be float32 [B, Hq, score_stride]")
    need = c_size_t(0)
    _call("sfi_dense_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), 1, ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_dense_attn_with_head_stats", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(), seq_lens.data_ptr(),
          n_sink, n_recent, out.data_ptr(), _ptr(lse), scores.data_ptr(), stride, _ptr(ws), _nbytes(ws),
          _stream(stream, dev))
    return out, lse, scores


def mixed_attn(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, modes: Sequence[int], t_q: Sequence[int], compact_k: torch.Tensor,
               compact_v: torch.Tensor, n_compact: torch.Tensor, *, n_sink: int, n_recent: int, max_seq_len: int,
               scale: Optional[float] = None, with_scores: bool = True, score_stride: Optional[int] = None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
               scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Drafting (mode 0) and verifying (mode 1) requests in one launch.  q [R, Hq, d] with R = sum(t_q)
    -> (out [R, Hq, d], lse [R, Hq], scores [B, Hkv, stride] or None)."""
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    _i32(n_compact, "n_compact")
    if q.dim() != 3:
        raise ValueError("q must be [R, Hq, d]")
    R, Hq, d = q.shape
    B = len(modes)
    if len(t_q) != B or sum(int(x) for x in t_q) != R:
        raise ValueError("t_q must have one entry per request and sum to q's rows")
    Hkv, cap = compact_k.shape[1], compact_k.shape[2]
    kv = _kv(k_pool, v_pool, block_table, max_seq_len)
    if _check_pool(k_pool, v_pool, block_table, B, d) != Hkv:
        raise ValueError(f"compact_k has {Hkv} KV heads; the pools hold {k_pool.shape[1]}")
    for tt, n in ((compact_k, "compact_k"), (compact_v, "compact_v")):
        _dev(tt, n)
        if tt.dtype != k_pool.dtype or tuple(tt.shape) != (B, Hkv, cap, d):
            raise ValueError(f"{n} must be [B, Hkv, cap, d] in the pool dtype")
    if q.dtype != k_pool.dtype or tuple(seq_lens.shape) != (B,) or tuple(n_compact.shape) != (B,):
        raise ValueError("q must share the pool dtype; seq_lens and n_compact must be [B]")
    shape = _shape(B, Hq, Hkv, d, _dtype_code(q), scale)
    dev = q.device
    _f32_out(out, (R, Hq, d), "out")
    _f32_out(lse, (R, Hq), "lse")
    m = (c_int32 * B)(*[int(x) for x in modes])
    t = (c_int32 * B)(*[int(x) for x in t_q])
    if out is None:
        out = torch.empty((R, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, Hq), dtype=torch.float32, device=dev)
    if with_scores and scores is None:
        stride = int(score_stride if score_stride is not None else max_seq_len)
        scores = torch.empty((B, Hkv, stride), dtype=torch.float32, device=dev)
    if scores is not None:
        _f32_out(scores, (B, Hkv, scores.shape[-1]), "scores")
    stride = scores.shape[-1] if scores is not None else 0
    need = c_size_t(0)
    _call("sfi_mixed_attn_workspace_size", ctypes.byref(shape), ctypes.byref(kv), m, t, cap, n_recent,
          ctypes.byref(need))
    ws = _workspace(need.value, workspace, dev, stream)
    _call("sfi_mixed_attn", ctypes.byref(shape), ctypes.byref(kv), q.data_ptr(), m, t, seq_lens.data_ptr(),
          n_sink, n_recent, compact_k.data_ptr(), compact_v.data_ptr(), cap, n_compact.data_ptr(), out.data_ptr(),
          _ptr(lse), _ptr(scores), stride, _ptr(ws), _nbytes(ws), _stream(stream, dev))
    return out, lse, scores


def plan_splits(op: int, *, B: int, Hq: int, Hkv: int, d: int, bf16: bool, max_pages: int, num_pages: int,
                max_seq_len: int, t_q: int = 1, cap: int = 0, n_recent: int = 0):
    """(tokens per split, splits per (request, KV head)) chosen by the library; host only."""
    shape = _shape(B, Hq, Hkv, d, SFI_BF16 if bf16 else SFI_F32, None)
    kv = SfiPagedKV(16, 16, 16, max_pages, PAGE_SIZE, num_pages, max_seq_len)  # addresses unused by planning
    st, ns = c_int32(0), c_int32(0)
    _call("sfi_plan_splits", op, ctypes.byref(shape), ctypes.byref(kv), t_q, cap, n_recent, ctypes.byref(st),
          ctypes.byref(ns))
    return st.value, ns.value


def stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Calibration copy (not part of the decode path)."""
    _dev(src, "src")
    _dev(dst, "dst")
    n = min(_nbytes(src), _nbytes(dst))
    _call("sfi_stream_copy", src.data_ptr(), dst.data_ptr(), n, _stream(stream, src.device))


def stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Streaming read of src (measurement helper, not part of the decode path); sink is a device
    int32 tensor of at least one element."""
    _dev(src, "src")
    _dev(sink, "sink")
    _call("sfi_stream_read", src.data_ptr(), _nbytes(src) // 16 * 16, sink.data_ptr(), _stream(stream, src.device))
