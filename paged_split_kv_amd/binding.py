"""Thin Python binding over libpa.so (include/pa.h).  Argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are passed as raw device
pointers with the current torch stream; no computation of the decode path happens here.  If the
library is not built, every call raises: there is no fallback path.

torch must be imported before the library is loaded so that libpa.so binds to the same HIP runtime
(libamdhip64.so.7) that owns torch's device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_OK, PA_INVALID_ARG, PA_UNSUPPORTED, PA_CAPACITY, PA_HIP_ERROR = 0, 1, 2, 3, 4
PA_MAX_SEQS = 8192
PA_MAX_GROUP_ROWS = 64
PA_INLINE_PLAN_SEQS = 256
PA_NOALLOC_SCRATCH_BYTES = 32 << 20

_DTYPE_OF_NAME = {"f32": PA_F32, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}
_TORCH_OF_NAME = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}

SYMBOLS = ("pa_plan_capacity", "pa_workspace_bytes", "pa_plan", "pa_decode", "pa_merge",
           "pa_attention", "pa_attention_noalloc", "pa_prefill", "pa_prefill_workspace_bytes", "pa_attention_mixed",
           "pa_split_decode_first", "pa_status_string", "pa_device_cu_count")


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load(path: str = LIB_PATH):
    """Load libpa.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_split_kv_amd.build` "
                           "(the decode path has no fallback)")
    lib = ctypes.CDLL(path)
    i32 = ctypes.c_int32
    vp = ctypes.c_void_p
    f32 = ctypes.c_float
    lib.pa_plan_capacity.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
    lib.pa_plan_capacity.restype = ctypes.c_int
    lib.pa_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.pa_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_plan.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.pa_plan.restype = ctypes.c_int
    lib.pa_decode.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, ctypes.c_int, i32, i32, i32,
                              vp, i32, vp, i32, vp, i32, i32, f32, f32, f32, vp, vp, vp, vp, i32, i32, vp,
                              ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_merge.argtypes = [i32, i32, i32, i32, vp, i32, vp, i32, vp, ctypes.c_size_t, vp,
                             ctypes.c_int, vp]
    lib.pa_merge.restype = ctypes.c_int
    lib.pa_attention.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, ctypes.c_int, i32, i32, i32,
                                 vp, i32, vp, i32, vp, i32, i32, f32, f32, f32, i32, i32, i32, i32, i32,
                                 vp, vp, vp, vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.pa_attention.restype = ctypes.c_int
    lib.pa_attention_noalloc.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, ctypes.c_int, i32, i32, i32,
                                         vp, i32, vp, i32, vp, i32, i32, f32, f32, f32, i32, i32, i32, i32, i32,
                                         vp, vp, vp, vp, ctypes.c_int, vp]
    lib.pa_attention_noalloc.restype = ctypes.c_int
    lib.pa_prefill.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, ctypes.c_int, i32, i32, i32, vp, i32,
                               vp, i32, vp, i32, f32, f32, f32, i32, vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pa_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_attention_mixed.argtypes = [vp, ctypes.c_int, i32, i32, i32, vp, vp, ctypes.c_int, i32, i32, i32,
                                       vp, i32, vp, i32, vp, i32, i32, i32, i32, f32, f32, f32, i32, i32,
                                       i32, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.pa_attention_mixed.restype = ctypes.c_int
    lib.pa_split_decode_first.argtypes = [ctypes.POINTER(i32), i32, i32, ctypes.POINTER(i32),
                                          ctypes.POINTER(i32)]
    lib.pa_split_decode_first.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_device_cu_count.argtypes = [i32, ctypes.POINTER(i32)]
    lib.pa_device_cu_count.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PaError(status, where)


class Prepared:
    """One C entry point with its arguments already marshalled (pointers, sizes and the stream as
    they were when it was prepared): calling it issues the same call again.  For timed loops, where
    re-checking and re-marshalling every argument would add host time per launch."""

    def __init__(self, fn, args, where: str):
        self.fn = fn
        self.args = args
        self.where = where

    def __call__(self) -> None:
        _check(self.fn(*self.args), self.where)


def _issue(fn, args, where: str, prepare: bool):
    if prepare:
        return Prepared(fn, args, where)
    _check(fn(*args), where)
    return None


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# ---------------------------------------------------------------------------------------------
# C entry points
# ---------------------------------------------------------------------------------------------

def pa_plan_capacity(num_seqs: int, num_kv_heads: int, cu_count: int, budget_mult: int = 2,
                     max_partitions: int = 256) -> int:
    out = ctypes.c_int32(0)
    _check(load().pa_plan_capacity(num_seqs, num_kv_heads, cu_count, budget_mult, max_partitions,
                                   ctypes.byref(out)), "pa_plan_capacity")
    return int(out.value)


def pa_workspace_bytes(capacity: int, max_q_len: int, num_q_heads: int, head_dim: int) -> int:
    return int(load().pa_workspace_bytes(capacity, max_q_len, num_q_heads, head_dim))


def pa_device_cu_count(device: Optional[int] = None) -> int:
    dev = torch.cuda.current_device() if device is None else int(device)
    out = ctypes.c_int32(0)
    _check(load().pa_device_cu_count(dev, ctypes.byref(out)), "pa_device_cu_count")
    return int(out.value)


def pa_plan(context_lens: torch.Tensor, num_kv_heads: int, *, cu_count: int, budget_mult: int = 2,
            max_partitions: int = 256, tile_tokens: int = 256, capacity: Optional[int] = None,
            work_info: Optional[torch.Tensor] = None, reduce_info: Optional[torch.Tensor] = None,
            num_work: Optional[torch.Tensor] = None, cu_query_lens: Optional[torch.Tensor] = None,
            sliding_window: int = 0, dispatch_info: Optional[torch.Tensor] = None, stream=None,
            prepare: bool = False):
    """Plan on the device.  Returns (work_info [capacity, 4], reduce_info [B, 2], num_work [2] =
    (used slots, tiles of the largest slot)), all int32 on the device of context_lens; passed-in
    buffers are refilled in place.  With a sliding window the plan covers the windowed key ranges
    (cu_query_lens gives the query lengths).  dispatch_info (int32 [capacity, 4]) also receives the
    decode's dispatch order.  With prepare=True nothing is launched and a Prepared call is returned
    instead."""
    _need(context_lens, "context_lens", torch.int32)
    dev = context_lens.device
    B = int(context_lens.shape[0])
    if cu_query_lens is not None:
        _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
        if cu_query_lens.shape[0] != B + 1:
            raise ValueError("cu_query_lens must be [num_seqs + 1]")
    if capacity is None:
        capacity = pa_plan_capacity(B, num_kv_heads, cu_count, budget_mult, max_partitions)
    if work_info is None:
        work_info = torch.empty((capacity, 4), dtype=torch.int32, device=dev)
    if reduce_info is None:
        reduce_info = torch.empty((B, 2), dtype=torch.int32, device=dev)
    if num_work is None:
        num_work = torch.empty((2,), dtype=torch.int32, device=dev)
    _need(work_info, "work_info", torch.int32, dev)
    _need(reduce_info, "reduce_info", torch.int32, dev)
    _need(num_work, "num_work", torch.int32, dev)
    if work_info.numel() < 4 * capacity or reduce_info.numel() < 2 * B or num_work.numel() < 2:
        raise ValueError("plan buffers smaller than capacity / num_seqs / 2")
    if dispatch_info is not None:
        _need(dispatch_info, "dispatch_info", torch.int32, dev)
        if dispatch_info.numel() < 4 * capacity:
            raise ValueError("dispatch_info smaller than capacity")
    args = (_ptr(context_lens), _ptr(cu_query_lens), B, num_kv_heads, cu_count, budget_mult, max_partitions,
            tile_tokens, sliding_window, capacity, _ptr(work_info), _ptr(reduce_info), _ptr(num_work),
            _ptr(dispatch_info), _stream(stream))
    prepared = _issue(load().pa_plan, args, "pa_plan", prepare)
    return prepared if prepare else (work_info, reduce_info, num_work)


def pa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: str,
              block_tables: torch.Tensor, context_lens: torch.Tensor, work_info: torch.Tensor,
              num_work: torch.Tensor, workspace: torch.Tensor, *, scale: float,
              cu_query_lens: Optional[torch.Tensor] = None, max_q_len: int = 1,
              k_scale: float = 1.0, v_scale: float = 1.0, tile_tokens: int = 256,
              reduce_info: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              sliding_window: int = 0, dispatch_info: Optional[torch.Tensor] = None, stream=None,
              prepare: bool = False):
    """Split-KV decode into the workspace (see include/pa.h).  kv_dtype is "f32", "bf16" or
    "fp8" (uint8 tensors holding OCP e4m3fn codes).  With ``out`` (and ``reduce_info``) the merge
    runs in the same call.  With prepare=True nothing is launched and a Prepared call is returned."""
    dev = q.device
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", q.dtype)
    _need(k_cache, "k_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(v_cache, "v_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    _need(work_info, "work_info", torch.int32, dev)
    _need(num_work, "num_work", torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if cu_query_lens is not None:
        _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    if out is not None:
        _need(out, "out", q.dtype, dev)
        if tuple(out.shape) != tuple(q.shape):
            raise ValueError("out must have the shape of q")
        if reduce_info is None:
            raise ValueError("reduce_info is required when out is given")
    if reduce_info is not None:
        _need(reduce_info, "reduce_info", torch.int32, dev)
    if dispatch_info is not None:
        _need(dispatch_info, "dispatch_info", torch.int32, dev)
        if dispatch_info.numel() < work_info.numel():
            raise ValueError("dispatch_info smaller than work_info")
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    B = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    if cu_query_lens is not None and cu_query_lens.shape[0] != B + 1:
        raise ValueError("cu_query_lens must be [num_seqs + 1]")
    capacity = int(work_info.shape[0])
    args = (_ptr(q), PA_F32 if q.dtype == torch.float32 else PA_BF16, R, Hq, D,
            _ptr(k_cache), _ptr(v_cache), _DTYPE_OF_NAME[kv_dtype], nb, Hkv, bs,
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B,
            _ptr(cu_query_lens), max_q_len, sliding_window, scale, k_scale, v_scale,
            _ptr(work_info), _ptr(reduce_info), _ptr(num_work), _ptr(dispatch_info), capacity, tile_tokens,
            _ptr(workspace), workspace.numel(), _ptr(out),
            PA_F32 if q.dtype == torch.float32 else PA_BF16, _stream(stream))
    return _issue(load().pa_decode, args, "pa_decode", prepare)


def pa_merge(out: torch.Tensor, reduce_info: torch.Tensor, workspace: torch.Tensor, *, capacity: int,
             cu_query_lens: Optional[torch.Tensor] = None, max_q_len: int = 1, stream=None,
             prepare: bool = False):
    """Log-sum-exp merge of the workspace into out ([R, Hq, D], float32 or bfloat16), in place.  With
    prepare=True nothing is launched and a Prepared call is returned."""
    dev = out.device
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _need(out, "out", out.dtype)
    _need(reduce_info, "reduce_info", torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if cu_query_lens is not None:
        _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    R, Hq, D = out.shape
    B = int(reduce_info.shape[0])
    args = (R, Hq, D, B, _ptr(cu_query_lens), max_q_len, _ptr(reduce_info), capacity,
            _ptr(workspace), workspace.numel(), _ptr(out),
            PA_F32 if out.dtype == torch.float32 else PA_BF16, _stream(stream))
    return _issue(load().pa_merge, args, "pa_merge", prepare)


def pa_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: str,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, work_info: torch.Tensor,
                 reduce_info: torch.Tensor, num_work: torch.Tensor, workspace: torch.Tensor,
                 out: torch.Tensor, *, scale: float, cu_count: int, budget_mult: int = 2,
                 max_partitions: int = 256, tile_tokens: int = 256,
                 cu_query_lens: Optional[torch.Tensor] = None, max_q_len: int = 1,
                 k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0,
                 stream=None, prepare: bool = False):
    """Plan, decode and merge in one call (see include/pa.h); the plan buffers are outputs.  With
    prepare=True nothing is launched and a Prepared call is returned."""
    dev = q.device
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", q.dtype)
    _need(k_cache, "k_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(v_cache, "v_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    _need(work_info, "work_info", torch.int32, dev)
    _need(reduce_info, "reduce_info", torch.int32, dev)
    _need(num_work, "num_work", torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    _need(out, "out", q.dtype, dev)
    if cu_query_lens is not None:
        _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    B = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    if cu_query_lens is not None and cu_query_lens.shape[0] != B + 1:
        raise ValueError("cu_query_lens must be [num_seqs + 1]")
    capacity = int(work_info.shape[0])
    if reduce_info.numel() < 2 * B or num_work.numel() < 2:
        raise ValueError("plan buffers smaller than num_seqs / 2")
    qd = PA_F32 if q.dtype == torch.float32 else PA_BF16
    args = (_ptr(q), qd, R, Hq, D, _ptr(k_cache), _ptr(v_cache), _DTYPE_OF_NAME[kv_dtype],
            nb, Hkv, bs, _ptr(block_tables), int(block_tables.shape[1]),
            _ptr(context_lens), B, _ptr(cu_query_lens), max_q_len, sliding_window,
            scale, k_scale, v_scale, cu_count, budget_mult, max_partitions, tile_tokens, capacity,
            _ptr(work_info), _ptr(reduce_info), _ptr(num_work), _ptr(workspace),
            workspace.numel(), _ptr(out), qd, _stream(stream))
    return _issue(load().pa_attention, args, "pa_attention", prepare)


def pa_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: str,
                         block_tables: torch.Tensor, context_lens: torch.Tensor, work_info: torch.Tensor,
                         reduce_info: torch.Tensor, num_work: torch.Tensor, out: torch.Tensor, *, scale: float,
                         cu_count: int, budget_mult: int = 2, max_partitions: int = 256, tile_tokens: int = 256,
                         cu_query_lens: Optional[torch.Tensor] = None, max_q_len: int = 1, k_scale: float = 1.0,
                         v_scale: float = 1.0, sliding_window: int = 0, stream=None, prepare: bool = False):
    """pa_attention without a workspace argument: the library's per-device static array holds the
    partial states (see include/pa.h).  Same checks as pa_attention otherwise."""
    dev = q.device
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", q.dtype)
    _need(k_cache, "k_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(v_cache, "v_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    _need(work_info, "work_info", torch.int32, dev)
    _need(reduce_info, "reduce_info", torch.int32, dev)
    _need(num_work, "num_work", torch.int32, dev)
    _need(out, "out", q.dtype, dev)
    if cu_query_lens is not None:
        _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    B = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    if cu_query_lens is not None and cu_query_lens.shape[0] != B + 1:
        raise ValueError("cu_query_lens must be [num_seqs + 1]")
    if reduce_info.numel() < 2 * B or num_work.numel() < 2:
        raise ValueError("plan buffers smaller than num_seqs / 2")
    qd = PA_F32 if q.dtype == torch.float32 else PA_BF16
    args = (_ptr(q), qd, R, Hq, D, _ptr(k_cache), _ptr(v_cache), _DTYPE_OF_NAME[kv_dtype],
            nb, Hkv, bs, _ptr(block_tables), int(block_tables.shape[1]),
            _ptr(context_lens), B, _ptr(cu_query_lens), max_q_len, sliding_window,
            scale, k_scale, v_scale, cu_count, budget_mult, max_partitions, tile_tokens, int(work_info.shape[0]),
            _ptr(work_info), _ptr(reduce_info), _ptr(num_work), _ptr(out), qd, _stream(stream))
    return _issue(load().pa_attention_noalloc, args, "pa_attention_noalloc", prepare)


def pa_attention_mixed(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: str,
                       block_tables: torch.Tensor, context_lens: torch.Tensor, cu_query_lens: torch.Tensor,
                       num_decodes: int, num_decode_rows: int, work_info: torch.Tensor,
                       reduce_info: torch.Tensor, num_work: torch.Tensor, workspace: torch.Tensor,
                       out: torch.Tensor, *, scale: float, cu_count: int, budget_mult: int = 2,
                       max_partitions: int = 256, tile_tokens: int = 256, max_q_len: int = 1,
                       k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0,
                       stream=None, prepare: bool = False):
    """A decodes-first mixed batch in one call (see include/pa.h): the plan buffers are sized for the
    num_decodes decode requests; out receives every row.  With prepare=True nothing is launched and a
    Prepared call is returned."""
    dev = q.device
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", q.dtype)
    _need(k_cache, "k_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(v_cache, "v_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    _need(work_info, "work_info", torch.int32, dev)
    _need(reduce_info, "reduce_info", torch.int32, dev)
    _need(num_work, "num_work", torch.int32, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    _need(out, "out", q.dtype, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    B = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    if cu_query_lens.shape[0] != B + 1:
        raise ValueError("cu_query_lens must be [num_seqs + 1]")
    if reduce_info.numel() < 2 * num_decodes or num_work.numel() < 2:
        raise ValueError("plan buffers smaller than num_decodes / 2")
    qd = PA_F32 if q.dtype == torch.float32 else PA_BF16
    args = (_ptr(q), qd, R, Hq, D, _ptr(k_cache), _ptr(v_cache), _DTYPE_OF_NAME[kv_dtype], nb, Hkv, bs,
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B, _ptr(cu_query_lens),
            num_decodes, num_decode_rows, max_q_len, sliding_window, scale, k_scale, v_scale, cu_count,
            budget_mult, max_partitions, tile_tokens, int(work_info.shape[0]), _ptr(work_info),
            _ptr(reduce_info), _ptr(num_work), _ptr(workspace), workspace.numel(), _ptr(out), qd,
            _stream(stream))
    return _issue(load().pa_attention_mixed, args, "pa_attention_mixed", prepare)


def pa_prefill_workspace_bytes(num_rows: int, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                               head_dim: int, cu_count: int) -> int:
    return int(load().pa_prefill_workspace_bytes(num_rows, num_seqs, num_q_heads, num_kv_heads, head_dim, cu_count))


def pa_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: str,
               block_tables: torch.Tensor, context_lens: torch.Tensor, cu_query_lens: torch.Tensor,
               out: torch.Tensor, workspace: Optional[torch.Tensor] = None, *, scale: float, cu_count: int = 0,
               k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0, stream=None,
               prepare: bool = False):
    """Prefill rows of the given requests into out (see include/pa.h).  q and out are the whole
    batch's [R, Hq, D] arrays; cu_query_lens holds absolute row numbers (a slice of the batch's).
    Without a workspace the one-launch form runs; with one (a uint8 device tensor of
    pa_prefill_workspace_bytes(...) bytes, and cu_count) the split form."""
    dev = q.device
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    _need(q, "q", q.dtype)
    _need(out, "out", q.dtype, dev)
    _need(k_cache, "k_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(v_cache, "v_cache", _TORCH_OF_NAME[kv_dtype], dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    _need(cu_query_lens, "cu_query_lens", torch.int32, dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    B = int(context_lens.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] != B or cu_query_lens.shape[0] != B + 1:
        raise ValueError("block_tables must be [num_seqs, max_blocks], cu_query_lens [num_seqs + 1]")
    qd = PA_F32 if q.dtype == torch.float32 else PA_BF16
    args = (_ptr(q), qd, R, Hq, D, _ptr(k_cache), _ptr(v_cache), _DTYPE_OF_NAME[kv_dtype], nb, Hkv, bs,
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B, _ptr(cu_query_lens),
            sliding_window, scale, k_scale, v_scale, int(cu_count), _ptr(workspace),
            0 if workspace is None else workspace.numel(), _ptr(out), qd, _stream(stream))
    return _issue(load().pa_prefill, args, "pa_prefill", prepare)


def pa_split_decode_first(cu_query_lens_host, threshold: int) -> Tuple[int, int]:
    """(decode requests, decode rows) of a decode-first batch, from HOST cumulative query lengths."""
    import numpy as np
    cu = np.ascontiguousarray(np.asarray(cu_query_lens_host, dtype=np.int32))
    nd = ctypes.c_int32(0)
    ndt = ctypes.c_int32(0)
    _check(load().pa_split_decode_first(cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(cu.shape[0]) - 1,
                                        threshold, ctypes.byref(nd), ctypes.byref(ndt)), "pa_split_decode_first")
    return int(nd.value), int(ndt.value)
