"""Thin binding over libpa_probe.so (include/pa_probe.h): the benchmark's read-only bandwidth probes.
Argument marshalling only; the probes compute nothing of the decode path."""
from __future__ import annotations

import ctypes
import os

import torch

from . import binding as B

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_probe.so")
SYMBOLS = ("pa_probe_read", "pa_probe_gather")

_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_split_kv_amd.build`")
    B.load()                       # torch's HIP runtime first, then libpa (status strings)
    lib = ctypes.CDLL(path)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    lib.pa_probe_read.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    lib.pa_probe_read.restype = ctypes.c_int
    lib.pa_probe_gather.argtypes = [vp, vp, ctypes.c_int, i32, i32, i32, i32, vp, i32, vp, i32, vp, vp, i32, i32,
                                    vp, vp]
    lib.pa_probe_gather.restype = ctypes.c_int
    _lib = lib
    return lib


def sink_for(words: int, device) -> torch.Tensor:
    return torch.empty((max(words, 1),), dtype=torch.int32, device=device)


def pa_probe_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if sink.numel() < 4 * workgroups:
        raise ValueError("sink holds fewer than 4 words per workgroup")
    st = load().pa_probe_read(B._ptr(src), src.numel() * src.element_size(), int(workgroups), B._ptr(sink),
                              B._stream(stream))
    B._check(st, "pa_probe_read")


def pa_probe_gather(k_cache, v_cache, kv_dtype: str, block_tables, context_lens, work_info, num_work,
                    sink: torch.Tensor, tile_tokens: int = 256, stream=None, prepare: bool = False):
    nb, hkv, bs, d = (int(x) for x in k_cache.shape)
    cap = int(work_info.shape[0])
    if sink.numel() < 4 * cap * hkv:
        raise ValueError("sink holds fewer than 4 words per (slot, kv head) workgroup")
    args = (B._ptr(k_cache), B._ptr(v_cache), B._DTYPE_OF_NAME[kv_dtype], nb, hkv, bs, d,
            B._ptr(block_tables), int(block_tables.shape[1]), B._ptr(context_lens),
            int(context_lens.shape[0]), B._ptr(work_info), B._ptr(num_work), cap,
            int(tile_tokens), B._ptr(sink), B._stream(stream))
    return B._issue(load().pa_probe_gather, args, "pa_probe_gather", prepare)
