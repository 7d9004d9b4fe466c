"""CPU oracle for paged split-KV decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The product library never calls it and shares no code with it.

The arithmetic lives in ``pa_oracle.c`` (plain C, integer planner, IEEE double attention), built
with gcc into ``liboracle.so`` beside this file.  This module only marshals numpy arrays.

Functions:
  plan_capacity, plan    -- O1, the length-proportional planner (integer, bit-exact contract)
  attention_direct       -- O2, softmax attention of every row over its visible keys (optionally
                            limited to the last `window` of them)
  attention_split        -- O3, the same computed per plan slot and merged by log-sum-exp
  attention_rows         -- O2 for selected (row, head) pairs of a full-size problem
  decode_values          -- element decoding of the storage types (bf16 bits, e4m3fn codes)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "bf16": 1, "fp8": 2}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}

OK = 0
INVALID = 1


class OracleError(RuntimeError):
    pass


def compile_source(src: str, lib_path: str) -> str:
    """gcc with strict IEEE (no fast-math, no contraction): `src` -> shared library `lib_path`."""
    tmp = lib_path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


def build(force: bool = False) -> str:
    """Compile the oracle (pa_oracle.c -> liboracle.so) when missing or older than its source."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


_lib = None

# A test that plants a mistake in a copy of pa_oracle.c builds that copy elsewhere and names the
# library here, so the pin tests run against it in a child process.
_OVERRIDE_ENV = "PA_ORACLE_LIB"


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(_OVERRIDE_ENV)
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        vp = ctypes.c_void_p
        c_int = ctypes.c_int
        dbl = ctypes.c_double
        lib.orc_plan_capacity.argtypes = [c_int, c_int, c_int, c_int, c_int, i32p]
        lib.orc_plan.argtypes = [vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, vp, vp,
                                 vp]
        prob = [vp, c_int, c_int, c_int, c_int, vp, vp, c_int, c_int, c_int, c_int, vp, c_int, vp,
                c_int, vp, dbl, dbl, dbl, c_int]
        lib.orc_attention_direct.argtypes = prob + [vp, c_int]
        lib.orc_attention_split.argtypes = prob + [vp, vp, c_int, vp, c_int]
        lib.orc_attention_rows.argtypes = prob + [vp, vp, c_int, vp]
        lib.orc_decode_array.argtypes = [vp, c_int, ctypes.c_int64, vp]
        for f in ("orc_plan_capacity", "orc_plan", "orc_attention_direct", "orc_attention_split",
                  "orc_attention_rows", "orc_decode_array"):
            getattr(lib, f).restype = c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


# ---------------------------------------------------------------------------------------------
# O1: planner
# ---------------------------------------------------------------------------------------------

def plan_capacity(num_seqs: int, num_kv_heads: int, cu_count: int = 256, budget_mult: int = 2,
                  max_partitions: int = 256) -> int:
    out = ctypes.c_int32(0)
    st = _load().orc_plan_capacity(num_seqs, num_kv_heads, cu_count, budget_mult, max_partitions,
                                   ctypes.byref(out))
    if st != OK:
        raise OracleError("invalid planner arguments")
    return int(out.value)


def plan(context_lens, num_kv_heads: int, cu_count: int = 256, budget_mult: int = 2,
         max_partitions: int = 256, tile_tokens: int = 256, capacity: Optional[int] = None,
         with_largest: bool = False, cu_query_lens=None, window: int = 0):
    """Returns (work_info int32 [capacity, 4], reduce_info int32 [B, 2], num_work) and, with
    with_largest, also the tile count of the largest slot.  cu_query_lens and window only matter
    together: with a window the plan covers each request's windowed key range."""
    ctx = _i32(context_lens)
    B = int(ctx.shape[0])
    cu = None if cu_query_lens is None else _i32(cu_query_lens)
    if cu is not None and cu.shape[0] != B + 1:
        raise OracleError("cu_query_lens shape")
    cap = plan_capacity(B, num_kv_heads, cu_count, budget_mult, max_partitions)
    if capacity is None:
        capacity = cap
    work = np.zeros((max(capacity, 0), 4), dtype=np.int32)
    red = np.zeros((B, 2), dtype=np.int32)
    nw = np.zeros(2, dtype=np.int32)
    st = _load().orc_plan(_ptr(ctx), _ptr(cu), B, num_kv_heads, cu_count, budget_mult, max_partitions,
                          tile_tokens, int(window), capacity, _ptr(work), _ptr(red), _ptr(nw))
    if st != OK:
        raise OracleError("invalid planner arguments")
    if with_largest:
        return work, red, int(nw[0]), int(nw[1])
    return work, red, int(nw[0])


# ---------------------------------------------------------------------------------------------
# O2 / O3: attention
# ---------------------------------------------------------------------------------------------

def _problem(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, cu_query_lens,
             scale, k_scale, v_scale, window=0):
    q = np.ascontiguousarray(q, dtype=_STORAGE[q_dtype])
    k = np.ascontiguousarray(k_cache, dtype=_STORAGE[kv_dtype])
    v = np.ascontiguousarray(v_cache, dtype=_STORAGE[kv_dtype])
    bt = _i32(block_tables)
    ctx = _i32(context_lens)
    cu = None if cu_query_lens is None else _i32(cu_query_lens)
    R, Hq, D = q.shape
    nb, Hkv, bs, D2 = k.shape
    if D2 != D or v.shape != k.shape:
        raise OracleError("shape mismatch")
    B = int(ctx.shape[0])
    if bt.ndim != 2 or bt.shape[0] != B:
        raise OracleError("block table shape")
    if cu is not None and cu.shape[0] != B + 1:
        raise OracleError("cu_query_lens shape")
    keep = (q, k, v, bt, ctx, cu)
    args = [_ptr(q), DTYPE_CODES[q_dtype], R, Hq, D, _ptr(k), _ptr(v), DTYPE_CODES[kv_dtype], nb, Hkv,
            bs, _ptr(bt), int(bt.shape[1]), _ptr(ctx), B, _ptr(cu), float(scale), float(k_scale),
            float(v_scale), int(window)]
    return args, keep, (R, Hq, D)


def attention_direct(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                     cu_query_lens, scale, k_scale=1.0, v_scale=1.0,
                     threads: Optional[int] = None, window: int = 0) -> np.ndarray:
    args, keep, (R, Hq, D) = _problem(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                      context_lens, cu_query_lens, scale, k_scale, v_scale, window)
    out = np.empty((R, Hq, D), dtype=np.float64)
    st = _load().orc_attention_direct(*args, _ptr(out), threads or default_threads())
    if st != OK:
        raise OracleError("invalid attention problem")
    return out


def attention_split(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                    cu_query_lens, scale, work_info, reduce_info, tile_tokens, k_scale=1.0,
                    v_scale=1.0, threads: Optional[int] = None, window: int = 0) -> np.ndarray:
    args, keep, (R, Hq, D) = _problem(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                      context_lens, cu_query_lens, scale, k_scale, v_scale, window)
    work = _i32(work_info)
    red = _i32(reduce_info)
    out = np.empty((R, Hq, D), dtype=np.float64)
    st = _load().orc_attention_split(*args, _ptr(work), _ptr(red), int(tile_tokens), _ptr(out),
                                     threads or default_threads())
    if st != OK:
        raise OracleError("invalid attention problem")
    return out


def attention_rows(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                   cu_query_lens, scale, rows, heads, k_scale=1.0, v_scale=1.0,
                   window: int = 0) -> np.ndarray:
    args, keep, (R, Hq, D) = _problem(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                                      context_lens, cu_query_lens, scale, k_scale, v_scale, window)
    rows = _i32(rows)
    heads = _i32(heads)
    out = np.empty((rows.shape[0], D), dtype=np.float64)
    st = _load().orc_attention_rows(*args, _ptr(rows), _ptr(heads), int(rows.shape[0]), _ptr(out))
    if st != OK:
        raise OracleError("invalid attention problem")
    return out


def decode_values(bits: np.ndarray, dtype: str) -> np.ndarray:
    src = np.ascontiguousarray(bits, dtype=_STORAGE[dtype])
    out = np.empty(src.shape, dtype=np.float64)
    st = _load().orc_decode_array(_ptr(src), DTYPE_CODES[dtype], int(src.size), _ptr(out))
    if st != OK:
        raise OracleError("bad dtype")
    return out


def run_case(case, threads: Optional[int] = None) -> np.ndarray:
    """O2 on a workload Case (any device; data is copied to the host)."""
    h = case.host()
    return attention_direct(h["q"], case.q_dtype, h["k_cache"], h["v_cache"], case.kv_dtype,
                            h["block_tables"], h["context_lens"], h["cu_query_lens"], case.scale,
                            case.k_scale, case.v_scale, threads=threads,
                            window=getattr(case, "window", 0))
