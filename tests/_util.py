"""Shared helpers for the GPU parity tests: tolerances and oracle calls on workload cases."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Tolerances of the decode output against the fp64 oracle, by the least precise input involved:
# fp32 1e-4 absolute; bf16 2e-2 absolute + 1e-2 relative (numpy allclose form); fp8 KV 5e-2 absolute.
TOL = {"f32": (1e-4, 0.0), "bf16": (2e-2, 1e-2), "fp8": (5e-2, 0.0)}


def tolerance_kind(case) -> str:
    if case.kv_dtype == "fp8":
        return "fp8"
    if case.kv_dtype == "bf16" or case.q.dtype == torch.bfloat16:
        return "bf16"
    return "f32"


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, kind: str, what: str = "") -> None:
    atol, rtol = TOL[kind]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"({kind}: atol {atol}, rtol {rtol}); max err {err.max():.3e}; first {idx}")


def oracle_plan_of(case, cu_count, budget_mult=2, max_partitions=256, tile_tokens=256, capacity=None,
                   with_largest=False):
    ctx = case.context_lens.cpu().numpy()
    cu = None if case.cu_query_lens is None else case.cu_query_lens.cpu().numpy()
    return oracle.plan(ctx, case.num_kv_heads, cu_count, budget_mult, max_partitions, tile_tokens,
                       capacity, with_largest=with_largest, cu_query_lens=cu, window=case.window)


def oracle_direct(case) -> np.ndarray:
    return oracle.run_case(case)


def announce(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()
