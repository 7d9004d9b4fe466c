"""pa_attention_noalloc (the entry point for callers that cannot allocate) against pa_attention: two
calls in a row through the C ABI, the second with a smaller input, each compared bit for bit with
pa_attention given a workspace of the size the no-allocation call uses (the same kernels on the same
arguments), plan buffers included, and with the fp64 oracle at the decode tolerances."""
import numpy as np
import pytest
import torch

from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import PlanConfig
from _util import announce, assert_close, oracle_direct, to_f64, tolerance_kind

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc_bytes(capacity, max_q_len, hq, d):
    full = B.pa_workspace_bytes(capacity, max_q_len, hq, d)
    if full <= B.PA_NOALLOC_SCRATCH_BYTES:
        return full
    up = lambda x: (x + 255) // 256 * 256
    return up(capacity * max_q_len * hq * d * 4) + up(capacity * max_q_len * hq * 2 * 4)


def _both(case, cfg):
    cap = B.pa_plan_capacity(case.num_seqs, case.num_kv_heads, cfg.cu_count, cfg.budget_mult, cfg.max_partitions)
    Hq, D = case.num_q_heads, case.head_dim
    kw = dict(scale=case.scale, cu_count=cfg.cu_count, budget_mult=cfg.budget_mult,
              max_partitions=cfg.max_partitions, tile_tokens=cfg.tile_tokens, cu_query_lens=case.cu_query_lens,
              max_q_len=case.max_q_len, k_scale=case.k_scale, v_scale=case.v_scale, sliding_window=case.window)
    res = []
    for noalloc in (True, False):
        work = torch.full((cap, 4), 7, dtype=torch.int32, device=DEV)
        red = torch.full((case.num_seqs, 2), 7, dtype=torch.int32, device=DEV)
        nw = torch.full((2,), 7, dtype=torch.int32, device=DEV)
        out = torch.full_like(case.q, float("nan"))
        if noalloc:
            B.pa_attention_noalloc(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables,
                                   case.context_lens, work, red, nw, out, **kw)
        else:
            ws = torch.empty((_noalloc_bytes(cap, case.max_q_len, Hq, D),), dtype=torch.uint8, device=DEV)
            B.pa_attention(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables, case.context_lens,
                           work, red, nw, ws, out, **kw)
        torch.cuda.synchronize()
        res.append((out, work, red, nw))
    return res


def _check(case, cfg, what):
    (o1, w1, r1, n1), (o2, w2, r2, n2) = _both(case, cfg)
    assert torch.equal(w1, w2) and torch.equal(r1, r2) and torch.equal(n1, n2), f"{what}: plan buffers differ"
    assert torch.equal(o1, o2), f"{what}: pa_attention_noalloc differs from pa_attention"
    assert_close(to_f64(o1), oracle_direct(case), tolerance_kind(case), what)


def test_noalloc_matches_pa_attention_twice_smaller_second():
    cfg = PlanConfig(cu_count=B.pa_device_cu_count(0))
    big = W.make_config("skewed_bf16", device=DEV)
    announce(f"noalloc first call: skewed step ({int(big.context_lens.sum().item())} tokens)")
    _check(big, cfg, "noalloc skewed")
    small = W.build_case("noalloc_small", [700, 33, 1, 300], num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=3, q_lens=[3, 1, 1, 2], pad_rows=2,
                         device=DEV)
    announce("noalloc second call: 4 requests with verify rows")
    _check(small, cfg, "noalloc small")


def test_noalloc_slot_states_only_when_the_region_does_not_fit():
    """The verify workload's full workspace (with the shared-slot region) exceeds the array; its slot
    states fit, so the call runs with those alone, like pa_attention given that much."""
    cfg = PlanConfig(cu_count=B.pa_device_cu_count(0))
    case = W.make_config("verify_bf16", device=DEV)
    cap = B.pa_plan_capacity(case.num_seqs, case.num_kv_heads, cfg.cu_count, cfg.budget_mult, cfg.max_partitions)
    assert B.pa_workspace_bytes(cap, case.max_q_len, case.num_q_heads, case.head_dim) > B.PA_NOALLOC_SCRATCH_BYTES
    announce("noalloc verify (slot states only)")
    _check(case, cfg, "noalloc verify")
    tiny = W.make_config("tiny_fp32", device=DEV)
    announce("noalloc tiny fp32 after it")
    _check(tiny, cfg, "noalloc tiny")


def test_noalloc_refuses_states_beyond_the_array():
    case = W.build_case("noalloc_over", [64] * 8, num_q_heads=16, num_kv_heads=1, head_dim=256, block_size=16,
                        kv_dtype="bf16", q_dtype="bf16", seed=5, q_lens=[4] * 8, device=DEV)
    # capacity 8 x 256 partitions at a large budget: slot states far beyond 32 MiB
    cap = B.pa_plan_capacity(8, 1, 1 << 20, 2, 256)
    work = torch.empty((cap, 4), dtype=torch.int32, device=DEV)
    red = torch.empty((8, 2), dtype=torch.int32, device=DEV)
    nw = torch.empty((2,), dtype=torch.int32, device=DEV)
    out = torch.empty_like(case.q)
    with pytest.raises(B.PaError) as e:
        B.pa_attention_noalloc(case.q, case.k_cache, case.v_cache, "bf16", case.block_tables, case.context_lens,
                               work, red, nw, out, scale=case.scale, cu_count=1 << 20,
                               cu_query_lens=case.cu_query_lens, max_q_len=4)
    assert e.value.status == B.PA_CAPACITY
