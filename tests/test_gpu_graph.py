"""Capture-safe plan refresh and graph replay.

The plan is a pure function of context_lens, minted once per batch shape and refreshed in place on
every step; draft passes advance context_lens and must re-plan (ROCm/ATOM PR #2366 section 3 "Plan
lifetime vs cudagraph" and review item 2; ROCm/ATOM PR #2514 Design).  Here one HIP graph holds three
draft passes -- advance the lengths, pa_plan, pa_decode, pa_merge, copy the rows out -- and is replayed
several times, with eager work and synchronisation between replays; every pass of every replay is
checked against the oracle at that pass's lengths.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import DecodeStep, MixedStep, PlanConfig
from _util import announce, assert_close, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PASSES = 3


def _oracle_at(case, lens):
    h = case.host()
    return oracle.attention_direct(h["q"], case.q_dtype, h["k_cache"], h["v_cache"], case.kv_dtype,
                                   h["block_tables"], np.asarray(lens, np.int32), h["cu_query_lens"],
                                   case.scale, case.k_scale, case.v_scale)


@pytest.mark.parametrize("mode", ["separate_merge", "merge_in_call", "attention", "attention_shared_slots"])
def test_graph_replays_draft_passes(mode):
    """attention_shared_slots: a budget of 2 compute units leaves every request one slot, so
    pa_attention cuts the slots into pieces; the piece table is rewritten on every replay."""
    fused = mode == "merge_in_call"
    cu_count = 2 if mode == "attention_shared_slots" else 256
    final = [1300, 40, 2, 5000, 777, 256]
    q_lens = [2, 1, 2, 3, 1, 2]
    # pages exist for the final lengths; the graph starts PASSES tokens earlier
    case = W.build_case("graph", final, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        kv_dtype="bf16", q_dtype="bf16", seed=31, q_lens=q_lens, pad_rows=2,
                        device=DEV, poison_tail=False)
    start = np.asarray(final) - PASSES
    lens = torch.from_numpy(start.astype(np.int32)).to(DEV)
    case.context_lens = lens
    step = DecodeStep.for_case(case, PlanConfig(cu_count=cu_count))
    assert step.shares_slots(case.kv_dtype, case.num_q_heads, case.head_dim) == (mode == "attention_shared_slots")
    outs = [torch.empty_like(step.out) for _ in range(PASSES)]

    def passes():
        for p in range(PASSES):
            lens.add_(1)                                   # the draft step advances every length
            if mode.startswith("attention"):               # plans in place inside the decode launch
                step.attention(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables, lens,
                               scale=case.scale, cu_query_lens=case.cu_query_lens)
            else:
                step.plan(lens)                            # refresh the plan in place
                step.decode(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables, lens,
                            scale=case.scale, cu_query_lens=case.cu_query_lens, merge=fused)
                if not fused:
                    step.merge(case.cu_query_lens)
            outs[p].copy_(step.out)

    # warm up eagerly (the recorded path must be the planned one), then capture
    passes()
    torch.cuda.synchronize()
    lens.copy_(torch.from_numpy(start.astype(np.int32)))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            passes()
    torch.cuda.synchronize()

    refs = [_oracle_at(case, start + p + 1) for p in range(PASSES)]
    other = W.build_case("eager", [900, 60], num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                         kv_dtype="bf16", q_dtype="bf16", seed=32, q_lens=[1, 2], device=DEV)
    other_step = DecodeStep.for_case(other, PlanConfig(cu_count=256))
    for rep in range(4):
        announce(f"graph replay {rep} {mode}")
        lens.copy_(torch.from_numpy(start.astype(np.int32)))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p in range(PASSES):
            assert_close(to_f64(outs[p]), refs[p], "bf16", f"replay {rep} pass {p}")
        assert int(lens.cpu().numpy().sum()) == int(np.sum(final))
        ow, orr, on, olarge = oracle.plan(final, 2, cu_count, with_largest=True)
        assert step.num_work.cpu().numpy().tolist() == [on, olarge]
        assert np.array_equal(step.work_info.cpu().numpy(), ow)
        assert np.array_equal(step.reduce_info.cpu().numpy(), orr)
        # eager work between replays, on the same device and stream
        o = other_step.run_case(other, fused=True)
        torch.cuda.synchronize()
        assert_close(to_f64(o), oracle.run_case(other), "bf16", f"eager between replays {rep}")


def test_graph_replays_mixed_batch_one_call():
    """pa_attention_mixed inside a graph: decodes and a prompt share one launch, then the merge.
    Three passes advance every length by one; each replay is checked against the oracle."""
    final = [1300, 40, 5000, 777, 300]
    q_lens = [1, 1, 1, 1, 9]
    case = W.build_case("graph_mixed", final, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        kv_dtype="bf16", q_dtype="bf16", seed=33, q_lens=q_lens, pad_rows=1, device=DEV,
                        poison_tail=False)
    start = np.asarray(final) - PASSES
    lens = torch.from_numpy(start.astype(np.int32)).to(DEV)
    case.context_lens = lens
    step = MixedStep(case, 1, PlanConfig(cu_count=256), one_call=True)
    outs = [torch.empty_like(step.out) for _ in range(PASSES)]

    def passes():
        for p in range(PASSES):
            lens.add_(1)
            step.run(case)
            outs[p].copy_(step.out)

    passes()
    torch.cuda.synchronize()
    lens.copy_(torch.from_numpy(start.astype(np.int32)))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            passes()
    torch.cuda.synchronize()
    refs = [_oracle_at(case, start + p + 1) for p in range(PASSES)]
    for rep in range(3):
        announce(f"mixed graph replay {rep}")
        lens.copy_(torch.from_numpy(start.astype(np.int32)))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p in range(PASSES):
            assert_close(to_f64(outs[p]), refs[p], "bf16", f"mixed replay {rep} pass {p}")
