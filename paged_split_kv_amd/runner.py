"""One decode step on the device: pa_plan -> pa_decode -> pa_merge on one stream, or the same step
as one pa_attention call (the decode plans in place: two launches).

``DecodeStep`` owns the plan buffers, the workspace and the output for one batch geometry, so a
timed loop issues only library calls and allocates nothing.  All arithmetic happens in libpa.so.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as B


@dataclass
class PlanConfig:
    cu_count: int
    budget_mult: int = 2
    max_partitions: int = 256
    tile_tokens: int = 256


class DecodeStep:
    def __init__(self, *, num_seqs: int, num_rows: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, max_q_len: int, out_dtype: torch.dtype, device,
                 plan: Optional[PlanConfig] = None):
        self.device = torch.device(device)
        self.plan_cfg = plan or PlanConfig(cu_count=B.pa_device_cu_count(self.device.index or 0))
        p = self.plan_cfg
        self.num_seqs = num_seqs
        self.num_kv_heads = num_kv_heads
        self.use_dispatch = True          # decode() follows the plan's dispatch order
        self.max_q_len = max_q_len
        self.capacity = B.pa_plan_capacity(num_seqs, num_kv_heads, p.cu_count, p.budget_mult,
                                           p.max_partitions)
        self.work_info = torch.empty((self.capacity, 4), dtype=torch.int32, device=self.device)
        # the decode's dispatch order, written by the plan beside it
        self.dispatch_info = torch.empty((self.capacity, 4), dtype=torch.int32, device=self.device)
        self.reduce_info = torch.empty((num_seqs, 2), dtype=torch.int32, device=self.device)
        self.num_work = torch.empty((2,), dtype=torch.int32, device=self.device)
        nbytes = B.pa_workspace_bytes(self.capacity, max_q_len, num_q_heads, head_dim)
        self.workspace = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=self.device)
        self.out = torch.empty((num_rows, num_q_heads, head_dim), dtype=out_dtype, device=self.device)

    def shares_slots(self, kv_dtype: str, num_q_heads: int, head_dim: int) -> bool:
        """Whether the decode (``decode`` without the merge, or ``attention``) streams slots with
        several workgroups each: the plan gives every request one slot (capacity <= batch <= 256),
        head_dim <= 128, and the workspace (sized by pa_workspace_bytes) holds the region."""
        return 0 < self.capacity <= self.num_seqs <= B.PA_INLINE_PLAN_SEQS and head_dim <= 128

    @classmethod
    def for_case(cls, case, plan: Optional[PlanConfig] = None) -> "DecodeStep":
        return cls(num_seqs=case.num_seqs, num_rows=case.num_rows, num_q_heads=case.num_q_heads,
                   num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, max_q_len=case.max_q_len,
                   out_dtype=case.q.dtype, device=case.q.device, plan=plan)

    def plan(self, context_lens: torch.Tensor, stream=None, cu_query_lens=None,
             sliding_window: int = 0) -> None:
        p = self.plan_cfg
        B.pa_plan(context_lens, self.num_kv_heads, cu_count=p.cu_count, budget_mult=p.budget_mult,
                  max_partitions=p.max_partitions, tile_tokens=p.tile_tokens, capacity=self.capacity,
                  work_info=self.work_info, reduce_info=self.reduce_info, num_work=self.num_work,
                  cu_query_lens=cu_query_lens, sliding_window=sliding_window, dispatch_info=self.dispatch_info,
                  stream=stream)

    def decode(self, q, k_cache, v_cache, kv_dtype, block_tables, context_lens, *, scale,
               cu_query_lens=None, k_scale=1.0, v_scale=1.0, merge: bool = False,
               sliding_window: int = 0, stream=None) -> None:
        """pa_decode; with merge=True the call also runs the log-sum-exp merge into self.out (the
        merge launch follows the decode launch on the same stream)."""
        B.pa_decode(q, k_cache, v_cache, kv_dtype, block_tables, context_lens, self.work_info,
                    self.num_work, self.workspace, scale=scale, cu_query_lens=cu_query_lens,
                    max_q_len=self.max_q_len, k_scale=k_scale, v_scale=v_scale,
                    tile_tokens=self.plan_cfg.tile_tokens,
                    reduce_info=self.reduce_info if merge else None,
                    out=self.out if merge else None, sliding_window=sliding_window,
                    dispatch_info=self.dispatch_info if self.use_dispatch else None, stream=stream)

    def attention(self, q, k_cache, v_cache, kv_dtype, block_tables, context_lens, *, scale,
                  cu_query_lens=None, k_scale=1.0, v_scale=1.0, sliding_window: int = 0,
                  stream=None) -> torch.Tensor:
        """pa_attention: plan, decode and merge into self.out; the plan buffers are refreshed."""
        p = self.plan_cfg
        B.pa_attention(q, k_cache, v_cache, kv_dtype, block_tables, context_lens, self.work_info,
                       self.reduce_info, self.num_work, self.workspace, self.out, scale=scale,
                       cu_count=p.cu_count, budget_mult=p.budget_mult, max_partitions=p.max_partitions,
                       tile_tokens=p.tile_tokens, cu_query_lens=cu_query_lens, max_q_len=self.max_q_len,
                       k_scale=k_scale, v_scale=v_scale, sliding_window=sliding_window, stream=stream)
        return self.out

    def merge(self, cu_query_lens=None, stream=None) -> torch.Tensor:
        B.pa_merge(self.out, self.reduce_info, self.workspace, capacity=self.capacity,
                   cu_query_lens=cu_query_lens, max_q_len=self.max_q_len, stream=stream)
        return self.out

    def run_case(self, case, stream=None, replan: bool = True, fused: bool = True,
                 whole: bool = False) -> torch.Tensor:
        """Plan, decode and merge one Case.  fused=True passes out to pa_decode, which then merges
        in the same call; fused=False calls pa_merge separately; whole=True makes the one pa_attention
        call."""
        w = case.window
        if whole:
            return self.attention(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables,
                                  case.context_lens, scale=case.scale, cu_query_lens=case.cu_query_lens,
                                  k_scale=case.k_scale, v_scale=case.v_scale, sliding_window=w,
                                  stream=stream)
        if replan:
            self.plan(case.context_lens, stream, cu_query_lens=case.cu_query_lens, sliding_window=w)
        self.decode(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables,
                    case.context_lens, scale=case.scale, cu_query_lens=case.cu_query_lens,
                    k_scale=case.k_scale, v_scale=case.v_scale, merge=fused, sliding_window=w,
                    stream=stream)
        if fused:
            return self.out
        return self.merge(case.cu_query_lens, stream)


def run_case(case, plan: Optional[PlanConfig] = None, fused: bool = True,
             whole: bool = False) -> torch.Tensor:
    """Plan, decode and merge one workload Case; returns the output tensor (device)."""
    return DecodeStep.for_case(case, plan).run_case(case, fused=fused, whole=whole)


class MixedStep:
    """The decode-first split of a mixed batch (requests ordered decodes first): the leading requests
    with at most `threshold` query tokens go through pa_attention (split-KV decode, rows written to a
    view of the output), the rest through pa_prefill's one-launch form (short prompts) on the same
    stream.  The split is taken from a
    host copy of the cumulative query lengths, as a batch builder holds them; buffers are made once.
    With concurrent=True the two parts, which read the same inputs and write disjoint rows, run on
    two streams (the prefill on a second stream of default priority) and join before returning.
    With one_call=True the step is one pa_attention_mixed call (decode and prompts share a launch
    where they fit one, then the merge)."""

    def __init__(self, case, threshold: int, plan: Optional[PlanConfig] = None, concurrent: bool = False,
                 one_call: bool = False):
        self.threshold = threshold
        self.one_call = one_call
        self.side = torch.cuda.Stream(device=case.q.device) if concurrent else None
        self.nd, self.ndt = B.pa_split_decode_first(case.cu_query_lens.cpu().numpy(), threshold)
        self.out = torch.empty_like(case.q)
        self.dec = None
        if self.nd > 0:
            self.dec = DecodeStep(num_seqs=self.nd, num_rows=self.ndt, num_q_heads=case.num_q_heads,
                                  num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                                  max_q_len=threshold, out_dtype=case.q.dtype, device=case.q.device,
                                  plan=plan)
            self.dec.out = self.out[:self.ndt]

    def run(self, case, stream=None) -> torch.Tensor:
        nd, ndt = self.nd, self.ndt
        main = stream if stream is not None else torch.cuda.current_stream(case.q.device)
        if self.one_call and self.dec is not None:
            d, p = self.dec, self.dec.plan_cfg
            B.pa_attention_mixed(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables,
                                 case.context_lens, case.cu_query_lens, nd, ndt, d.work_info, d.reduce_info,
                                 d.num_work, d.workspace, self.out, scale=case.scale, cu_count=p.cu_count,
                                 budget_mult=p.budget_mult, max_partitions=p.max_partitions,
                                 tile_tokens=p.tile_tokens, max_q_len=self.threshold, k_scale=case.k_scale,
                                 v_scale=case.v_scale, sliding_window=case.window, stream=main)
            return self.out
        pre = main
        if self.side is not None and self.dec is not None:
            self.side.wait_stream(main)
            pre = self.side
        B.pa_prefill(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables[nd:],
                     case.context_lens[nd:], case.cu_query_lens[nd:], self.out, scale=case.scale,
                     k_scale=case.k_scale, v_scale=case.v_scale, sliding_window=case.window, stream=pre)
        if self.dec is not None:
            self.dec.attention(case.q[:ndt], case.k_cache, case.v_cache, case.kv_dtype, case.block_tables[:nd],
                               case.context_lens[:nd], scale=case.scale,
                               cu_query_lens=case.cu_query_lens[:nd + 1], k_scale=case.k_scale,
                               v_scale=case.v_scale, sliding_window=case.window, stream=main)
        if pre is not main:
            main.wait_stream(pre)
        return self.out


def mixed_step(case, threshold: int, plan: Optional[PlanConfig] = None, stream=None,
               concurrent: bool = False, one_call: bool = False) -> torch.Tensor:
    """One decode-first split step of a mixed batch (see MixedStep)."""
    return MixedStep(case, threshold, plan, concurrent, one_call).run(case, stream)
