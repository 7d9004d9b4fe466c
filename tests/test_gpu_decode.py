"""GPU decode + merge (pa_decode, pa_merge) against the fp64 oracle, element by element.

Tolerances: fp32 1e-4 abs; bf16 2e-2 abs + 1e-2 rel; fp8 KV 5e-2 abs (see _util.TOL).
Semantics pinned: per-token causal range S - (L - 1 - i) (opengfx1030/vllm-rdna PR #29, Change 1),
exact zeros for padding rows and empty rows, bitwise equality with and without cumulative query
lengths when every request has one token, independence from the plan's slot order.
"""
import math

import numpy as np
import pytest
import torch

from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import DecodeStep, PlanConfig
from _util import announce, assert_close, oracle_direct, to_f64, tolerance_kind

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (name, ctx, q_lens, Hq, Hkv, D, bs, kv, q, pad, P, T)
SMALL = [
    ("bf16_d128_g8", [700, 33, 1, 2000, 256, 257], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256),
    ("bf16_d64_verify", [37, 5, 64, 1290], [3, 1, 2, 4], 8, 2, 64, 64, "bf16", "bf16", 2, 256, 256),
    ("bf16_d256_verify3", [1500, 900, 2, 700], [3, 3, 1, 1], 6, 1, 256, 16, "bf16", "bf16", 2, 256, 256),
    ("bf16_d128_64rows", [3000, 17, 600], [4, 4, 1], 16, 1, 128, 16, "bf16", "bf16", 1, 64, 64),
    ("bf16_d128_bs128", [5000, 129, 128, 4000], None, 8, 1, 128, 128, "bf16", "bf16", 3, 256, 512),
    ("bf16_zero_len", [0, 300, 0, 2, 40], [2, 2, 1, 3, 1], 4, 2, 128, 16, "bf16", "bf16", 1, 8, 16),
    ("qf32_kvbf16", [800, 64, 3], None, 16, 2, 128, 16, "bf16", "f32", 0, 256, 256),
    ("fp8_d128", [900, 1, 4000, 77], None, 16, 2, 128, 16, "fp8", "bf16", 0, 256, 256),
    ("fp8_d64_verify", [300, 45], [2, 3], 12, 4, 64, 64, "fp8", "bf16", 1, 256, 64),
    ("fp8_d256", [1200, 600], [1, 2], 8, 2, 256, 16, "fp8", "f32", 0, 256, 256),
    ("f32_d64", [1, 17, 100, 300, 0], None, 4, 1, 64, 16, "f32", "f32", 2, 256, 256),
    ("f32_d128_verify", [500, 31, 2], [3, 2, 2], 8, 2, 128, 64, "f32", "f32", 1, 8, 64),
    ("f32_d256_qbf16", [700, 90], [1, 2], 4, 2, 256, 16, "f32", "bf16", 0, 256, 256),
    ("bf16_many_slots", [4096, 4096, 100, 5000], None, 8, 1, 128, 16, "bf16", "bf16", 0, 256, 16),
    # one query head per kv head (G = 1: one-row blocks), verify rows included
    ("bf16_g1_verify", [900, 2, 300], [1, 2, 3], 8, 8, 128, 16, "bf16", "bf16", 1, 256, 256),
    # fp8 at head_dim 64 on 128-token pages, tile 256 = two pages
    ("fp8_d64_bs128", [5000, 129, 700], None, 8, 2, 64, 128, "fp8", "bf16", 0, 256, 256),
    # the largest row block: 32 query heads per kv head x 2 tokens = 64 rows
    ("bf16_g32_64rows", [1200, 64], [2, 1], 32, 1, 128, 16, "bf16", "bf16", 1, 256, 256),
    # eight kv heads at head_dim 256 (G = 2)
    ("bf16_hkv8_d256", [800, 3000], [2, 1], 16, 8, 256, 16, "bf16", "bf16", 0, 256, 256),
    # last tile holds fewer keys than the request has query tokens: early tokens see nothing in the
    # wave that owns it while the last token does (regression: such rows must stay (-inf, 0, 0))
    ("bf16_short_last_tile", [257, 513, 258, 769], [3, 3, 2, 4], 8, 2, 128, 16, "bf16", "bf16", 1, 1, 256),
    ("fp8_short_last_tile", [257, 1025], [3, 4], 8, 2, 64, 16, "fp8", "bf16", 0, 1, 256),
    # head_dim 256 (the waves split the head dimension): four 16-row blocks, fp32 queries, one-chunk
    # slots, and a last tile shorter than the query length
    ("bf16_d256_64rows", [2100, 40, 700], [6, 1, 6], 6, 1, 256, 16, "bf16", "bf16", 1, 64, 64),
    ("fp8_d256_40rows", [900, 3000, 1], [5, 2, 1], 8, 1, 256, 64, "fp8", "bf16", 0, 256, 128),
    ("qf32_d256_tiny_tiles", [17, 1, 300, 4097], None, 6, 1, 256, 16, "bf16", "f32", 0, 4, 16),
    ("bf16_d256_short_last_tile", [257, 513], [3, 2], 6, 2, 256, 16, "bf16", "bf16", 0, 1, 256),
    # 128-token pages with an fp32 cache; 64-token pages with fp8 at head_dim 128 and verify rows
    ("f32_d128_bs128", [3000, 129, 128], None, 4, 1, 128, 128, "f32", "f32", 1, 256, 256),
    ("fp8_d128_bs64_verify", [2000, 65, 700], [2, 1, 3], 16, 2, 128, 64, "fp8", "bf16", 1, 256, 128),
]


def _small_case(spec, seed):
    name, ctx, ql, Hq, Hkv, D, bs, kv, qd, pad, P, T = spec
    return W.build_case(name, ctx, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                        kv_dtype=kv, q_dtype=qd, seed=seed, q_lens=ql, pad_rows=pad, device=DEV), P, T


def _partial_bytes(step):
    """Bytes of the workspace's slot partial-state regions (the shared-slot region follows them)."""
    up = lambda x: (x + 255) // 256 * 256
    c, l, h, d = step.capacity, step.max_q_len, step.out.shape[1], step.out.shape[2]
    return up(c * l * h * d * 4) + up(c * l * h * 2 * 4)


def _run(case, P=256, T=256, cu_count=256, fused=True):
    step = DecodeStep.for_case(case, PlanConfig(cu_count=cu_count, max_partitions=P, tile_tokens=T))
    step.out.fill_(float("nan"))
    step.workspace[:_partial_bytes(step)].fill_(0xFF)    # NaN pattern in every partial-state slot
    out = step.run_case(case, fused=fused)
    torch.cuda.synchronize()
    return out, step


def _zero_rows(case):
    """Rows that must be exactly zero: padding rows, rows of empty requests, tokens with no keys."""
    R = case.num_rows
    ctx = case.context_lens.cpu().numpy()
    zero = np.ones(R, dtype=bool)
    if case.cu_query_lens is None:
        for b, s in enumerate(ctx):
            zero[b] = s <= 0
    else:
        cu = case.cu_query_lens.cpu().numpy()
        for b, s in enumerate(ctx):
            L = cu[b + 1] - cu[b]
            for i in range(L):
                zero[cu[b] + i] = (s - (L - 1 - i)) <= 0
    return zero


@pytest.mark.parametrize("fused", [True, False], ids=["merge_in_call", "separate_merge"])
@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases_match_oracle(spec, fused):
    case, P, T = _small_case(spec, seed=11)
    announce(f"small {spec[0]} fused={fused}")
    out, _ = _run(case, P, T, fused=fused)
    got = to_f64(out)
    ref = oracle_direct(case)
    assert_close(got, ref, tolerance_kind(case), spec[0])
    z = _zero_rows(case)
    assert (got[z] == 0.0).all()
    assert (np.abs(got[~z]).sum(axis=(1, 2)) > 0).all()


ONE_SLOT = [s for s in SMALL if s[5] <= 128]


@pytest.mark.parametrize("mode", ["merge_in_call", "separate_merge", "attention"])
@pytest.mark.parametrize("spec", ONE_SLOT, ids=[s[0] for s in ONE_SLOT])
def test_one_slot_per_request(spec, mode):
    """A budget of at most one workgroup per request (cu_count 1): the capacity is the batch, every
    request is one slot, and the decode shares the slots (pieces, folded by the merge) where that
    applies (batch <= 256, head_dim <= 128), with or without out."""
    case, P, T = _small_case(spec, seed=12)
    announce(f"one slot per request {spec[0]} {mode}")
    if mode == "attention":
        step = DecodeStep.for_case(case, PlanConfig(cu_count=1, max_partitions=P, tile_tokens=T))
        step.out.fill_(float("nan"))
        out = step.run_case(case, whole=True)
        torch.cuda.synchronize()
    else:
        out, step = _run(case, P, T, cu_count=1, fused=(mode == "merge_in_call"))
    assert step.capacity == case.num_seqs
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), spec[0])
    z = _zero_rows(case)
    assert (got[z] == 0.0).all()


# The decode deals a slot's chunks evenly over its waves when the plan's largest slot holds at least
# 48 16-key chunks (12 per wave), and in units of the largest slot below that.  With at most two
# partitions per request (P = 2) the longest request's halves are the largest slots: 48 chunks at the
# boundary, 47 or 32 just below it; short requests leave some waves without chunks under either rule.
DEALING = [
    # (name, ctx, q_lens, kv, P, T)
    ("even_at_48_chunks_t16", [1536, 300, 17, 0, 5], None, "bf16", 2, 16),
    ("unit_at_47_chunks_t16", [1504, 300, 17, 0, 5], None, "bf16", 2, 16),
    ("even_at_3_tiles_verify", [1480, 1025, 2, 255], [3, 1, 2, 1], "bf16", 2, 256),
    ("unit_at_2_tiles_verify", [1024, 600, 2, 255], [3, 1, 2, 1], "bf16", 2, 256),
    ("even_fp8_at_4_tiles", [1537, 64, 1], None, "fp8", 2, 256),
    ("unit_fp8_at_2_tiles", [1000, 64, 1], None, "fp8", 2, 256),
]


@pytest.mark.parametrize("spec", DEALING, ids=[s[0] for s in DEALING])
def test_dealing_rule_boundaries(spec):
    name, ctx, ql, kv, P, T = spec
    case = W.build_case(name, ctx, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                        kv_dtype=kv, q_dtype="bf16", seed=41, q_lens=ql, device=DEV)
    announce(f"dealing {name}")
    out, step = _run(case, P, T, cu_count=256)
    assert step.capacity > case.num_seqs          # several slots per request: no shared slots
    largest = int(step.num_work[1].item())
    chunks = largest * (T // 16)
    assert (chunks >= 48) == name.startswith("even"), (largest, chunks)
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), name)
    z = _zero_rows(case)
    assert (got[z] == 0.0).all()


@pytest.mark.parametrize("name", ["tiny_fp32", "long_bf16", "verify_bf16", "fp8_kv"])
def test_full_size_workloads(name):
    announce(f"full {name}")
    case = W.make_config(name, device=DEV)
    out, step = _run(case, cu_count=256)
    got = to_f64(out)
    ref = oracle_direct(case)
    assert_close(got, ref, tolerance_kind(case), name)
    z = _zero_rows(case)
    assert (got[z] == 0.0).all()
    if name == "verify_bf16":
        assert z.sum() == 2 and z[-2:].all()     # the two rows past the last cumulative length


@pytest.mark.parametrize("which", ["p50", "p90", "max_tokens"])
def test_skewed_steps(which):
    steps = W.skewed_step_set()
    idx = W.skewed_named_steps(steps)[which]
    announce(f"skewed step {which} (#{idx}, {int(steps[idx].sum())} tokens)")
    case = W.make_config("skewed_bf16", device=DEV, step=idx)
    out, _ = _run(case, cu_count=256)
    assert_close(to_f64(out), oracle_direct(case), "bf16", f"skewed {which}")


@pytest.mark.parametrize("fused", [True, False], ids=["merge_in_call", "separate_merge"])
def test_sparse_topk_workload_with_cap_8(fused):
    announce(f"sparse top-k, cap 8, fused={fused}")
    case = W.make_sparse_case(device=DEV)
    out, step = _run(case, P=8, T=256, cu_count=256, fused=fused)
    assert (step.reduce_info[:, 1] <= 8).all()
    assert_close(to_f64(out), oracle_direct(case), "bf16", "sparse top-k")


# The merge's launch shapes: with at least 8 x CU (row, head) pairs one 64-thread workgroup per pair
# (no lane fold at head_dim 256, where a wave is exactly the 64 float4 columns); with fewer pairs than
# compute units each pair's columns over four workgroups; in between one 256-thread workgroup per pair.
MANY_PAIRS = [
    # (name, requests, Hq, Hkv, D, kv, q dtype): 300 x 8 = 2400 pairs >= 2048
    ("d256_bf16_2400pairs", 300, 8, 2, 256, "bf16", "bf16"),
    ("d256_qf32_2400pairs", 300, 8, 2, 256, "bf16", "f32"),
    ("d128_qf32_kvf32_2400pairs", 300, 8, 1, 128, "f32", "f32"),
    ("d64_fp8_qf32_2400pairs", 300, 8, 4, 64, "fp8", "f32"),
    ("d256_qf32_fewpairs", 20, 4, 1, 256, "bf16", "f32"),
    ("d128_qf32_midpairs", 100, 8, 2, 128, "bf16", "f32"),
]


@pytest.mark.parametrize("fused", [True, False], ids=["merge_in_call", "separate_merge"])
@pytest.mark.parametrize("spec", MANY_PAIRS, ids=[s[0] for s in MANY_PAIRS])
def test_merge_launch_shapes(spec, fused):
    name, n, hq, hkv, d, kv, qd = spec
    rng = np.random.default_rng(31)
    ctx = rng.integers(0, 700, size=n).tolist()
    ctx[3] = 0                                    # an empty request: its rows are zeros
    case = W.build_case(name, ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=16,
                        kv_dtype=kv, q_dtype=qd, seed=32, device=DEV)
    announce(f"merge launch shape {name} fused={fused}")
    # a large budget (planner argument only) and 16-token tiles, so that requests get several
    # partitions and each merge folds several states
    out, step = _run(case, P=256, T=16, cu_count=4096, fused=fused)
    assert int(step.num_work[0].item()) > 2 * n
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), name)
    z = _zero_rows(case)
    assert z[3] and (got[z] == 0.0).all()


@pytest.mark.parametrize("name", ["skewed_p90", "verify_bf16", "long_bf16", "small_mixed_lengths"])
def test_dispatch_order_changes_nothing(name):
    """pa_decode following the plan's dispatch order writes every slot's state where slot order
    writes it, bit for bit, and the merged rows are bitwise equal."""
    if name == "skewed_p90":
        steps = W.skewed_step_set()
        case = W.make_config("skewed_bf16", device=DEV, step=W.skewed_named_steps(steps)["p90"])
    elif name == "small_mixed_lengths":
        case = W.build_case(name, [9000, 33, 700, 0, 4096, 1], num_q_heads=8, num_kv_heads=2, head_dim=128,
                            block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=45, q_lens=[2, 1, 3, 1, 1, 1],
                            pad_rows=1, device=DEV)
    else:
        case = W.make_config(name, device=DEV)
    announce(f"dispatch order {name}")
    outs, states = [], []
    for use in (True, False):
        step = DecodeStep.for_case(case, PlanConfig(cu_count=256))
        step.use_dispatch = use
        step.workspace.fill_(0xFF)
        step.out.fill_(float("nan"))
        step.run_case(case, fused=False)
        torch.cuda.synchronize()
        outs.append(step.out.clone())
        states.append(step.workspace[:_partial_bytes(step)].clone())
        disp = step.dispatch_info.cpu().numpy()
    assert sorted(disp[:, 3].tolist()) == list(range(disp.shape[0]))       # a permutation of the slots
    assert torch.equal(states[0], states[1]), f"{name}: slot states differ with the dispatch order"
    assert torch.equal(outs[0], outs[1])
    assert_close(to_f64(outs[0]), oracle_direct(case), tolerance_kind(case), name)


def test_full_size_separate_merge_fp8():
    announce("full fp8_kv, separate merge")
    case = W.make_config("fp8_kv", device=DEV)
    out, _ = _run(case, cu_count=256, fused=False)
    assert_close(to_f64(out), oracle_direct(case), "fp8", "fp8 separate merge")


def test_merging_calls_back_to_back_reuse_the_workspace():
    # one step object (one workspace) across several different batches, pa_decode with out (the decode
    # and the merge launch in one call): nothing of a call may leak into the next
    specs = [("a", [700, 33, 1, 2000], [2, 1, 1, 3], 8, 2, 128, 16, "bf16", "bf16", 2, 256, 256),
             ("b", [90, 5000, 12, 64], [1, 3, 2, 1], 8, 2, 128, 16, "bf16", "bf16", 2, 256, 256),
             ("c", [0, 300, 4096, 7], [2, 1, 3, 1], 8, 2, 128, 16, "bf16", "bf16", 2, 256, 256)]
    cases = [_small_case(sp, seed=20 + k)[0] for k, sp in enumerate(specs)]
    step = DecodeStep.for_case(cases[0], PlanConfig(cu_count=256))
    for rep in range(2):
        for k, case in enumerate(cases):
            announce(f"back-to-back {rep} {k}")
            step.out.fill_(float("nan"))
            out = step.run_case(case, fused=True)
            torch.cuda.synchronize()
            assert_close(to_f64(out), oracle_direct(case), "bf16", f"back-to-back {rep} {k}")
            # the call with out is exactly the decode followed by pa_merge
            got = out.clone()
            sep = step.run_case(case, fused=False)
            torch.cuda.synchronize()
            assert torch.equal(got, sep), f"back-to-back {rep} {k}: pa_decode with out differs from pa_merge"


def test_workspace_switches_between_pieces_and_slots():
    """One workspace, one plan capacity (every request one slot), bf16 and fp32 caches: the bf16
    decode cuts the slots into pieces (the shared-slot region), the fp32 decode keeps slot states;
    alternating them, with and without out, must leave every call right."""
    ctx = [1, 17, 100, 3000, 5000]
    cases = [W.build_case(f"switch_{kv}", ctx, num_q_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                          kv_dtype=kv, q_dtype="f32", seed=41, device=DEV) for kv in ("bf16", "f32")]
    step = DecodeStep.for_case(cases[0], PlanConfig(cu_count=1, tile_tokens=16))
    assert step.capacity == len(ctx) and step.shares_slots("bf16", 4, 64)
    refs = [oracle_direct(c) for c in cases]
    for rep in range(2):
        for fused in (False, True):
            for case, ref in zip(cases, refs):
                announce(f"pieces/slots switch {rep} fused={fused} {case.kv_dtype}")
                step.out.fill_(float("nan"))
                out = step.run_case(case, fused=fused)
                torch.cuda.synchronize()
                assert_close(to_f64(out), ref, tolerance_kind(case), f"switch {rep} {fused} {case.kv_dtype}")


@pytest.mark.parametrize("fused", [True, False], ids=["merge_in_call", "separate_merge"])
def test_workspace_of_slot_states_only(fused):
    """A workspace that holds the slot states but not the shared-slot region is accepted; the decode
    and the merge then both keep slot states (no pieces), and agree with the oracle.  A smaller one is
    refused before any launch."""
    ctx = [1, 17, 100, 3000, 5000, 640]
    case = W.build_case("short_ws", ctx, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                        kv_dtype="bf16", q_dtype="bf16", seed=43, device=DEV)
    step = DecodeStep.for_case(case, PlanConfig(cu_count=1, tile_tokens=16))
    assert step.capacity == len(ctx)
    nbytes = _partial_bytes(step)
    assert nbytes < step.workspace.numel()
    step.workspace = step.workspace[:nbytes]
    announce(f"slot-state workspace ({nbytes} bytes) fused={fused}")
    step.out.fill_(float("nan"))
    out = step.run_case(case, fused=fused)
    torch.cuda.synchronize()
    assert_close(to_f64(out), oracle_direct(case), "bf16", "slot-state workspace")
    step.workspace = step.workspace[:nbytes - 256]
    with pytest.raises(B.PaError) as e:
        step.run_case(case, fused=fused)
    assert e.value.status == B.PA_CAPACITY


def test_single_key_row_is_the_value_row_fp32():
    case = W.make_config("tiny_fp32", device=DEV)   # request 0 has exactly one key
    out, _ = _run(case)
    blk = int(case.block_tables[0, 0].item())
    v0 = case.v_cache[blk, 0, 0, :].cpu()
    for h in range(case.num_q_heads):
        assert torch.equal(out[0, h].cpu(), v0)


def test_without_cu_equals_cu_of_ones_bitwise():
    spec = ("x", [700, 33, 1, 2000, 0, 513], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256)
    case, P, T = _small_case(spec, seed=5)
    a, _ = _run(case, P, T)
    a = a.clone()
    case.cu_query_lens = torch.arange(case.num_seqs + 1, dtype=torch.int32, device=DEV)
    b, _ = _run(case, P, T)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_slot_order_does_not_change_the_output():
    spec = ("x", [3000, 33, 1, 2000, 900], [2, 1, 1, 3, 1], 8, 2, 128, 16, "bf16", "bf16", 1, 256, 256)
    case, P, T = _small_case(spec, seed=6)
    ref, step = _run(case, P, T)
    ref = ref.clone()
    work = step.work_info.cpu().numpy()
    red = step.reduce_info.cpu().numpy()
    nw = int(step.num_work[0].item())
    # reverse the order of the requests' slot blocks; each request keeps its own slots in order
    new_work = np.tile(np.array([-1, 0, 0, 0], np.int32), (work.shape[0], 1))
    new_red = red.copy()
    pos = 0
    for b in reversed(range(case.num_seqs)):
        first, parts = red[b]
        new_work[pos:pos + parts] = work[first:first + parts]
        new_red[b] = (pos, parts)
        pos += parts
    assert pos == nw
    step.work_info.copy_(torch.from_numpy(new_work))
    step.reduce_info.copy_(torch.from_numpy(new_red))
    step.use_dispatch = False         # the dispatch order belongs to the plan pa_plan wrote, not this one
    step.out.fill_(float("nan"))
    out = step.run_case(case, replan=False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_output_guard_bands_untouched():
    spec = ("x", [400, 30], [2, 1], 8, 2, 128, 16, "bf16", "bf16", 2, 256, 256)
    case, P, T = _small_case(spec, seed=7)
    step = DecodeStep.for_case(case, PlanConfig(cu_count=256, max_partitions=P, tile_tokens=T))
    n = step.out.numel()
    big = torch.full((n + 2048,), -3.0, dtype=torch.bfloat16, device=DEV)
    step.out = big[1024:1024 + n].view(step.out.shape)
    step.run_case(case)
    torch.cuda.synchronize()
    assert (big[:1024] == -3.0).all() and (big[1024 + n:] == -3.0).all()
    assert_close(to_f64(step.out), oracle_direct(case), "bf16", "guard")


@pytest.mark.parametrize("P,T", [(1, 256), (2, 64), (8, 16), (256, 16), (256, 512)])
def test_split_count_invariance(P, T):
    spec = ("x", [6000, 2500, 40], [1, 2, 1], 8, 1, 128, 16, "bf16", "bf16", 0, P, T)
    case, _, _ = _small_case(spec, seed=8)
    announce(f"split invariance P={P} T={T}")
    out, step = _run(case, P, T)
    assert_close(to_f64(out), oracle_direct(case), "bf16", f"P={P} T={T}")


def test_repeated_calls_are_deterministic():
    spec = ("x", [3000, 700], [3, 1], 6, 1, 256, 16, "bf16", "bf16", 1, 256, 256)
    case, P, T = _small_case(spec, seed=9)
    a, _ = _run(case, P, T)
    a = a.clone()
    b, _ = _run(case, P, T)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
