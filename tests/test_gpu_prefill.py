"""Prefill rows and the decode-first split of mixed batches, against the fp64 oracle.

The decode-first split (opengfx1030/vllm-rdna PR #29, Change 2): requests are ordered decodes first;
the leading requests with at most 1 + k query tokens take the split-KV decode, the rest a prefill
kernel on the rebased remainder, both writing slices of the layer output.  Token i of a request with
L tokens and S keys sees S - (L - 1 - i) keys (Change 1), the window applying per token.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import PlanConfig, mixed_step
from _util import announce, assert_close, oracle_direct, to_f64, tolerance_kind
from test_gpu_decode import _zero_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (name, ctx, q_lens, Hq, Hkv, D, bs, kv, q, pad, window)
PREFILL = [
    ("bf16_d128_prompts", [100, 300, 64, 9], [100, 300, 64, 9], 16, 2, 128, 16, "bf16", "bf16", 2, 0),
    ("bf16_d128_chunk_behind_prefix", [1300, 5000], [200, 77], 16, 2, 128, 16, "bf16", "bf16", 0, 0),
    ("bf16_d256_g6", [100, 700], [100, 33], 12, 2, 256, 16, "bf16", "bf16", 1, 0),
    ("bf16_d64_g4_bs64", [520, 70], [250, 70], 8, 2, 64, 64, "bf16", "bf16", 0, 0),
    ("fp8_d128", [400, 2100], [150, 100], 16, 2, 128, 16, "fp8", "bf16", 0, 0),
    ("bf16_window50", [300, 1000], [120, 64], 16, 2, 128, 16, "bf16", "bf16", 1, 50),
    ("fp8_d256_window32", [900], [96], 12, 2, 256, 16, "fp8", "bf16", 0, 32),
    ("qf32_tokens_without_keys", [10, 40], [30, 40], 8, 1, 128, 16, "bf16", "f32", 2, 0),
    # one query head per kv head: 64 tokens per block
    ("bf16_g1_prompts", [333, 90], [200, 90], 4, 4, 128, 16, "bf16", "bf16", 1, 0),
    # 32 query heads per kv head: 2 tokens per 64-row block, with a window
    ("bf16_g32_window", [700, 129], [41, 7], 32, 1, 64, 16, "bf16", "bf16", 0, 100),
    # the direct-load path at head_dim 256: fp32 queries under a window (chunks wholly before a row's
    # window), and slots of fewer chunks than the ring holds (one to two 32-key chunks, ragged)
    ("bf16_d256_qf32_window40", [500, 45], [200, 45], 12, 2, 256, 16, "bf16", "f32", 1, 40),
    ("bf16_d256_short_slots", [20, 60, 3, 33], [20, 10, 3, 1], 8, 2, 256, 16, "bf16", "bf16", 0, 0),
]


def _prefill(case, out, *, requests=slice(None), cu_count=256, split=True):
    """pa_prefill over the given requests (a slice of the batch): the split form with its own workspace,
    or the one-launch form."""
    bt, ctx = case.block_tables[requests], case.context_lens[requests]
    n = int(ctx.shape[0])
    cu = case.cu_query_lens[requests.start or 0:(requests.start or 0) + n + 1]
    ws = None
    if split:
        nbytes = B.pa_prefill_workspace_bytes(case.num_rows, n, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                              cu_count)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)     # no initial contents needed
    B.pa_prefill(case.q, case.k_cache, case.v_cache, case.kv_dtype, bt, ctx, cu, out, ws, scale=case.scale,
                 cu_count=cu_count, k_scale=case.k_scale, v_scale=case.v_scale, sliding_window=case.window)


def _case(spec, seed):
    name, ctx, ql, Hq, Hkv, D, bs, kv, qd, pad, win = spec
    c = W.build_case(name, ctx, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs, kv_dtype=kv,
                     q_dtype=qd, seed=seed, q_lens=ql, pad_rows=pad, device=DEV)
    c.window = win
    return c


@pytest.mark.parametrize("split", [True, False], ids=["split", "one_launch"])
@pytest.mark.parametrize("spec", PREFILL, ids=[p[0] for p in PREFILL])
def test_prefill_matches_oracle(spec, split):
    case = _case(spec, seed=41)
    announce(f"prefill {spec[0]} split={split}")
    out = torch.full_like(case.q, float("nan"))
    _prefill(case, out, split=split)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), spec[0])
    assert (got[_zero_rows(case)] == 0.0).all()


@pytest.mark.parametrize("split", [True, False], ids=["split", "one_launch"])
def test_prefill_leaves_rows_before_its_first_request_alone(split):
    case = _case(PREFILL[0], seed=42)
    # treat requests 1.. as the prefill part: rows [cu[1], R) are written, rows before stay poisoned
    out = torch.full_like(case.q, float("nan"))
    _prefill(case, out, requests=slice(1, None), split=split)
    torch.cuda.synchronize()
    c1 = int(case.cu_query_lens[1].item())
    got = to_f64(out)
    assert np.isnan(got[:c1]).all()
    assert_close(got[c1:], oracle_direct(case)[c1:], "bf16", "prefill part")


# prompt chunks behind long prefixes: several blocks per request, each block's keys split over several
# workgroups by the plan; a small budget (cu_count) makes slots of many tiles, a large one many slots
LONG_PREFIX = [
    ("d256_g6_chunk_behind_3000", [3096], [96], 12, 2, 256, 16, "bf16", "bf16", 1, 0, 256),
    ("d128_g8_two_chunks", [4100, 2600], [200, 130], 16, 2, 128, 16, "bf16", "bf16", 0, 0, 256),
    ("d128_fp8_small_budget", [5000, 64], [150, 64], 16, 2, 128, 64, "fp8", "bf16", 2, 0, 8),
    ("d64_g4_window", [6000], [300], 8, 2, 64, 16, "bf16", "bf16", 0, 500, 256),
    ("d256_fp8_window", [3000, 700], [70, 40], 12, 2, 256, 16, "fp8", "bf16", 0, 1000, 64),
    # more blocks than the budget's slots: every block one slot
    ("d128_g16_many_blocks", [3000, 2000], [1100, 900], 16, 1, 128, 16, "bf16", "bf16", 0, 0, 64),
    # a request whose query outnumbers its keys (precondition edge): early tokens see nothing
    ("d128_tokens_without_keys", [40, 900], [100, 50], 8, 2, 128, 16, "bf16", "f32", 1, 0, 256),
    # pages of 64 and 128 tokens on the direct-load path (both halves of a 32-key chunk in one page)
    ("d256_bs64_bf16", [2500, 900], [120, 60], 12, 2, 256, 64, "bf16", "bf16", 1, 0, 256),
    ("d128_bs128_bf16_window", [3000, 1000], [200, 33], 16, 2, 128, 128, "bf16", "bf16", 0, 300, 64),
    ("d256_bs128_bf16_qf32", [2100, 700], [90, 40], 12, 2, 256, 128, "bf16", "f32", 0, 0, 16),
]


@pytest.mark.parametrize("spec", LONG_PREFIX, ids=[p[0] for p in LONG_PREFIX])
def test_prefill_chunks_behind_long_prefixes(spec):
    case = _case(spec[:11], seed=44)
    cu_count = spec[11]
    announce(f"prefill behind a prefix {spec[0]}")
    out = torch.full_like(case.q, float("nan"))
    _prefill(case, out, cu_count=cu_count)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), spec[0])
    assert (got[_zero_rows(case)] == 0.0).all()


def test_prefill_chunk_of_the_bench_at_full_size():
    """The 512-token chunk behind a 16384-token prefix (Hq 12 / Hkv 2, D 256) that bench.py times:
    sampled rows against the oracle, computed one by one."""
    case = W.make_prefill_chunk_case(device=DEV)
    announce("prefill chunk 512 behind 16384, full size")
    out = torch.full_like(case.q, float("nan"))
    _prefill(case, out, cu_count=B.pa_device_cu_count(0))
    torch.cuda.synchronize()
    # block edges (21 tokens per block at G = 6, head_dim 256) and the chunk's ends, every head of each row
    rows = np.repeat(np.array([0, 1, 20, 21, 22, 41, 42, 251, 252, 400, 503, 504, 510, 511]), case.num_q_heads)
    heads = np.tile(np.arange(case.num_q_heads), rows.shape[0] // case.num_q_heads)
    h = case.host()
    ref = oracle.attention_rows(h["q"], case.q_dtype, h["k_cache"], h["v_cache"], case.kv_dtype, h["block_tables"],
                                h["context_lens"], h["cu_query_lens"], case.scale, rows, heads, case.k_scale,
                                case.v_scale)
    got = to_f64(out)
    assert_close(got[rows, heads], ref, "bf16", "prefill chunk rows")
    assert np.isfinite(got).all()


# (name, ctx, q_lens, Hq, Hkv, D, bs, kv, q, pad, window, threshold)
MIXED = [
    # 7 decodes + a new 100-token prompt, TP=2 shapes (H 12/2, D 256) as on the vllm-rdna page
    ("seven_decodes_and_a_prompt", [2000] * 7 + [100], [1] * 7 + [100], 12, 2, 256, 16, "bf16", "bf16", 1, 0, 1),
    # MTP verify rows (1 + 2 speculative tokens), then two prefill chunks
    ("verify_then_chunks", [3000, 900, 17, 1500, 260], [3, 3, 3, 200, 60], 16, 2, 128, 16, "bf16", "bf16", 2, 0, 3),
    ("fp8_mixed_window", [5000, 40, 700], [1, 1, 300], 16, 2, 128, 16, "fp8", "bf16", 0, 64, 1),
    ("all_decode", [700, 33, 1], [1, 1, 1], 16, 2, 128, 16, "bf16", "bf16", 1, 0, 1),
    ("all_prefill", [700, 333], [70, 33], 16, 2, 128, 16, "bf16", "bf16", 1, 0, 1),
    # short prompts after decodes: in one call the prompts' query blocks are cut to the decode's
    # 16 query rows per workgroup and share its launch
    ("short_prompts_d128", [900, 4000, 50, 30], [1, 1, 20, 9], 16, 2, 128, 16, "bf16", "bf16", 1, 0, 1),
    ("short_prompts_fp8_window", [900, 4000, 50, 30], [1, 1, 20, 9], 8, 1, 64, 16, "fp8", "bf16", 0, 16, 1),
]


@pytest.mark.parametrize("mode", ["one_stream", "two_streams", "one_call"])
@pytest.mark.parametrize("spec", MIXED, ids=[m[0] for m in MIXED])
def test_mixed_batch_decode_first_split(spec, mode):
    *base, threshold = spec
    case = _case(tuple(base), seed=43)
    announce(f"mixed {spec[0]} threshold {threshold} {mode}")
    out = mixed_step(case, threshold, PlanConfig(cu_count=256), concurrent=(mode == "two_streams"),
                     one_call=(mode == "one_call"))
    torch.cuda.synchronize()
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), spec[0])
    assert (got[_zero_rows(case)] == 0.0).all()


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
def test_seven_decodes_at_16k_and_a_prompt_full_size(one_call):
    """The vllm-rdna table's second scenario at its sizes: 7 decodes at 16384 tokens and a new
    100-token prompt, TP=2 per rank (H 12/2), D 256."""
    case = W.build_case("mixed_16k", [16384] * 7 + [100], num_q_heads=12, num_kv_heads=2, head_dim=256,
                        block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=44, q_lens=[1] * 7 + [100],
                        device=DEV)
    announce(f"mixed 7 x 16k + 100-token prompt one_call={one_call}")
    out = mixed_step(case, 1, PlanConfig(cu_count=256), one_call=one_call)
    torch.cuda.synchronize()
    assert_close(to_f64(out), oracle_direct(case), "bf16", "mixed full size")


def test_one_call_with_more_decodes_than_plan_in_place():
    """300 single-token decodes and two prompts: the decode part is beyond the in-place plan's 256
    requests, so pa_attention_mixed plans with the plan kernel and launches the parts apart."""
    rng = np.random.default_rng(45)
    ctx = list(rng.integers(1, 600, size=300)) + [200, 90]
    ql = [1] * 300 + [40, 90]
    case = W.build_case("many_decodes", ctx, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                        kv_dtype="bf16", q_dtype="bf16", seed=46, q_lens=ql, pad_rows=2, device=DEV)
    announce("mixed one call, 300 decodes + 2 prompts")
    out = mixed_step(case, 1, PlanConfig(cu_count=256), one_call=True)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert_close(got, oracle_direct(case), "bf16", "many decodes")
    assert (got[_zero_rows(case)] == 0.0).all()
