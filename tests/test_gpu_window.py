"""Per-token sliding window on the GPU: plan and decode against the oracle.

A query token with n visible keys sees only [max(0, n - W), n) (opengfx1030/vllm-rdna PR #29, Change 1:
the sliding window applies per token; its Test Plan runs windows 0, 1, 3 and 50).  The plan must
cover exactly the keys the kernel reads under the window (ROCm/ATOM PR #2366 review, window logic),
so pa_plan's buffers are compared bit for bit with the oracle's windowed plan, through pa_plan and
through pa_attention's in-place plan.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import DecodeStep, PlanConfig
from _util import announce, assert_close, oracle_direct, oracle_plan_of, to_f64, tolerance_kind
from test_gpu_decode import _partial_bytes, _zero_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (name, ctx, q_lens, Hq, Hkv, D, bs, kv, q, pad, P, T, window)
CASES = [
    ("bf16_g8_w1", [700, 33, 1, 2000, 256, 257], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256, 1),
    ("bf16_g8_w3", [700, 33, 1, 2000, 256, 257], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256, 3),
    ("bf16_g8_w50", [700, 33, 1, 2000, 256, 257], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256, 50),
    ("bf16_g8_w700", [700, 33, 1, 2000, 256, 257], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256, 700),
    ("bf16_d64_verify_w3", [37, 5, 64, 1290], [3, 1, 2, 4], 8, 2, 64, 64, "bf16", "bf16", 2, 256, 256, 3),
    ("bf16_d64_verify_w50", [37, 5, 64, 1290], [3, 1, 2, 4], 8, 2, 64, 64, "bf16", "bf16", 2, 256, 256, 50),
    ("bf16_d256_verify_w1000", [1500, 900, 2, 700], [3, 3, 1, 1], 6, 1, 256, 16, "bf16", "bf16", 2, 256, 256, 1000),
    ("bf16_64rows_w257", [3000, 17, 600], [4, 4, 1], 16, 1, 128, 16, "bf16", "bf16", 1, 64, 64, 257),
    ("bf16_zero_len_w3", [0, 300, 0, 2, 40], [2, 2, 1, 3, 1], 4, 2, 128, 16, "bf16", "bf16", 1, 8, 16, 3),
    ("bf16_long_w4096", [20000, 5000, 4100], None, 16, 2, 128, 16, "bf16", "bf16", 0, 256, 256, 4096),
    ("fp8_d128_w50", [900, 1, 4000, 77], None, 16, 2, 128, 16, "fp8", "bf16", 0, 256, 256, 50),
    ("fp8_verify_w255", [3000, 45], [2, 3], 12, 4, 64, 64, "fp8", "bf16", 1, 256, 64, 255),
    ("f32_d64_w1", [1, 17, 100, 300, 0], None, 4, 1, 64, 16, "f32", "f32", 2, 256, 256, 1),
    ("f32_d128_verify_w50", [500, 31, 2], [3, 2, 2], 8, 2, 128, 64, "f32", "f32", 1, 8, 64, 50),
]


def _case(spec, seed):
    name, ctx, ql, Hq, Hkv, D, bs, kv, qd, pad, P, T, win = spec
    c = W.build_case(name, ctx, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs, kv_dtype=kv,
                     q_dtype=qd, seed=seed, q_lens=ql, pad_rows=pad, device=DEV)
    c.window = win
    return c, PlanConfig(cu_count=256, max_partitions=P, tile_tokens=T)


def _check_plan(step, case, cfg):
    ow, orr, on, olarge = oracle_plan_of(case, cfg.cu_count, cfg.budget_mult, cfg.max_partitions,
                                         cfg.tile_tokens, step.capacity, with_largest=True)
    assert step.num_work.cpu().numpy().tolist() == [on, olarge]
    assert np.array_equal(step.reduce_info.cpu().numpy(), orr)
    assert np.array_equal(step.work_info.cpu().numpy(), ow)


@pytest.mark.parametrize("mode", ["separate", "merge_in_call", "attention"])
@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_window_cases_match_oracle(spec, mode):
    case, cfg = _case(spec, seed=21)
    announce(f"window {spec[0]} {mode}")
    step = DecodeStep.for_case(case, cfg)
    step.out.fill_(float("nan"))
    step.workspace[:_partial_bytes(step)].fill_(0xFF)
    step.work_info.fill_(0x5A5A5A5A)
    out = step.run_case(case, fused=mode == "merge_in_call", whole=mode == "attention")
    torch.cuda.synchronize()
    _check_plan(step, case, cfg)
    got = to_f64(out)
    assert_close(got, oracle_direct(case), tolerance_kind(case), f"{spec[0]} {mode}")
    z = _zero_rows(case)
    assert (got[z] == 0.0).all()


def test_window_at_least_the_context_is_bitwise_the_plain_path():
    spec = ("bf16_d64_verify", [37, 5, 64, 1290], [3, 1, 2, 4], 8, 2, 64, 64, "bf16", "bf16", 2, 256, 256, 0)
    case, cfg = _case(spec, seed=22)
    plain = DecodeStep.for_case(case, cfg).run_case(case, fused=False).clone()
    case.window = 1290
    wide = DecodeStep.for_case(case, cfg).run_case(case, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(plain, wide)


@pytest.mark.parametrize("seed", range(16))
def test_window_plan_fuzz(seed):
    rng = np.random.default_rng(4100 + seed)
    Bn = int(rng.choice([1, 5, 32, 64, 65, 200, 256, 300, 1000]))
    hkv = int(rng.choice([1, 2, 8]))
    P = int(rng.choice([1, 8, 256]))
    T = int(rng.choice([16, 64, 256]))
    win = int(rng.choice([1, 3, 50, 257, 4096, 100000]))
    ctx = np.where(rng.random(Bn) < 0.25, 0, rng.integers(1, 60000, size=Bn)).astype(np.int32)
    ql = rng.integers(0, 5, size=Bn)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    announce(f"window plan fuzz seed {seed} B={Bn} W={win}")
    c = torch.as_tensor(ctx, device=DEV)
    cut = torch.as_tensor(cu, device=DEV)
    cap = B.pa_plan_capacity(Bn, hkv, 256, 2, P) + int(rng.integers(0, 3)) * 5
    work = torch.full((cap, 4), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    red = torch.full((Bn, 2), -7, dtype=torch.int32, device=DEV)
    nw = torch.full((2,), -9, dtype=torch.int32, device=DEV)
    B.pa_plan(c, hkv, cu_count=256, max_partitions=P, tile_tokens=T, capacity=cap, work_info=work,
              reduce_info=red, num_work=nw, cu_query_lens=cut, sliding_window=win)
    torch.cuda.synchronize()
    ow, orr, on, olarge = oracle.plan(ctx, hkv, 256, 2, P, T, cap, with_largest=True, cu_query_lens=cu,
                                      window=win)
    assert nw.cpu().numpy().tolist() == [on, olarge]
    assert np.array_equal(red.cpu().numpy(), orr)
    assert np.array_equal(work.cpu().numpy(), ow)


@pytest.mark.parametrize("seed", range(6))
def test_window_plan_in_place_fuzz(seed):
    """pa_attention's in-place plan under a window, on a one-page cache (every table entry names
    page 0, so any length stays in bounds); the output must equal the three-call path bitwise."""
    rng = np.random.default_rng(4200 + seed)
    Bn = int(rng.choice([3, 40, 64, 65, 256]))
    win = int(rng.choice([1, 50, 700, 5000]))
    T = int(rng.choice([16, 256]))
    ctx = np.where(rng.random(Bn) < 0.2, 0, rng.integers(1, 30000, size=Bn)).astype(np.int32)
    ql = rng.integers(1, 4, size=Bn)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    R = int(cu[-1]) + 1
    announce(f"window in-place plan fuzz seed {seed} B={Bn} W={win}")
    g = torch.Generator(device=DEV).manual_seed(seed)
    k = torch.randn((2, 2, 16, 64), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((2, 2, 16, 64), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((R, 4, 64), generator=g, device=DEV).to(torch.bfloat16)
    bt = torch.zeros((Bn, max(1, -(-int(ctx.max()) // 16))), dtype=torch.int32, device=DEV)
    lens = torch.as_tensor(ctx, device=DEV)
    cut = torch.as_tensor(cu, device=DEV)
    cfg = PlanConfig(cu_count=256, tile_tokens=T)
    mk = lambda: DecodeStep(num_seqs=Bn, num_rows=R, num_q_heads=4, num_kv_heads=2, head_dim=64,
                            max_q_len=3, out_dtype=torch.bfloat16, device=DEV, plan=cfg)
    three, whole = mk(), mk()
    for s in (three, whole):
        s.out.fill_(float("nan"))
        s.work_info.fill_(0x5A5A5A5A)
    three.plan(lens, cu_query_lens=cut, sliding_window=win)
    three.decode(q, k, v, "bf16", bt, lens, scale=0.125, cu_query_lens=cut, sliding_window=win)
    three.merge(cut)
    whole.attention(q, k, v, "bf16", bt, lens, scale=0.125, cu_query_lens=cut, sliding_window=win)
    torch.cuda.synchronize()
    assert torch.equal(whole.out, three.out)
    for a, b in ((whole.work_info, three.work_info), (whole.reduce_info, three.reduce_info),
                 (whole.num_work, three.num_work)):
        assert torch.equal(a, b)
    ow, orr, on, olarge = oracle.plan(ctx, 2, 256, 2, 256, T, whole.capacity, with_largest=True,
                                      cu_query_lens=cu, window=win)
    assert np.array_equal(whole.work_info.cpu().numpy(), ow)


def test_skewed_max_step_with_window():
    steps = W.skewed_step_set()
    idx = W.skewed_named_steps(steps)["max_tokens"]
    announce(f"window 8192 on skewed step #{idx}")
    case = W.make_config("skewed_bf16", device=DEV, step=idx)
    case.window = 8192
    cfg = PlanConfig(cu_count=256)
    step = DecodeStep.for_case(case, cfg)
    out = step.run_case(case, whole=True)
    torch.cuda.synchronize()
    _check_plan(step, case, cfg)
    assert_close(to_f64(out), oracle_direct(case), "bf16", "skewed max, window 8192")
