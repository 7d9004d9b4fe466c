"""pa_attention -- plan, decode and merge in one call, the decode planning in place -- against the
three-call path (bitwise) and the fp64 oracle.

The in-place plan must be the planner's plan bit for bit (ROCm/ATOM PR #2366 section 1, review items 2
and 3): every workgroup evaluates the same integer rule, and the stored buffers are compared with the
oracle's plan on whole buffers, sentinels and the largest-slot word included.  Batches above the
in-place limit, and fp32 caches, take the three-launch route and must give the same results.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import DecodeStep, PlanConfig
from _util import announce, assert_close, oracle_direct, to_f64, tolerance_kind
from test_gpu_decode import DEALING, SMALL, _partial_bytes, _small_case, _zero_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _poison(step):
    step.out.fill_(float("nan"))
    step.workspace[:_partial_bytes(step)].fill_(0xFF)
    step.work_info.fill_(0x5A5A5A5A)
    step.reduce_info.fill_(-7)
    step.num_work.fill_(-9)


def _oracle_plan(ctx, hkv, cfg, capacity):
    return oracle.plan(np.asarray(ctx), hkv, cfg.cu_count, cfg.budget_mult, cfg.max_partitions,
                       cfg.tile_tokens, capacity, with_largest=True)


def _check_plan(step, ctx, hkv, cfg):
    ow, orr, on, olarge = _oracle_plan(ctx, hkv, cfg, step.capacity)
    assert step.num_work.cpu().numpy().tolist() == [on, olarge]
    assert np.array_equal(step.reduce_info.cpu().numpy(), orr)
    assert np.array_equal(step.work_info.cpu().numpy(), ow)


def _poison_pieces(step):
    """NaN pattern in the shared-slot region too (it follows the slot partials)."""
    step.workspace[_partial_bytes(step):].fill_(0xFF)


def _both_routes(case, cfg):
    three = DecodeStep.for_case(case, cfg)
    _poison(three)
    _poison_pieces(three)
    ref = three.run_case(case, fused=False).clone()
    whole = DecodeStep.for_case(case, cfg)
    _poison(whole)
    _poison_pieces(whole)
    got = whole.run_case(case, whole=True)
    torch.cuda.synchronize()
    return got, ref, whole


def _assert_same_as_three(got, ref, what=""):
    """Bit for bit: with shared slots both routes cut the slots into the same pieces."""
    assert torch.equal(got, ref), f"{what}: pa_attention differs from pa_plan + pa_decode + pa_merge"


@pytest.mark.parametrize("spec", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(spec):
    case, P, T = _small_case(spec, seed=12)
    announce(f"attention {spec[0]}")
    cfg = PlanConfig(cu_count=256, max_partitions=P, tile_tokens=T)
    got, ref, step = _both_routes(case, cfg)
    _assert_same_as_three(got, ref, spec[0])
    _check_plan(step, case.context_lens.cpu().numpy(), case.num_kv_heads, cfg)
    g = to_f64(got)
    assert_close(g, oracle_direct(case), tolerance_kind(case), spec[0])
    assert (g[_zero_rows(case)] == 0.0).all()


@pytest.mark.parametrize("spec", DEALING, ids=[s[0] for s in DEALING])
def test_dealing_rule_boundaries(spec):
    """Both sides of the decode's even/unit dealing boundary: the in-place plan's largest slot picks
    the same dealing as the stored plan's, so the two routes agree bit for bit."""
    name, ctx, ql, kv, P, T = spec
    case = W.build_case(name, ctx, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                        kv_dtype=kv, q_dtype="bf16", seed=43, q_lens=ql, device=DEV)
    announce(f"attention dealing {name}")
    cfg = PlanConfig(cu_count=256, max_partitions=P, tile_tokens=T)
    got, ref, step = _both_routes(case, cfg)
    _assert_same_as_three(got, ref, name)
    _check_plan(step, ctx, 2, cfg)
    assert_close(to_f64(got), oracle_direct(case), tolerance_kind(case), name)


@pytest.mark.parametrize("name", ["verify_bf16", "fp8_kv", "long_bf16"])
def test_full_size_workloads(name):
    announce(f"attention full {name}")
    case = W.make_config(name, device=DEV)
    cfg = PlanConfig(cu_count=256)
    got, ref, step = _both_routes(case, cfg)
    _assert_same_as_three(got, ref, name)
    _check_plan(step, case.context_lens.cpu().numpy(), case.num_kv_heads, cfg)
    assert_close(to_f64(got), oracle_direct(case), tolerance_kind(case), name)


def test_skewed_max_step():
    steps = W.skewed_step_set()
    idx = W.skewed_named_steps(steps)["max_tokens"]
    announce(f"attention skewed max step #{idx}")
    case = W.make_config("skewed_bf16", device=DEV, step=idx)
    cfg = PlanConfig(cu_count=256)
    got, ref, step = _both_routes(case, cfg)
    _assert_same_as_three(got, ref, "skewed max")
    _check_plan(step, steps[idx], 2, cfg)
    assert_close(to_f64(got), oracle_direct(case), "bf16", "skewed max")


SHARED = [
    # (name, context lens, query lens, Hq, Hkv, D, page, kv, cu_count, tile[, q dtype]): each batch
    # has at least 2 x cu_count / Hkv requests, so the capacity is the batch and the slots are shared
    # up to 64 requests (the plan in one wave); empty requests leave spare slots, so the long
    # requests get several slots, each cut into the same number of pieces (some of them empty)
    ("wave_plan_bf16", [0] * 6 + [16, 600, 33, 5000, 1, 9000, 250, 20000] * 4 + [77, 3, 1500, 40, 0, 0],
     None, 8, 1, 128, 16, "bf16", 8, 256),
    # more than 64 requests (the plan across waves), fp8, log-normal lengths
    ("threads_plan_fp8", "lognormal200", None, 16, 2, 128, 16, "fp8", 100, 256),
    # verify rows (G x L = 8 rows), head_dim 64, 16-token tiles
    ("verify_d64_tiles16", "lognormal70", "q2", 4, 1, 64, 16, "bf16", 16, 16),
    # one request, one slot (capacity 1): its pieces are the only parallelism
    ("single_request", [100000], None, 4, 2, 128, 64, "bf16", 1, 256),
    # mostly empty requests: the spare slots go to five long ones, ~9 slots each, then pieces
    ("mostly_empty", [0] * 45 + [30000, 7000, 65000, 12000, 300], None, 8, 1, 128, 16, "fp8", 8, 256),
    # two 16-row blocks (G x L = 32): the four-wave form with two column blocks
    ("two_row_blocks", "lognormal90", "q2", 16, 1, 128, 16, "bf16", 32, 256),
    # fp32 cache and queries: the vector kernel takes its piece from the same rule
    ("fp32_cache", "lognormal80", None, 8, 2, 64, 16, "f32", 64, 64, "f32"),
]


def _shared_case(spec, seed):
    name, ctx, ql, hq, hkv, d, bs, kv, cu_count, T = spec[:10]
    qd = spec[10] if len(spec) > 10 else "bf16"
    rng = np.random.default_rng(seed)
    if isinstance(ctx, str):
        n = int(ctx[len("lognormal"):])
        ctx = np.clip(np.rint(np.exp(rng.normal(6.5, 1.4, size=n))), 1, 30000).astype(int)
        ctx[rng.random(n) < 0.1] = 0
        ctx = ctx.tolist()
    q_lens = None if ql is None else rng.integers(1, int(ql[1:]) + 1, size=len(ctx)).tolist()
    case = W.build_case(name, ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                        kv_dtype=kv, q_dtype=qd, seed=seed, q_lens=q_lens, pad_rows=1, device=DEV)
    return case, PlanConfig(cu_count=cu_count, tile_tokens=T)


@pytest.mark.parametrize("spec", SHARED, ids=[s[0] for s in SHARED])
def test_shared_slots_match_oracle(spec):
    """Every request one slot: the decode cuts the slots into pieces streamed by workgroups of their
    own and the merge folds the pieces per request, in pa_attention and in pa_plan + pa_decode +
    pa_merge alike (bit for bit).  Output against the oracle, the stored plan against the oracle's
    plan, exact zeros where rows have no keys."""
    case, cfg = _shared_case(spec, seed=31)
    announce(f"shared slots {spec[0]}")
    got, ref, step = _both_routes(case, cfg)
    assert step.shares_slots(case.kv_dtype, case.num_q_heads, case.head_dim)
    _check_plan(step, case.context_lens.cpu().numpy(), case.num_kv_heads, cfg)
    g = to_f64(got)
    assert_close(g, oracle_direct(case), tolerance_kind(case), spec[0])
    assert (g[_zero_rows(case)] == 0.0).all()
    _assert_same_as_three(got, ref, spec[0])


def _one_page_case(ctx, hkv, seed):
    """Every block-table entry names page 0 of a tiny cache: any length stays in bounds, so the
    plan can be exercised at any size; the output is checked against the three-call path only."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    Bn, hq, d, bs = len(ctx), 2 * hkv, 64, 16
    k = torch.randn((2, hkv, bs, d), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((2, hkv, bs, d), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((Bn, hq, d), generator=g, device=DEV).to(torch.bfloat16)
    mb = max(1, -(-int(max(ctx, default=1)) // bs))
    bt = torch.zeros((Bn, mb), dtype=torch.int32, device=DEV)
    lens = torch.as_tensor(np.asarray(ctx, dtype=np.int32), device=DEV)
    return q, k, v, bt, lens


@pytest.mark.parametrize("seed", range(12))
def test_plan_in_place_fuzz(seed):
    rng = np.random.default_rng(900 + seed)
    Bn = int(rng.choice([1, 2, 31, 63, 64, 65, 128, 200, 255, 256, 257, 300]))
    hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([1, 8, 256]))
    T = int(rng.choice([16, 64, 256]))
    mult = int(rng.choice([1, 2, 3]))
    kind = seed % 3
    if kind == 0:
        ctx = rng.integers(0, 40000, size=Bn)
    elif kind == 1:
        ctx = np.where(rng.random(Bn) < 0.4, 0, rng.integers(1, 3000, size=Bn))
    else:
        ctx = np.clip(np.rint(np.exp(rng.normal(7.0, 1.5, size=Bn))), 0, 60000).astype(np.int64)
    announce(f"plan in place fuzz seed {seed} B={Bn} Hkv={hkv} P={P} T={T} x{mult}")
    q, k, v, bt, lens = _one_page_case(ctx, hkv, seed)
    cfg = PlanConfig(cu_count=256, budget_mult=mult, max_partitions=P, tile_tokens=T)
    mk = lambda: DecodeStep(num_seqs=Bn, num_rows=Bn, num_q_heads=2 * hkv, num_kv_heads=hkv, head_dim=64,
                            max_q_len=1, out_dtype=torch.bfloat16, device=DEV, plan=cfg)
    three, whole = mk(), mk()
    for s in (three, whole):
        _poison(s)
    three.plan(lens)
    three.decode(q, k, v, "bf16", bt, lens, scale=0.125)
    three.merge()
    whole.attention(q, k, v, "bf16", bt, lens, scale=0.125)
    torch.cuda.synchronize()
    _check_plan(whole, ctx, hkv, cfg)
    _assert_same_as_three(whole.out, three.out, f"fuzz seed {seed}")


def test_all_empty_and_empty_batch():
    for ctx in ([0, 0, 0], []):
        announce(f"attention empty {ctx}")
        q, k, v, bt, lens = _one_page_case(ctx or [0], 1, 0)
        n = len(ctx)
        q, bt, lens = q[:n], bt[:n], lens[:n]
        step = DecodeStep(num_seqs=n, num_rows=max(n, 2), num_q_heads=2, num_kv_heads=1, head_dim=64,
                          max_q_len=1, out_dtype=torch.bfloat16, device=DEV, plan=PlanConfig(cu_count=256))
        _poison(step)
        qq = torch.zeros((max(n, 2), 2, 64), dtype=torch.bfloat16, device=DEV)
        step.attention(qq, k, v, "bf16", bt, lens, scale=0.125)
        torch.cuda.synchronize()
        assert (step.out == 0).all()
        _check_plan(step, ctx, 1, PlanConfig(cu_count=256))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_batch_beyond_plan_in_place(kv):
    """600 requests: past the in-place plan's limit (pa_attention then launches the plan kernel) and
    past the shared-slot table, so every request is one slot streamed by the eight-wave form.
    Lengths are log-normal with zeros and verify rows; both routes against the oracle."""
    rng = np.random.default_rng(31)
    Bn = 600
    ctx = np.clip(np.rint(np.exp(rng.normal(5.5, 1.2, size=Bn))), 1, 6000).astype(np.int64)
    ctx[rng.random(Bn) < 0.05] = 0
    ql = rng.integers(1, 3, size=Bn)
    ctx = np.maximum(ctx, np.where(ctx > 0, ql, 0))
    announce(f"attention {Bn} requests {kv}")
    case = W.build_case(f"beyond_in_place_{kv}", ctx.tolist(), num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=16, kv_dtype=kv, q_dtype="bf16", seed=77, q_lens=ql.tolist(), pad_rows=3,
                        device=DEV)
    cfg = PlanConfig(cu_count=256)
    got, ref, step = _both_routes(case, cfg)
    assert step.capacity == Bn                   # one slot per request
    _assert_same_as_three(got, ref, f"{Bn} requests")
    _check_plan(step, ctx, case.num_kv_heads, cfg)
    g = to_f64(got)
    assert_close(g, oracle_direct(case), tolerance_kind(case), f"{Bn} requests {kv}")
    assert (g[_zero_rows(case)] == 0.0).all()
