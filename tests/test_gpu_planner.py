"""GPU planner (pa_plan) against the oracle's planner: bit-exact on whole buffers, sentinels included."""
import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from _util import announce

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _gpu_plan(ctx, hkv, cu, mult=2, P=256, T=256, capacity=None, poison=True):
    c = torch.as_tensor(np.asarray(ctx, dtype=np.int32), device=DEV)
    cap = B.pa_plan_capacity(len(ctx), hkv, cu, mult, P) if capacity is None else capacity
    work = torch.empty((cap, 4), dtype=torch.int32, device=DEV)
    red = torch.empty((len(ctx), 2), dtype=torch.int32, device=DEV)
    nw = torch.empty((2,), dtype=torch.int32, device=DEV)
    disp = torch.empty((cap, 4), dtype=torch.int32, device=DEV)
    if poison:
        work.fill_(0x5A5A5A5A)
        red.fill_(-7)
        nw.fill_(-9)
        disp.fill_(0x3C3C3C3C)
    B.pa_plan(c, hkv, cu_count=cu, budget_mult=mult, max_partitions=P, tile_tokens=T, capacity=cap,
              work_info=work, reduce_info=red, num_work=nw, dispatch_info=disp)
    torch.cuda.synchronize()
    _gpu_plan.dispatch = disp.cpu().numpy()
    return work.cpu().numpy(), red.cpu().numpy(), nw.cpu().numpy().tolist()


def expected_dispatch(work, used):
    """The dispatch order from its definition: slots ranked by tile count, largest first, ties by
    slot index, unused slots last; rank r at position r below half = ceil(C / 2), else at
    C + half - 1 - r; entries (request, tile_begin, tile_end, slot).  Identity above 1024 slots."""
    C = work.shape[0]
    out = np.empty((C, 4), dtype=np.int32)
    slots = np.arange(C)
    if C > 1024:
        out[:, :3] = work[:, :3]
        out[:, 3] = slots
        return out
    tiles = np.where(slots < used, work[:, 2] - work[:, 1], -1)
    order = sorted(range(C), key=lambda s: (-int(tiles[s]), s))
    half = (C + 1) // 2
    for r, s in enumerate(order):
        p = r if r < half else C + half - 1 - r
        out[p, :3] = work[s, :3]
        out[p, 3] = s
    return out


def _compare(ctx, hkv, cu, mult=2, P=256, T=256, capacity=None):
    gw, gr, gn = _gpu_plan(ctx, hkv, cu, mult, P, T, capacity)
    ow, orr, on, olarge = oracle.plan(np.asarray(ctx), hkv, cu, mult, P, T, capacity, with_largest=True)
    assert gn == [on, olarge]
    assert np.array_equal(gr, orr)
    assert np.array_equal(gw, ow)
    assert np.array_equal(_gpu_plan.dispatch, expected_dispatch(np.asarray(ow).reshape(-1, 4), on))


@pytest.mark.parametrize("name", W.CONFIG_NAMES)
def test_plan_bit_exact_on_the_five_workloads(name):
    announce(f"plan {name}")
    if name == "skewed_bf16":
        steps = W.skewed_step_set()
        for idx in range(0, steps.shape[0], 7):
            _compare(steps[idx], 2, 256)
        return
    ctx = {"tiny_fp32": [1, 17, 100, 300], "long_bf16": [131072], "verify_bf16": [16384] * 15,
           "fp8_kv": W.fp8_context_lens().tolist()}[name]
    hkv = {"tiny_fp32": 1, "long_bf16": 2, "verify_bf16": 1, "fp8_kv": 2}[name]
    _compare(ctx, hkv, 256)


def test_plan_bit_exact_on_sparse_steps_with_cap_8():
    steps = W.sparse_lengths(64, 16, seed=11)
    for idx in range(0, 64, 5):
        _compare(steps[idx], 2, 256, P=8)


def test_plan_uses_device_cu_count():
    cu = B.pa_device_cu_count()
    assert cu >= 1
    _compare([1000, 5, 70000, 0, 123456], 2, cu)


@pytest.mark.parametrize("seed", range(30))
def test_plan_fuzz(seed):
    rng = np.random.default_rng(500 + seed)
    Bn = int(rng.choice([1, 2, 5, 31, 32, 255, 1024, 4097, 8192]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([1, 8, 64, 256]))
    T = int(rng.choice([16, 64, 256]))
    cu = int(rng.choice([256, 80, 304]))
    mult = int(rng.choice([1, 2, 3]))
    kind = seed % 3
    if kind == 0:
        ctx = rng.integers(0, 1 << 20, size=Bn)
    elif kind == 1:
        ctx = np.where(rng.random(Bn) < 0.4, 0, rng.integers(1, 3000, size=Bn))
    else:
        ctx = np.clip(np.rint(np.exp(rng.normal(9.0, 2.0, size=Bn))), 0, 1 << 20).astype(np.int64)
    extra = int(rng.integers(0, 3)) * 17
    cap = B.pa_plan_capacity(Bn, hkv, cu, mult, P) + extra
    announce(f"plan fuzz seed {seed} B={Bn}")
    _compare(ctx, hkv, cu, mult, P, T, cap)


def test_replan_in_place_leaves_nothing_stale():
    c1 = torch.tensor([50000, 3, 70000, 900], dtype=torch.int32, device=DEV)
    c2 = torch.tensor([10, 0, 20, 30], dtype=torch.int32, device=DEV)
    work, red, nw = B.pa_plan(c1, 1, cu_count=256)
    B.pa_plan(c2, 1, cu_count=256, work_info=work, reduce_info=red, num_work=nw)
    torch.cuda.synchronize()
    ow, orr, on = oracle.plan([10, 0, 20, 30], 1, 256)
    assert int(nw[0].item()) == on
    assert np.array_equal(work.cpu().numpy(), ow) and np.array_equal(red.cpu().numpy(), orr)


def test_empty_and_all_zero_batches():
    _compare([0, 0, 0], 2, 256)
    _compare([0], 1, 256, capacity=600)


@pytest.mark.parametrize("cap", [1, 3, 6, 65, 511, 513, 1023, 1024, 1025, 2048])
def test_dispatch_order_at_capacity_edges(cap):
    """Capacities around the four-slot reads and the thread splits of the ranking, with tied slot
    sizes and unused slots; above 1024 slots the order is the identity."""
    announce(f"dispatch order capacity {cap}")
    rng = np.random.default_rng(cap)
    if cap < 64:
        ctx, P = [int(rng.integers(1, 5000))], 1
    else:
        ctx, P = rng.choice([768, 1280, 1000, 70000, 0, 256], size=40).tolist(), 256
    _compare(ctx, 8, 256, 2, P, 256, cap)


def test_dispatch_order_with_slots_beyond_the_packed_keys():
    """Slots of a million tiles and more are ranked by comparing their fields, not by packed keys."""
    announce("dispatch order, huge slots")
    _compare([20_000_000, 17_000_000, 5, 20_000_000, 0, 16_777_216], 8, 256, 2, 1, 16)
