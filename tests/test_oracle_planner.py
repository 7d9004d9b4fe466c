"""Pins for the oracle's planner (O1) against facts the pages fix, hand-worked plans and brute force.

Sources: ROCm/ATOM PR #2366 (section 1 Motivation, section 5 Test Result, review item 3) and
ROCm/ATOM PR #2514 (Design, default 2 x CU budget).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_tiny_plan_matches_hand_worked_fixture():
    g = _load("plan_tiny_fp32.json")
    inp = g["inputs"]
    assert oracle.plan_capacity(len(inp["context_lens"]), inp["num_kv_heads"], inp["cu_count"],
                                inp["budget_mult"], inp["max_partitions"]) == g["capacity"]
    work, red, nw = oracle.plan(inp["context_lens"], inp["num_kv_heads"], inp["cu_count"],
                                inp["budget_mult"], inp["max_partitions"], inp["tile_tokens"])
    assert nw == g["num_work"]
    assert work.shape == (g["capacity"], 4)
    assert work[:nw].tolist() == g["work_first"]
    assert (work[nw:] == np.array([-1, 0, 0, 0])).all()
    assert red.tolist() == g["reduce"]


def test_long_single_request_plan_closed_form():
    # batch 1, 131072 tokens, Hkv 2: C = min(256, max(1, 256)) = 256, 512 tiles, 256 parts of 2 tiles
    work, red, nw = oracle.plan([131072], 2)
    assert nw == 256 and red.tolist() == [[0, 256]]
    expect = [[0, 2 * j, 2 * j + 2, 131072] for j in range(256)]
    assert work.tolist() == expect


def test_verify_workload_plan_closed_form():
    # 15 requests at 16384 tokens, Hkv 1: C = 512, extra = 497, parts = min(256, 64, 1 + 33) = 34
    work, red, nw = oracle.plan([16384] * 15, 1)
    assert nw == 510
    assert red.tolist() == [[34 * b, 34] for b in range(15)]
    for b in range(15):
        for j in range(34):
            assert work[34 * b + j].tolist() == [b, (j * 64) // 34, ((j + 1) * 64) // 34, 16384]
    assert (work[510:] == np.array([-1, 0, 0, 0])).all()


def test_fp8_workload_gives_one_partition_each():
    # 256 requests at Hkv 2: C = min(256*256, max(256, 256)) = 256 = B, so no split is possible
    rng = np.random.default_rng(0)
    ctx = rng.integers(128, 65537, size=256)
    work, red, nw = oracle.plan(ctx, 2)
    assert nw == 256
    assert (red[:, 1] == 1).all()
    assert (red[:, 0] == np.arange(256)).all()
    tiles = -(-ctx // 256)
    assert (work[:, 0] == np.arange(256)).all() and (work[:, 1] == 0).all()
    assert (work[:, 2] == tiles).all() and (work[:, 3] == ctx).all()


def test_page_facts():
    facts = {f["id"]: f for f in _load("plan_page_facts.json")["facts"]}

    f = facts["capacity_512_at_one_kv_head"]
    for B in f["batches"]:
        assert oracle.plan_capacity(B, f["num_kv_heads"], f["cu_count"], f["budget_mult"],
                                    f["max_partitions"]) == f["capacity"]

    f = facts["batch_one_runs_at_the_ceiling"]
    for s in f["contexts"]:
        for P in f["max_partitions"]:
            work, red, nw = oracle.plan([s], f["num_kv_heads"], f["cu_count"], f["budget_mult"], P,
                                        f["tile_tokens"])
            assert red[0, 1] == P and nw == P

    f = facts["ceiling_64_vs_256_identical_at_batch_8_and_24"]
    for s in f["contexts"]:
        for B in f["batches"]:
            counts = {}
            for P in (64, 256):
                _, red, _ = oracle.plan([s] * B, f["num_kv_heads"], f["cu_count"], f["budget_mult"],
                                        P, f["tile_tokens"])
                counts[P] = red[:, 1].tolist()
            assert counts[64] == counts[256] == [f["expected_parts"][str(B)]] * B

    f = facts["share_is_512_over_batch"]
    for B in f["batches"]:
        _, red, _ = oracle.plan([f["context"]] * B, f["num_kv_heads"], f["cu_count"],
                                f["budget_mult"], f["max_partitions"], f["tile_tokens"])
        assert (red[:, 1] == max(1, min(256, 512 // B))).all()

    f = facts["tile_is_256_tokens"]
    for tok, page in zip(f["tokens"], f["page_tiles"]):
        assert abs(math.ceil(tok / 256) - page) <= 1
        assert abs(math.ceil(tok / 128) - page) > page // 2
        assert abs(math.ceil(tok / 512) - page) > page // 4


def _brute_parts(ctx, C, P, T):
    """Partition counts by search instead of division: the largest k with k * W <= extra * S_b."""
    ctx = [int(s) for s in ctx]
    W = sum(ctx)
    extra = C - sum(1 for s in ctx if s > 0)
    out = []
    for s in ctx:
        if s == 0:
            out.append(0)
            continue
        k = 0
        while (k + 1) * W <= extra * s:
            k += 1
        out.append(min(P, -(-s // T), 1 + k))
    return out


def test_largest_slot_is_the_largest_tile_range():
    rng = np.random.default_rng(77)
    for _ in range(30):
        ctx = rng.integers(0, 200000, size=int(rng.integers(1, 300)))
        work, red, nw, largest = oracle.plan(ctx, 2, 256, 2, 256, 256, with_largest=True)
        brute = 0
        for w in work[:nw]:
            brute = max(brute, int(w[2] - w[1]))
        assert largest == brute
    assert oracle.plan([0, 0], 1, with_largest=True)[3] == 0


def _check_invariants(ctx, Hkv, cu, mult, P, T, work, red, nw):
    B = len(ctx)
    C = min(B * P, max(B, -(-(mult * cu) // Hkv)))
    assert work.shape[0] >= C
    assert 0 <= nw <= C
    assert red[:, 1].sum() == nw
    slot = 0
    for b in range(B):
        s = int(ctx[b])
        tiles = -(-s // T)
        first, parts = int(red[b, 0]), int(red[b, 1])
        assert first == slot
        if s == 0:
            assert parts == 0
        else:
            assert 1 <= parts <= min(P, tiles)
        covered = 0
        for j in range(parts):
            w = work[first + j].tolist()
            assert w[0] == b and w[3] == s
            assert w[1] == covered and w[2] > w[1]
            size = w[2] - w[1]
            assert tiles // parts <= size <= -(-tiles // parts)  # balanced to within one tile
            covered = w[2]
        assert covered == (tiles if parts else 0)
        slot += parts
    assert (work[nw:] == np.array([-1, 0, 0, 0])).all()
    # longer requests never receive fewer partitions
    order = np.argsort(ctx, kind="stable")
    assert (np.diff(red[order, 1]) >= 0).all()


@pytest.mark.parametrize("seed", range(40))
def test_fuzz_invariants_and_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.choice([1, 2, 3, 7, 15, 32, 100, 256, 600, 1500]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([1, 8, 64, 256]))
    T = int(rng.choice([16, 64, 256]))
    cu = int(rng.choice([256, 304, 80]))
    mult = int(rng.choice([1, 2, 3]))
    kind = seed % 4
    if kind == 0:
        ctx = rng.integers(0, 1 << 20, size=B)
    elif kind == 1:
        ctx = np.where(rng.random(B) < 0.3, 0, rng.integers(1, 5000, size=B))
    elif kind == 2:
        ctx = np.full(B, int(rng.integers(1, 200000)))
    else:
        ctx = np.clip(np.rint(np.exp(rng.normal(8.0, 2.0, size=B))), 0, 1 << 20).astype(np.int64)
    work, red, nw = oracle.plan(ctx, Hkv, cu, mult, P, T)
    _check_invariants(ctx, Hkv, cu, mult, P, T, work, red, nw)
    if B <= 256 and int(ctx.max(initial=0)) < 300000:
        C = oracle.plan_capacity(B, Hkv, cu, mult, P)
        assert red[:, 1].tolist() == _brute_parts(ctx, C, P, T)


def test_all_zero_lengths_and_larger_buffer():
    work, red, nw = oracle.plan([0, 0, 0], 2, capacity=600)
    assert nw == 0 and red.tolist() == [[0, 0]] * 3
    assert work.shape == (600, 4) and (work == np.array([-1, 0, 0, 0])).all()


def test_rejects_bad_arguments():
    with pytest.raises(oracle.OracleError):
        oracle.plan([5, -1], 1)
    with pytest.raises(oracle.OracleError):
        oracle.plan([5, 6], 1, capacity=10)  # below the required capacity of 512
    with pytest.raises(oracle.OracleError):
        oracle.plan([5], 0)
    with pytest.raises(oracle.OracleError):
        oracle.plan([5], 1, tile_tokens=0)


# ---------------------------------------------------------------------------------------------
# with a sliding window the plan covers each request's windowed key range (ROCm/ATOM PR #2366
# review, the window logic: plan and kernel must agree on the range once windows are allowed)
# ---------------------------------------------------------------------------------------------

def _read_range(s, L, W):
    lo = max(0, s - (L - 1) - W) if W > 0 else 0
    return lo, s


@pytest.mark.parametrize("seed", range(20))
def test_window_plan_covers_the_windowed_range(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.choice([1, 3, 16, 40, 200]))
    W = int(rng.choice([1, 3, 50, 700, 5000]))
    T = int(rng.choice([16, 64, 256]))
    P = int(rng.choice([1, 8, 256]))
    ctx = np.where(rng.random(B) < 0.2, 0, rng.integers(1, 40000, size=B))
    ql = rng.integers(1, 5, size=B)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    work, red, nw, largest = oracle.plan(ctx, 2, 256, 2, P, T, with_largest=True, cu_query_lens=cu, window=W)
    C = oracle.plan_capacity(B, 2, 256, 2, P)
    lens = []
    for b in range(B):
        lo, hi = _read_range(int(ctx[b]), int(ql[b]), W)
        lens.append(hi - lo)
        first, parts = int(red[b, 0]), int(red[b, 1])
        if hi - lo == 0:
            assert parts == 0
            continue
        t0, t1 = lo // T, -(-hi // T)
        assert 1 <= parts <= min(P, t1 - t0)
        covered = t0
        for j in range(parts):
            w = work[first + j].tolist()
            assert w[0] == b and w[3] == ctx[b] and w[1] == covered and w[2] > w[1]
            covered = w[2]
        assert covered == t1
    assert red[:, 1].sum() == nw <= C
    # partition counts by search, weighted by the windowed lengths
    tot = sum(lens)
    extra = C - sum(1 for x in lens if x > 0)
    for b in range(B):
        if lens[b] == 0:
            continue
        k = 0
        while (k + 1) * tot <= extra * lens[b]:
            k += 1
        lo, hi = _read_range(int(ctx[b]), int(ql[b]), W)
        assert red[b, 1] == min(P, -(-hi // T) - lo // T, 1 + k)
    assert largest == max([int(w[2] - w[1]) for w in work[:nw]], default=0)


def test_window_zero_or_wide_equals_the_plain_plan():
    rng = np.random.default_rng(77)
    ctx = rng.integers(0, 100000, size=50)
    ql = rng.integers(1, 4, size=50)
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    plain = oracle.plan(ctx, 2, with_largest=True)
    for W in (0, 200000):
        got = oracle.plan(ctx, 2, with_largest=True, cu_query_lens=cu, window=W)
        assert all(np.array_equal(a, b) for a, b in zip(got, plain))


def test_window_plan_hand_worked():
    # S = 1000, L = 2, W = 300: keys [699, 1000) -> tiles [2, 4) at T = 256; a lone request at Hkv 1
    # has C = 512 slots, so parts = min(256, 2, 1 + 511) = 2: tiles [2, 3) and [3, 4)
    work, red, nw = oracle.plan([1000], 1, cu_query_lens=[0, 2], window=300)
    assert nw == 2 and red.tolist() == [[0, 2]]
    assert work[:2].tolist() == [[0, 2, 3, 1000], [0, 3, 4, 1000]]
