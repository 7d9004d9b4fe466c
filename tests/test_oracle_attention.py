"""Pins for the oracle's attention (O2 direct, O3 split) against a library routine, closed forms,
invariants and the element-decoding definitions.

Semantics come from opengfx1030/vllm-rdna PR #29, Change item 1 (token i of L attends to
S - (L - 1 - i) keys; rows past the last cumulative length and zero-length requests are zero;
without cumulative lengths each request has one row) and from ROCm/ATOM PR #2366 (split counts
must not change the answer: section 5 drift sweep).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _paged_from_dense(kd, vd, block_size, rng, extra_blocks=5):
    """Scatter per-request dense K/V ([S_b, Hkv, D] float64 lists) into a random page pool.
    Returns (k_cache, v_cache, block_tables) as float32 arrays + int32 table."""
    Hkv, D = kd[0].shape[1], kd[0].shape[2]
    pages = [-(-k.shape[0] // block_size) for k in kd]
    nb = sum(pages) + extra_blocks
    perm = rng.permutation(nb)
    kc = rng.standard_normal((nb, Hkv, block_size, D)).astype(np.float32) * 100.0
    vc = rng.standard_normal((nb, Hkv, block_size, D)).astype(np.float32) * 100.0
    bt = np.full((len(kd), max(max(pages), 1)), -1, dtype=np.int32)
    pos = 0
    for b, (k, v) in enumerate(zip(kd, vd)):
        for p in range(pages[b]):
            blk = perm[pos]
            pos += 1
            bt[b, p] = blk
            seg = slice(p * block_size, min((p + 1) * block_size, k.shape[0]))
            n = seg.stop - seg.start
            kc[blk, :, :n, :] = np.transpose(k[seg], (1, 0, 2))
            vc[blk, :, :n, :] = np.transpose(v[seg], (1, 0, 2))
    return kc, vc, bt


def _problem(rng, ctx, qlens, Hq, Hkv, D, bs, pad_rows=0):
    kd = [rng.standard_normal((s, Hkv, D)).astype(np.float32) for s in ctx]
    vd = [rng.standard_normal((s, Hkv, D)).astype(np.float32) for s in ctx]
    kc, vc, bt = _paged_from_dense(kd, vd, bs, rng)
    if qlens is None:
        cu = None
        R = len(ctx) + pad_rows
    else:
        cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        R = int(cu[-1]) + pad_rows
    q = rng.standard_normal((R, Hq, D)).astype(np.float32)
    return dict(q=q, kd=kd, vd=vd, kc=kc, vc=vc, bt=bt, ctx=np.asarray(ctx, np.int32), cu=cu)


def _sdpa_reference(pb, Hq, scale):
    """torch scaled_dot_product_attention in float64 on the dense, contiguous K/V of each request,
    with an explicit causal-offset mask and its own grouped-query head mapping."""
    q = pb["q"]
    R, _, D = q.shape
    out = np.zeros((R, Hq, D))
    for b, s in enumerate(pb["ctx"]):
        if pb["cu"] is None:
            r0, L = b, 1
        else:
            r0, L = int(pb["cu"][b]), int(pb["cu"][b + 1] - pb["cu"][b])
        if L == 0 or s == 0:
            continue
        qq = torch.from_numpy(q[r0:r0 + L].astype(np.float64)).permute(1, 0, 2)[None]
        kk = torch.from_numpy(pb["kd"][b].astype(np.float64)).permute(1, 0, 2)[None]
        vv = torch.from_numpy(pb["vd"][b].astype(np.float64)).permute(1, 0, 2)[None]
        i = torch.arange(L)[:, None]
        p = torch.arange(int(s))[None, :]
        mask = p < (int(s) - (L - 1 - i))
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
        o = o[0].permute(1, 0, 2).numpy()
        visible = (int(s) - (L - 1 - np.arange(L))) > 0
        o[~visible] = 0.0
        out[r0:r0 + L] = o
    return out


def _direct(pb, scale, **kw):
    return oracle.attention_direct(pb["q"], "f32", pb["kc"], pb["vc"], "f32", pb["bt"], pb["ctx"],
                                   pb["cu"], scale, **kw)


CASES = [
    # (ctx, qlens, Hq, Hkv, D, bs, pad_rows)
    ([1, 17, 100, 300], None, 4, 1, 64, 16, 0),
    ([37, 5, 64, 129], [3, 1, 2, 4], 8, 2, 32, 16, 2),
    ([2, 0, 7, 90, 3], [3, 2, 1, 3, 0], 6, 1, 16, 64, 3),
    ([513, 260], [2, 3], 12, 4, 128, 128, 1),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_direct_matches_library_sdpa(case):
    ctx, qlens, Hq, Hkv, D, bs, pad = CASES[case]
    rng = np.random.default_rng(case)
    pb = _problem(rng, ctx, qlens, Hq, Hkv, D, bs, pad)
    scale = 1.0 / math.sqrt(D)
    got = _direct(pb, scale, threads=3)
    ref = _sdpa_reference(pb, Hq, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("T,P,cu_count,mult", [(16, 1, 256, 2), (32, 2, 4, 2), (64, 8, 7, 3),
                                               (256, 256, 256, 2), (16, 256, 64, 1)])
def test_split_equals_direct(case, T, P, cu_count, mult):
    ctx, qlens, Hq, Hkv, D, bs, pad = CASES[case]
    rng = np.random.default_rng(10 + case)
    pb = _problem(rng, ctx, qlens, Hq, Hkv, D, bs, pad)
    scale = 1.0 / math.sqrt(D)
    work, red, nw = oracle.plan(pb["ctx"], Hkv, cu_count, mult, P, T)
    split = oracle.attention_split(pb["q"], "f32", pb["kc"], pb["vc"], "f32", pb["bt"], pb["ctx"],
                                   pb["cu"], scale, work, red, T)
    direct = _direct(pb, scale)
    np.testing.assert_allclose(split, direct, rtol=0, atol=1e-10)


def test_single_key_returns_that_value_row_exactly():
    rng = np.random.default_rng(3)
    pb = _problem(rng, [1, 1, 5], None, 4, 2, 16, 16)
    out = _direct(pb, 0.25)
    for b in (0, 1):
        for h in range(4):
            assert (out[b, h] == pb["vd"][b][0, h // 2].astype(np.float64)).all()


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(4)
    pb = _problem(rng, [9, 33], [3, 2], 4, 1, 8, 16)
    pb["q"][:] = 0.0
    out = _direct(pb, 0.3)
    for b, s in enumerate(pb["ctx"]):
        r0, L = int(pb["cu"][b]), int(pb["cu"][b + 1] - pb["cu"][b])
        for i in range(L):
            n = int(s) - (L - 1 - i)
            mean = pb["vd"][b][:n, 0].astype(np.float64).mean(axis=0)
            for h in range(4):
                np.testing.assert_allclose(out[r0 + i, h], mean, rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(5)
    pb = _problem(rng, [40], None, 2, 1, 8, 16)
    row = pb["kd"][0][0].copy()
    for p in range(40):
        pb["kd"][0][p] = row
    pb["kc"], pb["vc"], pb["bt"] = _paged_from_dense(pb["kd"], pb["vd"], 16, rng)
    out = _direct(pb, 0.7)
    mean = pb["vd"][0][:, 0].astype(np.float64).mean(axis=0)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], mean, rtol=0, atol=1e-12)


def test_padding_and_zero_length_rows_are_exactly_zero():
    rng = np.random.default_rng(6)
    # request 1 has no keys; request 2 has 2 query tokens but only 1 key, so its first token sees none
    pb = _problem(rng, [20, 0, 1], [2, 1, 2], 4, 2, 16, 16, pad_rows=3)
    out = _direct(pb, 0.25)
    cu = pb["cu"]
    assert (out[cu[1]:cu[2]] == 0.0).all()          # zero-length request
    assert (out[cu[2]] == 0.0).all()                 # token 0 of request 2: S-(L-1-0) = 0 keys
    assert (out[cu[2] + 1] != 0.0).any()
    assert (out[cu[3]:] == 0.0).all()                # padding rows past the last cumulative length
    T, P = 16, 256
    work, red, _ = oracle.plan(pb["ctx"], 2, 256, 2, P, T)
    split = oracle.attention_split(pb["q"], "f32", pb["kc"], pb["vc"], "f32", pb["bt"], pb["ctx"],
                                   pb["cu"], 0.25, work, red, T)
    assert (split[cu[1]:cu[2]] == 0.0).all() and (split[cu[3]:] == 0.0).all()
    assert (split[cu[2]] == 0.0).all()


def test_causal_range_per_token():
    rng = np.random.default_rng(7)
    ctx, L = 50, 4
    pb = _problem(rng, [ctx], [L], 4, 1, 16, 16)
    ref = _direct(pb, 0.25)
    for i in range(L - 1):
        n = ctx - (L - 1 - i)      # token i sees keys [0, n); key n is first visible to token i+1
        kd = [k.copy() for k in pb["kd"]]
        vd = [v.copy() for v in pb["vd"]]
        kd[0][n] += 3.0
        vd[0][n] -= 5.0
        pb2 = dict(pb, kd=kd, vd=vd)
        pb2["kc"], pb2["vc"], pb2["bt"] = _paged_from_dense(kd, vd, 16, np.random.default_rng(99))
        got = _direct(pb2, 0.25)
        assert (got[: i + 1] == ref[: i + 1]).all()
        assert (np.abs(got[i + 1:] - ref[i + 1:]).max(axis=-1) > 1e-6).all()


def test_no_cumulative_lengths_equals_one_token_each():
    rng = np.random.default_rng(8)
    pb = _problem(rng, [5, 40, 17], None, 4, 2, 32, 16)
    a = _direct(pb, 0.2)
    pb2 = dict(pb)
    pb2["cu"] = np.arange(4, dtype=np.int32)
    b = _direct(pb2, 0.2)
    assert (a == b).all()


def test_grouped_heads_use_their_own_kv_head():
    # with Hkv distinct heads, mapping q head h to kv head h // G is what the library SDPA does
    rng = np.random.default_rng(9)
    pb = _problem(rng, [30, 12], None, 8, 4, 16, 16)
    got = _direct(pb, 0.25)
    ref = _sdpa_reference(pb, 8, 0.25)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)
    wrong = got.copy()
    wrong[:, [0, 1]] = got[:, [2, 3]]
    assert np.abs(wrong - ref).max() > 1e-3


def test_rows_subset_equals_direct():
    rng = np.random.default_rng(11)
    pb = _problem(rng, [60, 3, 200], [2, 3, 1], 6, 3, 32, 64, pad_rows=2)
    full = _direct(pb, 0.2)
    rows = np.array([0, 1, 2, 3, 4, 5, 6, 7], np.int32)
    heads = np.array([0, 5, 3, 2, 1, 4, 0, 5], np.int32)
    sub = oracle.attention_rows(pb["q"], "f32", pb["kc"], pb["vc"], "f32", pb["bt"], pb["ctx"],
                                pb["cu"], 0.2, rows, heads)
    assert (sub == full[rows, heads]).all()


def test_fp8_e4m3fn_decode_matches_library_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_values(codes, "fp8")
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert (mine[ok] == lib[ok]).all()
    assert np.signbit(mine[ok]).tolist() == np.signbit(lib[ok]).tolist()
    assert mine[0x7E] == 448.0 and np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_bf16_decode_matches_library_for_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_values(codes, "bf16")
    lib = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert (mine[ok] == lib[ok]).all()


def test_storage_types_decode_before_the_arithmetic():
    # a bf16 / fp8 problem equals the f32 problem on the decoded (and scaled) values
    rng = np.random.default_rng(12)
    pb = _problem(rng, [33, 70], [2, 1], 4, 2, 16, 16)
    kb = torch.from_numpy(pb["kc"]).to(torch.bfloat16)
    vb = torch.from_numpy(pb["vc"]).to(torch.bfloat16)
    kbits = kb.view(torch.int16).numpy().view(np.uint16)
    vbits = vb.view(torch.int16).numpy().view(np.uint16)
    got = oracle.attention_direct(pb["q"], "f32", kbits, vbits, "bf16", pb["bt"], pb["ctx"], pb["cu"], 0.25)
    ref = oracle.attention_direct(pb["q"], "f32", kb.float().numpy(), vb.float().numpy(), "f32",
                                  pb["bt"], pb["ctx"], pb["cu"], 0.25)
    assert (got == ref).all()
    ks, vs = 0.037, 0.021
    k8 = (torch.from_numpy(pb["kc"]) / ks).clamp(-448, 448).to(torch.float8_e4m3fn)
    v8 = (torch.from_numpy(pb["vc"]) / vs).clamp(-448, 448).to(torch.float8_e4m3fn)
    got = oracle.attention_direct(pb["q"], "f32", k8.view(torch.uint8).numpy(), v8.view(torch.uint8).numpy(),
                                  "fp8", pb["bt"], pb["ctx"], pb["cu"], 0.25, k_scale=ks, v_scale=vs)
    kf = (k8.to(torch.float64) * ks).numpy()
    vf = (v8.to(torch.float64) * vs).numpy()
    # dense reference on the decoded values through the library SDPA
    kd, vd = [], []
    for b, s in enumerate(pb["ctx"]):
        ks_ = np.concatenate([kf[pb["bt"][b, p]].transpose(1, 0, 2) for p in range(-(-int(s) // 16))])[:s]
        vs_ = np.concatenate([vf[pb["bt"][b, p]].transpose(1, 0, 2) for p in range(-(-int(s) // 16))])[:s]
        kd.append(ks_)
        vd.append(vs_)
    ref = _sdpa_reference(dict(pb, kd=kd, vd=vd), 4, 0.25)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_rejects_out_of_range_pages():
    rng = np.random.default_rng(13)
    pb = _problem(rng, [20], None, 2, 1, 8, 16)
    pb["bt"][0, 1] = pb["kc"].shape[0]
    with pytest.raises(oracle.OracleError):
        _direct(pb, 0.25)


# ---------------------------------------------------------------------------------------------
# sliding window: token i with n visible keys sees [max(0, n - W), n) (opengfx1030/vllm-rdna PR #29,
# Change 1: the sliding window applies per token; Test Plan: windows 0, 1, 3, 50)
# ---------------------------------------------------------------------------------------------

def _sdpa_window_reference(pb, Hq, scale, W):
    """torch SDPA in float64 on the dense K/V with an explicit band mask n - W <= p < n."""
    q = pb["q"]
    R, _, D = q.shape
    out = np.zeros((R, Hq, D))
    for b, s in enumerate(pb["ctx"]):
        r0, L = (b, 1) if pb["cu"] is None else (int(pb["cu"][b]), int(pb["cu"][b + 1] - pb["cu"][b]))
        if L == 0 or s == 0:
            continue
        qq = torch.from_numpy(q[r0:r0 + L].astype(np.float64)).permute(1, 0, 2)[None]
        kk = torch.from_numpy(pb["kd"][b].astype(np.float64)).permute(1, 0, 2)[None]
        vv = torch.from_numpy(pb["vd"][b].astype(np.float64)).permute(1, 0, 2)[None]
        n = int(s) - (L - 1 - torch.arange(L))[:, None]
        p = torch.arange(int(s))[None, :]
        mask = (p < n) & (p >= n - W)
        visible = mask.any(dim=1).numpy()
        mask[~mask.any(dim=1)] = True          # rows with no key: computed, then zeroed below
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale, enable_gqa=True)
        o = o[0].permute(1, 0, 2).numpy()
        o[~visible] = 0.0
        out[r0:r0 + L] = o
    return out


WINDOW_CASES = [
    # (ctx, qlens, Hq, Hkv, D, bs, pad_rows, W)
    ([1, 17, 100, 300], None, 4, 1, 64, 16, 0, 1),
    ([37, 5, 64, 129], [3, 1, 2, 4], 8, 2, 32, 16, 2, 3),
    ([2, 0, 7, 90, 3], [3, 2, 1, 3, 0], 6, 1, 16, 64, 3, 50),
    ([513, 260], [2, 3], 12, 4, 128, 128, 1, 50),
    ([700, 33], [4, 2], 4, 2, 64, 16, 0, 256),
]


@pytest.mark.parametrize("case", range(len(WINDOW_CASES)))
def test_window_direct_matches_library_sdpa(case):
    ctx, qlens, Hq, Hkv, D, bs, pad, W = WINDOW_CASES[case]
    rng = np.random.default_rng(40 + case)
    pb = _problem(rng, ctx, qlens, Hq, Hkv, D, bs, pad)
    scale = 1.0 / math.sqrt(D)
    got = _direct(pb, scale, window=W)
    ref = _sdpa_window_reference(pb, Hq, scale, W)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_window_of_one_returns_the_last_visible_value_row():
    rng = np.random.default_rng(41)
    pb = _problem(rng, [9, 33, 1], [2, 3, 1], 4, 2, 16, 16)
    out = _direct(pb, 0.25, window=1)
    for b, s in enumerate(pb["ctx"]):
        r0, L = int(pb["cu"][b]), int(pb["cu"][b + 1] - pb["cu"][b])
        for i in range(L):
            n = int(s) - (L - 1 - i)
            for h in range(4):
                assert (out[r0 + i, h] == pb["vd"][b][n - 1, h // 2].astype(np.float64)).all()


def test_window_at_least_the_context_changes_nothing():
    rng = np.random.default_rng(42)
    pb = _problem(rng, [37, 5, 64, 129], [3, 1, 2, 4], 8, 2, 32, 16, 2)
    full = _direct(pb, 0.2)
    for W in (129, 130, 10_000):
        assert np.array_equal(_direct(pb, 0.2, window=W), full)


def test_window_range_per_token():
    rng = np.random.default_rng(43)
    ctx, L, W = 60, 3, 7
    pb = _problem(rng, [ctx], [L], 4, 1, 16, 16)
    ref = _direct(pb, 0.25, window=W)
    for i in range(L):
        n = ctx - (L - 1 - i)
        for pos, inside in ((n - W - 1, False), (n - W, True)):
            kd = [k.copy() for k in pb["kd"]]
            vd = [v.copy() for v in pb["vd"]]
            kd[0][pos] += 3.0
            vd[0][pos] -= 5.0
            pb2 = dict(pb, kd=kd, vd=vd)
            pb2["kc"], pb2["vc"], pb2["bt"] = _paged_from_dense(kd, vd, 16, np.random.default_rng(98))
            got = _direct(pb2, 0.25, window=W)
            changed = np.abs(got[i] - ref[i]).max() > 1e-6
            assert changed == inside, (i, pos, inside)


@pytest.mark.parametrize("case", range(len(WINDOW_CASES)))
@pytest.mark.parametrize("T,P,cu_count,mult", [(16, 1, 256, 2), (64, 8, 7, 3), (256, 256, 256, 2),
                                               (16, 256, 64, 1)])
def test_window_split_equals_direct(case, T, P, cu_count, mult):
    ctx, qlens, Hq, Hkv, D, bs, pad, W = WINDOW_CASES[case]
    if T % bs:
        pytest.skip("tile not a multiple of the page")
    rng = np.random.default_rng(50 + case)
    pb = _problem(rng, ctx, qlens, Hq, Hkv, D, bs, pad)
    scale = 1.0 / math.sqrt(D)
    work, red, nw = oracle.plan(pb["ctx"], Hkv, cu_count, mult, P, T, cu_query_lens=pb["cu"], window=W)
    split = oracle.attention_split(pb["q"], "f32", pb["kc"], pb["vc"], "f32", pb["bt"], pb["ctx"],
                                   pb["cu"], scale, work, red, T, window=W)
    direct = _direct(pb, scale, window=W)
    np.testing.assert_allclose(split, direct, rtol=0, atol=1e-10)
