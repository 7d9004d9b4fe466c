"""Randomised decode and prefill parity against the fp64 oracle, element by element.

Each seed draws one small batch over the whole supported space: head_dim 64/128/256; pages of
16/64/128 tokens and tiles that are multiples of them; bf16, fp8 (e4m3fn) and fp32 caches with bf16
or fp32 queries; group sizes 1-8 with or without verify rows (per-token causal ranges, opengfx1030/
vllm-rdna PR #29, Change 1) and padding rows; partition ceilings 1-256 and budgets from one slot
per request (where the decode shares the slots) to 2 x 256 compute units (ROCm/ATOM PR #2366,
section 1); sliding windows; and the three call forms (decode with the merge in the call, decode
then pa_merge, pa_attention).  The prefill draws are prompts and chunks behind prefixes of up to 2000
keys through both pa_prefill forms; the mixed draws are decodes-first batches (decodes of up to 1 + k
rows, then prompts) through the decode-first split in its three forms.  The cases are small enough for the oracle to finish in well under a
second each; the tolerances are the ones every parity test uses.
"""
import numpy as np
import pytest
import torch

from paged_split_kv_amd import binding as B
from paged_split_kv_amd import workloads as W
from paged_split_kv_amd.runner import DecodeStep, PlanConfig, mixed_step
from _util import announce, assert_close, oracle_direct, to_f64, tolerance_kind
from test_gpu_decode import _zero_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MODES = ("merge_in_call", "separate_merge", "attention")


def _draw(seed):
    rng = np.random.default_rng(4200 + seed)
    D = int(rng.choice([64, 128, 256]))
    kv = str(rng.choice(["bf16", "bf16", "fp8", "f32"]))
    qd = str(rng.choice(["bf16", "f32"]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 6, 8]))
    bs = int(rng.choice([16, 64, 128]))
    T = int(rng.choice([t for t in (16, 64, 128, 256, 512) if t % bs == 0]))
    P = int(rng.choice([1, 2, 8, 256]))
    cu = int(rng.choice([1, 8, 64, 256]))
    Bn = int(rng.integers(1, 12))
    ctx = rng.integers(1, 6000, size=Bn)
    ctx[rng.random(Bn) < 0.2] = 0
    ql = None
    if rng.random() < 0.5:
        lmax = min(4, 64 // G)
        ql = rng.integers(1, lmax + 1, size=Bn).tolist()
    pad = int(rng.integers(0, 3))
    window = int(rng.choice([0, 0, 0, 1, 37, 700, 4000]))
    return dict(D=D, kv=kv, qd=qd, hkv=hkv, G=G, bs=bs, T=T, P=P, cu=cu, ctx=ctx.tolist(), ql=ql, pad=pad,
                window=window, mode=MODES[seed % 3])


@pytest.mark.parametrize("seed", range(64))
def test_decode_fuzz(seed):
    c = _draw(seed)
    announce(f"fuzz seed {seed}: " + " ".join(f"{k}={v}" for k, v in c.items() if k != "ctx") +
             f" B={len(c['ctx'])}")
    case = W.build_case(f"fuzz{seed}", c["ctx"], num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"],
                        head_dim=c["D"], block_size=c["bs"], kv_dtype=c["kv"], q_dtype=c["qd"], seed=seed,
                        q_lens=c["ql"], pad_rows=c["pad"], device=DEV)
    case.window = c["window"]
    step = DecodeStep.for_case(case, PlanConfig(cu_count=c["cu"], max_partitions=c["P"], tile_tokens=c["T"]))
    step.out.fill_(float("nan"))
    step.workspace.fill_(0xFF)                      # NaN pattern in every partial and piece state
    if c["mode"] == "attention":
        out = step.run_case(case, whole=True)
    else:
        out = step.run_case(case, fused=c["mode"] == "merge_in_call")
    got = to_f64(out)
    ref = oracle_direct(case)
    assert_close(got, ref, tolerance_kind(case), f"fuzz seed {seed}")
    if case.window == 0:
        assert (got[_zero_rows(case)] == 0.0).all()
    else:
        assert (got[np.all(ref == 0.0, axis=(1, 2))] == 0.0).all()


def _draw_prefill(seed):
    rng = np.random.default_rng(5300 + seed)
    D = int(rng.choice([64, 128, 256]))
    kv = str(rng.choice(["bf16", "bf16", "fp8"]))
    qd = str(rng.choice(["bf16", "f32"]))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 6, 8]))
    bs = int(rng.choice([16, 64, 128]))
    Bn = int(rng.integers(1, 4))
    ql = rng.integers(1, 161, size=Bn)
    prefix = np.where(rng.random(Bn) < 0.4, 0, rng.integers(0, 2001, size=Bn))
    ctx = (ql + prefix).tolist()
    pad = int(rng.integers(0, 3))
    window = int(rng.choice([0, 0, 1, 29, 300, 1500]))
    cu = int(rng.choice([8, 64, 256]))
    return dict(D=D, kv=kv, qd=qd, hkv=hkv, G=G, bs=bs, ctx=ctx, ql=ql.tolist(), pad=pad, window=window, cu=cu,
                split=bool(seed % 2 == 0))


@pytest.mark.parametrize("seed", range(32))
def test_prefill_fuzz(seed):
    """pa_prefill on random prompts and chunks behind prefixes, in the split form (query blocks planned,
    computed by the query-block kernel, merged) and the one-launch form."""
    c = _draw_prefill(seed)
    announce(f"prefill fuzz seed {seed}: " + " ".join(f"{k}={v}" for k, v in c.items()))
    case = W.build_case(f"pfuzz{seed}", c["ctx"], num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"],
                        head_dim=c["D"], block_size=c["bs"], kv_dtype=c["kv"], q_dtype=c["qd"], seed=seed,
                        q_lens=c["ql"], pad_rows=c["pad"], device=DEV)
    case.window = c["window"]
    out = torch.full_like(case.q, float("nan"))
    ws = None
    if c["split"]:
        nbytes = B.pa_prefill_workspace_bytes(case.num_rows, case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                              case.head_dim, c["cu"])
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    B.pa_prefill(case.q, case.k_cache, case.v_cache, case.kv_dtype, case.block_tables, case.context_lens,
                 case.cu_query_lens, out, ws, scale=case.scale, cu_count=c["cu"], k_scale=case.k_scale,
                 v_scale=case.v_scale, sliding_window=case.window)
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle_direct(case)
    assert_close(got, ref, tolerance_kind(case), f"prefill fuzz seed {seed}")
    assert (got[np.all(ref == 0.0, axis=(1, 2))] == 0.0).all()


def _draw_mixed(seed):
    rng = np.random.default_rng(6100 + seed)
    D = int(rng.choice([64, 128, 256]))
    kv = str(rng.choice(["bf16", "fp8"]))
    qd = str(rng.choice(["bf16", "f32"]))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 6, 8]))
    bs = int(rng.choice([16, 64]))
    k = int(rng.choice([0, 0, 1, 2]))                # draft tokens: decodes carry up to 1 + k rows
    nd = int(rng.integers(1, 9))
    npr = int(rng.integers(0, 3))
    dq = rng.integers(1, 2 + k, size=nd)
    pq = rng.integers(2 + k, 130, size=npr)
    ql = np.concatenate([dq, pq]).astype(np.int64)
    prefix = np.where(rng.random(nd + npr) < 0.2, 0, rng.integers(0, 3000, size=nd + npr))
    ctx = (ql + prefix).tolist()
    window = int(rng.choice([0, 0, 0, 64, 900]))
    mode = ("one_call", "two_calls", "two_streams")[seed % 3]
    return dict(D=D, kv=kv, qd=qd, hkv=hkv, G=G, bs=bs, threshold=1 + k, ctx=ctx, ql=ql.tolist(),
                window=window, mode=mode)


@pytest.mark.parametrize("seed", range(24))
def test_mixed_fuzz(seed):
    """Decodes-first mixed batches through the decode-first split: pa_attention_mixed in one call, and
    pa_prefill then pa_attention on one stream and on two."""
    c = _draw_mixed(seed)
    announce(f"mixed fuzz seed {seed}: " + " ".join(f"{k}={v}" for k, v in c.items() if k != "ctx"))
    case = W.build_case(f"mfuzz{seed}", c["ctx"], num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"],
                        head_dim=c["D"], block_size=c["bs"], kv_dtype=c["kv"], q_dtype=c["qd"], seed=seed,
                        q_lens=c["ql"], device=DEV)
    case.window = c["window"]
    out = mixed_step(case, c["threshold"], PlanConfig(cu_count=256), concurrent=c["mode"] == "two_streams",
                     one_call=c["mode"] == "one_call")
    torch.cuda.synchronize()
    got = to_f64(out)
    ref = oracle_direct(case)
    assert_close(got, ref, tolerance_kind(case), f"mixed fuzz seed {seed}")
    assert (got[np.all(ref == 0.0, axis=(1, 2))] == 0.0).all()
