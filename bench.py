"""Benchmark of the paged split-KV decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--window W]
                    [--no-graph] [--no-cold] [--no-cpu-baseline] [--cpu-seconds S] [--step-only]

Default workload: the skewed 32-request bf16 decode (Hq 16 / Hkv 2, D 128, pages of 16 tokens): 128
decode steps whose in-batch max/min context ratio follows the agentic trace (p50 ~2.5, p90 ~21), every
step drawing its pages at random from a 4 GiB K/V pool so that the 256 MB last-level cache cannot
carry a step's data to the next.  Inputs are resident in HBM.

One timed step = pa_decode + pa_merge for one attention layer, with the step's plan made once
beforehand (the pages build the plan once per forward and share it across layers: ROCm/ATOM PR #2366,
section 3, "Plan lifetime vs cudagraph").  The K timed steps sample the whole step set: whole passes
over all 128 steps in one seeded order, and for the remainder r < 128 the r steps at the set's
quantiles (j + 1/2) / r, so any K is a stratified sample (step_order).  value = KV bytes of exactly
the timed steps / their time (GB/s); ms_per_step = time / K.

Reported beside it: the same step over whole passes of all 128 steps (full_set); a HIP-graph replay
of it; pa_plan alone (the per-forward refresh); the one-call pa_attention (plan in place, two
launches) and the three-call form; per-kernel times with events around each launch; each step once
with the 256 MB last-level cache evicted before it; the decode kernel alone back to back (roofline);
the read-only ceilings of the same device (pa_probe_read: a contiguous read; pa_probe_gather: exactly
the decode's K/V bytes over the same plans, with the decode's launch shape and dispatch order, no
arithmetic; also timed in slot order); and the
CPU oracle on a bounded sample plus one timing per named configuration (cpu_baseline).

The roofline object is for the decode kernel: algorithmic bytes per launch (context length x Hkv x 2 x
D x element size summed over the batch, averaged over exactly the launches timed) over the mean
launch duration, measured with HIP events on the launch stream around K launches issued back to back
over the same step order as the headline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 matrix-core peak of the chip
METRIC = "µs/step + achieved KV-read HBM GB/s (% peak), skewed 32-req bf16 decode"
DECODE_SRC = os.path.join(ROOT, "paged_split_kv_amd", "csrc", "pa_decode.hip")
PREFILL_SRC = os.path.join(ROOT, "paged_split_kv_amd", "csrc", "pa_prefill.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_{workload}_counters.json")


# ------------------------------------------------------------------------------------------------
# step order and the headline arithmetic (host only; tested on the CPU)
# ------------------------------------------------------------------------------------------------

def step_order(K: int, nsteps: int, seed: int = 0) -> np.ndarray:
    """Indices of the K timed steps into a step set of nsteps (the skewed set is sorted by ratio):
    K // nsteps whole passes over every step in one seeded random order, then for the remainder r the
    r steps at the quantiles (j + 1/2) / r of the set, in a seeded random order."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nsteps)
    full, r = divmod(int(K), int(nsteps))
    parts = [perm] * full
    if r:
        strat = np.floor((np.arange(r) + 0.5) * nsteps / r).astype(np.int64)
        parts.append(rng.permutation(strat))
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def shared_slot_pieces(work_info: np.ndarray, used: int, factor: int = 2):
    """The pieces the decode streams when every request is one slot (shared slots): each slot of n
    tiles in X = max(1, ceil(n / per)) pieces, per = max(1, ceil((tiles + used) / (factor * used))),
    piece k covering the slot's tiles [floor(k n / X), floor((k + 1) n / X)); pieces in slot order.
    Returns the pieces as plan entries (request, tile_begin, tile_end, 0) and the bound per."""
    w = np.asarray(work_info).reshape(-1, 4)[:used]
    n = np.maximum(w[:, 2] - w[:, 1], 0).astype(np.int64)
    per = max(1, -(-(int(n.sum()) + used) // (factor * max(used, 1))))
    out = []
    for (b, t0, _, _), ns in zip(w, n):
        X = max(1, -(-int(ns) // per))
        for k in range(X):
            out.append((int(b), int(t0) + (k * int(ns)) // X, int(t0) + ((k + 1) * int(ns)) // X, 0))
    return np.asarray(out, dtype=np.int32).reshape(-1, 4), per


def rate(bytes_per_step: np.ndarray, order: np.ndarray, total_ms: float) -> dict:
    """Throughput of a timed run over `order`: bytes of exactly those steps over the total time."""
    K = len(order)
    done = float(np.asarray(bytes_per_step, dtype=np.float64)[order].sum())
    ms = total_ms / K
    gbps = done / (total_ms * 1e-3) / 1e9
    return {"steps": K, "distinct_steps": int(len(np.unique(order))), "bytes": done,
            "mean_bytes": done / K, "ms_per_step": ms, "us_per_step": ms * 1e3, "gbps": gbps,
            "pct_peak": 100.0 * gbps / HBM_PEAK_GBPS}


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per launch of the workload's main kernel from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    try:
        with open(COUNTERS_FILE.format(workload=workload)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("decode_source_sha") != source_sha(DECODE_SRC):
        return None
    if workload == "prefill" and c.get("prefill_source_sha") != source_sha(PREFILL_SRC):
        return None
    return c.get("traffic_bytes_per_launch")


def traffic_gbps(traffic_bytes, duration_us):
    """Counter-measured HBM GB/s of a launch: its FETCH + WRITE bytes over the measured duration."""
    if traffic_bytes is None or duration_us <= 0:
        return None
    return round(traffic_bytes / (duration_us * 1e-6) / 1e9, 1)


def attention_flops(context_lens, cu_query_lens, num_q_heads: int, head_dim: int, window: int = 0) -> float:
    """Matrix-core flops of one attention call: every (query token, head) row multiplies each key it
    sees twice (Q.K and P.V), 2 D flops each; token i of a request with L tokens and S keys sees
    S - (L - 1 - i) keys, the last W of them under a window."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    cu = np.asarray(cu_query_lens, dtype=np.int64)
    pairs = 0
    for b in range(ctx.shape[0]):
        L = int(cu[b + 1] - cu[b])
        n = np.maximum(ctx[b] - (L - 1 - np.arange(L)), 0)
        if window > 0:
            n = np.minimum(n, window)
        pairs += int(n.sum())
    return 4.0 * head_dim * num_q_heads * pairs


# ------------------------------------------------------------------------------------------------
# timing helpers
# ------------------------------------------------------------------------------------------------

def timed(calls, stream, warm_calls=()) -> float:
    """Run the warm-up calls, then the calls between two events on `stream`, synchronised on both
    sides; returns the elapsed milliseconds."""
    for f in warm_calls:
        f()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for f in calls:
        f()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def read_ceiling(dev, cu_count: int) -> dict:
    """pa_probe_read over a 2 GiB buffer, best of 10: the device's practical streaming read rate."""
    from paged_split_kv_amd import probe as P

    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    wgs = 2 * cu_count
    sink = P.sink_for(4 * wgs, dev)
    stream = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(3):
        P.pa_probe_read(src, wgs, sink)
    for _ in range(10):
        best = min(best, timed([lambda: P.pa_probe_read(src, wgs, sink)], stream))
    del src
    gbps = n / (best * 1e-3) / 1e9
    return {"gbps": round(gbps, 1), "pct_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 1), "bytes": n,
            "kernel": f"pa_probe_read: contiguous 2 GiB, {wgs} workgroups x 256 threads, 16-byte "
                      "non-temporal loads; best of 10"}


# ------------------------------------------------------------------------------------------------
# CPU oracle timings
# ------------------------------------------------------------------------------------------------

def _pool_step_host(pool, i):
    """Host arrays of skewed/sparse step i (pages gathered from the pool, block table renumbered)."""
    ctx = pool.steps[i]
    bs = pool.block_size
    pages = (ctx + bs - 1) // bs
    bt = pool.block_tables[i].cpu().numpy()
    used = np.concatenate([bt[b, :pages[b]] for b in range(len(ctx))])
    idx = torch.from_numpy(used.astype(np.int64)).to(pool.k_cache.device)
    k = pool.k_cache.index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
    v = pool.v_cache.index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
    remap = np.full(bt.shape, -1, dtype=np.int32)
    pos = 0
    for b in range(len(ctx)):
        remap[b, :pages[b]] = np.arange(pos, pos + pages[b], dtype=np.int32)
        pos += pages[b]
    q = pool.q[i].cpu().view(torch.int16).numpy().view(np.uint16)
    return q, k, v, remap, ctx.astype(np.int32)


def cpu_baseline_pool(pool, budget_s: float, window: int = 0) -> dict:
    """The CPU oracle (direct fp64 attention over the gathered pages) on a bounded sample of the
    pool's steps, in seeded random order, until the budget is spent."""
    import oracle

    threads = oracle.default_threads()
    done_bytes, spent, n = 0, 0.0, 0
    for i in np.random.default_rng(0).permutation(len(pool.steps)):
        q, k, v, remap, ctx = _pool_step_host(pool, i)
        t0 = time.perf_counter()
        oracle.attention_direct(q, "bf16", k, v, "bf16", remap, ctx, None, pool.scale, threads=threads,
                                window=window)
        spent += time.perf_counter() - t0
        keys = np.minimum(ctx, window) if window > 0 else ctx
        done_bytes += int(keys.astype(np.int64).sum()) * k.shape[1] * 2 * k.shape[3] * 2
        n += 1
        if spent >= budget_s:
            break
    used = min(threads, len(pool.steps[0]) * pool.k_cache.shape[1])
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "us_per_step": round(spent / n * 1e6, 1),
            "sample": f"{n} of the {len(pool.steps)} steps (seeded random order, stopped after "
                      f"{budget_s:.0f} s of oracle time), fp64 direct attention over the gathered pages, "
                      f"{spent:.1f} s"}


def _oracle_case_us(case, threads, budget_s: float = 1.0):
    import oracle

    h = case.host()
    spent, n = 0.0, 0
    while n == 0 or spent < budget_s:
        t0 = time.perf_counter()
        oracle.attention_direct(h["q"], case.q_dtype, h["k_cache"], h["v_cache"], case.kv_dtype,
                                h["block_tables"], h["context_lens"], h["cu_query_lens"], case.scale,
                                case.k_scale, case.v_scale, threads=threads, window=case.window)
        spent += time.perf_counter() - t0
        n += 1
    return spent / n * 1e6, min(threads, case.num_seqs * case.num_kv_heads), n


def cpu_oracle_per_config(dev, pool=None) -> dict:
    """The oracle's µs per step on every named configuration: tiny; the skewed steps nearest the p50
    and p90 ratio and the step with most tokens; long; verify; fp8 (each run once, or repeated for
    about a second when fast)."""
    import oracle
    from paged_split_kv_amd import workloads as W

    threads = oracle.default_threads()
    out = {}
    cases = [("tiny_fp32", None)]
    steps = W.skewed_step_set()
    for tag, idx in W.skewed_named_steps(steps).items():
        cases.append((f"skewed_{tag}", idx))
    cases += [("long_bf16", None), ("verify_bf16", None), ("fp8_kv", None)]
    for name, idx in cases:
        if name.startswith("skewed"):
            c = W.make_config("skewed_bf16", device=dev, step=idx)
        else:
            c = W.make_config(name, device=dev)
        us, busy, runs = _oracle_case_us(c, threads)
        out[name] = {"us_per_step": round(us, 1), "runs": runs, "kv_bytes": c.kv_bytes(), "busy_threads": busy,
                     "kv_gbps": round(c.kv_bytes() / (us * 1e-6) / 1e9, 3)}
        del c
    return out


def cpu_baseline_case(case, budget_s: float, kv_bytes: float) -> dict:
    """The CPU oracle on one full-size configuration, repeated while the budget lasts (at least once);
    the host copy of the case is made before the clock starts."""
    import oracle

    threads = oracle.default_threads()
    us, busy, n = _oracle_case_us(case, threads, budget_s)
    return {"value": round(kv_bytes / (us * 1e-6) / 1e9, 4), "unit": "GB/s", "cores": busy, "kind": "oracle",
            "us_per_step": round(us, 1),
            "sample": f"the whole configuration (one batch) {n} time(s), fp64 direct attention over the "
                      f"gathered pages"}


# ------------------------------------------------------------------------------------------------
# mixed batches
# ------------------------------------------------------------------------------------------------

def bench_mixed(args, batches, cu_count):
    """The decode-first split of a mixed batch: one pa_attention_mixed call per step (decode and
    prompt in one launch, then the merge); the two-call form (pa_prefill, then pa_attention), the
    same on two streams, and the parts alone are timed beside it.  Every timed call is marshalled
    beforehand (prepare=True), so the loops measure the device, not the host's argument checks."""
    from paged_split_kv_amd import binding as B
    from paged_split_kv_amd.runner import MixedStep, PlanConfig

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream(device=stream.device)         # default priority
    steps = [MixedStep(c, 1, PlanConfig(cu_count=cu_count)) for c in batches]
    one, dec, pre, pre_side, pre_split = [], [], [], [], []
    c0 = batches[0]
    ws_pre = torch.empty((B.pa_prefill_workspace_bytes(c0.num_rows, c0.num_seqs, c0.num_q_heads, c0.num_kv_heads,
                                                       c0.head_dim, cu_count),), dtype=torch.uint8,
                         device=stream.device)
    for c, m in zip(batches, steps):
        if m.dec is None:
            raise ValueError("the mixed workload has decode requests")
        d, p = m.dec, m.dec.plan_cfg
        one.append(B.pa_attention_mixed(
            c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, c.cu_query_lens, m.nd, m.ndt,
            d.work_info, d.reduce_info, d.num_work, d.workspace, m.out, scale=c.scale, cu_count=p.cu_count,
            budget_mult=p.budget_mult, max_partitions=p.max_partitions, tile_tokens=p.tile_tokens,
            max_q_len=m.threshold, k_scale=c.k_scale, v_scale=c.v_scale, sliding_window=c.window, stream=stream,
            prepare=True))
        dec.append(B.pa_attention(
            c.q[:m.ndt], c.k_cache, c.v_cache, c.kv_dtype, c.block_tables[:m.nd], c.context_lens[:m.nd],
            d.work_info, d.reduce_info, d.num_work, d.workspace, d.out, scale=c.scale, cu_count=p.cu_count,
            budget_mult=p.budget_mult, max_partitions=p.max_partitions, tile_tokens=p.tile_tokens,
            cu_query_lens=c.cu_query_lens[:m.nd + 1], max_q_len=d.max_q_len, k_scale=c.k_scale,
            v_scale=c.v_scale, sliding_window=c.window, stream=stream, prepare=True))
        for s_, lst in ((stream, pre), (side, pre_side)):
            lst.append(B.pa_prefill(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables[m.nd:],
                                    c.context_lens[m.nd:], c.cu_query_lens[m.nd:], m.out, scale=c.scale,
                                    k_scale=c.k_scale, v_scale=c.v_scale, sliding_window=c.window, stream=s_,
                                    prepare=True))
        # the prompt alone in the split form (query blocks planned over a workspace)
        pre_split.append(B.pa_prefill(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables[m.nd:],
                                      c.context_lens[m.nd:], c.cu_query_lens[m.nd:], m.out, ws_pre, scale=c.scale,
                                      cu_count=cu_count, k_scale=c.k_scale, v_scale=c.v_scale,
                                      sliding_window=c.window, stream=stream, prepare=True))
    n = len(batches)
    K = args.steps
    order = np.arange(K) % n

    def part(i, which):
        if which == "step":
            one[i]()
        elif which == "two_calls":
            pre[i]()
            dec[i]()
        elif which == "two_streams":
            side.wait_stream(stream)
            pre_side[i]()
            dec[i]()
            stream.wait_stream(side)
        elif which == "decode":
            dec[i]()
        elif which == "prefill":
            pre[i]()
        elif which == "prefill_split":
            pre_split[i]()

    def run(which, warm):
        return timed([lambda i=i: part(i, which) for i in order], stream,
                      [lambda i=i: part(i % n, which) for i in range(warm)])

    step_ms = run("step", args.warmup)
    c0, m0 = batches[0], steps[0]
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[c0.kv_dtype]
    per_key = c0.num_kv_heads * 2 * c0.head_dim * elem
    lens = c0.context_lens.cpu().numpy().astype(np.int64)
    all_bytes = np.full(n, float(lens.sum() * per_key))
    if args.step_only:
        head = rate(all_bytes, order, step_ms)
        return {"metric": "µs/step, mixed batch through the decode-first split (one pa_attention_mixed call)",
                "value": round(head["gbps"], 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
                "ms_per_step": round(head["ms_per_step"], 6), "us_per_step": round(head["us_per_step"], 2),
                "all_kv_bytes_per_step": float(all_bytes[0]),
                "decode_kv_bytes_per_step": float(lens[:m0.nd].sum() * per_key)}
    two_calls_ms = run("two_calls", 8)
    two_ms = run("two_streams", 8)
    dec_ms = run("decode", 8)
    pre_ms = run("prefill", 8)
    pre_split_ms = run("prefill_split", 8)
    dec_bytes = np.full(n, float(lens[:m0.nd].sum() * per_key))
    head = rate(all_bytes, order, step_ms)
    dec = rate(dec_bytes, order, dec_ms)
    return {
        "metric": "µs/step + achieved KV-read HBM GB/s (% peak), mixed batch through the decode-first split",
        "value": round(head["gbps"], 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"7 decodes at 16384 tokens + a new 100-token prompt, decodes first, Hq 12 / Hkv 2, "
                               f"D 256, page 16, bf16; {n} independent copies rotated",
                   "num_decodes": m0.nd, "decode_rows": m0.ndt, "threshold": 1,
                   "planner": {"budget": "2 x CU", "cu_count": cu_count, "max_partitions": 256, "tile_tokens": 256}},
        "us_per_step": round(head["us_per_step"], 2), "pct_hbm_peak": round(head["pct_peak"], 1),
        "step": "pa_split_decode_first on the host; pa_attention_mixed: the decodes (planned in place) and "
                "the prompt's query blocks in one launch, then pa_merge",
        "decode_part_us": round(dec["us_per_step"], 2), "prefill_part_us": round(pre_ms * 1e3 / K, 2),
        "prefill_part_split_form_us": round(pre_split_ms * 1e3 / K, 2),
        "two_calls_us_per_step": round(two_calls_ms * 1e3 / K, 2),
        "two_streams_us_per_step": round(two_ms * 1e3 / K, 2),
        "roofline": {"bound": "hbm", "achieved": round(dec["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec["gbps"] / HBM_PEAK_GBPS, 4), "traffic": counter_traffic("mixed"),
                     "traffic_gbps": traffic_gbps(counter_traffic("mixed"), dec["us_per_step"]),
                     "kernel": "pa_attention over the decode part (decode + merge launches)",
                     "duration_us": round(dec["us_per_step"], 2),
                     "algorithmic_bytes_per_launch": round(dec["mean_bytes"], 1)},
        "read_ceiling": read_ceiling(stream.device, cu_count),
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_case(c0, args.cpu_seconds,
                                                                             float(all_bytes[0])),
    }


def bench_prefill(args, batches, cu_count):
    """A prompt chunk behind a long prefix through pa_prefill alone: every query token of the chunk
    reads all the keys it sees.  Bytes counted: the request's K/V once (the algorithmic bytes); the
    rocprofv3 FETCH_SIZE of the same command gives the re-read factor of the query blocks.  One
    workspace serves the rotated copies (calls on one stream do not overlap)."""
    from paged_split_kv_amd import binding as B

    stream = torch.cuda.current_stream()
    n = len(batches)
    K = args.steps
    order = np.arange(K) % n
    outs = [torch.empty_like(c.q) for c in batches]
    c0 = batches[0]
    ws = torch.empty((B.pa_prefill_workspace_bytes(c0.num_rows, c0.num_seqs, c0.num_q_heads, c0.num_kv_heads,
                                                   c0.head_dim, cu_count),), dtype=torch.uint8, device=c0.q.device)
    calls = [B.pa_prefill(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, c.cu_query_lens,
                          outs[i], ws, scale=c.scale, cu_count=cu_count, sliding_window=c.window, prepare=True)
             for i, c in enumerate(batches)]
    ms = timed([lambda i=i: calls[i]() for i in order], stream, [lambda i=i: calls[i % n]() for i in range(args.warmup)])
    single = None
    if not args.step_only:
        one = [B.pa_prefill(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, c.cu_query_lens,
                            outs[i], scale=c.scale, sliding_window=c.window, prepare=True)
               for i, c in enumerate(batches)]
        single = timed([lambda i=i: one[i]() for i in order], stream, [lambda: one[0]()] * 4) * 1e3 / K
    kv = np.array([float(c.kv_bytes()) for c in batches])
    r = rate(kv, order, ms)
    G = c0.num_q_heads // c0.num_kv_heads
    flops = np.array([attention_flops(c.context_lens.cpu().numpy(), c.cu_query_lens.cpu().numpy(), c.num_q_heads,
                                      c.head_dim, c.window) for c in batches])
    tflops = float(flops[order].sum()) / (ms * 1e-3) / 1e12
    result = {
        "metric": "µs/step + achieved KV-read HBM GB/s (% peak), prompt chunk behind a long prefix (pa_prefill)",
        "value": round(r["gbps"], 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"one request: a {int(np.diff(c0.cu_query_lens.cpu().numpy())[0])}-token prompt chunk "
                               f"behind a {int(c0.context_lens[0].item()) - int(np.diff(c0.cu_query_lens.cpu().numpy())[0])}"
                               f"-token prefix, Hq {c0.num_q_heads} / Hkv {c0.num_kv_heads}, D {c0.head_dim}, page "
                               f"{c0.block_size}, bf16; {n} independent copies rotated",
                   "group": G},
        "us_per_step": round(r["us_per_step"], 2), "pct_hbm_peak": round(r["pct_peak"], 1),
        "step": "pa_prefill, split form: the chunk's query blocks cut and planned, each plan slot computed "
                "by the query-block kernel (waves share each K/V chunk through LDS), the slots merged "
                "(three launches)",
        "one_launch_form_us_per_step": None if single is None else round(single, 2),
        "tflops": round(tflops, 1),
        # 512 query tokens against 16.9k keys are a dense contraction: the matrix cores bound it
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": counter_traffic("prefill"),
                     "traffic_gbps": traffic_gbps(counter_traffic("prefill"), r["us_per_step"]),
                     "kernel": "pa_prefill (all three launches)",
                     "duration_us": round(r["us_per_step"], 3),
                     "algorithmic_flops_per_launch": round(float(flops[order].mean()), 1),
                     "algorithmic_bytes_per_launch": round(r["mean_bytes"], 1),
                     "note": "flops: 4 D per visible (query row, key) pair; bytes: the request's K/V once; "
                             "traffic: FETCH + WRITE of the query-block kernel"},
    }
    if not args.step_only:
        result["read_ceiling"] = read_ceiling(stream.device, cu_count)
    return result


# ------------------------------------------------------------------------------------------------
# the decode workloads
# ------------------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", dest="graph", action="store_true", default=True,
                    help="time a HIP-graph replay of the step set too (the default)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="skip the HIP-graph replay")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-step timing with the last-level cache evicted between steps")
    ap.add_argument("--step-only", action="store_true",
                    help="time only the headline step (for profiler runs: warm-up, then K steps)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device copy first (the reference kernel for the HBM counters)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in keys per query token (0 = none); the bytes counted are the "
                         "windowed ranges")
    ap.add_argument("--workload", choices=("skewed", "sparse", "long", "verify", "fp8", "mixed", "prefill"),
                    default="skewed",
                    help="skewed: the 32-request agentic batch (default, the headline metric); "
                         "sparse: 16 near-uniform top-k requests with a partition cap of 8; "
                         "long / verify / fp8: the other full-size configurations, reported beside it; "
                         "mixed: 7 decodes at 16k + a 100-token prompt through the decode-first split; "
                         "prefill: a 512-token prompt chunk behind a 16384-token prefix through pa_prefill")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode (it would shard by kv "
              "head, each GPU running the same op on its share of the heads)",
              file=sys.stderr)
        sys.exit(2)

    from paged_split_kv_amd import binding as B
    from paged_split_kv_amd import probe as P
    from paged_split_kv_amd import workloads as W
    from paged_split_kv_amd.runner import DecodeStep, PlanConfig

    B.load()
    P.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    win = args.window
    cu_count = B.pa_device_cu_count(0)
    pool = None
    T = 256
    if args.workload in ("skewed", "sparse"):
        print(f"[bench] building the 4 GiB page pool and the {args.workload} steps", file=sys.stderr, flush=True)
        if args.workload == "skewed":
            pool = W.skewed_pool(dev)
            max_parts = 256
        else:
            pool = W.skewed_pool(dev, steps=W.sparse_lengths(64, 16, seed=11))
            max_parts = 8
        batches = [W.Case(name=f"{args.workload}_{i}", q=pool.q[i], k_cache=pool.k_cache, v_cache=pool.v_cache,
                          kv_dtype="bf16", block_tables=pool.block_tables[i], context_lens=pool.context_lens[i],
                          cu_query_lens=None, max_q_len=1, scale=pool.scale)
                   for i in range(pool.steps.shape[0])]
        lens = [pool.steps[i] for i in range(len(batches))]
        qlens = [np.ones_like(x) for x in lens]
    else:
        # one named configuration; independent copies (own pages and values) are rotated so that
        # consecutive steps do not find each other's pages in the 256 MB last-level cache
        if args.workload == "mixed":
            make = lambda sd: W.make_mixed_case(device=dev, seed=sd)
            first = make(5)
        elif args.workload == "prefill":
            make = lambda sd: W.make_prefill_chunk_case(device=dev, seed=sd)
            first = make(6)
        else:
            name = {"long": "long_bf16", "verify": "verify_bf16", "fp8": "fp8_kv"}[args.workload]
            make = lambda sd: W.make_config(name, device=dev, seed=sd)
            first = make(None)
        copies = max(1, min(8, -(-(640 << 20) // first.kv_bytes())))
        print(f"[bench] building {copies} copies of the {args.workload} workload", file=sys.stderr, flush=True)
        batches = [first] + [make(1000 + c) for c in range(1, copies)]
        max_parts = 256
        lens = [c.context_lens.cpu().numpy() for c in batches]
        qlens = [np.ones_like(x) if c.cu_query_lens is None else np.diff(c.cu_query_lens.cpu().numpy())
                 for c, x in zip(batches, lens)]
    for c in batches:
        c.window = win
    if args.workload == "mixed":
        print(json.dumps(bench_mixed(args, batches, cu_count)), flush=True)
        return
    if args.workload == "prefill":
        print(json.dumps(bench_prefill(args, batches, cu_count)), flush=True)
        return
    nsteps = len(batches)
    c0 = batches[0]
    B_, Hq, D, Hkv = c0.num_seqs, c0.num_q_heads, c0.head_dim, c0.num_kv_heads
    cfg = PlanConfig(cu_count=cu_count, max_partitions=max_parts, tile_tokens=T)
    step = DecodeStep.for_case(c0, cfg)
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[c0.kv_dtype]

    def keys_read(S, L):
        """Keys a request reads: all S, or with a window the union of its tokens' windows."""
        return S - (np.maximum(0, S - (L - 1) - win) if win > 0 else 0)

    keys = np.array([keys_read(np.asarray(x, np.int64), np.asarray(l, np.int64)).sum()
                     for x, l in zip(lens, qlens)])
    kv_bytes = (keys * Hkv * 2 * D * elem).astype(np.float64)          # per step
    stream = torch.cuda.current_stream()
    K = args.steps
    order = step_order(K, nsteps)
    full_order = step_order(4 * nsteps, nsteps, seed=1)                # four whole passes

    # every step's plan, made once beforehand (as a forward shares one plan across its layers), with
    # the decode's dispatch order beside it
    plans, disps = [], []
    for c in batches:
        d = torch.empty((step.capacity, 4), dtype=torch.int32, device=dev)
        w, r, n = B.pa_plan(c.context_lens, Hkv, cu_count=cu_count, max_partitions=max_parts, tile_tokens=T,
                            capacity=step.capacity, cu_query_lens=c.cu_query_lens, sliding_window=win,
                            dispatch_info=d)
        plans.append((w, r, n))
        disps.append(d)
    torch.cuda.synchronize()
    ws, out = step.workspace, step.out

    def dec_call(i, prepare=True, dispatch=True):
        c, (w, r, n) = batches[i], plans[i]
        return B.pa_decode(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, w, n, ws,
                           scale=c.scale, cu_query_lens=c.cu_query_lens, max_q_len=c.max_q_len, k_scale=c.k_scale,
                           v_scale=c.v_scale, tile_tokens=T, sliding_window=win,
                           dispatch_info=disps[i] if dispatch else None, prepare=prepare)

    def mrg_call(i, prepare=True):
        c, (w, r, n) = batches[i], plans[i]
        return B.pa_merge(out, r, ws, capacity=step.capacity, cu_query_lens=c.cu_query_lens,
                          max_q_len=c.max_q_len, prepare=prepare)

    dec_p = [dec_call(i) for i in range(nsteps)]
    mrg_p = [mrg_call(i) for i in range(nsteps)]

    def headline(i):
        dec_p[i]()
        mrg_p[i]()

    warm = [lambda i=i: headline(i % nsteps) for i in range(args.warmup)]
    t0 = time.perf_counter()
    head_ms = timed([lambda i=i: headline(i) for i in order], stream, warm)
    wall = time.perf_counter() - t0
    head = rate(kv_bytes, order, head_ms)
    if args.workload == "skewed" and win == 0:
        metric = METRIC
        workload = ("skewed 32-request bf16 decode, Hq 16 / Hkv 2, D 128, page 16, 128 stratified steps "
                    "over a 4 GiB pool")
    elif args.workload == "skewed":
        metric = f"µs/step + achieved KV-read HBM GB/s (% peak), skewed 32-req bf16 decode, window {win}"
        workload = (f"skewed 32-request bf16 decode with a {win}-key sliding window, Hq 16 / Hkv 2, D 128, "
                    "page 16, 128 stratified steps over a 4 GiB pool; bytes = windowed keys")
    elif args.workload == "sparse":
        metric = "µs/step + achieved KV-read HBM GB/s (% peak), sparse top-k 16-req bf16 decode, cap 8"
        workload = ("sparse top-k bf16 decode: 16 requests of 2048 selected + 1..256 local tokens, "
                    "Hq 16 / Hkv 2, D 128, page 16, 64 steps over a 4 GiB pool, partition cap 8")
    else:
        desc = {"long": "one 131072-token bf16 request, Hq 16 / Hkv 2, D 128, page 64",
                "verify": "8 verify requests of 3 tokens + 7 single-token requests at 16384 tokens, bf16, "
                          "Hq 6 / Hkv 1, D 256, page 16, 2 padding rows",
                "fp8": "256 requests of 128..65536 tokens (log-normal), fp8 e4m3fn K/V with per-tensor "
                       "scales, bf16 q, Hq 16 / Hkv 2, D 128, page 16"}[args.workload]
        metric = f"µs/step + achieved KV-read HBM GB/s (% peak), {args.workload} workload"
        workload = f"{desc}; {nsteps} independent copies rotated" + (f"; window {win}" if win else "")
    result = {
        "metric": metric,
        "value": round(head["gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c0.kv_dtype if c0.kv_dtype != "fp8" else "fp8 KV, bf16 MFMA",
        "data": "synthetic",
        "config": {"workload": workload, "sliding_window": win, "num_seqs": B_, "max_q_len": c0.max_q_len,
                   "timed_steps": {"count": K, "distinct": head["distinct_steps"], "of": nsteps,
                                   "rule": "whole passes over every step in a seeded order, then the "
                                           "remainder at the set's quantiles (j + 1/2) / r",
                                   "mean_kv_bytes": round(head["mean_bytes"], 1),
                                   "set_mean_kv_bytes": round(float(kv_bytes.mean()), 1)},
                   "mean_keys_read_per_step": round(float(keys.mean()), 1),
                   "planner": {"budget": "2 x CU", "cu_count": cu_count, "max_partitions": max_parts,
                               "tile_tokens": T, "capacity": step.capacity}},
        "us_per_step": round(head["us_per_step"], 2),
        "pct_hbm_peak": round(head["pct_peak"], 1),
        "step": "pa_decode (in the plan's dispatch order) + pa_merge (two launches), each step's plan and "
                "dispatch order made once beforehand",
        "timed_wall_s": round(wall, 3),
    }
    if args.step_only:
        print(json.dumps(result), flush=True)
        return

    # the decode kernel alone, back to back over the same order (the roofline kernel); and in slot
    # order, without the plan's dispatch order
    dec_ms = timed([lambda i=i: dec_p[i]() for i in order], stream, [lambda: dec_p[0]()] * 8)
    dec = rate(kv_bytes, order, dec_ms)
    dec_s = [dec_call(i, dispatch=False) for i in range(nsteps)]
    dec_slot_ms = timed([lambda i=i: dec_s[i]() for i in order], stream, [lambda: dec_s[0]()] * 8)
    # the decode-shaped gather over the same plans and steps, its workgroups taking the slots in the
    # decode's dispatch order (the entries carry the slot's request and tile range first): the same
    # K/V bytes, no arithmetic; and the same gather in slot order
    sink = P.sink_for(4 * step.capacity * Hkv, dev)
    gat_p = [P.pa_probe_gather(c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, d, n, sink,
                               tile_tokens=T, prepare=True) for c, (w, r, n), d in zip(batches, plans, disps)]
    gat_ms = timed([lambda i=i: gat_p[i]() for i in order], stream, [lambda: gat_p[0]()] * 8)
    gat = rate(kv_bytes, order, gat_ms)
    gat_s = [P.pa_probe_gather(c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, w, n, sink,
                               tile_tokens=T, prepare=True) for c, (w, r, n) in zip(batches, plans)]
    gat_slot_ms = timed([lambda i=i: gat_s[i]() for i in order], stream, [lambda: gat_s[0]()] * 8)
    # where the decode shares the slots (every request one slot), the same gather over its pieces
    gat_pc = None
    if 0 < step.capacity <= B_ <= 256 and D <= 128:
        pcs = []
        for (w, r, n) in plans:
            used = int(n[0].item())
            ent, per = shared_slot_pieces(w.cpu().numpy(), used)
            pcs.append((torch.as_tensor(ent, device=dev),
                        torch.tensor([ent.shape[0], per], dtype=torch.int32, device=dev)))
        sink_pc = P.sink_for(4 * max(e.shape[0] for e, _ in pcs) * Hkv, dev)
        gat_pp = [P.pa_probe_gather(c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, e, nw, sink_pc,
                                    tile_tokens=T, prepare=True) for c, (e, nw) in zip(batches, pcs)]
        gat_pc = rate(kv_bytes, order, timed([lambda i=i: gat_pp[i]() for i in order], stream,
                                             [lambda: gat_pp[0]()] * 8))
    # the headline step over four whole passes of the set
    full = rate(kv_bytes, full_order, timed([lambda i=i: headline(i) for i in full_order], stream))
    # the plan alone (its per-forward refresh), the one-call and three-call forms, same order
    plan_p = [B.pa_plan(c.context_lens, Hkv, cu_count=cu_count, max_partitions=max_parts, tile_tokens=T,
                        capacity=step.capacity, work_info=step.work_info, reduce_info=step.reduce_info,
                        num_work=step.num_work, cu_query_lens=c.cu_query_lens, sliding_window=win,
                        dispatch_info=step.dispatch_info, prepare=True)
              for c in batches]
    plan_ms = timed([lambda i=i: plan_p[i]() for i in order], stream, [lambda: plan_p[0]()] * 8)
    att_p = [B.pa_attention(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, step.work_info,
                            step.reduce_info, step.num_work, ws, out, scale=c.scale, cu_count=cu_count,
                            max_partitions=max_parts, tile_tokens=T, cu_query_lens=c.cu_query_lens,
                            max_q_len=c.max_q_len, k_scale=c.k_scale, v_scale=c.v_scale, sliding_window=win,
                            prepare=True) for c in batches]
    att_ms = timed([lambda i=i: att_p[i]() for i in order], stream, [lambda: att_p[0]()] * 8)
    dec_3 = [B.pa_decode(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, step.work_info,
                         step.num_work, ws, scale=c.scale, cu_query_lens=c.cu_query_lens, max_q_len=c.max_q_len,
                         k_scale=c.k_scale, v_scale=c.v_scale, tile_tokens=T, sliding_window=win,
                         dispatch_info=step.dispatch_info, prepare=True)
             for c in batches]
    mrg_3 = [B.pa_merge(out, step.reduce_info, ws, capacity=step.capacity, cu_query_lens=c.cu_query_lens,
                        max_q_len=c.max_q_len, prepare=True) for c in batches]

    def three(i):
        plan_p[i]()
        dec_3[i]()
        mrg_3[i]()

    three_ms = timed([lambda i=i: three(i) for i in order], stream, [lambda: three(0)] * 8)

    # per-kernel durations with events around each launch of the headline step
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(len(order))]
    torch.cuda.synchronize()
    for e, i in zip(evs, order):
        e[0].record(stream)
        dec_p[i]()
        e[1].record(stream)
        mrg_p[i]()
        e[2].record(stream)
    torch.cuda.synchronize()
    ev_dec = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
    ev_mrg = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3

    graph = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        # at least 32 steps in the graph (whole passes over the step set), so that one replay's launch
        # is spread over as many steps as in the skewed set's graph
        in_graph = np.arange(nsteps * max(1, -(-32 // nsteps))) % nsteps
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in in_graph:
                    dec_call(int(i), prepare=False)
                    mrg_call(int(i), prepare=False)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = 4
        g_ms = timed([g.replay] * reps, stream)
        gr = rate(kv_bytes, np.tile(in_graph, reps), g_ms)
        graph = {"us_per_step": round(gr["us_per_step"], 2), "kv_gbps": round(gr["gbps"], 1),
                 "pct_peak": round(gr["pct_peak"], 1),
                 "replayed": f"{reps} replays of one graph holding {len(in_graph)} steps, whole passes over "
                             f"the {nsteps} of the set (decode + merge each)"}

    cold = None
    if args.workload == "skewed" and not args.no_cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def per_step(evict):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(nsteps)]
            for i in range(nsteps):
                if evict:
                    scratch.fill_(i & 0xff)
                ev[i][0].record(stream)
                headline(i)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3

        per_step(True)
        t_cold, t_warm = per_step(True), per_step(False)
        del scratch
        cold = {"steps": nsteps,
                "evicted_us_mean": round(float(t_cold.mean()), 2),
                "evicted_us_p50": round(float(np.median(t_cold)), 2),
                "evicted_us_p90": round(float(np.quantile(t_cold, 0.9)), 2),
                "evicted_kv_gbps": round(float(kv_bytes.sum()) / (float(t_cold.sum()) * 1e-6) / 1e9, 1),
                "not_evicted_us_mean": round(float(t_warm.mean()), 2),
                "note": "each step (decode + merge) between its own events; 512 MB written before each "
                        "evicted step, outside its events"}

    traffic = counter_traffic(args.workload) if win == 0 else None
    rc = read_ceiling(dev, cu_count)
    result.update({
        "full_set": {"steps": full["steps"], "distinct": full["distinct_steps"],
                     "us_per_step": round(full["us_per_step"], 2), "kv_gbps": round(full["gbps"], 1),
                     "pct_peak": round(full["pct_peak"], 1),
                     "note": "the headline step over four whole passes of every step, seeded order"},
        "pa_plan_us": round(plan_ms * 1e3 / K, 2),
        "plan_decode_merge_us_per_step": round(three_ms * 1e3 / K, 2),
        "pa_attention_us_per_step": round(att_ms * 1e3 / K, 2),
        "kernel_us": {"pa_decode_back_to_back": round(dec["us_per_step"], 2),
                      "pa_decode_in_slot_order": round(dec_slot_ms * 1e3 / K, 2),
                      "decode_shaped_gather_back_to_back": round(gat["us_per_step"], 2),
                      "decode_shaped_gather_in_slot_order": round(gat_slot_ms * 1e3 / K, 2),
                      "decode_shaped_gather_over_shared_slot_pieces":
                          None if gat_pc is None else round(gat_pc["us_per_step"], 2),
                      "evented": {"pa_decode": round(float(ev_dec.mean()), 2),
                                  "pa_merge": round(float(ev_mrg.mean()), 2),
                                  "step_p50": round(float(np.median(ev_dec + ev_mrg)), 2),
                                  "step_p90": round(float(np.quantile(ev_dec + ev_mrg, 0.9)), 2)}},
        "roofline": {"bound": "hbm", "achieved": round(dec["gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "traffic_gbps": traffic_gbps(traffic, dec["us_per_step"]),
                     "kernel": "pa_decode",
                     "duration_us": round(dec["us_per_step"], 3),
                     "algorithmic_bytes_per_launch": round(dec["mean_bytes"], 1),
                     "launches": K},
        "ceilings": {"read": rc,
                     "decode_shaped_gather": {"gbps": round(gat["gbps"], 1), "pct_peak": round(gat["pct_peak"], 1),
                                              "us_per_launch": round(gat["us_per_step"], 2),
                                              "kernel": "pa_probe_gather: the decode's K/V bytes over the same "
                                                        "plans and step order, its launch shape and dispatch "
                                                        "order, no arithmetic"},
                     "decode_shaped_gather_over_shared_slot_pieces": None if gat_pc is None else {
                         "gbps": round(gat_pc["gbps"], 1), "pct_peak": round(gat_pc["pct_peak"], 1),
                         "us_per_launch": round(gat_pc["us_per_step"], 2),
                         "kernel": "pa_probe_gather over the pieces the decode streams when every request is "
                                   "one slot (shared slots), in piece order, no arithmetic"},
                     "decode_pct_of_gather": round(100.0 * dec["gbps"] / (gat if gat_pc is None else gat_pc)["gbps"], 1),
                     "decode_pct_of_read": round(100.0 * dec["gbps"] / rc["gbps"], 1),
                     "step_pct_of_read": round(100.0 * head["gbps"] / rc["gbps"], 1)},
        "hip_graph": graph,
        "cold_cache": cold,
        "cpu_baseline": None,
    })
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        if pool is not None:
            cb = cpu_baseline_pool(pool, args.cpu_seconds, win)
        else:
            cb = cpu_baseline_case(c0, min(args.cpu_seconds, 10.0), float(kv_bytes[0]))
        if args.workload == "skewed" and win == 0:
            cb["per_config"] = cpu_oracle_per_config(dev)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
