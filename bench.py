"""Benchmark of the paged split-KV decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--graph] [--no-cold]

Workload: the skewed 32-request bf16 decode (Hq 16 / Hkv 2, D 128, pages of 16 tokens).  128 decode
steps whose in-batch max/min context ratio follows the agentic trace (p50 ~2.5, p90 ~21); every step
draws its pages at random from a 4 GiB K/V pool, so the 256 MB last-level cache cannot hold a step's
data across steps.  One timed step = one pa_attention call over one batch (plan, decode and merge; the
decode launch plans in place, so two launches), inputs resident in HBM.  value = KV bytes read / step
time (GB/s).  The three-call form (pa_plan + pa_decode + pa_merge) and the form with the merge inside
the decode launch are timed too and reported beside it, and so is each step between its own events
with the 256 MB last-level cache evicted before it (a 512 MB write outside the events) and without.
A 1 GiB device copy gives the box's measured copy ceiling beside the 8 TB/s peak, and the CPU oracle
is timed on a bounded sample of every workload (cpu_baseline).

The roofline object is for the decode kernel: algorithmic bytes (sum of context lengths x Hkv x 2 x D
x 2 bytes per launch, averaged over the batches) over its average launch duration, measured with HIP
events on the launch stream around K pa_decode launches issued back to back over the batches, each
with its own plan made beforehand.
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
METRIC = "µs/step + achieved KV-read HBM GB/s (% peak), skewed 32-req bf16 decode"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_skewed_bf16_counters.json")
DECODE_SRC = os.path.join(ROOT, "paged_split_kv_amd", "csrc", "pa_decode.hip")


def decode_source_sha() -> str:
    with open(DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was taken on
    the current decode source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("decode_source_sha") != decode_source_sha():
        return None
    return c.get("traffic_bytes_per_launch")


def cpu_baseline(pool, budget_s: float, max_steps: int, window: int = 0):
    """The CPU oracle (direct fp64 attention over the gathered pages) on a bounded sample of steps."""
    import oracle

    threads = oracle.default_threads()
    done_bytes = 0
    spent = 0.0
    n = 0
    picks = np.random.default_rng(0).permutation(len(pool.steps))
    for i in picks[:max_steps]:
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
        t0 = time.perf_counter()
        oracle.attention_direct(q, "bf16", k, v, "bf16", remap, ctx.astype(np.int32), None, pool.scale,
                                threads=threads, window=window)
        spent += time.perf_counter() - t0
        keys = np.minimum(ctx, window) if window > 0 else ctx
        done_bytes += int(keys.sum()) * k.shape[1] * 2 * k.shape[3] * 2
        n += 1
        if spent >= budget_s:
            break
    # the oracle splits the work into (request, kv head) tasks: no more threads than tasks are busy
    used = min(threads, len(pool.steps[0]) * pool.k_cache.shape[1])
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "us_per_step": round(spent / n * 1e6, 1),
            "sample": f"{n} of the {len(pool.steps)} steps (seeded random order, stopped after "
                      f"{budget_s:.0f} s), fp64 direct attention over the gathered pages, {spent:.1f} s"}


def cpu_baseline_case(case, budget_s: float, kv_bytes: float):
    """The CPU oracle (direct fp64 attention) on one full-size configuration, repeated while the
    budget lasts (at least once); the host copy of the case is made before the clock starts."""
    import oracle

    threads = oracle.default_threads()
    h = case.host()
    spent, n = 0.0, 0
    while n == 0 or spent < budget_s:
        t0 = time.perf_counter()
        oracle.attention_direct(h["q"], case.q_dtype, h["k_cache"], h["v_cache"], case.kv_dtype,
                                h["block_tables"], h["context_lens"], h["cu_query_lens"], case.scale,
                                case.k_scale, case.v_scale, threads=threads, window=case.window)
        spent += time.perf_counter() - t0
        n += 1
    used = min(threads, case.num_seqs * case.num_kv_heads)   # busy threads: one (request, kv head) task each
    return {"value": round(kv_bytes * n / spent / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle", "us_per_step": round(spent / n * 1e6, 1),
            "sample": f"{n} run(s) of the whole configuration (one batch), fp64 direct attention over the "
                      f"gathered pages, {spent:.1f} s"}


def copy_ceiling(dev) -> dict:
    """A device-to-device copy of 1 GiB (torch's copy kernel), best of 10: read + written bytes over
    time, the box's measured streaming ceiling beside the 8 TB/s published peak."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(10):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return {"gbps": round(2 * n / (best * 1e-3) / 1e9, 1), "bytes_moved": 2 * n,
            "kernel": "torch copy_, 1 GiB device to device, best of 10"}


def bench_mixed(args, batches, cu_count):
    """The decode-first split of a mixed batch: one pa_attention_mixed call per step (decode and
    prompt in one launch, then the merge); the two-call form (pa_prefill, then pa_attention), the
    same on two streams, and the parts alone are timed beside it."""
    from paged_split_kv_amd import binding as B
    from paged_split_kv_amd.runner import MixedStep, PlanConfig

    stream = torch.cuda.current_stream()
    steps = [MixedStep(c, 1, PlanConfig(cu_count=cu_count), concurrent=True) for c in batches]
    m_side = [m.side for m in steps]
    for m in steps:
        m.side = None                  # the two-call forms run on one stream unless timed otherwise
    n = len(batches)
    K = args.steps

    def part(i, which):
        c, m = batches[i % n], steps[i % n]
        if which == "step":
            m.one_call = True
            m.run(c, stream)
            m.one_call = False
            return
        if which == "two_calls":
            m.run(c, stream)
            return
        if which == "two_streams":
            m.side = m_side[i % n]
            m.run(c, stream)
            m.side = None
            return
        if which == "decode" and m.dec is not None:
            m.dec.attention(c.q[:m.ndt], c.k_cache, c.v_cache, c.kv_dtype, c.block_tables[:m.nd],
                            c.context_lens[:m.nd], scale=c.scale, cu_query_lens=c.cu_query_lens[:m.nd + 1],
                            sliding_window=c.window)
        if which == "prefill":
            B.pa_prefill(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables[m.nd:], c.context_lens[m.nd:],
                         c.cu_query_lens[m.nd:], m.out, scale=c.scale, sliding_window=c.window)

    def timed(which, warm):
        for i in range(warm):
            part(i, which)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            part(i, which)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K

    step_ms = timed("step", args.warmup)
    two_calls_ms = timed("two_calls", 8)
    two_ms = timed("two_streams", 8)
    dec_ms = timed("decode", 8)
    pre_ms = timed("prefill", 8)
    c0, m0 = batches[0], steps[0]
    ceil = copy_ceiling(stream.device)
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[c0.kv_dtype]
    per_key = c0.num_kv_heads * 2 * c0.head_dim * elem
    lens = c0.context_lens.cpu().numpy().astype(np.int64)
    dec_bytes = float(lens[:m0.nd].sum() * per_key)
    all_bytes = float(lens.sum() * per_key)
    gbps = all_bytes / (step_ms * 1e-3) / 1e9
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9
    return {
        "metric": "µs/step + achieved KV-read HBM GB/s (% peak), mixed batch through the decode-first split",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"7 decodes at 16384 tokens + a new 100-token prompt, decodes first, Hq 12 / Hkv 2, "
                               f"D 256, page 16, bf16; {n} independent copies rotated",
                   "num_decodes": m0.nd, "decode_rows": m0.ndt, "threshold": 1,
                   "planner": {"budget": "2 x CU", "cu_count": cu_count, "max_partitions": 256, "tile_tokens": 256}},
        "us_per_step": round(step_ms * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 1),
        "step": "pa_split_decode_first on the host; pa_attention_mixed: the decodes (planned in place) and "
                "the prompt's query blocks in one launch, then pa_merge",
        "decode_part_us": round(dec_ms * 1e3, 2), "prefill_part_us": round(pre_ms * 1e3, 2),
        "two_calls_us_per_step": round(two_calls_ms * 1e3, 2),
        "two_streams_us_per_step": round(two_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "pa_attention over the decode part (decode + merge launches)",
                     "duration_us": round(dec_ms * 1e3, 2), "algorithmic_bytes_per_launch": round(dec_bytes, 1)},
        "copy_ceiling": ceil,
        "pct_of_copy_ceiling": {"step": round(100.0 * gbps / ceil["gbps"], 1)},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_case(c0, args.cpu_seconds, all_bytes),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--graph", action="store_true", help="also time a HIP-graph replay of the steps")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the per-step timing with the last-level cache evicted between steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a 1 GiB device copy first (reference kernel for the HBM counters)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in keys per query token (0 = none); the bytes counted are the "
                         "windowed ranges")
    ap.add_argument("--workload", choices=("skewed", "sparse", "long", "verify", "fp8", "mixed"),
                    default="skewed",
                    help="skewed: the 32-request agentic batch (default, the headline metric); "
                         "sparse: 16 near-uniform top-k requests with a partition cap of 8; "
                         "long / verify / fp8: the other full-size configurations, reported beside it; "
                         "mixed: 7 decodes at 16k + a 100-token prompt through the decode-first split")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU mode (it would shard by kv "
              "head, each GPU running the same op on its share of the heads)",
              file=sys.stderr)
        sys.exit(2)

    from paged_split_kv_amd import binding as B
    from paged_split_kv_amd import workloads as W
    from paged_split_kv_amd.runner import DecodeStep, MixedStep, PlanConfig

    B.load()
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
    if args.workload in ("skewed", "sparse"):
        print(f"[bench] building the 4 GiB page pool and the {args.workload} steps", file=sys.stderr, flush=True)
        if args.workload == "skewed":
            pool = W.skewed_pool(dev)
            max_parts = 256
        else:
            pool = W.skewed_pool(dev, steps=W.sparse_lengths(64, 16, seed=11))
            max_parts = 8
        batches = [W.Case(f"{args.workload}_{i}", pool.q[i], pool.k_cache, pool.v_cache, "bf16",
                          pool.block_tables[i], pool.context_lens[i], None, 1, pool.scale)
                   for i in range(pool.steps.shape[0])]
        lens = [pool.steps[i] for i in range(len(batches))]
        qlens = [np.ones_like(x) for x in lens]
    else:
        # one named configuration; independent copies (own pages and values) are rotated so that
        # consecutive steps do not find each other's pages in the 256 MB last-level cache
        if args.workload == "mixed":
            name = "mixed_7x16k_prompt100"
            make = lambda sd: W.make_mixed_case(device=dev, seed=sd)
        else:
            name = {"long": "long_bf16", "verify": "verify_bf16", "fp8": "fp8_kv"}[args.workload]
            make = lambda sd: W.make_config(name, device=dev, seed=sd)
        first = make(None) if args.workload != "mixed" else make(5)
        copies = max(1, min(8, -(-(640 << 20) // first.kv_bytes())))
        print(f"[bench] building {copies} copies of {name}", file=sys.stderr, flush=True)
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
    nsteps = len(batches)
    c0 = batches[0]
    B_, Hq, D, Hkv = c0.num_seqs, c0.num_q_heads, c0.head_dim, c0.num_kv_heads
    step = DecodeStep.for_case(c0, PlanConfig(cu_count=cu_count, max_partitions=max_parts))
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[c0.kv_dtype]

    def keys_read(S, L):
        """Keys a request reads: all S, or with a window the union of its tokens' windows."""
        return S - (np.maximum(0, S - (L - 1) - win) if win > 0 else 0)

    keys = np.array([keys_read(np.asarray(x, np.int64), np.asarray(l, np.int64)).sum()
                     for x, l in zip(lens, qlens)])
    kv_bytes = keys * Hkv * 2 * D * elem                                    # per step
    stream = torch.cuda.current_stream()

    def run(i, ev=None, mode="attention"):
        """One step over batch i.  attention: one pa_attention call (the decode plans in place, then
        the merge: two launches).  three: pa_plan, pa_decode writing partial states, pa_merge.
        fused: pa_plan, then pa_decode with the merge inside its launch."""
        c = batches[i % nsteps]
        if mode == "attention":
            step.attention(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens,
                           scale=c.scale, cu_query_lens=c.cu_query_lens, k_scale=c.k_scale,
                           v_scale=c.v_scale, sliding_window=win)
            return
        if ev is not None:
            ev[0].record(stream)
        step.plan(c.context_lens, cu_query_lens=c.cu_query_lens, sliding_window=win)
        if ev is not None:
            ev[1].record(stream)
        step.decode(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, scale=c.scale,
                    cu_query_lens=c.cu_query_lens, k_scale=c.k_scale, v_scale=c.v_scale,
                    merge=mode == "fused", sliding_window=win)
        if ev is not None:
            ev[2].record(stream)
        if mode == "three":
            step.merge(c.cu_query_lens)
        if ev is not None:
            ev[3].record(stream)

    def timed(mode, warm=8):
        for i in range(warm):
            run(i, mode=mode)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            run(i, mode=mode)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    K = args.steps
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # the timed region: K steps of the whole path, synchronised on both sides
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        run(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    plain_ms = start.elapsed_time(end)
    bytes_done = float(sum(kv_bytes[i % nsteps] for i in range(K)))

    # per-kernel durations: the three-call form of the same steps with events around each launch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for i in range(8):
        run(i, mode="three")
    torch.cuda.synchronize()
    for i in range(K):
        run(i, evs[i], mode="three")
    torch.cuda.synchronize()
    plan_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    mrg_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = plan_ms + dec_ms + mrg_ms

    # the decode kernel alone: launches back to back over the batches, each with its own plan made
    # beforehand, so consecutive launches read different pages and no event sits between them
    plans = []
    for c in batches:
        w, r, n = B.pa_plan(c.context_lens, Hkv, cu_count=cu_count, max_partitions=max_parts,
                            capacity=step.capacity, cu_query_lens=c.cu_query_lens, sliding_window=win)
        plans.append((w, n))
    torch.cuda.synchronize()

    def decode_only(i):
        c = batches[i % nsteps]
        w, n = plans[i % nsteps]
        B.pa_decode(c.q, c.k_cache, c.v_cache, c.kv_dtype, c.block_tables, c.context_lens, w, n, step.workspace,
                    scale=c.scale, cu_query_lens=c.cu_query_lens, max_q_len=c.max_q_len, k_scale=c.k_scale,
                    v_scale=c.v_scale, sliding_window=win)

    for i in range(8):
        decode_only(i)
    da = torch.cuda.Event(enable_timing=True)
    db = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    da.record(stream)
    for i in range(K):
        decode_only(i)
    db.record(stream)
    torch.cuda.synchronize()
    decode_ms = da.elapsed_time(db) / K

    three_ms = timed("three")          # pa_plan + pa_decode + pa_merge, no events in between
    fused_ms = timed("fused")          # pa_plan + pa_decode with the merge in its launch

    graph = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(nsteps):
                    run(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gs = torch.cuda.Event(enable_timing=True)
        ge = torch.cuda.Event(enable_timing=True)
        reps = max(1, K // nsteps)
        gs.record(stream)
        for _ in range(reps):
            g.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        g_ms = gs.elapsed_time(ge) / (reps * nsteps)
        graph = {"us_per_step": round(g_ms * 1e3, 2),
                 "kv_gbps": round(float(kv_bytes.mean()) / (g_ms * 1e-3) / 1e9, 1)}

    # one step per batch with events around it, each after a 512 MB write that evicts the 256 MB
    # last-level cache (outside the events), and the same without the write
    cold = None
    if args.workload == "skewed" and not args.no_cold:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def per_step(evict):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(nsteps)]
            for i in range(nsteps):
                if evict:
                    scratch.fill_(i & 0xff)
                evs[i][0].record(stream)
                run(i)
                evs[i][1].record(stream)
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in evs]) * 1e3

        per_step(True)                                # warm-up of the pattern
        t_cold, t_warm = per_step(True), per_step(False)
        del scratch
        cold = {"steps": nsteps,
                "evicted_us_mean": round(float(t_cold.mean()), 2),
                "evicted_us_p50": round(float(np.median(t_cold)), 2),
                "evicted_us_p90": round(float(np.quantile(t_cold, 0.9)), 2),
                "evicted_kv_gbps": round(float(kv_bytes.mean()) / (float(t_cold.mean()) * 1e-6) / 1e9, 1),
                "not_evicted_us_mean": round(float(t_warm.mean()), 2),
                "note": "pa_attention per step between its own events; 512 MB written before each "
                        "evicted step, outside its events"}

    us_step = plain_ms * 1e3 / K
    gbps = bytes_done / (plain_ms * 1e-3) / 1e9
    dec_gbps = float(kv_bytes.mean()) / (decode_ms * 1e-3) / 1e9
    traffic = counter_traffic()
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
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(plain_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c0.kv_dtype if c0.kv_dtype != "fp8" else "fp8 KV, bf16 MFMA",
        "data": "synthetic",
        "config": {"workload": workload, "sliding_window": win,
                   "num_seqs": B_, "max_q_len": c0.max_q_len,
                   "mean_tokens_per_step": round(float(np.mean([x.sum() for x in lens])), 1),
                   "mean_keys_read_per_step": round(float(keys.mean()), 1),
                   "planner": {"budget": "2 x CU", "cu_count": cu_count, "max_partitions": max_parts,
                               "tile_tokens": 256}},
        "us_per_step": round(us_step, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 1),
        "step": "pa_attention: the decode launch plans in place, then pa_merge",
        "three_call_us_per_step": round(three_ms * 1e3 / K, 2),
        "merge_in_decode_launch_us_per_step": round(fused_ms * 1e3 / K, 2),
        "evented_three_call_us_p50": round(float(np.median(step_ms)) * 1e3, 2),
        "evented_three_call_us_p90": round(float(np.quantile(step_ms, 0.9)) * 1e3, 2),
        "kernel_us": {"pa_decode_back_to_back": round(decode_ms * 1e3, 2),
                      "evented": {"pa_plan": round(float(plan_ms.mean()) * 1e3, 2),
                                  "pa_decode": round(float(dec_ms.mean()) * 1e3, 2),
                                  "pa_merge": round(float(mrg_ms.mean()) * 1e3, 2)}},
        "timed_wall_s": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic if args.workload == "skewed" and win == 0 else None,
                     "kernel": "pa_decode",
                     "duration_us": round(decode_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": round(float(kv_bytes.mean()), 1)},
        "hip_graph": graph,
        "cold_cache": cold,
        "cpu_baseline": None,
    }
    ceil = copy_ceiling(dev)
    result["copy_ceiling"] = ceil
    result["pct_of_copy_ceiling"] = {"step": round(100.0 * gbps / ceil["gbps"], 1),
                                     "decode_kernel": round(100.0 * dec_gbps / ceil["gbps"], 1)}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if pool is not None:
            result["cpu_baseline"] = cpu_baseline(pool, args.cpu_seconds, nsteps, win)
        else:
            result["cpu_baseline"] = cpu_baseline_case(c0, min(args.cpu_seconds, 10.0), float(kv_bytes[0]))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
