"""bench.py's command-line contract on the host: more than one GPU is refused with a message before
any device work, and the JSON fields the benchmark line carries are the ones its docstring names."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_distributed_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_workloads_and_options():
    r = _run(["--help"])
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--gpus", "--workload", "--window", "--graph", "--no-graph",
                "--no-cold", "--no-cpu-baseline", "--step-only"):
        assert opt in r.stdout
    for w in ("skewed", "sparse", "long", "verify", "fp8", "mixed", "prefill"):
        assert w in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_step_order_samples_the_whole_set():
    import numpy as np
    bench = _bench_module()
    n = 128
    # fewer steps than the set: a stratified sample, the j-th smallest index at quantile (j + 1/2) / K
    for K in (1, 5, 20, 100, 127):
        order = bench.step_order(K, n)
        assert len(order) == K and len(np.unique(order)) == K
        target = (np.arange(K) + 0.5) * n / K
        assert (np.abs(np.sort(order) - target) < 1.0).all(), K
    # whole passes: every step equally often; a remainder adds a stratified sample
    for K in (128, 512, 300):
        order = bench.step_order(K, n)
        counts = np.bincount(order, minlength=n)
        assert len(order) == K
        assert counts.min() >= K // n and counts.max() <= K // n + 1
    # the same K gives the same order
    assert (bench.step_order(20, n) == bench.step_order(20, n)).all()


def test_rate_counts_exactly_the_timed_steps():
    import numpy as np
    bench = _bench_module()
    rng = np.random.default_rng(3)
    per_step = rng.uniform(50e6, 400e6, size=128)        # bytes of each step of the set, unequal
    for K in (20, 128, 200):
        order = bench.step_order(K, 128)
        r = bench.rate(per_step, order, total_ms=K * 0.045)
        assert abs(r["mean_bytes"] - per_step[order].mean()) <= 1e-6 * r["mean_bytes"]
        # value x ms_per_step = mean bytes of the timed steps
        assert abs(r["gbps"] * 1e9 * r["ms_per_step"] * 1e-3 - per_step[order].mean()) <= 1e-6 * r["mean_bytes"]
        assert abs(r["pct_peak"] - 100 * r["gbps"] / bench.HBM_PEAK_GBPS) < 1e-9
    # a stratified sample of 20 stays near the set's mean, where the first 20 of a sorted set would not
    sorted_bytes = np.sort(per_step)
    r20 = bench.rate(sorted_bytes, bench.step_order(20, 128), 1.0)
    assert abs(r20["mean_bytes"] / sorted_bytes.mean() - 1) < 0.05
    assert sorted_bytes[:20].mean() / sorted_bytes.mean() < 0.7


def test_attention_flops_counts_each_visible_pair():
    """Matrix-core flops of the prefill bench: 4 D per visible (query row, key) pair, counted here by
    brute force over the tokens of small requests, with and without a window."""
    import numpy as np
    bench = _bench_module()
    rng = np.random.default_rng(5)
    for _ in range(20):
        B = int(rng.integers(1, 5))
        L = rng.integers(0, 40, size=B)
        S = L + rng.integers(0, 300, size=B)
        cu = np.concatenate([[0], np.cumsum(L)])
        hq, d = int(rng.choice([4, 12])), int(rng.choice([64, 256]))
        for W in (0, 1, 17, 1000):
            pairs = 0
            for b in range(B):
                for i in range(int(L[b])):
                    n = int(S[b]) - (int(L[b]) - 1 - i)
                    keys = range(max(n - W, 0) if W else 0, n)
                    pairs += len(keys)
            assert bench.attention_flops(S, cu, hq, d, W) == 4.0 * d * hq * pairs


def test_shared_slot_pieces_cover_each_slot_once():
    """The piece-shaped gather reads what the decode streams under shared slots: every slot's tiles
    exactly once, in slot order, in at most (factor + 1) x used pieces of at most `per` tiles."""
    import numpy as np
    bench = _bench_module()
    rng = np.random.default_rng(7)
    for _ in range(50):
        used = int(rng.integers(1, 257))
        n = rng.integers(1, 300, size=used)
        t0 = rng.integers(0, 50, size=used)
        w = np.zeros((used + int(rng.integers(0, 5)), 4), dtype=np.int32)
        w[:used, 0] = np.arange(used)
        w[:used, 1] = t0
        w[:used, 2] = t0 + n
        w[used:, 0] = -1
        ent, per = bench.shared_slot_pieces(w, used)
        assert per == max(1, -(-(int(n.sum()) + used) // (2 * used)))
        assert len(ent) <= 3 * used
        sizes = ent[:, 2] - ent[:, 1]
        assert (sizes >= 0).all() and (sizes <= per).all()
        for s in range(used):
            mine = ent[ent[:, 0] == s]
            # consecutive, contiguous, covering [t0, t0 + n) exactly
            assert mine[0, 1] == t0[s] and mine[-1, 2] == t0[s] + n[s]
            assert (mine[1:, 1] == mine[:-1, 2]).all()
        assert (np.diff(ent[:, 0]) >= 0).all()
