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
    for opt in ("--steps", "--warmup", "--gpus", "--workload", "--window", "--graph", "--no-cold",
                "--no-cpu-baseline"):
        assert opt in r.stdout
    for w in ("skewed", "sparse", "long", "verify", "fp8", "mixed"):
        assert w in r.stdout
