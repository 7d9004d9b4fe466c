"""The oracle's pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of oracle/pa_oracle.c (a dropped term, a wrong sign,
index or bias, an off-by-one range, a transposed layout), builds the copy with the oracle's own gcc
line and runs the oracle pin tests against it in a child process (the oracle loads the library
named by PA_ORACLE_LIB).  A case passes when at least one pin fails on the planted mistake.  The
unmodified source, built the same way, must pass every pin, so a failure of the harness itself is
not mistaken for a caught mistake.  Everything here runs on the CPU.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(REPO, "oracle", "pa_oracle.c")
PIN_FILES = ["tests/test_oracle_planner.py", "tests/test_oracle_attention.py"]

# (name, text in pa_oracle.c, replacement).  Each text occurs exactly once in the source.
MUTATIONS = [
    # element decoding
    ("bf16_wrong_shift", "uint32_t w = ((uint32_t)bits) << 16;", "uint32_t w = ((uint32_t)bits) << 15;"),
    ("fp8_normal_bias_8", "mag = ldexp(1.0 + (double)man / 8.0, exp - 7);",
     "mag = ldexp(1.0 + (double)man / 8.0, exp - 8);"),
    ("fp8_subnormal_exponent", "mag = ldexp((double)man / 8.0, 1 - 7);",
     "mag = ldexp((double)man / 8.0, 0 - 7);"),
    ("fp8_nan_code_finite", "if (exp == 0xF && man == 0x7) return NAN;", ""),
    ("fp8_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    # attention arithmetic
    ("kv_head_interleaved", "const int g = h / G;", "const int g = h % p->num_kv_heads;"),
    ("softmax_scale_dropped", "double s = p->scale * dot;", "double s = dot;"),
    ("k_scale_dropped", "orc_cache_index(p, blk, g, slot, d)) * p->k_scale)",
     "orc_cache_index(p, blk, g, slot, d)))"),
    ("v_scale_dropped", "orc_cache_index(p, blk, g, slot, d)) * p->v_scale)",
     "orc_cache_index(p, blk, g, slot, d)))"),
    ("exp_base_2", "double w = exp(scores[pos - lo] - m);", "double w = exp2(scores[pos - lo] - m);"),
    ("direct_not_normalised", "for (int d = 0; d < D; ++d) o[d] = acc[d] / l;",
     "for (int d = 0; d < D; ++d) o[d] = acc[d];"),
    ("cache_layout_transposed", "return ((block * p->num_kv_heads + g) * p->block_size + slot)",
     "return ((block * p->block_size + slot) * p->num_kv_heads + g)"),
    ("causal_range_short_by_one", "return S - (int64_t)(L - 1 - i);", "return S - (int64_t)(L - i);"),
    ("window_one_key_wide", "return n - p->window > 0 ? n - p->window : 0;",
     "return n - p->window - 1 > 0 ? n - p->window - 1 : 0;"),
    ("rows_owner_inclusive_end", "if (r >= r0 && r < r0 + qlen)", "if (r >= r0 && r <= r0 + qlen)"),
    # log-sum-exp merge of partials
    ("merge_unweighted_sums", "den += f * pl[j];", "den += pl[j];"),
    ("merge_unweighted_values", "for (int d = 0; d < D; ++d) o[d] += f * pacc[(int64_t)j * D + d];",
     "for (int d = 0; d < D; ++d) o[d] += pacc[(int64_t)j * D + d];"),
    ("split_ignores_causal_limit", "if (hi > n) hi = n;", ""),
    ("split_ignores_window", "if (lo < orc_window_start(p, n)) lo = orc_window_start(p, n);", ""),
    # planner
    ("capacity_no_batch_floor", "int64_t b = num_seqs > budget ? num_seqs : budget;", "int64_t b = budget;"),
    ("capacity_ignores_kv_heads",
     "int64_t budget = orc_ceil_div((int64_t)budget_mult * cu_count, num_kv_heads);",
     "int64_t budget = (int64_t)budget_mult * cu_count;"),
    ("share_rounded_up", "parts = 1 + (extra * len) / total;",
     "parts = 1 + (extra * len + total - 1) / total;"),
    ("share_without_base_partition", "parts = 1 + (extra * len) / total;", "parts = (extra * len) / total + (len > 0 && extra == 0);"),
    ("partition_clamp_dropped", "if (parts > max_partitions) parts = max_partitions;", ""),
    ("partition_begin_rounded_up", "w[1] = (int32_t)(t0 + (j * tiles) / parts);",
     "w[1] = (int32_t)(t0 + (j * tiles + parts - 1) / parts);"),
    ("tiles_from_length", "int64_t tiles = len > 0 ? orc_ceil_div(s, tile_tokens) - t0 : 0;",
     "int64_t tiles = len > 0 ? orc_ceil_div(len, tile_tokens) : 0;"),
    ("read_start_without_verify_tokens", "int64_t lo = S - (int64_t)(L - 1) - window;",
     "int64_t lo = S - window;"),
    ("largest_slot_not_tracked", "if (w[2] - w[1] > largest) largest = w[2] - w[1];", ""),
    ("unused_slots_not_marked", "work_info[4 * w + 0] = -1;", "work_info[4 * w + 0] = 0;"),
]


def _run_pins(lib_path: str) -> tuple[int, str]:
    env = dict(os.environ)
    env["PA_ORACLE_LIB"] = lib_path
    env["OMP_NUM_THREADS"] = "2"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *PIN_FILES]
    res = subprocess.run(cmd, cwd=REPO, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout[-3000:] + res.stderr[-2000:]


def _build(tmp_dir: str, name: str, text: str) -> str:
    src = os.path.join(tmp_dir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text)
    return oracle.compile_source(src, os.path.join(tmp_dir, f"lib{name}.so"))


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    tmp_dir = str(tmp_path_factory.mktemp("oracle_mutants"))
    with open(SRC) as f:
        original = f.read()
    libs = {"unmodified": _build(tmp_dir, "unmodified", original)}
    bad = {}
    for name, old, new in MUTATIONS:
        count = original.count(old)
        if count != 1:
            bad[name] = f"text occurs {count} times in pa_oracle.c"
            continue
        libs[name] = _build(tmp_dir, name, original.replace(old, new))
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = dict(zip(libs, pool.map(_run_pins, libs.values())))
    return results, bad


def test_unmodified_oracle_passes_its_pins(outcomes):
    results, _ = outcomes
    rc, log = results["unmodified"]
    assert rc == 0, log


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(outcomes, name):
    results, bad = outcomes
    assert name not in bad, bad.get(name)
    rc, log = results[name]
    # exit status 1: the pins ran and at least one failed (not a crash, not a collection error)
    assert rc == 1, f"mistake {name!r} survived the oracle pins (pytest exit {rc}):\n{log}"
