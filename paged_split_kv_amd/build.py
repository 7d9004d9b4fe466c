"""Compile libpa.so and libpa_probe.so (the gfx950 HIP libraries behind include/pa.h and include/pa_probe.h) in-tree.

    python -m paged_split_kv_amd.build

Each translation unit is compiled in parallel with hipcc for gfx950, then linked into
``paged_split_kv_amd/libpa.so`` (the decode path, include/pa.h) and
``paged_split_kv_amd/libpa_probe.so`` (the benchmark's read-only bandwidth probes,
include/pa_probe.h).  Packed-fp32 instruction selection is switched off for device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_api.hip", "pa_plan.hip", "pa_decode.hip", "pa_prefill.hip", "pa_merge.hip"]
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
PROBE_SOURCES = ["pa_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def device_flags() -> List[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False) -> str:
    """Build libpa.so and libpa_probe.so; returns the path of libpa.so."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="pa_build_", dir=PKG)
    try:
        procs = []
        objs = []
        for src in SOURCES + PROBE_SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *device_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            if p.returncode != 0:
                failed.append(f"--- {src} ---\n{text}")
            elif verbose and text.strip():
                print(text)
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
        for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
            lib_objs = [o for o, src in zip(objs, SOURCES + PROBE_SOURCES) if src in srcs]
            out_tmp = lib + f".tmp{os.getpid()}"
            cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *lib_objs]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            os.replace(out_tmp, lib)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
