"""CPU-side checks of the C ABI: the library loads, exports every declared entry point, and the
host-side argument checks return their status codes before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from paged_split_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="pa.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.load()
    names = _declared_functions()
    assert set(names) == set(B.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_noalloc_refuses_states_beyond_its_array():
    # the size check comes first: no device lookup and no launch for states beyond the static array
    lib = B.load()
    vp = ctypes.c_void_p
    cap = B.pa_plan_capacity(8, 1, 1 << 20, 2, 256)
    st = lib.pa_attention_noalloc(vp(256), B.PA_BF16, 32, 16, 256, vp(256), vp(256), B.PA_BF16, 64, 1, 16, vp(256),
                                  4, vp(256), 8, vp(256), 4, 0, 0.0625, 1.0, 1.0, 1 << 20, 2, 256, 256, cap,
                                  vp(256), vp(256), vp(256), vp(256), B.PA_BF16, None)
    assert st == B.PA_CAPACITY


def test_probe_library_exports_every_declared_function():
    from paged_split_kv_amd import probe as P
    lib = P.load()
    names = _declared_functions("pa_probe.h")
    assert set(names) == set(P.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_argument_checks():
    # refused before any launch: null pointers, misalignment, unsupported shapes
    from paged_split_kv_amd import probe as P
    lib = P.load()
    v = ctypes.c_void_p
    assert lib.pa_probe_read(None, 1024, 4, v(256), None) == B.PA_INVALID_ARG
    assert lib.pa_probe_read(v(256), 1024, 0, v(256), None) == B.PA_INVALID_ARG
    assert lib.pa_probe_read(v(258), 1024, 4, v(256), None) == B.PA_INVALID_ARG
    assert lib.pa_probe_read(v(256), 0, 4, v(256), None) == B.PA_OK        # nothing to read
    g = dict(k=v(256), v=v(512), dt=B.PA_BF16, nb=8, hkv=2, bs=16, d=128, bt=v(256), mb=4, ctx=v(256), ns=2,
             wi=v(256), nw=v(256), cap=8, T=256, sink=v(256))

    def gather(**kw):
        a = dict(g)
        a.update(kw)
        return lib.pa_probe_gather(a["k"], a["v"], a["dt"], a["nb"], a["hkv"], a["bs"], a["d"], a["bt"], a["mb"],
                                   a["ctx"], a["ns"], a["wi"], a["nw"], a["cap"], a["T"], a["sink"], None)
    assert gather(k=None) == B.PA_INVALID_ARG
    assert gather(wi=v(264)) == B.PA_INVALID_ARG
    assert gather(d=96) == B.PA_UNSUPPORTED
    assert gather(bs=32) == B.PA_UNSUPPORTED
    assert gather(T=24) == B.PA_UNSUPPORTED
    assert gather(dt=7) == B.PA_INVALID_ARG
    assert gather(cap=0) == B.PA_OK                                            # no workgroup


def test_status_strings():
    assert B.status_string(B.PA_OK) == "ok"
    for s in (B.PA_INVALID_ARG, B.PA_UNSUPPORTED, B.PA_CAPACITY, B.PA_HIP_ERROR):
        assert B.status_string(s) not in ("ok", "unknown status")
    assert B.status_string(99) == "unknown status"


@pytest.mark.parametrize("seed", range(5))
def test_capacity_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        Bn = int(rng.integers(0, 9000))
        hkv = int(rng.choice([1, 2, 3, 4, 8, 16]))
        cu = int(rng.choice([1, 80, 256, 304, 1000]))
        mult = int(rng.choice([1, 2, 3, 4]))
        P = int(rng.choice([1, 8, 64, 256, 1000]))
        assert B.pa_plan_capacity(Bn, hkv, cu, mult, P) == oracle.plan_capacity(Bn, hkv, cu, mult, P)


def test_workspace_bytes():
    # fp32 partials [C, Lmax, Hq, D] and (m, l) pairs [C, Lmax, Hq, 2], then (C > 0) the shared-slot
    # region: partials and (m, l) pairs of 3 C pieces and 256 int32 pairs; each region rounded up to
    # 256 bytes
    def expect(c, l, h, d):
        up = lambda x: (x + 255) // 256 * 256
        slots = up(c * l * h * d * 4) + up(c * l * h * 2 * 4)
        pieces = up(3 * c * l * h * d * 4) + up(3 * c * l * h * 2 * 4) + up(256 * 2 * 4)
        return slots + pieces if c > 0 else slots
    for args in [(512, 1, 4, 64), (256, 1, 16, 128), (512, 3, 6, 256), (1, 1, 1, 64), (0, 1, 1, 64)]:
        assert B.pa_workspace_bytes(*args) == expect(*args)
    assert B.pa_workspace_bytes(10, 0, 1, 64) == 0
    assert B.pa_workspace_bytes(-1, 1, 1, 64) == 0


def _plan_status(**kw):
    a = dict(ctx=ctypes.c_void_p(16), cuq=None, B=4, hkv=1, cu=256, mult=2, P=256, T=256, win=0, cap=512,
             work=ctypes.c_void_p(256), red=ctypes.c_void_p(256), nw=ctypes.c_void_p(256), disp=None)
    a.update(kw)
    return B.load().pa_plan(a["ctx"], a["cuq"], a["B"], a["hkv"], a["cu"], a["mult"], a["P"], a["T"],
                            a["win"], a["cap"], a["work"], a["red"], a["nw"], a["disp"], None)


def test_plan_argument_checks():
    # (no valid call is made: every case below must be refused before a launch)
    assert _plan_status(disp=ctypes.c_void_p(264)) == B.PA_INVALID_ARG   # dispatch order 16-byte aligned
    assert _plan_status(cap=511) == B.PA_CAPACITY
    assert _plan_status(B=-1) == B.PA_INVALID_ARG
    assert _plan_status(hkv=0) == B.PA_INVALID_ARG
    assert _plan_status(cu=0) == B.PA_INVALID_ARG
    assert _plan_status(mult=0) == B.PA_INVALID_ARG
    assert _plan_status(P=0) == B.PA_INVALID_ARG
    assert _plan_status(T=0) == B.PA_INVALID_ARG
    assert _plan_status(nw=None) == B.PA_INVALID_ARG
    assert _plan_status(ctx=None) == B.PA_INVALID_ARG
    assert _plan_status(work=None) == B.PA_INVALID_ARG
    assert _plan_status(work=ctypes.c_void_p(8)) == B.PA_INVALID_ARG       # misaligned int4 entries
    assert _plan_status(nw=ctypes.c_void_p(260)) == B.PA_INVALID_ARG       # num_work pair misaligned
    assert _plan_status(B=B.PA_MAX_SEQS + 1, cap=1 << 22) == B.PA_UNSUPPORTED
    assert _plan_status(win=-1) == B.PA_INVALID_ARG


_GOOD = dict(q=256, qd=B.PA_BF16, R=4, Hq=16, D=128, k=256, v=256, kvd=B.PA_BF16, nb=10, Hkv=2, bs=16,
             bt=256, mb=4, ctx=256, Bn=4, cu=None, ql=1, win=0, scale=0.1, ks=1.0, vs=1.0, work=256, red=256,
             nw=256, cap=256, T=256, ws=256, wsb=1 << 30, out=None, od=B.PA_BF16)


def _decode_status(**kw):
    a = dict(_GOOD)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.load().pa_decode(vp(a["q"]), a["qd"], a["R"], a["Hq"], a["D"], vp(a["k"]), vp(a["v"]),
                              a["kvd"], a["nb"], a["Hkv"], a["bs"], vp(a["bt"]), a["mb"], vp(a["ctx"]),
                              a["Bn"], vp(a["cu"]), a["ql"], a["win"], a["scale"], a["ks"], a["vs"], vp(a["work"]),
                              vp(a["red"]), vp(a["nw"]), vp(a.get("disp")), a["cap"], a["T"], vp(a["ws"]), a["wsb"],
                              vp(a["out"]), a["od"], None)


def test_decode_argument_checks():
    assert _decode_status(disp=264) == B.PA_INVALID_ARG                 # dispatch order 16-byte aligned
    assert _decode_status(qd=B.PA_FP8_E4M3) == B.PA_INVALID_ARG        # q must be f32 or bf16
    assert _decode_status(kvd=7) == B.PA_INVALID_ARG
    assert _decode_status(Hq=15) == B.PA_INVALID_ARG                   # Hq % Hkv != 0
    assert _decode_status(D=96) == B.PA_UNSUPPORTED
    assert _decode_status(D=512) == B.PA_UNSUPPORTED
    assert _decode_status(bs=32) == B.PA_UNSUPPORTED
    assert _decode_status(mb=1 << 27) == B.PA_UNSUPPORTED              # keys a table reaches exceed int32
    assert _decode_status(T=200) == B.PA_UNSUPPORTED                   # tile not a multiple of bs
    assert _decode_status(Hq=32, Hkv=1, cu=256, ql=3) == B.PA_UNSUPPORTED   # 96 rows per group
    assert _decode_status(ql=2) == B.PA_INVALID_ARG                    # no cu but max_q_len 2
    assert _decode_status(R=3) == B.PA_INVALID_ARG                     # no cu and fewer rows than requests
    assert _decode_status(q=None) == B.PA_INVALID_ARG
    assert _decode_status(k=None) == B.PA_INVALID_ARG
    assert _decode_status(bt=None) == B.PA_INVALID_ARG
    assert _decode_status(work=None) == B.PA_INVALID_ARG
    assert _decode_status(ws=None) == B.PA_INVALID_ARG
    assert _decode_status(ws=512 + 16) == B.PA_INVALID_ARG             # workspace not 256-aligned
    assert _decode_status(q=8) == B.PA_INVALID_ARG                     # q not 16-aligned
    assert _decode_status(wsb=1000) == B.PA_CAPACITY
    assert _decode_status(scale=float("nan")) == B.PA_INVALID_ARG
    assert _decode_status(Bn=-1) == B.PA_INVALID_ARG
    assert _decode_status(win=-5) == B.PA_INVALID_ARG
    assert _decode_status(out=512, od=B.PA_F32) == B.PA_INVALID_ARG    # merged output dtype != q dtype
    assert _decode_status(out=512, red=None, D=96) == B.PA_UNSUPPORTED
    assert _decode_status(out=512, red=None) == B.PA_INVALID_ARG       # merging needs reduce_info
    assert _decode_status(out=520) == B.PA_INVALID_ARG                 # out not 16-aligned
    assert _decode_status(out=512, red=260) == B.PA_INVALID_ARG        # reduce_info entries misaligned
    assert _decode_status(cap=0) == B.PA_OK                            # nothing to do: no launch
    assert _decode_status(Bn=0) == B.PA_OK


def _merge_status(**kw):
    a = dict(R=4, Hq=16, D=128, Bn=4, cu=None, ql=1, red=256, cap=256, ws=256, wsb=1 << 30, out=256,
             od=B.PA_BF16)
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.load().pa_merge(a["R"], a["Hq"], a["D"], a["Bn"], vp(a["cu"]), a["ql"], vp(a["red"]),
                             a["cap"], vp(a["ws"]), a["wsb"], vp(a["out"]), a["od"], None)


def test_merge_argument_checks():
    assert _merge_status(od=B.PA_FP8_E4M3) == B.PA_INVALID_ARG
    assert _merge_status(D=80) == B.PA_UNSUPPORTED
    assert _merge_status(out=None) == B.PA_INVALID_ARG
    assert _merge_status(red=None) == B.PA_INVALID_ARG
    assert _merge_status(ws=None) == B.PA_INVALID_ARG
    assert _merge_status(ql=2) == B.PA_INVALID_ARG
    assert _merge_status(wsb=10) == B.PA_CAPACITY
    assert _merge_status(red=260) == B.PA_INVALID_ARG                  # int2 entries misaligned
    assert _merge_status(R=0) == B.PA_OK


def test_binding_refuses_host_tensors():
    ctx = torch.tensor([1, 2], dtype=torch.int32)
    with pytest.raises(ValueError):
        B.pa_plan(ctx, 1, cu_count=256)


def _attention_status(**kw):
    a = dict(_GOOD)
    a.update(dict(out=512, cuc=256, mult=2, P=256))
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.load().pa_attention(vp(a["q"]), a["qd"], a["R"], a["Hq"], a["D"], vp(a["k"]), vp(a["v"]),
                                 a["kvd"], a["nb"], a["Hkv"], a["bs"], vp(a["bt"]), a["mb"], vp(a["ctx"]),
                                 a["Bn"], vp(a["cu"]), a["ql"], a["win"], a["scale"], a["ks"], a["vs"], a["cuc"],
                                 a["mult"], a["P"], a["T"], a["cap"], vp(a["work"]), vp(a["red"]),
                                 vp(a["nw"]), vp(a["ws"]), a["wsb"], vp(a["out"]), a["od"], None)


def test_attention_argument_checks():
    # the union of the three calls' checks, all before any launch
    assert _attention_status(cap=255) == B.PA_CAPACITY                 # plan: below the formula (256)
    assert _attention_status(P=0) == B.PA_INVALID_ARG
    assert _attention_status(cuc=0) == B.PA_INVALID_ARG
    assert _attention_status(nw=260) == B.PA_INVALID_ARG               # num_work pair misaligned
    assert _attention_status(red=None) == B.PA_INVALID_ARG
    assert _attention_status(Bn=B.PA_MAX_SEQS + 1, cap=1 << 22) == B.PA_UNSUPPORTED
    assert _attention_status(D=96) == B.PA_UNSUPPORTED                 # decode checks
    assert _attention_status(bs=32) == B.PA_UNSUPPORTED
    assert _attention_status(T=200) == B.PA_UNSUPPORTED
    assert _attention_status(qd=B.PA_FP8_E4M3) == B.PA_INVALID_ARG
    assert _attention_status(ws=None) == B.PA_INVALID_ARG
    assert _attention_status(wsb=1000) == B.PA_CAPACITY
    assert _attention_status(out=None) == B.PA_INVALID_ARG             # merge checks
    assert _attention_status(out=520) == B.PA_INVALID_ARG
    assert _attention_status(od=B.PA_F32) == B.PA_INVALID_ARG
    assert _attention_status(ql=2) == B.PA_INVALID_ARG
    assert _attention_status(win=-1) == B.PA_INVALID_ARG


def test_merge_refuses_misaligned_out():
    assert _merge_status(out=264) == B.PA_INVALID_ARG


def _prefill_status(**kw):
    a = dict(_GOOD)
    a.update(dict(cu=256, out=512, cuc=256, pws=1024, pwsb=1 << 30))
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.load().pa_prefill(vp(a["q"]), a["qd"], a["R"], a["Hq"], a["D"], vp(a["k"]), vp(a["v"]), a["kvd"],
                               a["nb"], a["Hkv"], a["bs"], vp(a["bt"]), a["mb"], vp(a["ctx"]), a["Bn"],
                               vp(a["cu"]), a["win"], a["scale"], a["ks"], a["vs"], a["cuc"], vp(a["pws"]),
                               a["pwsb"], vp(a["out"]), a["od"], None)


def test_prefill_workspace_bytes():
    # blocks of T = 256 / G tokens (128 / G at head_dim 256), at most ceil(R / T) + B of them; capacity
    # formula over the blocks (budget 1 x CU, ceiling 256); regions: lengths, first rows (+1), request
    # indices, work_info, reduce_info, num_work, then the partial states [C, T, Hq, D] fp32 and (m, l)
    # pairs, each 256-aligned
    up = lambda x: (x + 255) // 256 * 256
    for R, Bn, hq, hkv, d, cu in [(512, 1, 12, 2, 256, 256), (33, 4, 16, 2, 128, 256), (1000, 7, 8, 8, 64, 80),
                                  (0, 0, 4, 1, 128, 256)]:
        T = max(1, (128 if d == 256 else 256) // (hq // hkv))
        nb = (R + T - 1) // T + Bn
        cap = min(nb * 256, max(nb, -(-cu // hkv)))
        want = (up(4 * nb) + up(4 * (nb + 1)) + up(4 * nb) + up(16 * cap) + up(8 * nb) + up(8)
                + up(cap * T * hq * d * 4) + up(cap * T * hq * 2 * 4))
        assert B.pa_prefill_workspace_bytes(R, Bn, hq, hkv, d, cu) == want, (R, Bn, hq, hkv, d, cu)
    assert B.pa_prefill_workspace_bytes(8192 * 256, 1, 64, 1, 128, 256) == 0         # more than 8192 blocks
    assert B.pa_prefill_workspace_bytes(10, 1, 12, 5, 128, 256) == 0                  # heads not a multiple
    assert B.pa_prefill_workspace_bytes(10, 1, 4, 1, 128, 0) == 0


def test_prefill_argument_checks():
    assert _prefill_status(cu=None) == B.PA_INVALID_ARG             # the query lengths are required
    assert _prefill_status(kvd=B.PA_F32) == B.PA_UNSUPPORTED        # matrix-core path only
    assert _prefill_status(D=96) == B.PA_UNSUPPORTED
    assert _prefill_status(bs=32) == B.PA_UNSUPPORTED
    assert _prefill_status(mb=1 << 27) == B.PA_UNSUPPORTED           # keys a table reaches exceed int32
    assert _prefill_status(Hq=15) == B.PA_INVALID_ARG
    assert _prefill_status(od=B.PA_F32) == B.PA_INVALID_ARG
    assert _prefill_status(out=None) == B.PA_INVALID_ARG
    assert _prefill_status(out=520) == B.PA_INVALID_ARG
    assert _prefill_status(win=-1) == B.PA_INVALID_ARG
    assert _prefill_status(scale=float("nan")) == B.PA_INVALID_ARG
    assert _prefill_status(cuc=0) == B.PA_INVALID_ARG
    assert _prefill_status(pws=None, R=0) == B.PA_OK                # the one-launch form: no workspace
    assert _prefill_status(pws=1032) == B.PA_INVALID_ARG            # workspace 256-byte aligned
    assert _prefill_status(pwsb=4096) == B.PA_CAPACITY
    assert _prefill_status(R=0) == B.PA_OK                         # nothing to write: no launch


def _mixed_status(**kw):
    a = dict(_GOOD)
    a.update(dict(cu=256, out=512, cuc=256, mult=2, P=256, nd=2, ndt=2))
    a.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return B.load().pa_attention_mixed(vp(a["q"]), a["qd"], a["R"], a["Hq"], a["D"], vp(a["k"]), vp(a["v"]),
                                       a["kvd"], a["nb"], a["Hkv"], a["bs"], vp(a["bt"]), a["mb"], vp(a["ctx"]),
                                       a["Bn"], vp(a["cu"]), a["nd"], a["ndt"], a["ql"], a["win"], a["scale"],
                                       a["ks"], a["vs"], a["cuc"], a["mult"], a["P"], a["T"], a["cap"],
                                       vp(a["work"]), vp(a["red"]), vp(a["nw"]), vp(a["ws"]), a["wsb"],
                                       vp(a["out"]), a["od"], None)


def test_mixed_attention_argument_checks():
    # the split itself, then the decode part's checks (plan, decode, merge), then the prompts'
    assert _mixed_status(nd=5) == B.PA_INVALID_ARG                  # more decodes than requests
    assert _mixed_status(nd=-1) == B.PA_INVALID_ARG
    assert _mixed_status(ndt=5) == B.PA_INVALID_ARG                 # decode rows past the rows
    assert _mixed_status(cu=None) == B.PA_INVALID_ARG
    assert _mixed_status(cap=255) == B.PA_CAPACITY                  # formula for 2 requests: 256
    assert _mixed_status(D=96) == B.PA_UNSUPPORTED
    assert _mixed_status(od=B.PA_F32) == B.PA_INVALID_ARG
    assert _mixed_status(out=None) == B.PA_INVALID_ARG
    assert _mixed_status(out=520) == B.PA_INVALID_ARG
    assert _mixed_status(kvd=B.PA_F32) == B.PA_UNSUPPORTED          # the prompts need bf16 / fp8
    assert _mixed_status(win=-1) == B.PA_INVALID_ARG


def test_split_decode_first_on_the_host():
    # 7 decodes then a 100-token prompt (opengfx1030/vllm-rdna PR #29 table: 7 decodes + a new prompt)
    cu = [0, 1, 2, 3, 4, 5, 6, 7, 107]
    assert B.pa_split_decode_first(cu, 1) == (7, 7)
    # verify rows of 3 (1 + 2 speculative tokens) first, then two prefill chunks
    cu = [0, 3, 6, 9, 209, 259]
    assert B.pa_split_decode_first(cu, 3) == (3, 9)
    assert B.pa_split_decode_first(cu, 1) == (0, 0)
    assert B.pa_split_decode_first(cu, 1000) == (5, 259)
    assert B.pa_split_decode_first([0], 1) == (0, 0)
    # a decode after a prefill is not moved: the split is the leading run only
    assert B.pa_split_decode_first([0, 1, 50, 51], 1) == (1, 1)
    with pytest.raises(B.PaError):
        B.pa_split_decode_first([0, 1], 0)
