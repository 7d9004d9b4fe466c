"""Seeded synthetic inputs for paged split-KV decode.

This module only draws and lays out inputs: context lengths, block tables,
query rows and K/V page pools.  It holds none of the attention or planning
arithmetic, so both the GPU path and the CPU oracle can consume what it makes.

Workloads (shapes and value distributions follow the problem statements on the
pages; the agentic-trace statistics come from ATOM PR #2366 "Route the paged
decode to aiter's FlyDSL kernel with work planner", section 1 Motivation):

* ``tiny_fp32``      4 requests, lengths {1, 17, 100, 300}, Hq 4 / Hkv 1,
                     D 64, pages of 16, fp32.
* ``skewed_bf16``    32 single-token requests, Hq 16 / Hkv 2, D 128, pages of
                     16, bf16.  Lengths come from a stratified set of 128 steps
                     whose max/min ratio matches the trace (p50 ~2.5, p90 ~22).
* ``long_bf16``      one request of 131072 tokens, pages of 64, Hq 16 / Hkv 2,
                     D 128, bf16.
* ``verify_bf16``    8 requests x 3 verify tokens + 7 single-token requests,
                     all at 16384 tokens, plus 2 padding rows past the last
                     cumulative query length; Hq 6 / Hkv 1, D 256, pages of 16.
* ``fp8_kv``         256 single-token requests, lengths log-normal in
                     [128, 65536], e4m3fn K/V with per-tensor scales, bf16 q.

Value recipe: q/K/V ~ N(0, 1) drawn in float32 from a seeded torch generator,
then rounded to the storage type (RNE for bf16; fp8 codes are the e4m3fn
round-to-nearest of value/scale with scale = amax/448, saturated to +-448).
Page ids are a random permutation of the pool; table entries past a request's
last page are -1; cache slots past a request's length in its last page hold
NaN (poison: they must never influence an output).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

KV_DTYPES = ("f32", "bf16", "fp8")
Q_DTYPES = ("f32", "bf16")

_TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
FP8_MAX = 448.0


@dataclass
class Case:
    """One decode call's inputs, all tensors on ``device``."""

    name: str
    q: torch.Tensor                 # [R, Hq, D] float32 or bfloat16
    k_cache: torch.Tensor           # [num_blocks, Hkv, bs, D]: float32, bfloat16, or uint8 e4m3fn codes
    v_cache: torch.Tensor
    kv_dtype: str                   # "f32" | "bf16" | "fp8"
    block_tables: torch.Tensor      # int32 [B, max_blocks_per_seq]
    context_lens: torch.Tensor      # int32 [B]
    cu_query_lens: Optional[torch.Tensor]  # int32 [B + 1] or None (one token per request)
    max_q_len: int
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    window: int = 0                 # sliding window in keys per query token; 0 = none
    meta: Dict = field(default_factory=dict)

    @property
    def q_dtype(self) -> str:
        return "f32" if self.q.dtype == torch.float32 else "bf16"

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[1])

    @property
    def block_size(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of K plus V that the step must read: sum_b S_b * Hkv * 2 * D * elem."""
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]
        total = int(self.context_lens.to(torch.int64).sum().item())
        return total * self.num_kv_heads * 2 * self.head_dim * elem

    def to(self, device) -> "Case":
        def mv(t):
            return None if t is None else t.to(device)
        return Case(name=self.name, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
                    kv_dtype=self.kv_dtype, block_tables=mv(self.block_tables),
                    context_lens=mv(self.context_lens), cu_query_lens=mv(self.cu_query_lens),
                    max_q_len=self.max_q_len, scale=self.scale, k_scale=self.k_scale,
                    v_scale=self.v_scale, window=self.window, meta=dict(self.meta))

    def host(self) -> Dict[str, np.ndarray]:
        """Host numpy views of the storage bytes (bf16 as uint16 bits, fp8 as uint8 codes)."""
        def np_of(t):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        out = {
            "q": np_of(self.q), "k_cache": np_of(self.k_cache), "v_cache": np_of(self.v_cache),
            "block_tables": np_of(self.block_tables), "context_lens": np_of(self.context_lens),
        }
        out["cu_query_lens"] = None if self.cu_query_lens is None else np_of(self.cu_query_lens)
        return out


# ----------------------------------------------------------------------------------------------
# value drawing helpers (layout and storage rounding only)
# ----------------------------------------------------------------------------------------------

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _store(x: torch.Tensor, dtype: str):
    """Round float32 values to the storage type. Returns (tensor, scale)."""
    if dtype == "f32":
        return x.contiguous(), 1.0
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous(), 1.0
    if dtype == "fp8":
        amax = float(x.abs().max().item()) if x.numel() else 1.0
        scale = amax / FP8_MAX if amax > 0 else 1.0
        codes = (x / scale).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes.contiguous(), scale
    raise ValueError(dtype)


def _poison_value(dtype: str):
    return 0x7F if dtype == "fp8" else float("nan")


def build_case(name: str, context_lens: Sequence[int], *, num_q_heads: int, num_kv_heads: int,
               head_dim: int, block_size: int, kv_dtype: str, q_dtype: str, seed: int,
               q_lens: Optional[Sequence[int]] = None, pad_rows: int = 0, device="cpu",
               extra_blocks: int = 3, max_blocks_per_seq: Optional[int] = None,
               poison_tail: bool = True, scale: Optional[float] = None) -> Case:
    """Lay out one decode call.

    ``q_lens`` (per request query tokens) switches on ``cu_query_lens``; without it every request
    has one query row and no cumulative lengths are passed.  ``pad_rows`` appends rows past the
    last cumulative length (graph padding).
    """
    assert kv_dtype in KV_DTYPES and q_dtype in Q_DTYPES
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int64)
    B = int(ctx.shape[0])
    pages = [(int(s) + block_size - 1) // block_size for s in ctx]
    need = int(sum(pages))
    num_blocks = need + extra_blocks
    mbps = max(max(pages) if pages else 1, 1) if max_blocks_per_seq is None else max_blocks_per_seq
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((B, mbps), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[pos:pos + pages[b]]
        pos += pages[b]

    if q_lens is None:
        cu = None
        R = B + pad_rows
        max_q = 1
    else:
        ql = np.asarray(q_lens, dtype=np.int64)
        assert ql.shape[0] == B
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(ql)
        R = int(cu[-1]) + pad_rows
        max_q = int(max(ql.max() if B else 1, 1))

    g = _gen(seed, device)
    q = _randn((R, num_q_heads, head_dim), g, device)
    k = _randn((num_blocks, num_kv_heads, block_size, head_dim), g, device)
    v = _randn((num_blocks, num_kv_heads, block_size, head_dim), g, device)
    q = q.to(torch.bfloat16) if q_dtype == "bf16" else q
    k, k_scale = _store(k, kv_dtype)
    v, v_scale = _store(v, kv_dtype)

    if poison_tail:
        pv = _poison_value(kv_dtype)
        for b in range(B):
            s = int(ctx[b])
            if s % block_size and pages[b]:
                blk = int(bt[b, pages[b] - 1])
                k[blk, :, s % block_size:, :] = pv
                v[blk, :, s % block_size:, :] = pv

    dev = torch.device(device)
    return Case(
        name=name, q=q.contiguous(), k_cache=k, v_cache=v, kv_dtype=kv_dtype,
        block_tables=torch.from_numpy(bt).to(dev),
        context_lens=torch.from_numpy(ctx.astype(np.int32)).to(dev),
        cu_query_lens=None if cu is None else torch.from_numpy(cu).to(dev),
        max_q_len=max_q,
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
        k_scale=k_scale, v_scale=v_scale,
        meta={"seed": seed},
    )


# ----------------------------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------------------------

def skewed_step_set(num_steps: int = 128, batch: int = 32, seed: int = 1,
                    draws: int = 100_000) -> np.ndarray:
    """Stratified set of decode steps whose max/min context ratio follows the agentic trace.

    Per draw a spread sigma_s = exp(-1.49 + 0.94 z) is itself log-normal; the ``batch`` lengths of
    the draw are exp(mu + sigma_s z) with mu = ln sqrt(256 * 131072), rounded and clipped to
    [256, 131072].  Draws are sorted (stably) by max/min and ``num_steps`` are taken at the
    quantiles (k + 1/2) / num_steps.  Returns int64 [num_steps, batch], ordered by ratio.
    """
    rng = np.random.default_rng(seed)
    sig = np.exp(-1.49 + 0.94 * rng.standard_normal(draws))
    z = rng.standard_normal((draws, batch))
    mu = math.log(math.sqrt(256.0 * 131072.0))
    ctx = np.clip(np.rint(np.exp(mu + sig[:, None] * z)), 256, 131072).astype(np.int64)
    ratio = ctx.max(axis=1) / ctx.min(axis=1)
    order = np.argsort(ratio, kind="stable")
    k = np.arange(num_steps)
    pick = order[np.floor((k + 0.5) / num_steps * draws).astype(np.int64)]
    return ctx[pick]


def skewed_named_steps(steps: np.ndarray) -> Dict[str, int]:
    """Indices of the steps nearest the p50 and p90 ratio and of the step with most tokens."""
    ratio = steps.max(axis=1) / steps.min(axis=1)
    out = {}
    for tag, qv in (("p50", 0.5), ("p90", 0.9)):
        target = np.quantile(ratio, qv)
        out[tag] = int(np.argmin(np.abs(ratio - target)))
    out["max_tokens"] = int(np.argmax(steps.sum(axis=1)))
    return out


def fp8_context_lens(batch: int = 256, seed: int = 4) -> np.ndarray:
    rng = np.random.default_rng(seed)
    mu = math.log(math.sqrt(128.0 * 65536.0))
    z = rng.standard_normal(batch)
    return np.clip(np.rint(np.exp(mu + 1.27 * z)), 128, 65536).astype(np.int64)


def make_config(name: str, device="cpu", step: Optional[int] = None, seed: Optional[int] = None) -> Case:
    """The five named workloads at full size.  ``seed`` replaces the workload's own value seed (for
    independent copies of the same shape)."""
    def sd(own: int) -> int:
        return own if seed is None else seed

    if name == "tiny_fp32":
        return build_case(name, [1, 17, 100, 300], num_q_heads=4, num_kv_heads=1, head_dim=64,
                          block_size=16, kv_dtype="f32", q_dtype="f32", seed=sd(0), device=device)
    if name == "skewed_bf16":
        steps = skewed_step_set()
        idx = skewed_named_steps(steps)["p50"] if step is None else step
        c = build_case(name, steps[idx].tolist(), num_q_heads=16, num_kv_heads=2, head_dim=128,
                       block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=sd(100 + idx),
                       device=device)
        c.meta["step"] = idx
        return c
    if name == "long_bf16":
        return build_case(name, [131072], num_q_heads=16, num_kv_heads=2, head_dim=128,
                          block_size=64, kv_dtype="bf16", q_dtype="bf16", seed=sd(2), device=device)
    if name == "verify_bf16":
        return build_case(name, [16384] * 15, num_q_heads=6, num_kv_heads=1, head_dim=256,
                          block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=sd(3),
                          q_lens=[3] * 8 + [1] * 7, pad_rows=2, device=device)
    if name == "fp8_kv":
        return build_case(name, fp8_context_lens().tolist(), num_q_heads=16, num_kv_heads=2,
                          head_dim=128, block_size=16, kv_dtype="fp8", q_dtype="bf16", seed=sd(4),
                          device=device)
    raise KeyError(name)


CONFIG_NAMES: List[str] = ["tiny_fp32", "skewed_bf16", "long_bf16", "verify_bf16", "fp8_kv"]


def make_mixed_case(device="cpu", seed: int = 5) -> Case:
    """A mixed batch, decodes first: 7 decodes at 16384 tokens and a new 100-token prompt, at the
    per-rank shapes of TP=2 (12 query heads, 2 kv heads, head_dim 256), bf16 (opengfx1030/vllm-rdna
    PR #29, Problem table, second row)."""
    return build_case("mixed_7x16k_prompt100", [16384] * 7 + [100], num_q_heads=12, num_kv_heads=2,
                      head_dim=256, block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=seed,
                      q_lens=[1] * 7 + [100], device=device)


def make_prefill_chunk_case(device="cpu", seed: int = 6, prefix: int = 16384, chunk: int = 512) -> Case:
    """A prompt chunk behind a long prefix (chunked prefill): one request whose last `chunk` tokens are
    new query rows over prefix + chunk keys, at the per-rank shapes of the mixed batch (12 query heads,
    2 kv heads, head_dim 256), bf16 (opengfx1030/vllm-rdna PR #29, Change 2: prompt rows go to the
    prefill kernel on the rebased remainder)."""
    return build_case("prefill_chunk", [prefix + chunk], num_q_heads=12, num_kv_heads=2, head_dim=256,
                      block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=seed, q_lens=[chunk], device=device)


# ----------------------------------------------------------------------------------------------
# sparse / top-k layers: every request reads a fixed-size selection of pages, so lengths are
# near-uniform (ROCm/ATOM PR #2366 section 3: sparse sites read a fixed top-k window; PR #2514
# Design: sparse plans use a partition cap of 8)
# ----------------------------------------------------------------------------------------------

SPARSE_TOPK_TOKENS = 2048     # selected tokens per request
SPARSE_LOCAL_TOKENS = 256     # plus up to this many local (most recent) tokens


def sparse_lengths(num_steps: int, batch: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return SPARSE_TOPK_TOKENS + rng.integers(1, SPARSE_LOCAL_TOKENS + 1, size=(num_steps, batch))


def make_sparse_case(device="cpu", batch: int = 16, seed: int = 9) -> Case:
    ctx = sparse_lengths(1, batch, seed)[0]
    return build_case("sparse_topk", ctx.tolist(), num_q_heads=16, num_kv_heads=2, head_dim=128,
                      block_size=16, kv_dtype="bf16", q_dtype="bf16", seed=seed, device=device)


# ----------------------------------------------------------------------------------------------
# the skewed-batch pool used for timing: one large page pool, fresh random pages per step
# ----------------------------------------------------------------------------------------------

@dataclass
class StepPool:
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    q: torch.Tensor                   # [steps, B, Hq, D]
    block_tables: torch.Tensor        # [steps, B, max_blocks]
    context_lens: torch.Tensor        # [steps, B]
    steps: np.ndarray                 # int64 [steps, B]
    block_size: int
    scale: float


def skewed_pool(device, pool_bytes: int = 4 << 30, num_steps: int = 128, seed: int = 7,
                num_q_heads: int = 16, num_kv_heads: int = 2, head_dim: int = 128,
                block_size: int = 16, steps: Optional[np.ndarray] = None) -> StepPool:
    """K/V page pool much larger than the 256 MB last-level cache, with each step's pages drawn
    at random from it, so consecutive steps share almost no pages.  ``steps`` (int [num_steps, B])
    replaces the skewed step set."""
    if steps is None:
        steps = skewed_step_set(num_steps=num_steps)
    num_steps = steps.shape[0]
    elem = 2
    page_bytes = 2 * num_kv_heads * block_size * head_dim * elem
    num_blocks = pool_bytes // page_bytes
    need_max = int(((steps + block_size - 1) // block_size).sum(axis=1).max())
    assert num_blocks >= need_max, "pool too small for the largest step"
    g = _gen(seed, device)
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k = torch.empty(shape, dtype=torch.bfloat16, device=device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    chunk = max(1, (256 << 20) // (num_kv_heads * block_size * head_dim * 4))
    for t in (k, v):
        for s in range(0, num_blocks, chunk):
            e = min(num_blocks, s + chunk)
            t[s:e] = _randn((e - s,) + shape[1:], g, device).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    B = steps.shape[1]
    mbps = int(((steps.max() + block_size - 1) // block_size))
    bt = np.full((num_steps, B, mbps), -1, dtype=np.int32)
    for i in range(num_steps):
        pages = (steps[i] + block_size - 1) // block_size
        ids = rng.choice(num_blocks, size=int(pages.sum()), replace=False).astype(np.int32)
        pos = 0
        for b in range(B):
            bt[i, b, :pages[b]] = ids[pos:pos + pages[b]]
            pos += pages[b]
    q = _randn((num_steps, B, num_q_heads, head_dim), g, device).to(torch.bfloat16)
    dev = torch.device(device)
    return StepPool(k_cache=k, v_cache=v, q=q, block_tables=torch.from_numpy(bt).to(dev),
                    context_lens=torch.from_numpy(steps.astype(np.int32)).to(dev), steps=steps,
                    block_size=block_size, scale=1.0 / math.sqrt(head_dim))
