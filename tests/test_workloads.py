"""Host checks of the seeded input generator (paged_split_kv_amd/workloads.py): copying a Case keeps
every field, and the generator is deterministic."""
import numpy as np
import torch

from paged_split_kv_amd import workloads as W


def _case():
    c = W.build_case("to_copy", [5, 40, 17], num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                     kv_dtype="fp8", q_dtype="bf16", seed=7, q_lens=[1, 3, 2], pad_rows=1)
    c.window = 9
    return c


def test_case_to_keeps_every_field():
    c = _case()
    d = c.to("cpu")
    for f in ("name", "kv_dtype", "max_q_len", "scale", "k_scale", "v_scale", "window", "meta"):
        assert getattr(d, f) == getattr(c, f), f
    for f in ("q", "k_cache", "v_cache", "block_tables", "context_lens", "cu_query_lens"):
        a, b = getattr(c, f), getattr(d, f)
        assert a.dtype == b.dtype and torch.equal(a, b), f
    assert d.window == 9 and isinstance(d.meta, dict) and d.meta == {"seed": 7}
    assert d.meta is not c.meta


def test_case_to_keeps_a_missing_cu():
    c = W.build_case("no_cu", [3, 30], num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=16,
                     kv_dtype="bf16", q_dtype="bf16", seed=1)
    d = c.to("cpu")
    assert d.cu_query_lens is None and d.window == 0 and d.max_q_len == 1


def test_generator_is_deterministic():
    a, b = _case(), _case()
    for f in ("q", "k_cache", "v_cache", "block_tables", "context_lens", "cu_query_lens"):
        x, y = getattr(a, f), getattr(b, f)
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f
    assert np.array_equal(W.skewed_step_set(num_steps=8, draws=2000), W.skewed_step_set(num_steps=8, draws=2000))
