"""The seeded input generator: deterministic, the documented value ranges,
and the per-expert byte counts."""
import numpy as np
import torch

from sparse_moe_decode_q3moe_amd import inputs as gen


def test_same_seed_same_bytes():
    a = gen.moe_layer(gen.TINY, 5)
    b = gen.moe_layer(gen.TINY, 5)
    c = gen.moe_layer(gen.TINY, 6)
    assert torch.equal(a.gate, b.gate) and torch.equal(a.down, b.down)
    assert torch.equal(a.router, b.router)
    assert not torch.equal(a.gate, c.gate)


def test_fp16_scale_fields_in_range():
    g = gen.make_generator(1)
    q4 = gen.q4k_experts(2, 8, 512, g).view(2, 8, 2, 144)
    d = q4[..., 0:4].contiguous().view(torch.float16).float()
    lo, hi = float(np.float16(1e-3)), float(np.float16(1e-2))
    assert d.min() >= lo and d.max() <= hi
    q6 = gen.q6k_experts(2, 8, 512, g).view(2, 8, 2, 210)
    d6 = q6[..., 208:210].contiguous().view(torch.float16).float()
    assert d6.min() >= lo and d6.max() <= hi


def test_expert_strides():
    s = gen.QWEN3_30B_A3B
    assert s.gate_stride == 884736 and s.down_stride == 1290240
    assert gen.MoeShape(1, 2048, 128, 8, 768, gen.Q4_K).down_stride == 884736
    assert [gen.stack_down_qtype(l) for l in (0, 23, 24, 47)] == [gen.Q6_K, gen.Q6_K, gen.Q4_K, gen.Q4_K]


def test_skewed_routing_inputs():
    layer = gen.moe_layer(gen.MoeShape(T=64, H=256, E=8, k=2, F=256, down_qtype=gen.Q4_K), 3)
    x = gen.hidden_states(64, 256, 4)
    x2, r2 = gen.skewed_hidden_and_router(layer, x, 9)
    changed = (x2 != x).any(1)
    assert int(changed.sum()) == 32
    assert torch.equal(r2[4:], layer.router[4:]) and not torch.equal(r2[:4], layer.router[:4])
