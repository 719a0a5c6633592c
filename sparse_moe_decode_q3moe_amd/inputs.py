"""Seeded synthetic inputs for the Qwen3-MoE sparse FFN block.

This module only draws random bytes and numbers; it holds none of the
block's arithmetic.  Both the HIP path and the CPU oracle take their inputs
from here, so the two sides always see identical bytes.

Shapes follow the Qwen3-30B-A3B layer facts listed under "File facts" in
aprender issue #3714 (qwen3moe has NO working CUDA path): hidden 2048,
128 experts, top-8, expert FFN 768, f32 router [128 x 2048], gate/up Q4_K,
down Q6_K or Q4_K per layer, 32 q heads / 4 kv heads with head_dim 128,
rope base 1e7.

Value distributions (none are on the pages; they are the synthetic stand-in
for the real GGUF files, which are not available):

* router rows ~ N(0, 0.02) f32, hidden ~ N(0, 1) f32;
* Q4_K super-blocks: every byte uniform, then the fp16 ``d`` and ``dmin``
  fields overwritten with U[1e-3, 1e-2] rounded to fp16 (nearest-even);
* Q6_K super-blocks: every byte uniform (the 16 scales read as int8), then
  the fp16 ``d`` field overwritten with U[1e-3, 1e-2] rounded to fp16.

The attention side of the full decoder layer (the same "File facts"):

* projection weights W_q [4096 x 2048], W_k and W_v [512 x 2048], W_o
  [2048 x 4096] ~ N(0, 0.02) drawn in f32, then stored as bf16 (nearest-even);
* RMSNorm gains (input, post-attention, per-head q and k) ~ U[0.5, 1.5];
* the cached keys and values of earlier positions ~ N(0, 1) as bf16.

Generators are ``torch.Generator`` objects on the device the tensor is made
on; a tensor made on the GPU is copied to the host before the oracle sees it.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

QK_K = 256                      # weights per k-quant super-block
Q4_K, Q6_K = 1, 2               # qtype codes used across the library ABI
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}


@dataclasses.dataclass(frozen=True)
class MoeShape:
    """One sparse-MoE FFN layer: T tokens, hidden H, E experts, top-k, FFN F."""
    T: int
    H: int
    E: int
    k: int
    F: int
    down_qtype: int = Q6_K

    def expert_bytes(self, qtype: int, rows: int, cols: int) -> int:
        return rows * (cols // QK_K) * BLOCK_BYTES[qtype]

    @property
    def gate_stride(self) -> int:
        return self.expert_bytes(Q4_K, self.F, self.H)

    @property
    def down_stride(self) -> int:
        return self.expert_bytes(self.down_qtype, self.H, self.F)


# The tiny layer (4 tokens, all Q4_K) and the Qwen3-30B-A3B decode layer.
TINY = MoeShape(T=4, H=256, E=8, k=2, F=256, down_qtype=Q4_K)

# Vocabulary of the output head and the embedding table.  The pages give no
# size; the token ids they print (up to 151,645) need at least 151,646 rows,
# and 151,936 is the Qwen3 family's padded vocabulary.
QWEN3_VOCAB = 151936
QWEN3_30B_A3B = MoeShape(T=1, H=2048, E=128, k=8, F=768, down_qtype=Q6_K)
N_LAYERS_30B = 48               # down is Q6_K in layers 0-23, Q4_K in 24-47


def stack_down_qtype(layer: int) -> int:
    return Q6_K if layer < N_LAYERS_30B // 2 else Q4_K


def make_generator(seed: int, device: torch.device | str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _fp16_bytes_uniform(shape, lo: float, hi: float, gen, device) -> torch.Tensor:
    v = torch.empty(shape, dtype=torch.float32, device=device).uniform_(lo, hi, generator=gen)
    return v.to(torch.float16).view(torch.uint8)


def q4k_experts(n_experts: int, rows: int, cols: int, gen: torch.Generator,
                device="cpu") -> torch.Tensor:
    """uint8 [n_experts, rows * cols/256 * 144]: expert e's matrix at row-major offset e*stride."""
    assert cols % QK_K == 0
    nb = cols // QK_K
    raw = torch.randint(0, 256, (n_experts, rows, nb, 144), dtype=torch.uint8,
                        device=device, generator=gen)
    raw[..., 0:4] = _fp16_bytes_uniform((n_experts, rows, nb, 2), 1e-3, 1e-2, gen,
                                        device).view(n_experts, rows, nb, 4)
    return raw.view(n_experts, rows * nb * 144)


def q6k_experts(n_experts: int, rows: int, cols: int, gen: torch.Generator,
                device="cpu") -> torch.Tensor:
    """uint8 [n_experts, rows * cols/256 * 210]."""
    assert cols % QK_K == 0
    nb = cols // QK_K
    raw = torch.randint(0, 256, (n_experts, rows, nb, 210), dtype=torch.uint8,
                        device=device, generator=gen)
    raw[..., 208:210] = _fp16_bytes_uniform((n_experts, rows, nb, 1), 1e-3, 1e-2, gen,
                                            device).view(n_experts, rows, nb, 2)
    return raw.view(n_experts, rows * nb * 210)


def kquant_experts(qtype: int, n_experts: int, rows: int, cols: int, gen, device="cpu"):
    if qtype == Q4_K:
        return q4k_experts(n_experts, rows, cols, gen, device)
    if qtype == Q6_K:
        return q6k_experts(n_experts, rows, cols, gen, device)
    raise ValueError(f"unknown qtype {qtype}")


def normal_f32(shape, std: float, gen, device="cpu") -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32, device=device).normal_(0.0, std, generator=gen)


def uniform_f32(shape, lo: float, hi: float, gen, device="cpu") -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32, device=device).uniform_(lo, hi, generator=gen)


@dataclasses.dataclass
class MoeLayer:
    shape: MoeShape
    router: torch.Tensor          # f32 [E, H]
    gate: torch.Tensor            # uint8 [E, gate_stride]
    up: torch.Tensor              # uint8 [E, gate_stride]
    down: torch.Tensor            # uint8 [E, down_stride]

    def to(self, device) -> "MoeLayer":
        return MoeLayer(self.shape, self.router.to(device), self.gate.to(device),
                        self.up.to(device), self.down.to(device))


def moe_layer(shape: MoeShape, seed: int, device="cpu") -> MoeLayer:
    """One layer's router and expert tensors, all drawn from one seeded stream."""
    gen = make_generator(seed, device)
    router = normal_f32((shape.E, shape.H), 0.02, gen, device)
    gate = q4k_experts(shape.E, shape.F, shape.H, gen, device)
    up = q4k_experts(shape.E, shape.F, shape.H, gen, device)
    down = kquant_experts(shape.down_qtype, shape.E, shape.H, shape.F, gen, device)
    return MoeLayer(shape, router, gate, up, down)


def hidden_states(T: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    return normal_f32((T, H), 1.0, make_generator(seed, device), device)


def skewed_hidden_and_router(layer: MoeLayer, hidden: torch.Tensor, seed: int,
                             hot=(0, 1, 2, 3), frac: float = 0.5,
                             gamma: float = 16.0, delta: float = 0.5):
    """Skewed-routing variant: a seeded half of the tokens gets x += gamma*v and
    the hot experts' router rows get += delta*v for one seeded unit vector v,
    which lifts those experts' logits by about gamma*delta (8) for those tokens
    while adding only delta*(v.x) ~ N(0, delta^2) to the hot logits of the rest.
    Returns new (hidden, router) tensors; the inputs are not modified."""
    dev = hidden.device
    gen = make_generator(seed, dev)
    T, H = hidden.shape
    v = normal_f32((H,), 1.0, gen, dev)
    v = v / torch.linalg.vector_norm(v)
    pick = torch.randperm(T, generator=gen, device=dev)[: int(round(frac * T))]
    x = hidden.clone()
    x[pick] += gamma * v
    r = layer.router.clone()
    r[list(hot)] += delta * v
    return x, r


@dataclasses.dataclass(frozen=True)
class AttnShape:
    """The attention half of a decoder layer: hidden H, n_q query heads,
    n_kv key/value heads, head_dim D, KV-cache capacity S_max."""
    H: int = 2048
    n_q: int = 32
    n_kv: int = 4
    D: int = 128
    S_max: int = 4096
    eps: float = 1e-6
    rope_base: float = 1e7


QWEN3_30B_A3B_ATTN = AttnShape()


def bf16_normal(shape, std: float, gen, device="cpu") -> torch.Tensor:
    """N(0, std^2) drawn in f32 and stored as bfloat16 (nearest-even)."""
    return normal_f32(shape, std, gen, device).to(torch.bfloat16)


@dataclasses.dataclass
class AttnLayer:
    shape: AttnShape
    wq: torch.Tensor              # bf16 [n_q*D, H]
    wk: torch.Tensor              # bf16 [n_kv*D, H]
    wv: torch.Tensor              # bf16 [n_kv*D, H]
    wo: torch.Tensor              # bf16 [H, n_q*D]
    in_norm: torch.Tensor         # f32 [H]
    post_norm: torch.Tensor       # f32 [H]
    q_norm: torch.Tensor          # f32 [D]
    k_norm: torch.Tensor          # f32 [D]

    def to(self, device) -> "AttnLayer":
        return AttnLayer(self.shape, *(t.to(device) for t in (
            self.wq, self.wk, self.wv, self.wo, self.in_norm, self.post_norm, self.q_norm,
            self.k_norm)))


def attn_layer(shape: AttnShape, seed: int, device="cpu") -> AttnLayer:
    gen = make_generator(seed, device)
    qd, kd = shape.n_q * shape.D, shape.n_kv * shape.D
    wq = bf16_normal((qd, shape.H), 0.02, gen, device)
    wk = bf16_normal((kd, shape.H), 0.02, gen, device)
    wv = bf16_normal((kd, shape.H), 0.02, gen, device)
    wo = bf16_normal((shape.H, qd), 0.02, gen, device)
    gains = [uniform_f32((n,), 0.5, 1.5, gen, device) for n in (shape.H, shape.H, shape.D, shape.D)]
    return AttnLayer(shape, wq, wk, wv, wo, *gains)


def kv_caches(B: int, shape: AttnShape, seed: int, device="cpu"):
    """(k_cache, v_cache) bf16 [B, n_kv, S_max, D] ~ N(0, 1)."""
    gen = make_generator(seed, device)
    dims = (B, shape.n_kv, shape.S_max, shape.D)
    return bf16_normal(dims, 1.0, gen, device), bf16_normal(dims, 1.0, gen, device)


def bf16_bits(t: torch.Tensor):
    """The raw uint16 bits of a bfloat16 tensor, as a host NumPy array."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
