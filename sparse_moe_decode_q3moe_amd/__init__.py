"""Qwen3-MoE sparse FFN block on AMD Instinct MI355X (gfx950).

The compute path is libq3moe.so (hand-written HIP kernels behind a C ABI,
include/q3moe.h); this package is its Python binding plus the seeded input
generator.  Functions carry the C entry points' names.
"""
from ._lib import (  # noqa: F401
    EXPORTS, Experts, Q3MoeError, Q4_K, Q6_K, expert_ffn_status, library,
    q3moe_attn_prologue, q3moe_attn_prologue_kv, q3moe_bf16_gemv, q3moe_bf16_gemv3, q3moe_expert_ffn, q3moe_expert_ffn_status_offset,
    q3moe_expert_ffn_workspace_bytes, q3moe_gqa_attention,
    q3moe_gqa_attention_workspace_bytes, q3moe_group_by_expert, q3moe_kv_write,
    q3moe_moe_ffn, q3moe_moe_ffn_noalloc, q3moe_moe_ffn_prenorm, q3moe_moe_stack,
    q3moe_moe_stack_workspace_bytes, MoeLayer, q3moe_moe_ffn_workspace_bytes, q3moe_persistent_path,
    q3moe_rmsnorm, q3moe_route, q3moe_route_workspace_bytes, q3moe_embed, q3moe_output_head,
    q3moe_kv_write_rows, q3moe_prefill_attention,
    q3moe_expert_matrix_bytes,
)
