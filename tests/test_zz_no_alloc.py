"""q3moe_moe_ffn_noalloc (the MoE block with the library's own device
scratch as its workspace) against q3moe_moe_ffn with a caller workspace, on
consecutive calls that take both paths (two launches at 8 tokens, then the
one persistent kernel at 1 token, then 3 tokens) and reuse the scratch each
time: the same expert indices and routing weights, outputs equal to the
workspace entry point's bit for bit, and within 1e-4 relative L2 of the
oracle.  Shapes beyond the scratch are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_indices_equal, assert_rows_close, experts_of, oracle_moe, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()
    cpu = gen.moe_layer(gen.QWEN3_30B_A3B, 3131)
    return cpu, cpu.to(DEV)


def test_noalloc_matches_workspace_entry_point(layer):
    cpu, dev = layer
    g = gen.make_generator(3132)
    for T in (8, 1, 3):
        s = gen.MoeShape(T=T, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K)
        lay = gen.MoeLayer(s, cpu.router, cpu.gate, cpu.up, cpu.down)
        x = gen.normal_f32((T, 2048), 1.0, g)
        xd = x.to(DEV)
        say(f"noalloc call T={T} persistent={q3.q3moe_persistent_path(T, 2048, 768, 128, 8, gen.Q6_K, True)}")
        out_n, idx_n, w_n = q3.q3moe_moe_ffn_noalloc(xd, dev.router, 8, *experts_of(dev), F=768)
        ws = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(T, 2048, 768, 128, 8), dtype=torch.uint8,
                         device=DEV)
        out_w, idx_w, w_w = q3.q3moe_moe_ffn(xd, dev.router, 8, *experts_of(dev), F=768, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx_n.cpu(), idx_w.cpu())
        assert torch.equal(w_n.cpu(), w_w.cpu())
        assert torch.equal(out_n.cpu().view(torch.int32), out_w.cpu().view(torch.int32))
        ref_idx, ref_w, logits, ref = oracle_moe(lay, x.numpy())
        assert_indices_equal(idx_n.cpu().numpy(), ref_idx, logits, 8, f"noalloc T={T}")
        np.testing.assert_allclose(w_n.cpu().numpy(), ref_w, rtol=1e-6, atol=0)
        err = assert_rows_close(out_n.cpu().numpy(), ref, what=f"noalloc T={T}")
        say(f"  max rel L2 {err:.2e}")


def test_noalloc_accumulate_and_limit(layer):
    cpu, dev = layer
    x = gen.hidden_states(2, 2048, 3133)
    prev = gen.hidden_states(2, 2048, 3134)
    out = prev.to(DEV)
    q3.q3moe_moe_ffn_noalloc(x.to(DEV), dev.router, 8, *experts_of(dev), F=768, out=out,
                             accumulate=True)
    torch.cuda.synchronize()
    s = gen.MoeShape(T=2, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K)
    lay = gen.MoeLayer(s, cpu.router, cpu.gate, cpu.up, cpu.down)
    _, _, _, ref = oracle_moe(lay, x.numpy(), out=prev.numpy(), accumulate=True)
    assert_rows_close(out.cpu().numpy(), ref, what="noalloc accumulate")
    big = 64                                       # needs more than the 4 MiB scratch
    assert q3.q3moe_moe_ffn_workspace_bytes(big, 2048, 768, 128, 8) > (4 << 20)
    xb = torch.zeros((big, 2048), device=DEV)
    with pytest.raises(q3.Q3MoeError) as e:
        q3.q3moe_moe_ffn_noalloc(xb, dev.router, 8, *experts_of(dev), F=768)
    assert e.value.status == 5
