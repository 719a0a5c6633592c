"""The whole-model ends of a decode step against the oracle: the token
embedding gather (bit-exact, NaN rows for tokens outside the vocabulary),
the Q6_K output head at the full vocabulary and on ragged row counts
(within 1e-4 relative L2 per token, argmax equal), and a whole decode step
of a 2-layer model: embedding, two Qwen3-MoE decoder layers (attention and
the MoE block), final RMSNorm and the head."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_rows_close, experts_of, oracle_tensors, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
VOCAB = gen.QWEN3_VOCAB


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()


def _rows_host(W, rows, qtype, H):
    """Only the rows the oracle needs, copied to the host (compact table)."""
    rb = q3.q3moe_expert_matrix_bytes(qtype, 1, H)
    sel = torch.as_tensor(rows, dtype=torch.int64, device=W.device)
    return W.view(-1, rb)[sel].cpu().numpy().reshape(-1)


@pytest.mark.parametrize("qtype,V", [(gen.Q4_K, VOCAB), (gen.Q6_K, 37)])
def test_embed_bit_exact(qtype, V):
    H = 2048
    say(f"embed qtype={qtype} V={V}")
    table = gen.kquant_experts(qtype, 1, V, H, gen.make_generator(71, DEV), DEV)[0].contiguous()
    toks = np.array([0, V - 1, 5, 5, V // 2, 17 % V, 3, 1], np.int32)
    out = q3.q3moe_embed(torch.from_numpy(toks).to(DEV), table, qtype, V, H)
    torch.cuda.synchronize()
    uniq, inv = np.unique(toks, return_inverse=True)
    ref = oracle.oracle().embed(inv.astype(np.int32), _rows_host(table, uniq, qtype, H), qtype,
                                len(uniq), H)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    bad = q3.q3moe_embed(torch.tensor([-1, V, 2], dtype=torch.int32, device=DEV), table, qtype, V, H)
    torch.cuda.synchronize()
    b = bad.cpu().numpy()
    assert np.all(np.isnan(b[:2])) and np.array_equal(b[2].view(np.uint32),
                                                      oracle.oracle().embed(np.array([0], np.int32), _rows_host(table, [2], qtype, H), qtype, 1, H)[0].view(np.uint32))


@pytest.mark.parametrize("T,V", [(1, VOCAB), (2, VOCAB), (3, 4099), (1, 9), (2, 1)])
def test_output_head_parity(T, V):
    H = 2048
    say(f"output head T={T} V={V}")
    W = gen.kquant_experts(gen.Q6_K, 1, V, H, gen.make_generator(72 + V, DEV), DEV)[0].contiguous()
    x = gen.hidden_states(T, H, 73 + T)
    logits = q3.q3moe_output_head(x.to(DEV), W, V)
    torch.cuda.synchronize()
    ref = oracle.oracle().output_head(x.numpy(), W.cpu().numpy(), gen.Q6_K, V)
    err = assert_rows_close(logits.cpu().numpy(), ref, what=f"head T={T} V={V}")
    if V > 1:
        assert np.array_equal(logits.cpu().numpy().argmax(1), ref.argmax(1))
    say(f"  max rel L2 {err:.2e}")


def test_output_head_one_hot_columns():
    """A one-hot activation reads back one column of the dequantised matrix
    for every row: an index or plane mistake in any unit shows here."""
    H, V = 2048, 4099
    W = gen.kquant_experts(gen.Q6_K, 1, V, H, gen.make_generator(74, DEV), DEV)[0].contiguous()
    cols = [0, 31, 32, 127, 128, 255, 256, 1000, 2047]
    x = torch.zeros((len(cols), H))
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    got = []
    for i in range(0, len(cols), 2):                  # passes of two tokens and one
        got.append(q3.q3moe_output_head(x[i:i + 2].contiguous().to(DEV), W, V).cpu().numpy())
    got = np.concatenate(got)
    ref = oracle.oracle().output_head(x.numpy(), W.cpu().numpy(), gen.Q6_K, V)
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=0)


def test_two_layer_model_decode_step():
    """embedding -> 2 decoder layers (input RMSNorm, Q/K/V, QK-norm + RoPE,
    KV write, GQA attention, O projection, post-attention RMSNorm, route,
    expert FFN) -> final RMSNorm -> head, for two sequences, on the GPU
    entry points and on the oracle's functions."""
    s = gen.QWEN3_30B_A3B_ATTN
    H, V, B = 2048, 4099, 2
    o = oracle.oracle()
    g = gen.make_generator(75, DEV)
    emb = gen.kquant_experts(gen.Q4_K, 1, V, H, g, DEV)[0].contiguous()
    head = gen.kquant_experts(gen.Q6_K, 1, V, H, g, DEV)[0].contiguous()
    final_norm = gen.uniform_f32((H,), 0.5, 1.5, gen.make_generator(76))
    toks = np.array([11, 4000], np.int32)
    pos = np.array([s.S_max - 1, s.S_max - 300], np.int32)
    layers = []
    for l in range(2):
        att = gen.attn_layer(s, 80 + l)
        moe = gen.moe_layer(gen.MoeShape(T=B, H=H, E=128, k=8, F=768,
                                         down_qtype=gen.stack_down_qtype(47 * l)), 90 + l)
        kc, vc = gen.kv_caches(B, s, 95 + l)
        layers.append((att, moe, kc, vc))
    # GPU
    x = q3.q3moe_embed(torch.from_numpy(toks).to(DEV), emb, gen.Q4_K, V, H)
    posd = torch.from_numpy(pos).to(DEV)
    for att, moe, kc, vc in layers:
        A, M = att.to(DEV), moe.to(DEV)
        kcd, vcd = kc.to(DEV), vc.to(DEV)
        q, k, v = q3.q3moe_bf16_gemv3([A.wq, A.wk, A.wv], x, norm_gain=A.in_norm, eps=s.eps)
        q3.q3moe_attn_prologue_kv(q.view(B, s.n_q, s.D), k.view(B, s.n_kv, s.D), v.view(B, s.n_kv, s.D),
                                  A.q_norm, A.k_norm, posd, s.eps, s.rope_base, kcd, vcd)
        a = q3.q3moe_gqa_attention(q.view(B, s.n_q, s.D), kcd, vcd, posd + 1, 1.0 / np.sqrt(s.D))
        q3.q3moe_bf16_gemv(A.wo, a.view(B, -1), out=x, accumulate=True)
        q3.q3moe_moe_ffn_prenorm(x, A.post_norm, s.eps, M.router, 8, *experts_of(M), F=768, out=x,
                                 accumulate=True)
    xn = q3.q3moe_rmsnorm(x, final_norm.to(DEV), s.eps)
    logits = q3.q3moe_output_head(xn, head, V)
    torch.cuda.synchronize()
    # oracle
    xr = o.embed(toks, emb.cpu().numpy(), gen.Q4_K, V, H)
    for att, moe, kc, vc in layers:
        bits = [gen.bf16_bits(t) for t in (att.wq, att.wk, att.wv, att.wo)]
        gains = [t.numpy() for t in (att.in_norm, att.post_norm, att.q_norm, att.k_norm)]
        xr, _, _, _, _ = o.decoder_layer(xr, *bits, *gains, gen.bf16_bits(kc), gen.bf16_bits(vc), pos,
                                         s.n_q, s.n_kv, s.D, s.eps, s.rope_base, moe.router.numpy(), 8,
                                         *oracle_tensors(moe), F=768, E=128)
    ref = o.output_head(o.rmsnorm(xr, final_norm.numpy(), s.eps), head.cpu().numpy(), gen.Q6_K, V)
    err = assert_rows_close(logits.cpu().numpy(), ref, what="2-layer model logits")
    assert np.array_equal(logits.cpu().numpy().argmax(1), ref.argmax(1))
    say(f"2-layer model decode step: max rel L2 {err:.2e}")
