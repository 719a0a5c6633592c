"""The attention side of the decoder layer on the HIP path vs the CPU oracle:
bf16 projections, the KV-cache write, grouped-query decode attention, and
the whole Qwen3-30B-A3B decoder layer (input RMSNorm -> Q/K/V -> Q/K norm +
RoPE -> KV write -> attention -> O + residual -> post-attention RMSNorm ->
route -> expert FFN + residual) at batch 1 and 16 with 4096 cached
positions.

Bars: the KV write is bit-exact; f32 outputs agree within 1e-4 relative L2
per row; expert choices are equal.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_indices_equal, assert_rows_close, experts_of, oracle_tensors, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()


def _bits(t):
    return gen.bf16_bits(t)


# ------------------------------------------------------------------- GEMV --

GEMV_CASES = [  # (T, N, K, accumulate, seed)
    (1, 4096, 2048, False, 1),     # W_q at batch 1
    (1, 512, 2048, False, 2),      # W_k / W_v
    (1, 2048, 4096, True, 3),      # W_o with the residual add
    (16, 4096, 2048, False, 4),    # batch 16
    (16, 2048, 4096, True, 5),
    (16, 512, 2048, False, 6),
    (3, 100, 72, False, 7),        # ragged rows, K below one wave step
    (5, 37, 1032, True, 8),        # K not a multiple of 512, odd tokens
    (17, 300, 2056, False, 9),     # more than 16 tokens: two passes
    (1, 1, 8, False, 10),          # the smallest shape
    (2, 3000, 8200, False, 11),    # K beyond one staged chunk of every kernel shape
    (9, 2049, 520, True, 12),
    # the matrix-core form (9+ tokens, K a multiple of 256 up to 4096)
    (17, 300, 2048, False, 13),    # two passes (16 + 1), a partial row tile
    (40, 2049, 256, True, 14),     # one wave per tile, three passes (the last of 8 tokens)
    (63, 33, 4096, False, 15),     # sixteen waves per tile, four passes
    (9, 16, 512, True, 16),        # the fewest tokens it takes
]


@pytest.mark.parametrize("T,N,K,acc,seed", GEMV_CASES)
def test_bf16_gemv_parity(T, N, K, acc, seed):
    say(f"gemv T={T} N={N} K={K} acc={acc} seed={seed}")
    g = gen.make_generator(seed)
    W = gen.bf16_normal((N, K), 0.02, g)
    x = gen.normal_f32((T, K), 1.0, g)
    y0 = gen.normal_f32((T, N), 1.0, g) if acc else None
    ref = oracle.oracle().bf16_gemv(_bits(W), x.numpy(), y0.numpy() if acc else None, accumulate=acc)
    out = y0.to(DEV) if acc else None
    got = q3.q3moe_bf16_gemv(W.to(DEV), x.to(DEV), out=out, accumulate=acc)
    torch.cuda.synchronize()
    assert_rows_close(got.cpu().numpy(), ref, what=f"gemv T={T} N={N} K={K}")


GEMV3_CASES = [  # T, (N0, N1, N2), K, norm, seed
    (1, (4096, 512, 512), 2048, True, 21),     # the layer's Q/K/V after its input norm, batch 1
    (16, (4096, 512, 512), 2048, True, 22),    # batch 16
    (3, (4096, 512, 512), 2048, False, 23),    # no norm
    (5, (100, 37, 0), 1032, True, 24),         # ragged rows, two matrices, K not a multiple of 512
    (17, (300, 0, 0), 2056, True, 25),         # more than 16 tokens: two passes, one matrix
    (2, (3000, 64, 8), 8200, True, 26),        # K beyond one staged chunk
    (1, (1, 1, 1), 8, True, 27),               # the smallest shape
    # the matrix-core form, with and without the norm
    (17, (300, 40, 0), 2048, True, 28),        # two passes, partial row tiles
    (64, (128, 16, 16), 1024, True, 29),       # 64 tokens with the norm: four passes
    (20, (50, 7, 0), 768, True, 30),           # three waves per tile, two matrices
    (12, (4096, 512, 512), 2048, False, 31),   # no norm
]


@pytest.mark.parametrize("T,Ns,K,norm,seed", GEMV3_CASES)
def test_bf16_gemv3_parity(T, Ns, K, norm, seed):
    """Up to three projections in one launch, with the input RMSNorm inside:
    each output against the oracle's RMSNorm then its bf16 GEMV."""
    say(f"gemv3 T={T} N={Ns} K={K} norm={norm} seed={seed}")
    g = gen.make_generator(seed)
    Ws = [gen.bf16_normal((n, K), 0.02, g) for n in Ns if n]
    x = gen.normal_f32((T, K), 1.0, g)
    gain = gen.uniform_f32((K,), 0.5, 1.5, g)
    o = oracle.oracle()
    xn = o.rmsnorm(x.numpy(), gain.numpy(), 1e-6) if norm else x.numpy()
    got = q3.q3moe_bf16_gemv3([W.to(DEV) for W in Ws], x.to(DEV),
                              norm_gain=gain.to(DEV) if norm else None, eps=1e-6)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        ref = o.bf16_gemv(_bits(W), xn)
        assert_rows_close(got[i].cpu().numpy(), ref, what=f"gemv3 output {i}")


def test_bf16_gemv_zero_tokens():
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((0, 64), dtype=torch.float32, device=DEV)
    y = q3.q3moe_bf16_gemv(W, x)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


# ------------------------------------------------- prologue + KV write --

@pytest.mark.parametrize("B,pos_list", [(1, [4095]), (16, None), (3, [5, -1, 4096])])
def test_attn_prologue_kv_matches_two_calls(B, pos_list):
    """The fused prologue + KV write equals q3moe_attn_prologue followed by
    q3moe_kv_write bit for bit (q, k and both caches), including positions
    outside the cache (nothing written)."""
    say(f"prologue+kv B={B}")
    s = gen.QWEN3_30B_A3B_ATTN
    g = gen.make_generator(70 + B)
    q = gen.normal_f32((B, s.n_q, s.D), 1.0, g)
    k = gen.normal_f32((B, s.n_kv, s.D), 1.0, g)
    v = gen.normal_f32((B, s.n_kv, s.D), 1.0, g)
    qn = gen.uniform_f32((s.D,), 0.5, 1.5, g)
    kn = gen.uniform_f32((s.D,), 0.5, 1.5, g)
    pos = torch.tensor(pos_list if pos_list else [s.S_max - 1 - 211 * b for b in range(B)],
                       dtype=torch.int32)
    kc, vc = gen.kv_caches(B, s, 80 + B)
    q1, k1, kc1, vc1 = q.to(DEV), k.to(DEV), kc.to(DEV), vc.to(DEV)
    q3.q3moe_attn_prologue(q1, k1, qn.to(DEV), kn.to(DEV), pos.to(DEV), s.eps, s.rope_base)
    q3.q3moe_kv_write(k1, v.to(DEV), pos.to(DEV), kc1, vc1)
    q2, k2, kc2, vc2 = q.to(DEV), k.to(DEV), kc.to(DEV), vc.to(DEV)
    q3.q3moe_attn_prologue_kv(q2, k2, v.to(DEV), qn.to(DEV), kn.to(DEV), pos.to(DEV), s.eps,
                              s.rope_base, kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(q1.cpu().view(torch.int32), q2.cpu().view(torch.int32))
    assert torch.equal(k1.cpu().view(torch.int32), k2.cpu().view(torch.int32))
    assert np.array_equal(_bits(kc1), _bits(kc2))
    assert np.array_equal(_bits(vc1), _bits(vc2))


# --------------------------------------------------------------- KV write --

def test_kv_write_bit_exact():
    """Rounding ties, NaN, infinities, overflow to infinity and subnormals,
    one position per sequence, a position out of range (no write)."""
    B, nkv, S, D = 5, 4, 96, 128
    say(f"kv write B={B} S={S}")
    g = gen.make_generator(31)
    kc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    vc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    kn = gen.normal_f32((B, nkv, D), 3.0, g)
    vn = gen.normal_f32((B, nkv, D), 3.0, g)
    specials = torch.tensor([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, float("nan"),
                             float("inf"), -float("inf"), 3.4e38, 1e-40, -0.0, 2.0 ** -133],
                            dtype=torch.float32)
    kn[0, 0, :specials.numel()] = specials
    vn[1, 2, -specials.numel():] = specials
    pos = torch.tensor([0, 95, 17, 96, 40], dtype=torch.int32)       # 96 is out of range
    ref_k, ref_v = oracle.oracle().kv_write(kn.numpy(), vn.numpy(), np.clip(pos.numpy(), 0, S - 1),
                                            _bits(kc), _bits(vc))
    # the oracle refuses out-of-range positions; that sequence keeps its cache
    ref_k[3], ref_v[3] = _bits(kc)[3], _bits(vc)[3]
    kd, vd = kc.to(DEV), vc.to(DEV)
    q3.q3moe_kv_write(kn.to(DEV), vn.to(DEV), pos.to(DEV), kd, vd)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kd), ref_k)
    assert np.array_equal(_bits(vd), ref_v)


# -------------------------------------------------------------- attention --

ATTN_CASES = [  # (B, n_q, n_kv, D, S_max, lengths or None for S_max, q_std, seed)
    (1, 32, 4, 128, 4096, None, 1.0, 41),                     # the decode layer, full cache
    (16, 32, 4, 128, 4096, [4096, 1, 63, 64, 65, 4095, 128, 129, 2000, 4033, 700, 3,
                             1024, 4000, 257, 3999], 1.0, 42),  # batch 16, ragged lengths
    (2, 32, 4, 128, 4096, [4096, 2500], 6.0, 43),              # peaked softmax
    (3, 8, 8, 64, 300, [300, 1, 77], 1.0, 44),                 # D = 64, no grouping
    (2, 16, 1, 256, 200, [200, 129], 1.0, 45),                 # D = 256, group 16
    (2, 12, 4, 128, 130, [130, 66], 1.0, 46),                  # group 3: one wave idle
    (1, 40, 8, 128, 1000, [999], 1.0, 47),                     # group 5
    (64, 32, 4, 128, 512, None, 1.0, 48),                      # many sequences: 4 tiles per workgroup
]


@pytest.mark.parametrize("B,nq,nkv,D,S,lengths,qstd,seed", ATTN_CASES)
def test_gqa_attention_parity(B, nq, nkv, D, S, lengths, qstd, seed):
    say(f"attention B={B} nq={nq} nkv={nkv} D={D} S={S} seed={seed}")
    g = gen.make_generator(seed)
    q = gen.normal_f32((B, nq, D), qstd, g)
    kc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    vc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    lens = torch.tensor(lengths if lengths is not None else [S] * B, dtype=torch.int32)
    # positions at or past each length hold NaN: reading one would poison the output
    kb, vb = _bits(kc).copy(), _bits(vc).copy()
    for b in range(B):
        kb[b, :, lens[b]:] = BF16_NAN
        vb[b, :, lens[b]:] = BF16_NAN
    kc = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16)
    vc = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    ref = oracle.oracle().gqa_attention(q.numpy(), kb, vb, lens.numpy(), scale)
    got = q3.q3moe_gqa_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), scale)
    torch.cuda.synchronize()
    assert_rows_close(got.cpu().numpy().reshape(B * nq, D), ref.reshape(B * nq, D),
                      what=f"attention B={B} D={D}")


def test_gqa_attention_invalid_length_gives_nan():
    """A length of 0 or beyond S_max reads nothing and yields NaN for that
    sequence only."""
    B, nq, nkv, D, S = 3, 32, 4, 128, 256
    g = gen.make_generator(49)
    q = gen.normal_f32((B, nq, D), 1.0, g)
    kc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    vc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
    lens = torch.tensor([0, 100, S + 1], dtype=torch.int32)
    got = q3.q3moe_gqa_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), 0.0884).cpu()
    ref = oracle.oracle().gqa_attention(q[1:2].numpy(), _bits(kc)[1:2], _bits(vc)[1:2],
                                        np.array([100], np.int32), 0.0884)
    assert torch.isnan(got[0]).all() and torch.isnan(got[2]).all()
    assert_rows_close(got[1].numpy(), ref[0], what="attention valid row")


def test_gqa_attention_workspace_reuse():
    """One workspace through calls of several batch sizes."""
    nq, nkv, D, S = 32, 4, 128, 1024
    ws = torch.empty(q3.q3moe_gqa_attention_workspace_bytes(64, nq, nkv, D, S), dtype=torch.uint8,
                     device=DEV)
    g = gen.make_generator(50)
    for B in (64, 1, 16, 3):
        say(f"attention reuse B={B}")
        q = gen.normal_f32((B, nq, D), 1.0, g)
        kc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
        vc = gen.bf16_normal((B, nkv, S, D), 1.0, g)
        lens = torch.randint(1, S + 1, (B,), generator=g, dtype=torch.int32)
        ref = oracle.oracle().gqa_attention(q.numpy(), _bits(kc), _bits(vc), lens.numpy(), 0.0884)
        got = q3.q3moe_gqa_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), lens.to(DEV), 0.0884,
                                     workspace=ws)
        torch.cuda.synchronize()
        assert_rows_close(got.cpu().numpy().reshape(B * nq, D), ref.reshape(B * nq, D),
                          what=f"attention reuse B={B}")


# ------------------------------------------------------ whole decoder layer --

def _positions(B, S):
    if B == 1:
        return np.array([S - 1], np.int32)
    return np.array([S - 1 - 211 * b for b in range(B)], np.int32)


def oracle_layer(o, att, moe, x, kc, vc, pos):
    """The decoder layer on the oracle, step by step (f32 between steps)."""
    s = att.shape
    B = x.shape[0]
    xn = o.rmsnorm(x, att.in_norm.numpy(), s.eps)
    q = o.bf16_gemv(_bits(att.wq), xn).reshape(B, s.n_q, s.D)
    k = o.bf16_gemv(_bits(att.wk), xn).reshape(B, s.n_kv, s.D)
    v = o.bf16_gemv(_bits(att.wv), xn).reshape(B, s.n_kv, s.D)
    q, k = o.attn_prologue(q, k, att.q_norm.numpy(), att.k_norm.numpy(), pos, s.eps, s.rope_base)
    kc, vc = o.kv_write(k, v, pos, kc, vc)
    a = o.gqa_attention(q, kc, vc, pos + 1, 1.0 / np.sqrt(s.D))
    x1 = o.bf16_gemv(_bits(att.wo), a.reshape(B, -1), x, accumulate=True)
    h = o.rmsnorm(x1, att.post_norm.numpy(), s.eps)
    ms = moe.shape
    idx, w, logits = o.route(h, moe.router.numpy(), ms.k)
    out = o.expert_ffn(h, idx, w, *oracle_tensors(moe), F=ms.F, E=ms.E, out=x1, accumulate=True)
    return dict(a=a, x1=x1, idx=idx, logits=logits, out=out, kc=kc, vc=vc)


def gpu_layer(att, moe, x, kc, vc, pos, form="separate"):
    s = att.shape
    B = x.shape[0]
    if form == "prenorm":                # input norm + Q/K/V in one launch
        q, k, v = q3.q3moe_bf16_gemv3([att.wq, att.wk, att.wv], x, norm_gain=att.in_norm, eps=s.eps)
        q, k, v = q.view(B, s.n_q, s.D), k.view(B, s.n_kv, s.D), v.view(B, s.n_kv, s.D)
    else:
        xn = q3.q3moe_rmsnorm(x, att.in_norm, s.eps)
        q = q3.q3moe_bf16_gemv(att.wq, xn).view(B, s.n_q, s.D)
        k = q3.q3moe_bf16_gemv(att.wk, xn).view(B, s.n_kv, s.D)
        v = q3.q3moe_bf16_gemv(att.wv, xn).view(B, s.n_kv, s.D)
    if form == "prenorm":                # prologue and KV write in one launch
        q3.q3moe_attn_prologue_kv(q, k, v, att.q_norm, att.k_norm, pos, s.eps, s.rope_base, kc, vc)
    else:
        q3.q3moe_attn_prologue(q, k, att.q_norm, att.k_norm, pos, s.eps, s.rope_base)
        q3.q3moe_kv_write(k, v, pos, kc, vc)
    a = q3.q3moe_gqa_attention(q, kc, vc, pos + 1, 1.0 / np.sqrt(s.D))
    x1 = x.clone()
    q3.q3moe_bf16_gemv(att.wo, a.view(B, -1), out=x1, accumulate=True)
    ms = moe.shape
    out = x1.clone()
    if form == "prenorm":                # norm + route + FFN in one call, in place
        _, idx, _ = q3.q3moe_moe_ffn_prenorm(out, att.post_norm, s.eps, moe.router, ms.k,
                                             *experts_of(moe), F=ms.F, out=out, accumulate=True)
        return dict(a=a, x1=x1, idx=idx, out=out)
    h = q3.q3moe_rmsnorm(x1, att.post_norm, s.eps)
    idx, w = q3.q3moe_route(h, moe.router, ms.k)
    q3.q3moe_expert_ffn(h, idx, w, *experts_of(moe), F=ms.F, out=out, accumulate=True)
    return dict(a=a, x1=x1, idx=idx, out=out)


@pytest.mark.parametrize("form", ["separate", "prenorm"])
@pytest.mark.parametrize("B", [1, 16])
def test_decoder_layer_parity(B, form):
    say(f"decoder layer B={B} form={form}")
    att = gen.attn_layer(gen.QWEN3_30B_A3B_ATTN, 61)
    moe = gen.moe_layer(gen.QWEN3_30B_A3B, 62)
    s = att.shape
    x = gen.hidden_states(B, s.H, 63)
    kc, vc = gen.kv_caches(B, s, 64)
    pos = _positions(B, s.S_max)
    ref = oracle_layer(oracle.oracle(), att, moe, x.numpy(), _bits(kc), _bits(vc), pos)
    got = gpu_layer(att.to(DEV), moe.to(DEV), x.to(DEV), kc.to(DEV), vc.to(DEV),
                    torch.from_numpy(pos).to(DEV), form)
    torch.cuda.synchronize()
    assert_rows_close(got["a"].cpu().numpy().reshape(B, -1), ref["a"].reshape(B, -1), what="attention")
    assert_rows_close(got["x1"].cpu().numpy(), ref["x1"], what="residual after O")
    assert_indices_equal(got["idx"].cpu().numpy(), ref["idx"], ref["logits"], moe.shape.k, "route")
    err = assert_rows_close(got["out"].cpu().numpy(), ref["out"], what="layer output")
    say(f"decoder layer B={B}: max rel L2 {err:.2e}")
