"""The attention side of batched prefill against the oracle: the projections
of many tokens on the matrix cores (q3moe_bf16_gemv from 64 tokens on), the
KV rows of one sequence (bit-exact), causal prefill attention (from position
0 and after a 3,584-position prefix, ragged and unordered positions, MHA and
GQA groups, invalid positions, a causal probe with poisoned future rows), and
a whole Qwen3-MoE decoder layer over a 512-token prompt."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_rows_close, oracle_tensors, experts_of, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
S = gen.QWEN3_30B_A3B_ATTN


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()


def _bits(t):
    return gen.bf16_bits(t)


@pytest.mark.parametrize("T,N,K,acc", [(512, 4096, 2048, False), (512, 512, 2048, False),
                                       (100, 520, 2048, True), (64, 2048, 4096, True),
                                       (300, 136, 96, False)])
def test_bf16_gemm_parity(T, N, K, acc):
    say(f"bf16 GEMM T={T} N={N} K={K} acc={acc}")
    g = gen.make_generator(300 + T + N)
    W = gen.bf16_normal((N, K), 0.02, g)
    x = gen.normal_f32((T, K), 1.0, g)
    y0 = gen.normal_f32((T, N), 1.0, g)
    y = y0.to(DEV).clone()
    q3.q3moe_bf16_gemv(W.to(DEV), x.to(DEV), out=y, accumulate=acc)
    torch.cuda.synchronize()
    ref = oracle.oracle().bf16_gemv(_bits(W), x.numpy(), y0.numpy() if acc else None, accumulate=acc)
    err = assert_rows_close(y.cpu().numpy(), ref, what=f"GEMM T={T} N={N}")
    say(f"  max rel L2 {err:.2e}")


def test_bf16_gemv3_many_tokens_without_norm():
    """gemv3 without a norm at 512 tokens: three GEMMs, each equal to the
    single-matrix call bit for bit."""
    g = gen.make_generator(311)
    Ws = [gen.bf16_normal((n, 2048), 0.02, g).to(DEV) for n in (4096, 512, 512)]
    x = gen.normal_f32((512, 2048), 1.0, g).to(DEV)
    ys = q3.q3moe_bf16_gemv3(Ws, x)
    for W, y in zip(Ws, ys):
        y1 = q3.q3moe_bf16_gemv(W, x)
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), y1.cpu())


def test_kv_write_rows_bit_exact():
    g = gen.make_generator(312)
    T = 512
    k = gen.normal_f32((T, S.n_kv, S.D), 1.0, g)
    v = gen.normal_f32((T, S.n_kv, S.D), 1.0, g)
    kc, vc = (c[0] for c in gen.kv_caches(1, S, 313))
    pos = np.arange(3584, 3584 + T, dtype=np.int32)
    pos[5] = -1                                        # writes nothing
    pos[6] = S.S_max                                   # writes nothing
    kd, vd = kc.to(DEV).contiguous(), vc.to(DEV).contiguous()
    q3.q3moe_kv_write_rows(k.to(DEV), v.to(DEV), torch.from_numpy(pos).to(DEV), kd, vd)
    torch.cuda.synchronize()
    ok = (pos >= 0) & (pos < S.S_max)
    rk, rv = oracle.oracle().kv_write_rows(k.numpy()[ok], v.numpy()[ok], pos[ok], _bits(kc), _bits(vc))
    assert np.array_equal(_bits(kd), rk) and np.array_equal(_bits(vd), rv)


def _attn_case(T, nq, nkv, pos, seed, poison_after=None):
    g = gen.make_generator(seed)
    q = gen.normal_f32((T, nq, 128), 1.0, g)
    kc = gen.bf16_normal((nkv, S.S_max, 128), 1.0, g)
    vc = gen.bf16_normal((nkv, S.S_max, 128), 1.0, g)
    if poison_after is not None:                      # NaN in every row no query may read
        kc[:, poison_after + 1:] = float("nan")
        vc[:, poison_after + 1:] = float("nan")
    return q, kc, vc, np.asarray(pos, np.int32)


@pytest.mark.parametrize("name,T,nq,nkv,start", [
    ("prompt_512_gqa8", 512, 32, 4, 0),
    ("chunk_512_after_3584", 512, 32, 4, 3584),
    ("ragged_37", 37, 32, 4, 1000),
    ("mha_70", 70, 4, 4, 10),
    ("gqa4_33", 33, 16, 4, 63),
])
def test_prefill_attention_parity(name, T, nq, nkv, start):
    say(f"prefill attention {name}")
    pos = np.arange(start, start + T)
    q, kc, vc, pos = _attn_case(T, nq, nkv, pos, 320 + T, poison_after=int(pos.max()))
    out = q3.q3moe_prefill_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(pos).to(DEV),
                                     1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    ref = oracle.oracle().prefill_attention(q.numpy(), _bits(kc), _bits(vc), pos, 1.0 / math.sqrt(128))
    err = assert_rows_close(out.cpu().numpy().reshape(T * nq, 128), ref.reshape(T * nq, 128),
                            what=name)
    say(f"  max rel L2 {err:.2e}")


def test_prefill_attention_unordered_and_invalid_positions():
    """Positions in any order, repeated, and out of range (NaN rows, and no
    cache row past each query's position is read: those rows hold NaN)."""
    T = 50
    rng = np.random.default_rng(7)
    pos = rng.integers(0, 700, size=T).astype(np.int32)
    pos[3] = pos[4]
    pos[10] = -1
    pos[11] = S.S_max
    q, kc, vc, pos = _attn_case(T, 32, 4, pos, 331)
    kc[:, 700:] = float("nan")
    vc[:, 700:] = float("nan")
    out = q3.q3moe_prefill_attention(q.to(DEV), kc.to(DEV), vc.to(DEV), torch.from_numpy(pos).to(DEV), 0.09)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ok = (pos >= 0) & (pos < S.S_max)
    assert np.all(np.isnan(got[~ok]))
    ref = oracle.oracle().prefill_attention(q.numpy()[ok], _bits(kc), _bits(vc), pos[ok], 0.09)
    assert_rows_close(got[ok].reshape(-1, 128), ref.reshape(-1, 128), what="unordered positions")


def test_decoder_layer_prefill_512():
    """A whole decoder layer over a 512-token prompt (positions 0..511):
    RMSNorm, Q/K/V GEMMs, QK-norm + RoPE rows, KV rows, causal attention, O
    GEMM with the residual, then the MoE block on the grouped prefill path.
    Every stage is checked on the oracle's own input (as the 48-layer test
    checks each layer on the oracle's stream): projections + prologue, the
    new cache rows (one bf16 step at most: the two sides' k and v differ by
    f32 rounding before they are rounded to bf16), attention on the oracle's
    caches, the O projection, the MoE block (exact routing).  The
    free-running layer is held to 2e-3: a token early in the prompt attends
    to few rows, so one bf16 step of its own v row reaches its output."""
    T = 512
    say("decoder layer prefill T=512")
    att = gen.attn_layer(S, 340)
    moe = gen.moe_layer(gen.MoeShape(T=T, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K), 341)
    kc, vc = (c[0].contiguous() for c in gen.kv_caches(1, S, 342))
    x = gen.hidden_states(T, 2048, 343)
    pos = np.arange(T, dtype=np.int32)
    A, M = att.to(DEV), moe.to(DEV)
    kd, vd = kc.to(DEV), vc.to(DEV)
    posd = torch.from_numpy(pos).to(DEV)
    scale = 1.0 / math.sqrt(S.D)
    o = oracle.oracle()
    bits = [_bits(t) for t in (att.wq, att.wk, att.wv, att.wo)]
    # oracle, stage by stage
    xn_r = o.rmsnorm(x.numpy(), att.in_norm.numpy(), S.eps)
    q_r = o.bf16_gemv(bits[0], xn_r).reshape(T, S.n_q, S.D)
    k_r = o.bf16_gemv(bits[1], xn_r).reshape(T, S.n_kv, S.D)
    v_r = o.bf16_gemv(bits[2], xn_r).reshape(T, S.n_kv, S.D)
    q_r, k_r = o.attn_prologue(q_r, k_r, att.q_norm.numpy(), att.k_norm.numpy(), pos, S.eps, S.rope_base)
    kc_r, vc_r = o.kv_write_rows(k_r, v_r, pos, _bits(kc), _bits(vc))
    a_r = o.prefill_attention(q_r, kc_r, vc_r, pos, scale)
    x1_r = o.bf16_gemv(bits[3], a_r.reshape(T, -1), x.numpy(), accumulate=True)
    out_r, idx_r, _, _ = o.moe_block(x1_r, moe.router.numpy(), 8, *oracle_tensors(moe), F=768, E=128,
                                     norm_gain=att.post_norm.numpy(), eps=S.eps, residual=True)
    # GPU, free running
    xd = x.to(DEV)
    xn = q3.q3moe_rmsnorm(xd, A.in_norm, S.eps)
    q, k, v = q3.q3moe_bf16_gemv3([A.wq, A.wk, A.wv], xn)
    q, k, v = q.view(T, S.n_q, S.D), k.view(T, S.n_kv, S.D), v.view(T, S.n_kv, S.D)
    q3.q3moe_attn_prologue(q, k, A.q_norm, A.k_norm, posd, S.eps, S.rope_base)
    q3.q3moe_kv_write_rows(k, v, posd, kd, vd)
    a = q3.q3moe_prefill_attention(q, kd, vd, posd, scale)
    q3.q3moe_bf16_gemv(A.wo, a.view(T, -1), out=xd, accumulate=True)
    _, idx_free, _ = q3.q3moe_moe_ffn_prenorm(xd, A.post_norm, S.eps, M.router, 8, *experts_of(M),
                                              F=768, out=xd, accumulate=True)
    torch.cuda.synchronize()
    e_q = assert_rows_close(q.cpu().numpy().reshape(T, -1), q_r.reshape(T, -1), what="q after prologue")
    assert_rows_close(k.cpu().numpy().reshape(T, -1), k_r.reshape(T, -1), what="k after prologue")
    assert_rows_close(v.cpu().numpy().reshape(T, -1), v_r.reshape(T, -1), what="v")
    for got, ref in ((_bits(kd), kc_r), (_bits(vd), vc_r)):
        assert np.array_equal(got[:, T:], ref[:, T:])
        gv = (got[:, :T].astype(np.uint32) << 16).view(np.float32).reshape(-1, S.D)
        rv_ = (ref[:, :T].astype(np.uint32) << 16).view(np.float32).reshape(-1, S.D)
        bound = 2.0 ** -7 * np.maximum(np.abs(gv), np.abs(rv_)) + \
            1e-5 * np.abs(rv_).max(axis=1, keepdims=True)
        assert np.all(np.abs(gv - rv_) <= bound), "new cache rows differ by more than rounding"
        assert (gv != rv_).mean() < 1e-2
    # attention on the oracle's caches and queries, O projection on its output
    qo = torch.from_numpy(q_r).to(DEV)
    a2 = q3.q3moe_prefill_attention(qo, torch.from_numpy(kc_r.view(np.int16)).to(DEV).view(torch.bfloat16),
                                    torch.from_numpy(vc_r.view(np.int16)).to(DEV).view(torch.bfloat16),
                                    posd, scale)
    x1 = x.to(DEV)
    q3.q3moe_bf16_gemv(A.wo, torch.from_numpy(a_r.reshape(T, -1)).to(DEV), out=x1, accumulate=True)
    torch.cuda.synchronize()
    e_a = assert_rows_close(a2.cpu().numpy().reshape(T, -1), a_r.reshape(T, -1), what="attention")
    e_o = assert_rows_close(x1.cpu().numpy(), x1_r, what="O projection + residual")
    # the MoE half on the oracle's attention output: exact routing
    x1d = torch.from_numpy(x1_r).to(DEV)
    _, idx, _ = q3.q3moe_moe_ffn_prenorm(x1d, A.post_norm, S.eps, M.router, 8, *experts_of(M), F=768,
                                         out=x1d, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), idx_r)
    e_m = assert_rows_close(x1d.cpu().numpy(), out_r, what="MoE half")
    free = (idx_free.cpu().numpy() == idx_r).all(axis=1)
    e_f = assert_rows_close(xd.cpu().numpy()[free], out_r[free], tol=2e-3, what="free-running layer")
    say(f"  q {e_q:.2e}, attention {e_a:.2e}, O {e_o:.2e}, MoE {e_m:.2e}; free-running {e_f:.2e}, "
        f"routing equal on {int(free.sum())}/{T}")
    assert free.mean() >= 0.99
