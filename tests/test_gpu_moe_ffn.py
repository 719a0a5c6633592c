"""The one-call MoE block (q3moe_moe_ffn: route + expert FFN) vs the oracle.

For at most 4 tokens at H = 2048 the whole block is one persistent kernel
that routes inside (every workgroup computes a slice of the router logits,
publishes it as tagged words and selects the top-k from all slices); other
shapes run the route and expert-FFN kernels back to back.  Indices
bit-exact, routing weights to 1e-6 relative, outputs within 1e-4 relative
L2 per token.  Repeated calls through one workspace check that each call's
tags keep it from reading an earlier call's partial results.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_indices_equal, assert_rows_close, experts_of, oracle_moe, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = {  # name: (shape, seed); the first seven take the one-kernel path
    "a3b_T1": (gen.QWEN3_30B_A3B, 41),
    "a3b_T2": (gen.MoeShape(T=2, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K), 42),
    "a3b_q4k_down_T3": (gen.MoeShape(T=3, H=2048, E=128, k=8, F=768, down_qtype=gen.Q4_K), 43),
    "a3b_T4": (gen.MoeShape(T=4, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K), 44),
    "E256_k4_F512_T2": (gen.MoeShape(T=2, H=2048, E=256, k=4, F=512, down_qtype=gen.Q6_K), 45),
    "E64_k1_T1": (gen.MoeShape(T=1, H=2048, E=64, k=1, F=256, down_qtype=gen.Q4_K), 46),
    "E72_k6_T3": (gen.MoeShape(T=3, H=2048, E=72, k=6, F=512, down_qtype=gen.Q4_K), 51),
    # two launches: more tokens, other hidden sizes, more experts
    "a3b_T5": (gen.MoeShape(T=5, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K), 47),
    "tiny_T4": (gen.TINY, 48),
    "E300_T1": (gen.MoeShape(T=1, H=2048, E=300, k=8, F=256, down_qtype=gen.Q6_K), 49),
    "prefill_T40": (gen.MoeShape(T=40, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K), 50),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(name):
        if name not in cache:
            shape, seed = CASES[name]
            cpu = gen.moe_layer(shape, seed)
            x = gen.hidden_states(shape.T, shape.H, seed + 500)
            cache[name] = (cpu, cpu.to(DEV), x)
        return cache[name]
    return get


def _check(cpu, got, x, what, out=None, accumulate=False):
    s = cpu.shape
    ref_idx, ref_w, logits, ref = oracle_moe(cpu, x.numpy(), out=out, accumulate=accumulate)
    o, idx, w = got
    torch.cuda.synchronize()
    assert_indices_equal(idx.cpu().numpy(), ref_idx, logits, s.k, what)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-6, atol=0)
    return assert_rows_close(o.cpu().numpy(), ref, what=what)


@pytest.mark.parametrize("name", list(CASES))
def test_moe_ffn_parity(layers, name):
    cpu, dev, x = layers(name)
    s = cpu.shape
    say(f"moe_ffn {name}: T={s.T} H={s.H} E={s.E} k={s.k} F={s.F} down={s.down_qtype}")
    ws = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(s.T, s.H, s.F, s.E, s.k),
                     dtype=torch.uint8, device=DEV)
    got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, workspace=ws)
    err = _check(cpu, got, x, name)
    assert q3.expert_ffn_status(ws, s.T, s.H, s.F, s.E, s.k) == 0
    say(f"  max rel L2 {err:.2e}")


@pytest.mark.parametrize("name", ["a3b_T1", "a3b_q4k_down_T3", "tiny_T4"])
def test_moe_ffn_accumulate(layers, name):
    cpu, dev, x = layers(name)
    s = cpu.shape
    say(f"moe_ffn accumulate {name}")
    prev = (x * 100.0).contiguous()
    out = prev.to(DEV)
    got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, out=out,
                           accumulate=True)
    _check(cpu, got, x, f"{name} accumulate", out=prev.numpy(), accumulate=True)


def test_moe_ffn_workspace_reuse(layers):
    """One zeroed workspace through a sequence of calls with different
    inputs and token counts: every call must see only its own tagged words."""
    cpu1, dev1, x1 = layers("a3b_T1")
    cpu4, dev4, x4 = layers("a3b_T4")
    s4 = cpu4.shape
    ws = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(s4.T, s4.H, s4.F, s4.E, s4.k),
                     dtype=torch.uint8, device=DEV)
    g = gen.make_generator(77)
    for i in range(6):
        cpu, dev, x = (cpu1, dev1, x1) if i % 2 == 0 else (cpu4, dev4, x4)
        if i >= 2:                                  # fresh activations, same weights
            x = gen.normal_f32(tuple(x.shape), 1.0, g)
        s = cpu.shape
        say(f"workspace reuse call {i}: T={s.T}")
        got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, workspace=ws)
        _check(cpu, got, x, f"reuse call {i}")
    assert q3.expert_ffn_status(ws, s4.T, s4.H, s4.F, s4.E, s4.k) == 0


def test_moe_ffn_matches_two_calls(layers):
    """The one-kernel block and the two entry points agree on the routing
    and, to the last bits allowed by the summation orders, on the output."""
    cpu, dev, x = layers("a3b_T2")
    s = cpu.shape
    say("moe_ffn vs route + expert_ffn")
    xd = x.to(DEV)
    out, idx, w = q3.q3moe_moe_ffn(xd, dev.router, s.k, *experts_of(dev), F=s.F)
    idx2, w2 = q3.q3moe_route(xd, dev.router, s.k)
    out2 = q3.q3moe_expert_ffn(xd, idx2, w2, *experts_of(dev), F=s.F)
    torch.cuda.synchronize()
    assert torch.equal(idx.cpu(), idx2.cpu())
    np.testing.assert_allclose(w.cpu().numpy(), w2.cpu().numpy(), rtol=1e-6, atol=0)
    assert_rows_close(out.cpu().numpy(), out2.cpu().numpy().astype(np.float64), what="two calls")


def test_moe_ffn_routing_ties_and_specials(layers):
    """In-kernel routing on exactly equal logits, on two logits that differ
    by far less than an f32 ulp, and on a token whose input holds +inf (a
    run of equal infinite logits): the oracle's choices (the larger logit
    first, equal logits by the lower index)."""
    cpu, dev, x = layers("a3b_T2")
    s = cpu.shape
    say("moe_ffn routing ties")
    R = cpu.router.clone()
    x1 = x.clone()
    sgn = torch.sign(x1[0])
    R[[5, 9, 30, 101]] = 0.01 * sgn                 # four identical top logits of token 0
    R[77] = 0.01 * sgn
    j = int(torch.argmax(x1[0].abs()))
    R[77, j] += 1e-7 * sgn[j] / x1[0, j].abs()      # above them by ~1e-7 (an f32 ulp is ~2e-6)
    x1[1, 0] = float("inf")                         # token 1: +inf logits wherever R[e, 0] > 0
    lay = gen.MoeLayer(s, R, cpu.gate, cpu.up, cpu.down)
    lay_dev = gen.MoeLayer(s, R.to(DEV), dev.gate, dev.up, dev.down)
    out, idx, w = q3.q3moe_moe_ffn(x1.to(DEV), lay_dev.router, s.k, *experts_of(lay_dev), F=s.F)
    torch.cuda.synchronize()
    ref_idx, ref_w, logits, ref = oracle_moe(lay, x1.numpy())
    got = idx.cpu().numpy()
    assert ref_idx[0, :5].tolist() == [77, 5, 9, 30, 101], ref_idx[0]
    assert np.array_equal(got, ref_idx), (got, ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-6, atol=0)
    assert_rows_close(out.cpu().numpy()[:1], ref[:1], what="ties, token 0")


EPS = 1e-6
PRENORM_CASES = ["a3b_T1", "a3b_T4", "E72_k6_T3", "a3b_T5", "tiny_T4", "prefill_T40"]


def _gain(H, seed):
    return gen.uniform_f32((H,), 0.5, 1.5, gen.make_generator(seed))


@pytest.mark.parametrize("name", PRENORM_CASES)
def test_moe_ffn_prenorm_in_place(layers, name):
    """q3moe_moe_ffn_prenorm with out = hidden and accumulate: the residual
    update x += MoE(RMSNorm(x)) in one call (the norm inside the one-kernel
    block for the first three cases, a norm kernel first for the others),
    against the oracle's RMSNorm, routing and expert FFN."""
    cpu, dev, x = layers(name)
    s = cpu.shape
    say(f"moe_ffn_prenorm in place {name}: T={s.T} E={s.E} k={s.k}")
    g = _gain(s.H, 7 + s.T)
    xd = x.to(DEV).clone()
    out, idx, w = q3.q3moe_moe_ffn_prenorm(xd, g.to(DEV), EPS, dev.router, s.k, *experts_of(dev),
                                           F=s.F, out=xd, accumulate=True)
    assert out.data_ptr() == xd.data_ptr()
    xn = oracle.oracle().rmsnorm(x.numpy(), g.numpy(), EPS)
    err = _check(cpu, (out, idx, w), torch.from_numpy(xn), f"{name} prenorm in place",
                 out=x.numpy().copy(), accumulate=True)
    say(f"  max rel L2 {err:.2e}")


@pytest.mark.parametrize("name", ["a3b_T2", "a3b_T5"])
def test_moe_ffn_prenorm_matches_norm_then_block(layers, name):
    """The pre-norm block (out of place, no accumulate) equals q3moe_rmsnorm
    followed by q3moe_moe_ffn: the same routing, outputs to the summation
    orders; and q3moe_rmsnorm's rows equal the oracle's to the last bit."""
    cpu, dev, x = layers(name)
    s = cpu.shape
    say(f"moe_ffn_prenorm vs rmsnorm + moe_ffn {name}")
    g = _gain(s.H, 99).to(DEV)
    xd = x.to(DEV)
    out, idx, w = q3.q3moe_moe_ffn_prenorm(xd, g, EPS, dev.router, s.k, *experts_of(dev), F=s.F)
    xn = q3.q3moe_rmsnorm(xd, g, EPS)
    out2, idx2, w2 = q3.q3moe_moe_ffn(xn, dev.router, s.k, *experts_of(dev), F=s.F)
    torch.cuda.synchronize()
    ref_xn = oracle.oracle().rmsnorm(x.numpy(), g.cpu().numpy(), EPS)
    assert np.array_equal(xn.cpu().numpy().view(np.uint32), ref_xn.view(np.uint32))
    assert torch.equal(idx.cpu(), idx2.cpu())
    np.testing.assert_allclose(w.cpu().numpy(), w2.cpu().numpy(), rtol=1e-6, atol=0)
    assert_rows_close(out.cpu().numpy(), out2.cpu().numpy().astype(np.float64), what="prenorm vs two steps")


def test_moe_ffn_workspace_reuse_across_paths(layers):
    """One workspace, sized for 512 tokens, through calls that take every
    path: the batched prefill kernels (512 tokens fill the workspace with
    grouping data and activation pieces), the two-launch decode form (6 and
    8 tokens: its route kernel's arrival counter must be zero at launch) and
    the one-kernel block (1 token).  The route counter sits at one fixed
    offset for every size, so no call finds a larger call's data there."""
    full = gen.MoeShape(T=512, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K)
    cpu, dev, _ = layers("a3b_T1")
    ws = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(full.T, full.H, full.F, full.E, full.k),
                     dtype=torch.uint8, device=DEV)
    g = gen.make_generator(4242)
    for T in (512, 6, 1, 8, 5, 2):
        s = gen.MoeShape(T=T, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K)
        lay = gen.MoeLayer(s, cpu.router, cpu.gate, cpu.up, cpu.down)
        x = gen.normal_f32((T, 2048), 1.0, g)
        say(f"workspace reuse across paths: T={T}, persistent="
            f"{q3.q3moe_persistent_path(T, 2048, 768, 128, 8, gen.Q6_K, True)}")
        got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, 8, *experts_of(dev), F=768, workspace=ws)
        _check(lay, got, x, f"reuse across paths T={T}")
        assert q3.expert_ffn_status(ws, T, 2048, 768, 128, 8) == 0


def test_persistent_path_is_taken_at_decode(layers):
    """At the 30B-A3B decode shape (1 token) the MoE block is the one
    persistent kernel on this device: the occupancy check passes, the call
    advances the workspace's call counter (only that kernel does), and the
    status word stays zero."""
    cpu, dev, x = layers("a3b_T1")
    s = cpu.shape
    assert q3.q3moe_persistent_path(1, 2048, 768, 128, 8, gen.Q6_K, True) == 1
    assert q3.q3moe_persistent_path(1, 2048, 768, 128, 8, gen.Q6_K, False) == 1
    assert q3.q3moe_persistent_path(5, 2048, 768, 128, 8, gen.Q6_K, True) == 0
    assert q3.q3moe_persistent_path(512, 2048, 768, 128, 8, gen.Q6_K, False) == 0
    assert q3.q3moe_persistent_path(1, 2000, 768, 128, 8, gen.Q6_K, True) == -1
    ws = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(s.T, s.H, s.F, s.E, s.k),
                     dtype=torch.uint8, device=DEV)
    counter = lambda: int(ws[128:132].view(torch.int32).item())   # noqa: E731
    before = counter()
    got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, workspace=ws)
    _check(cpu, got, x, "persistent path")
    assert counter() == before + 1
    assert q3.expert_ffn_status(ws, s.T, s.H, s.F, s.E, s.k) == 0


# Error budget of the int8 activations against the f32 block (relative L2):
# over a batch of tokens 2e-2 (the oracle shows 0.5-0.6 % at the 30B-A3B
# shape), per token 0.25 (a token whose block output nearly cancels, as the
# large min offsets of random Q4_K down weights make some do, reaches ~15 %).
Q8_BUDGET_BATCH = 2e-2
Q8_BUDGET_TOKEN = 0.25


@pytest.mark.parametrize("name", ["a3b_T1", "a3b_T4", "a3b_q4k_down_T3", "E72_k6_T3"])
def test_moe_ffn_int8_activations(layers, name):
    """q3moe_moe_ffn_q8: routing identical to the f32 block; outputs within
    1e-4 of the oracle that quantises the gate/up input the same way (one
    int8 value per element, d = max|x|/127 per 32 values), and within the
    stated error budget of the f32 oracle."""
    cpu, dev, x = layers(name)
    s = cpu.shape
    say(f"moe_ffn int8 activations {name}")
    got = q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, int8_activations=True)
    torch.cuda.synchronize()
    o = oracle.oracle()
    ref_idx, ref_w, logits = o.route(x.numpy(), cpu.router.numpy(), s.k)
    from parity import oracle_tensors, rel_l2_rows
    ref_q8 = o.expert_ffn_q8(x.numpy(), ref_idx, ref_w, *oracle_tensors(cpu), F=s.F, E=s.E)
    ref_f32 = o.expert_ffn(x.numpy(), ref_idx, ref_w, *oracle_tensors(cpu), F=s.F, E=s.E)
    out, idx, w = got
    assert_indices_equal(idx.cpu().numpy(), ref_idx, logits, s.k, name)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-6, atol=0)
    err = assert_rows_close(out.cpu().numpy(), ref_q8, what=f"{name} int8 vs its oracle")
    budget = rel_l2_rows(out.cpu().numpy(), ref_f32)
    say(f"  vs the int8 oracle {err:.2e}; vs the f32 oracle max {budget.max():.2e}")
    assert budget.max() <= Q8_BUDGET_TOKEN
    # the mode really quantises: it is not the f32 block
    assert budget.min() > 1e-4


def test_moe_ffn_int8_activations_budget(layers):
    """64 tokens (16 calls of 4) through the int8 mode at the 30B-A3B shape
    with Q6_K and with Q4_K down: the relative L2 error against the f32
    oracle over the batch within 2e-2 and per token within 0.25, and every
    token within 1e-4 of the oracle that quantises the same way."""
    from parity import oracle_tensors, rel_l2_rows
    o = oracle.oracle()
    for name in ("a3b_T4", "a3b_q4k_down_T3"):
        cpu, dev, _ = layers(name)
        s = cpu.shape
        x = gen.hidden_states(64, 2048, 777 + s.down_qtype)
        outs = []
        for c in range(16):
            xc = x[4 * c:4 * c + 4].contiguous()
            out, _, _ = q3.q3moe_moe_ffn(xc.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F,
                                         int8_activations=True)
            outs.append(out)
        got = torch.cat(outs).cpu().numpy().astype(np.float64)
        ridx, rw, _ = o.route(x.numpy(), cpu.router.numpy(), s.k)
        ref_q8 = o.expert_ffn_q8(x.numpy(), ridx, rw, *oracle_tensors(cpu), F=s.F, E=s.E)
        ref = o.expert_ffn(x.numpy(), ridx, rw, *oracle_tensors(cpu), F=s.F, E=s.E).astype(np.float64)
        assert_rows_close(got, ref_q8, what=f"{name} int8 batch vs its oracle")
        per = rel_l2_rows(got, ref)
        agg = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        say(f"int8 budget {name}: batch {agg:.2e}, per token max {per.max():.2e} median {np.median(per):.2e}")
        assert agg <= Q8_BUDGET_BATCH and per.max() <= Q8_BUDGET_TOKEN


def test_moe_ffn_int8_activations_edge_cases(layers):
    """A group of zeros, a group of evenly spaced values, and a group whose
    values sit exactly on half steps (ties go to even)."""
    cpu, dev, x = layers("a3b_T2")
    s = cpu.shape
    x1 = x.clone()
    x1[0, :32] = 0.0
    x1[0, 32:64] = torch.arange(32, dtype=torch.float32) - 15.5       # d = 16.5/127
    x1[0, 64:96] = torch.tensor([127.0, 0.5, 1.5, 2.5] * 8)           # d = 1: ties to even
    got = q3.q3moe_moe_ffn(x1.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, int8_activations=True)
    torch.cuda.synchronize()
    o = oracle.oracle()
    from parity import oracle_tensors
    ref_idx, ref_w, logits = o.route(x1.numpy(), cpu.router.numpy(), s.k)
    ref = o.expert_ffn_q8(x1.numpy(), ref_idx, ref_w, *oracle_tensors(cpu), F=s.F, E=s.E)
    assert_indices_equal(got[1].cpu().numpy(), ref_idx, logits, s.k, "int8 edge cases")
    assert_rows_close(got[0].cpu().numpy(), ref, what="int8 edge cases")


def test_moe_ffn_int8_activations_rejects_other_shapes(layers):
    cpu, dev, x = layers("a3b_T5")
    s = cpu.shape
    with pytest.raises(q3.Q3MoeError) as e:
        q3.q3moe_moe_ffn(x.to(DEV), dev.router, s.k, *experts_of(dev), F=s.F, int8_activations=True)
    assert e.value.status == 2
