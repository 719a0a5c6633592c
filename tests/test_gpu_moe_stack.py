"""q3moe_moe_stack: n stacked MoE blocks, x <- x + MoE_l(RMSNorm_l(x)), in
one call (one persistent launch per 48 layers for the decode shapes).

Checked three ways:
  * against n q3moe_moe_ffn_prenorm calls in place on the same stream
    (same per-layer arithmetic, so x and every layer's routing are
    bit-identical);
  * against the oracle running the same stack on its own stream: routing
    identical at every layer, the final stream within the drift-derived
    tolerance of the free-running stack test (the oracle's own drift at a
    1e-6 relative input perturbation, x100, never below 1e-4);
  * its edge cases: more than 48 layers (several launches), a shape outside
    the persistent kernel (per-layer fallback), an expert count whose router
    units do not fill the grid, and a workspace shared with one-layer calls.
Layer sizes are Qwen3-30B-A3B's ("File facts", aprender issue #3714): H 2048,
128 experts, top-8, F 768, down Q6_K in layers 0-23 and Q4_K in 24-47, with
per-layer RMSNorm gains drawn uniformly from [0.5, 1.5]."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import assert_indices_equal, assert_rows_close, experts_of, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")


def _layers(T, n, E=128, k=8, F=768, seed=3000):
    """n seeded layers on the device (down type by depth as in the 48-layer
    model, scaled to n) with their gains."""
    out = []
    for l in range(n):
        lq = l if n == 48 else (0 if l < n // 2 else 47)
        shape = gen.MoeShape(T=T, H=2048, E=E, k=k, F=F, down_qtype=gen.stack_down_qtype(lq))
        lay = gen.moe_layer(shape, seed + l, device=DEV)
        g = gen.uniform_f32((2048,), 0.5, 1.5, gen.make_generator(seed + 500 + l))
        out.append((lay, g.to(DEV)))
    torch.cuda.synchronize()
    return out


def _stack_args(layers):
    return [q3.MoeLayer(g, lay.router, *experts_of(lay)) for lay, g in layers]


def _oracle_layer(o, lay, gain, x):
    """One layer on the oracle; only the experts it selects are copied to the
    host (same bytes, compact addressing)."""
    s = lay.shape
    xn = o.rmsnorm(x, gain.cpu().numpy(), EPS)
    idx, w, logits = o.route(xn, lay.router.cpu().numpy(), s.k)
    sel = np.unique(idx)
    remap = np.full(s.E, -1, np.int32)
    remap[sel] = np.arange(sel.size, dtype=np.int32)
    selt = torch.from_numpy(sel.astype(np.int64)).to(lay.gate.device)
    tens = ((lay.gate[selt].cpu().numpy(), gen.Q4_K), (lay.up[selt].cpu().numpy(), gen.Q4_K),
            (lay.down[selt].cpu().numpy(), s.down_qtype))
    out = o.expert_ffn(xn, remap[idx], w, *tens, F=s.F, E=sel.size, out=x, accumulate=True)
    return idx, logits, out


def _check_against_oracle(layers, x0, x_gpu, idx_gpu, what):
    """Free-running oracle over the stack: routing equal at every layer, the
    final stream within max(1e-4, 100 x the oracle's own drift)."""
    o = oracle.oracle()
    k = layers[0][0].shape.k
    rng = np.random.default_rng(5)
    x_ref = x0.copy()
    x_pert = (x0 * (1.0 + 1e-6 * rng.standard_normal(x0.shape))).astype(np.float32)
    idx_all = idx_gpu.cpu().numpy()
    for l, (lay, g) in enumerate(layers):
        ref_idx, logits, x_ref = _oracle_layer(o, lay, g, x_ref)
        _, _, x_pert = _oracle_layer(o, lay, g, x_pert)
        assert_indices_equal(idx_all[l], ref_idx, logits, k, f"{what} layer {l}")
    drift = float(np.max(np.linalg.norm(x_pert.astype(np.float64) - x_ref, axis=1) /
                         np.linalg.norm(x_ref, axis=1)))
    tol = max(1e-4, 100.0 * drift)
    err = assert_rows_close(x_gpu.cpu().numpy(), x_ref, tol=tol, what=f"{what} final stream")
    say(f"  {what}: final stream rel L2 {err:.2e} (tolerance {tol:.2e})")


def _ws(T, E=128, k=8, F=768):
    return torch.zeros(q3.q3moe_moe_stack_workspace_bytes(T, 2048, F, E, k), dtype=torch.uint8,
                       device=DEV)


@pytest.fixture(scope="module")
def full48():
    _need_gpu()
    return _layers(1, 48)


def test_full_stack_equals_per_layer_calls(full48):
    """48 full-size layers, one token: the one-launch stack against 48
    in-place pre-norm block calls, bit for bit."""
    say("stack vs 48 per-layer calls, T=1")
    x0 = gen.hidden_states(1, 2048, 77).to(DEV)
    ws = _ws(1)
    x = x0.clone()
    _, idx, w = q3.q3moe_moe_stack(x, _stack_args(full48), 8, 768, EPS, workspace=ws)
    assert q3.q3moe_persistent_path(1, 2048, 768, 128, 8, gen.Q6_K, 1) == 1
    ref = x0.clone()
    ws1 = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(1, 2048, 768, 128, 8), dtype=torch.uint8,
                      device=DEV)
    for l, (lay, g) in enumerate(full48):
        _, i1, w1 = q3.q3moe_moe_ffn_prenorm(ref, g, EPS, lay.router, 8, *experts_of(lay), F=768,
                                             out=ref, accumulate=True, workspace=ws1)
        assert torch.equal(i1, idx[l]), f"layer {l} indices"
        assert torch.equal(w1, w[l]), f"layer {l} weights"
    torch.cuda.synchronize()
    assert torch.equal(x, ref)
    assert q3.expert_ffn_status(ws, 1, 2048, 768, 128, 8) == 0


def test_full_stack_against_oracle(full48):
    """48 full-size layers, one token, against the oracle's own stream."""
    say("stack vs oracle, T=1, 48 layers")
    x0 = gen.hidden_states(1, 2048, 78)
    x = x0.to(DEV)
    ws = _ws(1)
    _, idx, _ = q3.q3moe_moe_stack(x, _stack_args(full48), 8, 768, EPS, workspace=ws)
    torch.cuda.synchronize()
    _check_against_oracle(full48, x0.numpy(), x, idx, "T=1 48 layers")
    assert q3.expert_ffn_status(ws, 1, 2048, 768, 128, 8) == 0


@pytest.mark.parametrize("T,n", [(2, 5), (3, 4), (4, 3)])
def test_batched_stack_against_oracle(T, n):
    """Several tokens (ragged token counts within the kernel's 1-4)."""
    _need_gpu()
    say(f"stack vs oracle, T={T}, {n} layers")
    layers = _layers(T, n, seed=3100 + 10 * T)
    x0 = gen.hidden_states(T, 2048, 79 + T)
    x = x0.to(DEV)
    ws = _ws(T)
    _, idx, _ = q3.q3moe_moe_stack(x, _stack_args(layers), 8, 768, EPS, workspace=ws)
    torch.cuda.synchronize()
    _check_against_oracle(layers, x0.numpy(), x, idx, f"T={T}")
    assert q3.expert_ffn_status(ws, T, 2048, 768, 128, 8) == 0


def test_more_layers_than_one_launch():
    """50 layers (a 48-layer launch and a 2-layer one) of a 16-expert top-4
    model, two tokens."""
    _need_gpu()
    say("stack of 50 layers, E=16 k=4, T=2")
    layers = _layers(2, 50, E=16, k=4, seed=3300)
    x0 = gen.hidden_states(2, 2048, 81)
    x = x0.to(DEV)
    ws = _ws(2, E=16, k=4)
    _, idx, _ = q3.q3moe_moe_stack(x, _stack_args(layers), 4, 768, EPS, workspace=ws)
    torch.cuda.synchronize()
    _check_against_oracle(layers, x0.numpy(), x, idx, "50 layers")
    assert q3.expert_ffn_status(ws, 2, 2048, 768, 16, 4) == 0


def test_shape_outside_the_persistent_kernel():
    """Five tokens take the per-layer path; same contract."""
    _need_gpu()
    say("stack fallback, T=5, 3 layers")
    assert q3.q3moe_persistent_path(5, 2048, 768, 128, 8, gen.Q6_K, 1) == 0
    layers = _layers(5, 3, seed=3400)
    x0 = gen.hidden_states(5, 2048, 82)
    x = x0.to(DEV)
    _, idx, _ = q3.q3moe_moe_stack(x, _stack_args(layers), 8, 768, EPS, workspace=_ws(5))
    torch.cuda.synchronize()
    _check_against_oracle(layers, x0.numpy(), x, idx, "T=5")


def test_expert_count_below_the_grid():
    """100 experts: the router units (100 x 2 column parts) do not fill a
    256-workgroup grid, so the in-place one-layer call and the stack run on
    200 workgroups (every workgroup must own a router unit for the in-place
    update).  Both against the oracle."""
    _need_gpu()
    say("E=100: in-place pre-norm block and a 3-layer stack")
    layers = _layers(2, 3, E=100, seed=3500)
    o = oracle.oracle()
    x0 = gen.hidden_states(2, 2048, 83)
    lay, g = layers[0]
    x = x0.to(DEV)
    ws1 = torch.zeros(q3.q3moe_moe_ffn_workspace_bytes(2, 2048, 768, 100, 8), dtype=torch.uint8,
                      device=DEV)
    _, idx1, _ = q3.q3moe_moe_ffn_prenorm(x, g, EPS, lay.router, 8, *experts_of(lay), F=768, out=x,
                                          accumulate=True, workspace=ws1)
    torch.cuda.synchronize()
    ref_idx, logits, x_ref = _oracle_layer(o, lay, g, x0.numpy())
    assert_indices_equal(idx1.cpu().numpy(), ref_idx, logits, 8, "E=100 one layer")
    assert_rows_close(x.cpu().numpy(), x_ref, what="E=100 one layer")
    assert q3.expert_ffn_status(ws1, 2, 2048, 768, 100, 8) == 0
    xs = x0.to(DEV)
    _, idx, _ = q3.q3moe_moe_stack(xs, _stack_args(layers), 8, 768, EPS, workspace=_ws(2, E=100))
    torch.cuda.synchronize()
    _check_against_oracle(layers, x0.numpy(), xs, idx, "E=100 stack")


def test_workspace_shared_with_block_calls():
    """One workspace through a pre-norm block call, a 3-layer stack (T=3), a
    plain block call and a 2-layer stack at T=1: the calls share the epoch
    counter and buffers, and every result matches the oracle."""
    _need_gpu()
    say("workspace shared between block and stack calls")
    layers = _layers(3, 3, seed=3600)
    o = oracle.oracle()
    ws = _ws(3)
    lay, g = layers[0]
    x0 = gen.hidden_states(3, 2048, 84)
    x = x0.to(DEV)
    _, i0, _ = q3.q3moe_moe_ffn_prenorm(x, g, EPS, lay.router, 8, *experts_of(lay), F=768, out=x,
                                        accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    ref_idx, logits, x_ref = _oracle_layer(o, lay, g, x0.numpy())
    assert_indices_equal(i0.cpu().numpy(), ref_idx, logits, 8, "block call")
    assert_rows_close(x.cpu().numpy(), x_ref, what="block call")

    x1 = gen.hidden_states(3, 2048, 85)
    xs = x1.to(DEV)
    _, idx, _ = q3.q3moe_moe_stack(xs, _stack_args(layers), 8, 768, EPS, workspace=ws)
    torch.cuda.synchronize()
    _check_against_oracle(layers, x1.numpy(), xs, idx, "stack after block")

    lay2, _ = layers[1]
    x2 = gen.hidden_states(3, 2048, 86)
    out, i2, w2 = q3.q3moe_moe_ffn(x2.to(DEV), lay2.router, 8, *experts_of(lay2), F=768, workspace=ws)
    torch.cuda.synchronize()
    ri, _, rl = o.route(x2.numpy(), lay2.router.cpu().numpy(), 8)
    assert_indices_equal(i2.cpu().numpy(), ri, rl, 8, "block after stack")

    x3 = gen.hidden_states(1, 2048, 87)
    two = [(gen.MoeLayer(gen.MoeShape(T=1, H=2048, E=128, k=8, F=768, down_qtype=l.shape.down_qtype),
                         l.router, l.gate, l.up, l.down), g_) for l, g_ in layers[:2]]
    xs3 = x3.to(DEV)
    _, idx3, _ = q3.q3moe_moe_stack(xs3, _stack_args(two), 8, 768, EPS, workspace=ws)
    torch.cuda.synchronize()
    _check_against_oracle(two, x3.numpy(), xs3, idx3, "T=1 stack after T=3 calls")
    assert q3.expert_ffn_status(ws, 3, 2048, 768, 128, 8) == 0
