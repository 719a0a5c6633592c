"""Fault injection on the GPU path: the parity check rejects a wrong routing.

The expert FFN runs on the GPU with routing faults planted in its inputs
(the same three faults the pages inject into their test builds: aprender
issue #3714, R1 receipt, "The oracle bites"), and its output is compared
with the oracle's block output under the TRUE routing at the bar every
parity test uses (1e-4 relative L2 per token).  A clean control passes;
each fault must fail it.  Readings of the three faults:
  WrongExpert     slot 0's expert replaced by the best expert outside the
                  selected set (the (k+1)-th largest logit), weight kept;
  DropTopExpert   slot 0 contributes nothing (its weight set to 0, the other
                  weights unchanged);
  UniformWeights  every selected slot weighted 1/k.
The faulted routings are valid inputs (indices in range), so every kernel
runs normally."""
import numpy as np
import pytest
import torch

import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import REL_L2_TOL, experts_of, oracle_moe, rel_l2_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _faults(idx, w, logits, k):
    order = np.argsort(-logits, axis=1, kind="stable")
    wrong = idx.copy()
    wrong[:, 0] = order[:, k]
    drop = w.copy()
    drop[:, 0] = 0.0
    uni = np.full_like(w, 1.0 / k)
    return {"WrongExpert": (wrong, w), "DropTopExpert": (idx, drop), "UniformWeights": (idx, uni)}


@pytest.mark.parametrize("T", [1, 4, 40])
def test_routing_faults_are_rejected(T):
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    shape = gen.MoeShape(T=T, H=2048, E=128, k=8, F=768, down_qtype=gen.Q6_K)
    cpu = gen.moe_layer(shape, 900 + T)
    dev = cpu.to(DEV)
    x = gen.hidden_states(T, 2048, 950 + T)
    ref_idx, ref_w, logits, ref = oracle_moe(cpu, x.numpy())
    xd = x.to(DEV)

    def gpu_ffn(idx, w):
        out = q3.q3moe_expert_ffn(xd, torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV),
                                  torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV),
                                  *experts_of(dev), F=768)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    clean = rel_l2_rows(gpu_ffn(ref_idx, ref_w), ref)
    say(f"fault injection T={T}: clean control max rel L2 {clean.max():.2e}")
    assert clean.max() <= REL_L2_TOL
    for name, (idx, w) in _faults(ref_idx, ref_w, logits, 8).items():
        got = gpu_ffn(idx, w)
        err = rel_l2_rows(got, ref)
        cos = float(np.sum(got.astype(np.float64) * ref) /
                    (np.linalg.norm(got) * np.linalg.norm(ref)))
        say(f"  {name}: min per-token rel L2 {err.min():.3e}, cosine {cos:.4f}")
        assert err.min() > REL_L2_TOL, f"{name} was not rejected (token {err.argmin()})"
