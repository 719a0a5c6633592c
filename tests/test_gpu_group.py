"""Token -> expert grouping on the GPU against the oracle: counts, offsets
and the pair list bit-exact (integer work), for decode and prefill sizes,
skewed routing, out-of-range indices, the largest E and T = 0."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen
from parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device visible")
    q3.library()


def _check(idx: np.ndarray, E: int, what: str):
    say(f"group {what}: T={idx.shape[0]} k={idx.shape[1]} E={E}")
    counts, offsets, pairs = q3.q3moe_group_by_expert(torch.from_numpy(idx).to(DEV), E)
    torch.cuda.synchronize()
    rc, ro, rp = oracle.oracle().group_by_expert(idx, E)
    assert np.array_equal(counts.cpu().numpy(), rc), what
    assert np.array_equal(offsets.cpu().numpy(), ro), what
    n = int(ro[E])
    assert np.array_equal(pairs.cpu().numpy()[:n], rp), what


def _routes(T, k, E, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,seed", [
    (1, 8, 128, 1),          # decode
    (4, 2, 8, 2),            # the tiny layer
    (16, 8, 128, 3),         # decode batch 16
    (512, 8, 128, 4),        # prefill 512
    (4096, 8, 128, 5),       # more pairs than one scatter pass per wave
    (37, 32, 1024, 6),       # largest E and k
    (9, 3, 5, 7),            # ragged
])
def test_group_matches_oracle(T, k, E, seed):
    _check(_routes(T, k, E, seed), E, f"random seed {seed}")


def test_group_out_of_range_indices_are_dropped():
    rng = np.random.default_rng(8)
    idx = rng.integers(-3, 131, size=(300, 8)).astype(np.int32)
    _check(idx, 128, "out of range")


def test_group_skewed_routing_from_the_route():
    """The prefill skew: half the tokens routed to the same 4 hot experts,
    produced by the GPU route itself."""
    T, H, E, k = 512, 2048, 128, 8
    g = gen.make_generator(9)
    router = gen.normal_f32((E, H), 0.02, g)
    layer = gen.MoeLayer(gen.MoeShape(T=T, H=H, E=E, k=k, F=256, down_qtype=gen.Q4_K),
                         router, None, None, None)
    x, R = gen.skewed_hidden_and_router(layer, gen.hidden_states(T, H, 10), seed=11)
    idx, _ = q3.q3moe_route(x.to(DEV), R.to(DEV), k)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    counts = np.bincount(idx_h.reshape(-1), minlength=128)
    assert np.sort(counts)[-4:].min() >= 200          # the hot experts are hot
    _check(idx_h, 128, "skewed")


def test_group_all_pairs_one_expert_and_empty():
    _check(np.full((100, 4), 7, np.int32), 16, "one expert")
    _check(np.zeros((0, 8), np.int32), 128, "T = 0")
