"""Shared helpers for the GPU-vs-oracle parity tests.

Tolerances: expert indices must match exactly; f32 outputs must agree with
the oracle within a relative L2 error of 1e-4 per token (row).  The oracle
accumulates in double; the kernels accumulate in f32, whose rounding error
over a 2048-term dot product is ~1e-6 relative, so 1e-4 leaves two orders
of margin while a wrong expert, a dropped term or a wrong scale gives
errors of order 1 (shown by the planted-mistake tests).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_moe_decode_q3moe_amd as q3
from sparse_moe_decode_q3moe_amd import inputs as gen

REL_L2_TOL = 1e-4


def say(msg: str):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, np.float64).reshape(got.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return num / den


def assert_rows_close(got, ref, tol=REL_L2_TOL, what=""):
    err = rel_l2_rows(got, ref)
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max per-row rel L2 {err.max():.3e} > {tol:.0e} (row {err.argmax()})"
    return float(err.max())


def near_tie_report(logits: np.ndarray, k: int, t: int) -> str:
    s = np.sort(logits[t])[::-1]
    return f"token {t}: gap between logit #{k} and #{k + 1} = {s[k - 1] - s[k]:.3e}"


def assert_indices_equal(got_idx, ref_idx, logits, k, what=""):
    got_idx = np.asarray(got_idx)
    bad = np.where((got_idx != ref_idx).any(1))[0]
    assert bad.size == 0, f"{what}: routing differs; " + "; ".join(
        near_tie_report(logits, k, int(t)) for t in bad[:4])


def experts_of(layer: gen.MoeLayer):
    s = layer.shape
    return (q3.Experts(layer.gate, gen.Q4_K), q3.Experts(layer.up, gen.Q4_K),
            q3.Experts(layer.down, s.down_qtype))


def oracle_tensors(layer: gen.MoeLayer):
    s = layer.shape
    return ((layer.gate.cpu().numpy(), gen.Q4_K), (layer.up.cpu().numpy(), gen.Q4_K),
            (layer.down.cpu().numpy(), s.down_qtype))


def gpu_moe(layer_dev: gen.MoeLayer, x_dev: torch.Tensor, out=None, accumulate=False):
    s = layer_dev.shape
    idx, w = q3.q3moe_route(x_dev, layer_dev.router, s.k)
    out = q3.q3moe_expert_ffn(x_dev, idx, w, *experts_of(layer_dev), F=s.F, out=out,
                              accumulate=accumulate)
    return idx, w, out


def oracle_moe(layer_cpu: gen.MoeLayer, x: np.ndarray, out=None, accumulate=False):
    o = oracle.oracle()
    s = layer_cpu.shape
    idx, w, logits = o.route(x, layer_cpu.router.numpy(), s.k)
    res = o.expert_ffn(x, idx, w, *oracle_tensors(layer_cpu), F=s.F, E=s.E, out=out,
                       accumulate=accumulate)
    return idx, w, logits, res
