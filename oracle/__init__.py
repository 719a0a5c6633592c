"""CPU oracle for the Qwen3-MoE sparse FFN block -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``q3moe_oracle.c`` (plain scalar C, double
accumulation).  Only the tests, the package's smoke check and the benchmark's
CPU-baseline leg may import this package; the HIP library never does.

Every function takes and returns NumPy arrays on the host.

Parity status per function (how each is pinned is listed in the tests):
  dequant_block / dequant_matrix  pinned: hand-built blocks with closed-form
                                  values, orientation probe, page byte counts
  qgemv                           pinned: dense NumPy product of the pinned
                                  dequantisation, row-constant probe
  route                           pinned: brute-force full sort, softmax
                                  closed forms, ties, shift invariance
  expert_ffn                      pinned: dense-over-all-experts brute force,
                                  single-expert dense MLP, zero cases
  quantize_act_q8 / expert_ffn_q8 pinned: hand-worked groups (ties to even,
                                  all-zero, non-finite), |x - d p| <= d/2,
                                  the f64 block on the dequantised values
  kv_write_rows /                 pinned: brute-force NumPy causal attention,
  prefill_attention               causal-window probes, slot contents
  embed / output_head             pinned: rows of the pinned dequantisation,
                                  NaN rows out of range, dense NumPy product,
                                  one-hot column probes
  rmsnorm / attn_prologue /       pinned: RMS closed form, rotation invariants,
  rope_neox                       NEOX-vs-interleaved discriminator
  group_by_expert                 pinned: a library sort of (expert, pair),
                                  a hand-worked example, count/offset invariants
  bf16 conversions                pinned: all 65,536 bf16 patterns and a sweep of
                                  f32 values against torch.bfloat16
  bf16_gemv                       pinned: dense NumPy product, one-hot probes
  kv_write                        pinned: torch.bfloat16 rounding, untouched slots
  gqa_attention                   pinned: brute-force NumPy softmax per head,
                                  one-position and equal-key closed forms,
                                  one-hot kv-head probe of the GQA mapping
Agreement with real GGUF files is not pinned (no files; the bit layout is
the GGUF k-quant reading).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "q3moe_oracle.c"
LIB = HERE / "libq3moe_oracle.so"

Q4_K, Q6_K = 1, 2
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}


def build(src: Path = SRC, out: Path = LIB, extra_flags=()) -> Path:
    """Compile the oracle with gcc (no fast-math: IEEE double throughout)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           "-o", str(out), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _stale() -> bool:
    return not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _declare(lib):
    sig = {
        "orc_max_threads": (ctypes.c_int, []),
        "orc_set_threads": (None, [ctypes.c_int]),
        "orc_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_block_bytes": (ctypes.c_int, [ctypes.c_int]),
        "orc_dequant_block": (ctypes.c_int, [ctypes.c_int, _P, _P]),
        "orc_dequant_row": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P]),
        "orc_dequant_matrix": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P]),
        "orc_qgemv": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, _P]),
        "orc_router_logits": (None, [_P, _I64, _I64, _P, _I32, _P]),
        "orc_topk_softmax": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P]),
        "orc_route": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I32, _P, _P, _P]),
        "orc_expert_ffn_f64": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _P, _P,
                                              _P, ctypes.c_int, _I64,
                                              _P, ctypes.c_int, _I64,
                                              _P, ctypes.c_int, _I64, _P]),
        "orc_expert_ffn": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _P, _P,
                                          _P, ctypes.c_int, _I64,
                                          _P, ctypes.c_int, _I64,
                                          _P, ctypes.c_int, _I64, _P, ctypes.c_int]),
        "orc_expert_ffn_q8": (ctypes.c_int, [_P, _I64, _I64, _I64, _I32, _I32, _P, _P,
                                             _P, ctypes.c_int, _I64,
                                             _P, ctypes.c_int, _I64,
                                             _P, ctypes.c_int, _I64, _P, ctypes.c_int]),
        "orc_quantize_act_q8": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
        "orc_kv_write_rows": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _I64]),
        "orc_prefill_attention": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P,
                                                 ctypes.c_double, _P]),
        "orc_embed": (ctypes.c_int, [_P, _I64, _P, ctypes.c_int, _I64, _I64, _P]),
        "orc_output_head": (ctypes.c_int, [_P, _I64, _P, ctypes.c_int, _I64, _I64, _P]),
        "orc_rmsnorm": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_float, _P]),
        "orc_group_by_expert": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
        "orc_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_float_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_bf16_gemv": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, ctypes.c_int]),
        "orc_kv_write": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _I64]),
        "orc_gqa_attention": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P, _I64, _P,
                                             ctypes.c_double, _P]),
        "orc_rope_neox": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, ctypes.c_double]),
        "orc_attn_prologue": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _I32, _P, _P, _P,
                                             ctypes.c_float, ctypes.c_float]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def load(path: Path | None = None):
    """Load the oracle library (building it first if the source is newer)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(str(path)))
    if _lib is None:
        if _stale():
            build()
        _lib = _declare(ctypes.CDLL(str(LIB)))
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Callable view of one oracle build (the real one, or a test variant)."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def max_threads(self) -> int:
        """Threads the oracle's parallel loops use now."""
        return self.lib.orc_max_threads()

    def set_threads(self, n: int) -> None:
        """Set the thread count of the parallel loops (results do not depend on it)."""
        self.lib.orc_set_threads(int(n))

    def half_to_double(self, bits: int) -> float:
        return self.lib.orc_half_to_double(bits)

    def dequant_block(self, qtype: int, blk: np.ndarray) -> np.ndarray:
        blk = _c(blk, np.uint8)
        assert blk.size == BLOCK_BYTES[qtype]
        out = np.empty(256, np.float64)
        assert self.lib.orc_dequant_block(qtype, _p(blk), _p(out)) == 0
        return out

    def dequant_matrix(self, qtype: int, mat: np.ndarray, rows: int, cols: int) -> np.ndarray:
        mat = _c(mat, np.uint8)
        assert mat.size >= rows * (cols // 256) * BLOCK_BYTES[qtype]
        out = np.empty((rows, cols), np.float64)
        assert self.lib.orc_dequant_matrix(qtype, _p(mat), rows, cols, _p(out)) == 0
        return out

    def qgemv(self, qtype: int, mat: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
        mat = _c(mat, np.uint8)
        x = _c(x, np.float64)
        y = np.empty(rows, np.float64)
        assert self.lib.orc_qgemv(qtype, _p(mat), rows, cols, _p(x), _p(y)) == 0
        return y

    def router_logits(self, x: np.ndarray, router: np.ndarray) -> np.ndarray:
        x = _c(x, np.float32)
        router = _c(router, np.float32)
        T, H = x.shape
        E = router.shape[0]
        out = np.empty((T, E), np.float64)
        self.lib.orc_router_logits(_p(x), T, H, _p(router), E, _p(out))
        return out

    def topk_softmax(self, logits: np.ndarray, k: int):
        logits = _c(logits, np.float64)
        T, E = logits.shape
        idx = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        assert self.lib.orc_topk_softmax(_p(logits), T, E, k, _p(idx), _p(w)) == 0
        return idx, w

    def route(self, x: np.ndarray, router: np.ndarray, k: int):
        """-> (idx int32 [T,k], w f32 [T,k], logits f64 [T,E])."""
        x = _c(x, np.float32)
        router = _c(router, np.float32)
        T, H = x.shape
        E = router.shape[0]
        idx = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float32)
        logits = np.empty((T, E), np.float64)
        assert self.lib.orc_route(_p(x), T, H, _p(router), E, k, _p(idx), _p(w), _p(logits)) == 0
        return idx, w, logits

    def group_by_expert(self, idx: np.ndarray, E: int):
        """idx int32 [T, k] -> (counts int32 [E], offsets int32 [E+1], pairs int32 [n])
        where n = offsets[E] (pairs with an index outside [0, E) are dropped)."""
        idx = _c(idx, np.int32)
        T, k = idx.shape
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        pairs = np.empty(max(1, T * k), np.int32)
        assert self.lib.orc_group_by_expert(_p(idx), T, k, E, _p(counts), _p(offsets),
                                            _p(pairs)) == 0
        return counts, offsets, pairs[:offsets[E]].copy()

    def float_to_bf16(self, f: float) -> int:
        return self.lib.orc_float_to_bf16(f)

    def bf16_to_double(self, b: int) -> float:
        return self.lib.orc_bf16_to_double(b)

    def bf16_gemv(self, W: np.ndarray, x: np.ndarray, y: np.ndarray | None = None,
                  accumulate: bool = False) -> np.ndarray:
        """W uint16 bf16 bits [N, K], x f32 [T, K] -> f32 [T, N] (y + W x when accumulating)."""
        W = _c(W, np.uint16)
        x = _c(x, np.float32)
        N, K = W.shape
        T = x.shape[0]
        out = np.zeros((T, N), np.float32) if y is None else _c(y, np.float32).copy()
        assert self.lib.orc_bf16_gemv(_p(W), N, K, _p(x), T, _p(out), 1 if accumulate else 0) == 0
        return out

    def kv_write(self, k_new, v_new, pos, kcache, vcache):
        """In place on copies of kcache / vcache (uint16 [B, n_kv, S_max, D]); returns them."""
        k_new = _c(k_new, np.float32)
        v_new = _c(v_new, np.float32)
        pos = _c(pos, np.int32)
        kc = _c(kcache, np.uint16).copy()
        vc = _c(vcache, np.uint16).copy()
        B, n_kv, S_max, D = kc.shape
        assert self.lib.orc_kv_write(_p(k_new), _p(v_new), B, n_kv, D, _p(pos), _p(kc), _p(vc),
                                     S_max) == 0
        return kc, vc

    def gqa_attention(self, q, kcache, vcache, lengths, scale: float) -> np.ndarray:
        """q f32 [B, n_q, D]; caches uint16 [B, n_kv, S_max, D]; lengths int32 [B]."""
        q = _c(q, np.float32)
        kc = _c(kcache, np.uint16)
        vc = _c(vcache, np.uint16)
        lengths = _c(lengths, np.int32)
        B, n_q, D = q.shape
        n_kv, S_max = kc.shape[1], kc.shape[2]
        out = np.empty_like(q)
        assert self.lib.orc_gqa_attention(_p(q), B, n_q, n_kv, D, _p(kc), _p(vc), S_max,
                                          _p(lengths), float(scale), _p(out)) == 0
        return out

    def kv_write_rows(self, k_new, v_new, pos, kcache, vcache):
        """T rows of one sequence: k_new, v_new f32 [T, n_kv, D] into slots pos[t] of
        copies of kcache / vcache (uint16 [n_kv, S_max, D]); returns them."""
        k_new = _c(k_new, np.float32)
        v_new = _c(v_new, np.float32)
        pos = _c(pos, np.int32)
        kc = _c(kcache, np.uint16).copy()
        vc = _c(vcache, np.uint16).copy()
        n_kv, S_max, D = kc.shape
        assert self.lib.orc_kv_write_rows(_p(k_new), _p(v_new), k_new.shape[0], n_kv, D, _p(pos),
                                          _p(kc), _p(vc), S_max) == 0
        return kc, vc

    def prefill_attention(self, q, kcache, vcache, pos, scale: float) -> np.ndarray:
        """q f32 [T, n_q, D]; one sequence's caches uint16 [n_kv, S_max, D];
        query t attends to positions 0..pos[t].  -> f32 [T, n_q, D]."""
        q = _c(q, np.float32)
        kc = _c(kcache, np.uint16)
        vc = _c(vcache, np.uint16)
        pos = _c(pos, np.int32)
        T, n_q, D = q.shape
        n_kv, S_max = kc.shape[0], kc.shape[1]
        out = np.empty_like(q)
        assert self.lib.orc_prefill_attention(_p(q), T, n_q, n_kv, D, _p(kc), _p(vc), S_max, _p(pos),
                                              float(scale), _p(out)) == 0
        return out

    def _ffn_args(self, x, idx, w, gate, up, down, F, E):
        x = _c(x, np.float32)
        idx = _c(idx, np.int32)
        w = _c(w, np.float32)
        T, H = x.shape
        k = idx.shape[1]
        tens = []
        for (buf, qt) in (gate, up, down):
            buf = _c(buf, np.uint8)
            E_ = buf.shape[0] if buf.ndim == 2 else E
            stride = buf.shape[1] if buf.ndim == 2 else buf.size // E_
            tens.append((buf, qt, stride))
        return x, idx, w, T, H, k, tens

    def expert_ffn(self, x, idx, w, gate, up, down, F: int, E: int,
                   out: np.ndarray | None = None, accumulate: bool = False) -> np.ndarray:
        """gate/up/down are (uint8 [E, stride], qtype) pairs.  -> f32 [T, H]."""
        x, idx, w, T, H, k, tens = self._ffn_args(x, idx, w, gate, up, down, F, E)
        res = np.zeros((T, H), np.float32) if out is None else _c(out, np.float32).copy()
        (g, gq, gs), (u, uq, us), (d, dq, ds) = tens
        rc = self.lib.orc_expert_ffn(_p(x), T, H, F, E, k, _p(idx), _p(w),
                                     _p(g), gq, gs, _p(u), uq, us, _p(d), dq, ds,
                                     _p(res), 1 if accumulate else 0)
        assert rc == 0, rc
        return res

    def quantize_act_q8(self, x: np.ndarray):
        """x f32 [T, H] -> (p int8 [T, H], d f32 [T, H/32], values d*p f64 [T, H])."""
        x = _c(x, np.float32)
        T, H = x.shape
        p = np.empty((T, H), np.int8)
        d = np.empty((T, H // 32), np.float32)
        xq = np.empty((T, H), np.float64)
        assert self.lib.orc_quantize_act_q8(_p(x), T, H, _p(p), _p(d), _p(xq)) == 0
        return p, d, xq

    def expert_ffn_q8(self, x, idx, w, gate, up, down, F: int, E: int,
                      out: np.ndarray | None = None, accumulate: bool = False) -> np.ndarray:
        """The expert FFN with the gate/up activations in the int8 form of
        quantize_act_q8.  -> f32 [T, H]."""
        x, idx, w, T, H, k, tens = self._ffn_args(x, idx, w, gate, up, down, F, E)
        res = np.zeros((T, H), np.float32) if out is None else _c(out, np.float32).copy()
        (g, gq, gs), (u, uq, us), (d, dq, ds) = tens
        rc = self.lib.orc_expert_ffn_q8(_p(x), T, H, F, E, k, _p(idx), _p(w),
                                        _p(g), gq, gs, _p(u), uq, us, _p(d), dq, ds,
                                        _p(res), 1 if accumulate else 0)
        assert rc == 0, rc
        return res

    def expert_ffn_f64(self, x, idx, w, gate, up, down, F: int, E: int) -> np.ndarray:
        x, idx, w, T, H, k, tens = self._ffn_args(x, idx, w, gate, up, down, F, E)
        res = np.empty((T, H), np.float64)
        (g, gq, gs), (u, uq, us), (d, dq, ds) = tens
        rc = self.lib.orc_expert_ffn_f64(_p(x), T, H, F, E, k, _p(idx), _p(w),
                                         _p(g), gq, gs, _p(u), uq, us, _p(d), dq, ds, _p(res))
        assert rc == 0, rc
        return res

    def embed(self, tokens: np.ndarray, table: np.ndarray, qtype: int, V: int, H: int) -> np.ndarray:
        """tokens int32 [T]; table uint8 (V rows of H/256 blocks) -> f32 [T, H]."""
        tokens = _c(tokens, np.int32).reshape(-1)
        table = _c(table, np.uint8)
        assert table.size >= V * (H // 256) * BLOCK_BYTES[qtype]
        out = np.empty((tokens.size, H), np.float32)
        assert self.lib.orc_embed(_p(tokens), tokens.size, _p(table), qtype, V, H, _p(out)) == 0
        return out

    def output_head(self, x: np.ndarray, W: np.ndarray, qtype: int, V: int) -> np.ndarray:
        """x f32 [T, H]; W uint8 (V rows of H/256 blocks) -> logits f32 [T, V]."""
        x = _c(x, np.float32)
        W = _c(W, np.uint8)
        T, H = x.shape
        assert W.size >= V * (H // 256) * BLOCK_BYTES[qtype]
        out = np.empty((T, V), np.float32)
        assert self.lib.orc_output_head(_p(x), T, _p(W), qtype, V, H, _p(out)) == 0
        return out

    def rmsnorm(self, x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
        x = _c(x, np.float32)
        gain = _c(gain, np.float32)
        T, n = x.shape
        out = np.empty_like(x)
        self.lib.orc_rmsnorm(_p(x), T, n, _p(gain), eps, _p(out))
        return out

    def rope_neox(self, x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
        """x f32 [T, n_heads, D] -> rotated copy."""
        x = _c(x, np.float32).copy()
        pos = _c(pos, np.int32)
        T, nh, D = x.shape
        assert self.lib.orc_rope_neox(_p(x), T, nh, D, _p(pos), base) == 0
        return x

    def attn_prologue(self, q, k, q_norm, k_norm, pos, eps: float, rope_base: float):
        """q f32 [T, n_q, D], k f32 [T, n_kv, D] -> normalised and rotated copies."""
        q = _c(q, np.float32).copy()
        k = _c(k, np.float32).copy()
        T, nq, D = q.shape
        nkv = k.shape[1]
        rc = self.lib.orc_attn_prologue(_p(q), _p(k), T, nq, nkv, D,
                                        _p(_c(q_norm, np.float32)), _p(_c(k_norm, np.float32)),
                                        _p(_c(pos, np.int32)), eps, rope_base)
        assert rc == 0
        return q, k


    def moe_block(self, x, router, k: int, gate, up, down, F: int, E: int,
                  norm_gain=None, eps: float = 0.0, residual: bool = False):
        """The MoE block as the layer runs it: optional RMSNorm of x, route,
        expert FFN; with residual the block output is added to x.
        -> (out f32 [T, H], idx, w, logits)."""
        h = x if norm_gain is None else self.rmsnorm(x, norm_gain, eps)
        idx, w, logits = self.route(h, router, k)
        out = self.expert_ffn(h, idx, w, gate, up, down, F=F, E=E,
                              out=x if residual else None, accumulate=residual)
        return out, idx, w, logits

    def decoder_layer(self, x, wq, wk, wv, wo, in_norm, post_norm, q_norm, k_norm, kcache,
                      vcache, pos, n_q: int, n_kv: int, D: int, eps: float, rope_base: float,
                      router, k: int, gate, up, down, F: int, E: int):
        """One decode step of the Qwen3-MoE decoder layer for B sequences:
        x += Wo attention(QKnorm+RoPE(Wq,Wk,Wv RMSNorm(x))), then
        x += MoE(RMSNorm(x)).  Weights are bf16 bits [N, K]; caches uint16
        [B, n_kv, S_max, D] (copies are written, the inputs are left alone).
        -> (x_out f32 [B, H], idx, w, kcache, vcache)."""
        B = x.shape[0]
        xn = self.rmsnorm(x, in_norm, eps)
        q = self.bf16_gemv(wq, xn).reshape(B, n_q, D)
        kk = self.bf16_gemv(wk, xn).reshape(B, n_kv, D)
        vv = self.bf16_gemv(wv, xn).reshape(B, n_kv, D)
        q, kk = self.attn_prologue(q, kk, q_norm, k_norm, pos, eps, rope_base)
        kc, vc = self.kv_write(kk, vv, pos, kcache, vcache)
        a = self.gqa_attention(q, kc, vc, np.asarray(pos, np.int32) + 1, 1.0 / np.sqrt(D))
        x1 = self.bf16_gemv(wo, a.reshape(B, -1), x, accumulate=True)
        out, idx, w, _ = self.moe_block(x1, router, k, gate, up, down, F, E,
                                        norm_gain=post_norm, eps=eps, residual=True)
        return out, idx, w, kc, vc


    def attention_prefill(self, x, wq, wk, wv, wo, in_norm, q_norm, k_norm, kcache, vcache, pos,
                          n_q: int, n_kv: int, D: int, eps: float, rope_base: float):
        """The attention half of a prefill step for T tokens of ONE sequence at
        positions pos[t]: x + Wo attention(...), their k, v rows written into
        copies of the caches (uint16 [n_kv, S_max, D]).  -> (x1, kcache, vcache)."""
        T = x.shape[0]
        xn = self.rmsnorm(x, in_norm, eps)
        q = self.bf16_gemv(wq, xn).reshape(T, n_q, D)
        kk = self.bf16_gemv(wk, xn).reshape(T, n_kv, D)
        vv = self.bf16_gemv(wv, xn).reshape(T, n_kv, D)
        q, kk = self.attn_prologue(q, kk, q_norm, k_norm, pos, eps, rope_base)
        kc, vc = self.kv_write_rows(kk, vv, pos, kcache, vcache)
        a = self.prefill_attention(q, kc, vc, pos, 1.0 / np.sqrt(D))
        return self.bf16_gemv(wo, a.reshape(T, -1), x, accumulate=True), kc, vc

    def decoder_layer_prefill(self, x, wq, wk, wv, wo, in_norm, post_norm, q_norm, k_norm, kcache,
                              vcache, pos, n_q: int, n_kv: int, D: int, eps: float, rope_base: float,
                              router, k: int, gate, up, down, F: int, E: int):
        """A prefill step of the decoder layer: attention_prefill, then
        x += MoE(RMSNorm(x)).  -> (x_out f32 [T, H], idx, w, kcache, vcache)."""
        x1, kc, vc = self.attention_prefill(x, wq, wk, wv, wo, in_norm, q_norm, k_norm, kcache, vcache,
                                            pos, n_q, n_kv, D, eps, rope_base)
        out, idx, w, _ = self.moe_block(x1, router, k, gate, up, down, F, E,
                                        norm_gain=post_norm, eps=eps, residual=True)
        return out, idx, w, kc, vc


_default = None


def oracle() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
