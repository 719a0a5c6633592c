"""Pins of the CPU oracle against facts other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a closed form, an invariant, a brute-force
computation or a number printed on the pages.  The same functions run
against the real oracle (tests/test_oracle_pins.py) and against deliberately
broken copies of it (tests/test_oracle_mutants.py), which shows that a
plausible mistake anywhere in the oracle fails at least one pin.
"""
from __future__ import annotations

import math
from pathlib import Path

import numpy as np
import scipy.special

from sparse_moe_decode_q3moe_amd import inputs as gen

Q4_K, Q6_K = gen.Q4_K, gen.Q6_K
GOLDEN = Path(__file__).resolve().parent / "golden"


def _close(a, b, rtol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)
    assert err <= rtol, f"{what}: rel L2 {err:.3e} > {rtol:.1e}"


def _f16(x: float) -> list[int]:
    b = np.array([x], np.float16).view(np.uint8)
    return [int(b[0]), int(b[1])]


# ---------------------------------------------------------------- fp16 -----

def pin_half_all_patterns(o):
    """All 65,536 binary16 patterns against NumPy's own float16 conversion."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ---------------------------------------------------------------- Q4_K -----

def _q4k_block(d: float, dmin: float, S: list[int], Q) -> np.ndarray:
    Q = list(Q)
    assert len(S) == 12 and len(Q) == 128
    return np.array(_f16(d) + _f16(dmin) + S + Q, np.uint8)


def pin_q4k_unit_scales(o):
    """d = 1, dmin = 0, every scale 1 and min 0, quant byte b = b.  The low
    nibble of byte 32c+l is weight 64c+l and equals l mod 16; the high nibble
    is weight 64c+32+l and equals (32c+l) >> 4 = 2c + l//16."""
    S = [1, 1, 1, 1, 0, 0, 0, 0, 0x01, 0x01, 0x01, 0x01]
    w = o.dequant_block(Q4_K, _q4k_block(1.0, 0.0, S, range(128)))
    # hand-checked spots
    spots = {0: 0, 1: 1, 15: 15, 16: 0, 31: 15, 32: 0, 47: 0, 48: 1, 63: 1,
             64: 0, 95: 15, 96: 2, 112: 3, 160: 4, 224: 6, 255: 7}
    for i, v in spots.items():
        assert w[i] == v, (i, w[i], v)
    exp = np.empty(256)
    for c in range(4):
        for l in range(32):
            exp[64 * c + l] = l % 16
            exp[64 * c + 32 + l] = 2 * c + l // 16
    assert np.array_equal(w, exp)


# scales sc_j = 1,2,3,4,17,33,49,63 and mins m_j = 5,6,7,8,52,20,36,13, packed
# by hand.  For j >= 4 the low 4 bits of sc_j / m_j sit in the low / high
# nibble of S[j+4] and their top 2 bits in bits 6-7 of S[j-4] / S[j]; the
# top bits of the scales (1,2,3,3) and of the mins (3,1,2,0) differ, so
# reading one set from the other's bytes is visible.
#   S[0] = 1 | 1<<6 = 65    S[4] = 5 | 3<<6 = 197    S[8]  = 1 | 4<<4  = 65
#   S[1] = 2 | 2<<6 = 130   S[5] = 6 | 1<<6 = 70     S[9]  = 1 | 4<<4  = 65
#   S[2] = 3 | 3<<6 = 195   S[6] = 7 | 2<<6 = 135    S[10] = 1 | 4<<4  = 65
#   S[3] = 4 | 3<<6 = 196   S[7] = 8 | 0<<6 = 8      S[11] = 15 | 13<<4 = 223
PACKED_S = [65, 130, 195, 196, 197, 70, 135, 8, 65, 65, 65, 223]


def pin_q4k_packed_scales(o):
    """d = 0.5, dmin = 0.25, every quant byte 0xF3 (low nibble 3, high 15):
    sub-block j holds d*sc_j*q - dmin*m_j, worked by hand."""
    w = o.dequant_block(Q4_K, _q4k_block(0.5, 0.25, PACKED_S, [0xF3] * 128))
    per_sub = [0.25, 13.5, 2.75, 28.0, 12.5, 242.5, 64.5, 469.25]
    for j, v in enumerate(per_sub):
        assert np.all(w[32 * j: 32 * j + 32] == v), (j, w[32 * j], v)


def pin_q4k_fp16_scales(o):
    """The fp16 d and dmin multiply: d = 2^-10, dmin = 3*2^-12 with unit
    scales/mins and q = 9 give 9*2^-10 - 3*2^-12 everywhere."""
    S = [1, 1, 1, 1, 1, 1, 1, 1, 0x11, 0x11, 0x11, 0x11]
    w = o.dequant_block(Q4_K, _q4k_block(2.0 ** -10, 3 * 2.0 ** -12, S, [0x99] * 128))
    assert np.all(w == 9 * 2.0 ** -10 - 3 * 2.0 ** -12)


# ---------------------------------------------------------------- Q6_K -----

def _q6k_block(L, Hb, s, d: float) -> np.ndarray:
    L, Hb = list(L), list(Hb)
    assert len(L) == 128 and len(Hb) == 64 and len(s) == 16
    sb = list(np.array(s, np.int8).view(np.uint8))
    return np.array(L + Hb + sb + _f16(d), np.uint8)


def pin_q6k_centre_is_zero(o):
    """q = 32 everywhere (low 0, high bits 2 = 0b10 in every field) -> 0."""
    w = o.dequant_block(Q6_K, _q6k_block([0] * 128, [0xAA] * 64, [7] * 16, 1.0))
    assert np.all(w == 0.0)


def pin_q6k_most_negative(o):
    """q = 0 with scale -128 and d = 1 -> (-128)*(0-32) = 4096."""
    w = o.dequant_block(Q6_K, _q6k_block([0] * 128, [0] * 64, [-128] * 16, 1.0))
    assert np.all(w == 4096.0)


def pin_q6k_positional(o):
    """Bytes built so that q_i = i mod 64: every low-nibble byte b holds
    (b & 15) in both nibbles; high-bit byte l of each half is 136 (fields
    0,2,0,2) for l < 16 and 221 (fields 1,3,1,3) for l >= 16.  With unit
    scales and d = 1 the weights read back as (i mod 64) - 32."""
    L = [(b & 15) * 17 for b in range(128)]
    Hb = [136 if (l % 32) < 16 else 221 for l in range(64)]
    w = o.dequant_block(Q6_K, _q6k_block(L, Hb, [1] * 16, 1.0))
    assert np.array_equal(w, np.arange(256) % 64 - 32.0)


def pin_q6k_nibble_halves(o):
    """Low-nibble bytes 0x31 (low nibble 1, high nibble 3), every high field
    2: the first two 32-runs of each 128 read q = 33 (value 1), the last two
    read q = 35 (value 3)."""
    w = o.dequant_block(Q6_K, _q6k_block([0x31] * 128, [0xAA] * 64, [1] * 16, 1.0))
    exp = np.array([1.0 if (i % 128) < 64 else 3.0 for i in range(256)])
    assert np.array_equal(w, exp)


def pin_q6k_low_byte_map(o):
    """Low-nibble byte b = b, no high bits, unit scales, d = 1.  Weight
    128n + 32r + l reads byte 64n + 32(r&1) + l, its low nibble for r < 2 and
    its high nibble for r >= 2; value q - 32.  Spots worked by hand."""
    w = o.dequant_block(Q6_K, _q6k_block(range(128), [0] * 64, [1] * 16, 1.0))
    spots = {0: -32, 5: -27, 31: -17, 32: -32, 50: -30, 64: -32, 80: -31, 96: -30,
             127: -29, 128: -32, 129: -31, 200: -28, 255: -25}
    for i, v in spots.items():
        assert w[i] == v, (i, w[i], v)


def pin_q6k_high_bit_map(o):
    """High-bit byte j = j, no low bits, unit scales, d = 1.  Weight
    128n + 32r + l takes bits 2r..2r+1 of byte 32n + l as q >> 4."""
    w = o.dequant_block(Q6_K, _q6k_block([0] * 128, range(64), [1] * 16, 1.0))
    spots = {0: -32, 1: -16, 3: 16, 33: -32, 36: -16, 44: 16, 98: -32, 144: -32,
             208: 16, 240: -32, 255: -32}
    for i, v in spots.items():
        assert w[i] == v, (i, w[i], v)


def pin_q6k_scale_index(o):
    """q = 33 everywhere (value 1 after the offset), scales s[m] = m + 1,
    d = 0.5: each run of 16 consecutive weights takes the next scale."""
    w = o.dequant_block(Q6_K, _q6k_block([0x11] * 128, [0xAA] * 64,
                                         list(range(1, 17)), 0.5))
    spots = {0: 1, 15: 1, 16: 2, 31: 2, 32: 3, 48: 4, 64: 5, 96: 7, 127: 8,
             128: 9, 200: 13, 255: 16}
    for i, v in spots.items():
        assert w[i] == 0.5 * v, (i, w[i])
    assert np.array_equal(w, 0.5 * (np.arange(256) // 16 + 1))


def pin_q6k_negative_scales(o):
    """Negative int8 scales keep their sign: s = -3, q = 40, d = 0.25 -> -6."""
    # q = 40 = 0b10_1000: low nibble 8 in every position, high field 2.
    w = o.dequant_block(Q6_K, _q6k_block([0x88] * 128, [0xAA] * 64, [-3] * 16, 0.25))
    assert np.all(w == -6.0)


# ------------------------------------------------------- sizes & layout -----

def page_sizes():
    rows = {}
    for line in (GOLDEN / "page_sizes.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            name, value, *_ = line.split()
            rows[name] = float(value)
    return rows


def pin_page_byte_counts(o):
    """Per-expert byte counts and the 48-layer expert total printed under
    "File facts" follow from 144 / 210 bytes per 256 weights."""
    ps = page_sizes()
    b4, b6 = o.lib.orc_block_bytes(Q4_K), o.lib.orc_block_bytes(Q6_K)
    gate = 768 * (2048 // 256) * b4
    down6 = 2048 * (768 // 256) * b6
    down4 = 2048 * (768 // 256) * b4
    assert gate == ps["gate_up_q4k_per_expert"]
    assert down6 == ps["down_q6k_per_expert"]
    assert down4 == ps["down_q4k_per_expert"]
    assert 128 * 4 == ps["router_logits_per_token_bytes"]
    total = 24 * 128 * (2 * gate + down6) + 24 * 128 * (2 * gate + down4)
    assert round(total / 1e9, 2) == ps["experts_all_layers_gb_2dp"]


def pin_row_orientation(o):
    """Rows are consecutive runs of cols/256 super-blocks: a Q4_K matrix whose
    row r has every quant nibble r mod 16 (unit scale, zero min) gives
    y[r] = (r mod 16) * sum(x); likewise a Q6_K matrix with q = 32 + r."""
    rows, cols = 20, 512
    S = [1, 1, 1, 1, 0, 0, 0, 0, 0x01, 0x01, 0x01, 0x01]
    mat = np.concatenate([_q4k_block(1.0, 0.0, S, [(r % 16) * 17] * 128)
                          for r in range(rows) for _ in range(cols // 256)])
    x = np.linspace(-1.0, 2.0, cols)
    y = o.qgemv(Q4_K, mat, rows, cols, x)
    assert np.allclose(y, (np.arange(rows) % 16) * x.sum(), rtol=1e-13, atol=1e-12)
    dense = o.dequant_matrix(Q4_K, mat, rows, cols)
    assert np.array_equal(dense, np.repeat((np.arange(rows) % 16.0)[:, None], cols, 1))
    mat6 = np.concatenate([_q6k_block([r * 17] * 128, [0xAA] * 64, [1] * 16, 1.0)
                           for r in range(8) for _ in range(cols // 256)])
    y6 = o.qgemv(Q6_K, mat6, 8, cols, x)
    assert np.allclose(y6, np.arange(8) * x.sum(), rtol=1e-13, atol=1e-12)


def pin_qgemv_dense_product(o):
    """qgemv equals NumPy's dense product with the dequantised matrix."""
    g = gen.make_generator(11)
    for qt, rows, cols in ((Q4_K, 24, 768), (Q6_K, 16, 512)):
        mat = gen.kquant_experts(qt, 1, rows, cols, g)[0].numpy()
        x = gen.normal_f32((cols,), 1.0, g).numpy().astype(np.float64)
        dense = o.dequant_matrix(qt, mat, rows, cols)
        _close(o.qgemv(qt, mat, rows, cols, x), dense @ x, 1e-13, "qgemv")


# --------------------------------------------------------------- router -----

def _router_case(T, H, E, seed):
    g = gen.make_generator(seed)
    return (gen.normal_f32((T, H), 1.0, g).numpy(), gen.normal_f32((E, H), 0.02, g).numpy())


def pin_route_bruteforce(o):
    """Logits equal NumPy's double product; the k selected experts are the
    first k of a full stable sort of all E logits (descending); weights are
    SciPy's softmax over those k logits."""
    x, R = _router_case(16, 2048, 128, 21)
    k = 8
    idx, w, logits = o.route(x, R, k)
    ref = x.astype(np.float64) @ R.astype(np.float64).T
    _close(logits, ref, 1e-14, "router logits")
    order = np.argsort(-ref, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, order)
    sel = np.take_along_axis(ref, order, 1)
    _close(w, scipy.special.softmax(sel, axis=1), 1e-7, "routing weights")
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(idx.shape[0]):
        assert len(set(idx[t].tolist())) == k
        assert idx[t].min() >= 0 and idx[t].max() < 128


def pin_route_k1_and_kE(o):
    """k = 1 gives weight exactly 1; k = E gives the full softmax, sorted."""
    x, R = _router_case(4, 256, 8, 22)
    idx, w, lg = o.route(x, R, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(lg, 1))
    idx, w, lg = o.route(x, R, 8)
    full = scipy.special.softmax(x.astype(np.float64) @ R.astype(np.float64).T, axis=1)
    assert np.array_equal(idx, np.argsort(-full, 1, kind="stable"))
    _close(w, np.take_along_axis(full, idx, 1), 1e-7, "k=E weights")


def pin_route_ties(o):
    """Duplicate router rows tie exactly; the lower expert index comes first."""
    x, R = _router_case(3, 512, 32, 23)
    R[[5, 9, 30]] = 0.01 * np.sign(x[0])[None, :]     # three identical, dominant rows
    idx, w, lg = o.route(x[:1], R, 4)
    assert lg[0, 5] == lg[0, 9] == lg[0, 30]
    assert list(idx[0, :3]) == [5, 9, 30]
    assert w[0, 0] == w[0, 1] == w[0, 2]


def pin_route_shift_invariance(o):
    """Adding the same constant to every logit (an extra input column equal
    to 1 and a constant router column) changes neither choice nor weights."""
    x, R = _router_case(8, 2047, 64, 24)
    x1 = np.concatenate([x, np.ones((8, 1), np.float32)], 1)
    R1 = np.concatenate([R, np.full((64, 1), 3.0, np.float32)], 1)
    i0, w0, _ = o.route(x, R, 6)
    i1, w1, _ = o.route(x1, R1, 6)
    assert np.array_equal(i0, i1)
    _close(w1, w0, 1e-7, "shifted weights")


# ------------------------------------------------------------ expert FFN -----

def _silu(z):
    return z * scipy.special.expit(z)


def _dense_experts(o, buf, qt, E, rows, cols):
    return [o.dequant_matrix(qt, buf[e], rows, cols) for e in range(E)]


def _ffn_case(shape: gen.MoeShape, seed: int):
    layer = gen.moe_layer(shape, seed)
    x = gen.hidden_states(shape.T, shape.H, seed + 1000).numpy()
    return layer, x


def _dense_moe(o, layer, x, gating):
    """sum over ALL experts of gating[t, e] * FFN_e(x[t]), NumPy float64."""
    s = layer.shape
    Wg = _dense_experts(o, layer.gate.numpy(), Q4_K, s.E, s.F, s.H)
    Wu = _dense_experts(o, layer.up.numpy(), Q4_K, s.E, s.F, s.H)
    Wd = _dense_experts(o, layer.down.numpy(), s.down_qtype, s.E, s.H, s.F)
    xd = x.astype(np.float64)
    out = np.zeros((x.shape[0], s.H))
    for e in range(s.E):
        y = (_silu(xd @ Wg[e].T) * (xd @ Wu[e].T)) @ Wd[e].T
        out += gating[:, e:e + 1] * y
    return out


def _tensors(layer):
    s = layer.shape
    return ((layer.gate.numpy(), Q4_K), (layer.up.numpy(), Q4_K),
            (layer.down.numpy(), s.down_qtype))


def pin_ffn_dense_bruteforce(o):
    """Sparse top-k FFN equals the dense mixture over all experts whose
    gating is w on the selected experts and 0 elsewhere (all-Q4_K tiny
    layer, and a Q6_K-down layer with F != H)."""
    for shape, seed in ((gen.TINY, 31),
                        (gen.MoeShape(T=3, H=256, E=6, k=3, F=512, down_qtype=Q6_K), 32)):
        layer, x = _ffn_case(shape, seed)
        idx, w, _ = o.route(x, layer.router.numpy(), shape.k)
        gating = np.zeros((shape.T, shape.E))
        for t in range(shape.T):
            gating[t, idx[t]] = w[t]
        ref = _dense_moe(o, layer, x, gating)
        got = o.expert_ffn_f64(x, idx, w, *_tensors(layer), F=shape.F, E=shape.E)
        _close(got, ref, 1e-12, f"dense brute force {shape}")


def pin_ffn_k_equals_E(o):
    """With k = E the block is the softmax mixture of every expert."""
    shape = gen.MoeShape(T=2, H=256, E=4, k=4, F=256, down_qtype=Q4_K)
    layer, x = _ffn_case(shape, 33)
    idx, w, lg = o.route(x, layer.router.numpy(), 4)
    ref = _dense_moe(o, layer, x, scipy.special.softmax(lg, axis=1))
    got = o.expert_ffn_f64(x, idx, w, *_tensors(layer), F=256, E=4)
    _close(got, ref, 3e-7, "k=E mixture")      # weights were rounded to f32


def pin_ffn_single_expert_is_dense_mlp(o):
    """E = 1, k = 1: a plain dense SwiGLU MLP Wd (silu(Wg x) * (Wu x))."""
    shape = gen.MoeShape(T=2, H=512, E=1, k=1, F=256, down_qtype=Q6_K)
    layer, x = _ffn_case(shape, 34)
    Wg = o.dequant_matrix(Q4_K, layer.gate.numpy()[0], 256, 512)
    Wu = o.dequant_matrix(Q4_K, layer.up.numpy()[0], 256, 512)
    Wd = o.dequant_matrix(Q6_K, layer.down.numpy()[0], 512, 256)
    xd = x.astype(np.float64)
    ref = (_silu(xd @ Wg.T) * (xd @ Wu.T)) @ Wd.T
    got = o.expert_ffn_f64(x, np.zeros((2, 1), np.int32), np.ones((2, 1), np.float32),
                           *_tensors(layer), F=256, E=1)
    _close(got, ref, 1e-12, "dense MLP")


def pin_ffn_zero_cases(o):
    """Zero input -> zero output; an all-zero up tensor -> zero output."""
    layer, x = _ffn_case(gen.TINY, 35)
    idx, w, _ = o.route(x, layer.router.numpy(), 2)
    t = _tensors(layer)
    assert np.all(o.expert_ffn_f64(np.zeros_like(x), idx, w, *t, F=256, E=8) == 0)
    zero_up = (np.zeros_like(t[1][0]), Q4_K)
    assert np.all(o.expert_ffn_f64(x, idx, w, t[0], zero_up, t[2], F=256, E=8) == 0)


def pin_ffn_tokens_independent(o):
    """A batch of T tokens equals T separate one-token calls, bit for bit."""
    layer, x = _ffn_case(gen.TINY, 36)
    idx, w, _ = o.route(x, layer.router.numpy(), 2)
    t = _tensors(layer)
    both = o.expert_ffn(x, idx, w, *t, F=256, E=8)
    for i in range(x.shape[0]):
        one = o.expert_ffn(x[i:i + 1], idx[i:i + 1], w[i:i + 1], *t, F=256, E=8)
        assert np.array_equal(one[0], both[i])


def pin_ffn_accumulate(o):
    """accumulate = 1 adds the block output to what the output buffer holds,
    rounding once: f32(prev + ffn)."""
    layer, x = _ffn_case(gen.TINY, 37)
    idx, w, _ = o.route(x, layer.router.numpy(), 2)
    t = _tensors(layer)
    prev = (x * 3.0).astype(np.float32)
    got = o.expert_ffn(x, idx, w, *t, F=256, E=8, out=prev, accumulate=True)
    ref = (prev.astype(np.float64) + o.expert_ffn_f64(x, idx, w, *t, F=256, E=8)).astype(np.float32)
    assert np.array_equal(got, ref)


def pin_ffn_expert_stride(o):
    """Expert e is read at base + e*stride: padding every expert with junk
    bytes (a larger stride) leaves the result unchanged, and the result
    depends on which expert is named."""
    layer, x = _ffn_case(gen.TINY, 38)
    idx, w, _ = o.route(x, layer.router.numpy(), 2)
    t = _tensors(layer)
    junk = np.random.default_rng(0)
    padded = []
    for buf, qt in t:
        pad = junk.integers(0, 256, (buf.shape[0], 160), dtype=np.uint8)
        padded.append((np.concatenate([buf, pad], 1), qt))
    a = o.expert_ffn_f64(x, idx, w, *t, F=256, E=8)
    b = o.expert_ffn_f64(x, idx, w, *padded, F=256, E=8)
    assert np.array_equal(a, b)
    c = o.expert_ffn_f64(x, (idx + 1) % 8, w, *t, F=256, E=8)
    assert np.linalg.norm(c - a) > 1e-3 * np.linalg.norm(a)


# --------------------------------------------------------- norm and RoPE -----

# ------------------------------------------------------ prefill attention -----

def _bf16_bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_prefill_attention_bruteforce(o):
    """T = 7 queries of one sequence at positions 3..9 (GQA, 4 query heads
    on 2 kv heads): each query attends to cache positions 0..pos[t]; against
    a NumPy float64 softmax over that causal window."""
    rng = np.random.default_rng(81)
    T, nq, nkv, D, S = 7, 4, 2, 16, 12
    q = rng.standard_normal((T, nq, D)).astype(np.float32)
    kc = _bf16_bits(rng.standard_normal((nkv, S, D)))
    vc = _bf16_bits(rng.standard_normal((nkv, S, D)))
    pos = np.arange(3, 10, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    got = o.prefill_attention(q, kc, vc, pos, scale)
    K, Vv = _bf16_vals(kc), _bf16_vals(vc)
    ref = np.empty((T, nq, D))
    for t in range(T):
        for h in range(nq):
            g = h // (nq // nkv)
            s_ = scale * (K[g, :pos[t] + 1] @ q[t, h].astype(np.float64))
            p = np.exp(s_ - s_.max())
            ref[t, h] = (p / p.sum()) @ Vv[g, :pos[t] + 1]
    _close(got, ref.astype(np.float32), 1e-6, "prefill attention brute force")


def pin_prefill_attention_causal_window(o):
    """Changing cache rows after pos[t] leaves query t unchanged; changing
    row pos[t] itself changes it; pos = 0 returns v at position 0 exactly."""
    rng = np.random.default_rng(82)
    nq, nkv, D, S = 2, 1, 8, 10
    q = rng.standard_normal((3, nq, D)).astype(np.float32)
    kc = _bf16_bits(rng.standard_normal((nkv, S, D)))
    vc = _bf16_bits(rng.standard_normal((nkv, S, D)))
    pos = np.array([0, 4, 6], np.int32)
    base = o.prefill_attention(q, kc, vc, pos, 0.3)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, 7:] ^= 0x4000
    vc2[:, 7:] ^= 0x4000
    assert np.array_equal(o.prefill_attention(q, kc2, vc2, pos, 0.3), base)
    vc3 = vc.copy()
    vc3[:, 6] ^= 0x0100
    after = o.prefill_attention(q, kc, vc3, pos, 0.3)
    assert np.array_equal(after[:2], base[:2]) and not np.array_equal(after[2], base[2])
    assert np.array_equal(base[0], np.broadcast_to(_bf16_vals(vc)[0, 0], (nq, D)).astype(np.float32))


def pin_kv_write_rows(o):
    """Row t of the new keys and values lands, rounded to bf16 (torch's
    round to nearest even), in slot pos[t] of the one sequence's caches;
    every other slot is untouched."""
    rng = np.random.default_rng(83)
    T, nkv, D, S = 3, 2, 8, 9
    k = rng.standard_normal((T, nkv, D)).astype(np.float32)
    v = rng.standard_normal((T, nkv, D)).astype(np.float32)
    kc = np.arange(nkv * S * D, dtype=np.uint16).reshape(nkv, S, D)
    vc = kc[::-1].copy()
    pos = np.array([4, 0, 8], np.int32)
    k2, v2 = o.kv_write_rows(k, v, pos, kc, vc)
    for t in range(T):
        assert np.array_equal(k2[:, pos[t]], _bf16_bits(k[t]))
        assert np.array_equal(v2[:, pos[t]], _bf16_bits(v[t]))
    keep = np.setdiff1d(np.arange(S), pos)
    assert np.array_equal(k2[:, keep], kc[:, keep]) and np.array_equal(v2[:, keep], vc[:, keep])


# ------------------------------------------------ embedding / output head -----

def pin_embed_rows(o):
    """The embedding gather returns the pinned dequantised rows of the
    chosen tokens (first, last, repeated), rounded once to f32, for Q4_K and
    Q6_K tables with a vocabulary that is not a multiple of anything; a token
    outside [0, V) gives a NaN row."""
    g = gen.make_generator(61)
    for qt in (Q4_K, Q6_K):
        V, H = 37, 512
        table = gen.kquant_experts(qt, 1, V, H, g)[0].numpy()
        dense = o.dequant_matrix(qt, table, V, H)
        toks = np.array([0, 36, 5, 5, 17], np.int32)
        got = o.embed(toks, table, qt, V, H)
        assert np.array_equal(got, dense[toks].astype(np.float32))
        bad = o.embed(np.array([3, -1, 37], np.int32), table, qt, V, H)
        assert np.array_equal(bad[0], dense[3].astype(np.float32))
        assert np.all(np.isnan(bad[1:]))


def pin_output_head_dense(o):
    """The head's logits equal a dense NumPy product of the pinned
    dequantised Q6_K matrix with x (V = 301 rows, 2 tokens), and a one-hot x
    reads back one column of the matrix."""
    g = gen.make_generator(62)
    V, H = 301, 512
    W = gen.kquant_experts(Q6_K, 1, V, H, g)[0].numpy()
    dense = o.dequant_matrix(Q6_K, W, V, H)
    x = gen.hidden_states(2, H, 63).numpy()
    got = o.output_head(x, W, Q6_K, V)
    _close(got, (x.astype(np.float64) @ dense.T).astype(np.float32), 1e-7, "head dense product")
    e = np.zeros((1, H), np.float32)
    e[0, 300] = 1.0
    assert np.array_equal(o.output_head(e, W, Q6_K, V)[0], dense[:, 300].astype(np.float32))


# ------------------------------------------------- int8 activations (Q8) -----

def pin_q8_hand_group(o):
    """A hand-worked 32-value group: max |x| = 127 gives d = 1 exactly, so
    p = x rounded to the nearest integer with ties to even (63.5 -> 64,
    -63.5 -> -64, 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2); a second group
    scaled by 2^-3 gives d = 2^-3 and the same integers; an all-zero group
    gives d = 0, p = 0; a group holding +inf or NaN gives NaN values."""
    g = np.array([127, 63.5, -63.5, 0.5, 1.5, 2.5, -2.5, -127, 3.25, -0.75] + [0.0] * 22, np.float32)
    want = np.array([127, 64, -64, 0, 2, 2, -2, -127, 3, -1] + [0] * 22, np.int8)
    zero = np.zeros(32, np.float32)
    bad = g.copy()
    bad[5] = np.inf
    nan = g.copy()
    nan[9] = np.nan
    x = np.stack([np.concatenate([g, g / 8]), np.concatenate([zero, bad]),
                  np.concatenate([nan, g])])
    p, d, xq = o.quantize_act_q8(x)
    assert np.array_equal(p[0, :32], want) and np.array_equal(p[0, 32:], want)
    assert d[0, 0] == 1.0 and d[0, 1] == 0.125
    assert np.array_equal(xq[0, :32], want.astype(np.float64))
    assert d[1, 0] == 0.0 and np.all(p[1, :32] == 0) and np.all(xq[1, :32] == 0.0)
    assert np.isnan(d[1, 1]) and np.all(np.isnan(xq[1, 32:]))
    assert np.isnan(d[2, 0]) and np.all(np.isnan(xq[2, :32]))
    assert np.array_equal(p[2, 32:], want)


def pin_q8_bounds(o):
    """On N(0, 1) rows: d = max|x| / 127 rounded to f32 (NumPy's own f32
    division), |p| <= 127 with the largest value at +-127, and every value
    within half a step of its group's scale: |x - d p| <= d / 2 (plus the
    f32 rounding of x / d)."""
    x = gen.hidden_states(3, 2048, 77).numpy()
    p, d, xq = o.quantize_act_q8(x)
    g = x.reshape(3, 64, 32)
    amax = np.abs(g).max(axis=2)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))
    assert np.abs(p.astype(np.int32)).max() <= 127
    pg = p.reshape(3, 64, 32).astype(np.int32)
    top = np.take_along_axis(pg, np.abs(g).argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.all(np.abs(top) == 127)
    err = np.abs(x.astype(np.float64) - xq).reshape(3, 64, 32)
    assert np.all(err <= d[..., None].astype(np.float64) * (0.5 + 1e-6))
    assert np.array_equal(xq, d.repeat(32, axis=1).astype(np.float64) * p)


def pin_q8_ffn_is_block_on_quantised_input(o):
    """The int8-activation block equals the dense NumPy block evaluated on
    the dequantised activations d * p for gate and up (the down projection
    on h as computed), summed over the selected experts with their weights."""
    shape = gen.MoeShape(T=3, H=256, E=6, k=3, F=512, down_qtype=Q6_K)
    layer, x = _ffn_case(shape, 38)
    idx, w, _ = o.route(x, layer.router.numpy(), shape.k)
    _, _, xq = o.quantize_act_q8(x)
    Wg = _dense_experts(o, layer.gate.numpy(), Q4_K, shape.E, shape.F, shape.H)
    Wu = _dense_experts(o, layer.up.numpy(), Q4_K, shape.E, shape.F, shape.H)
    Wd = _dense_experts(o, layer.down.numpy(), Q6_K, shape.E, shape.H, shape.F)
    ref = np.zeros((shape.T, shape.H))
    for t in range(shape.T):
        for s_ in range(shape.k):
            e = idx[t, s_]
            ref[t] += w[t, s_] * ((_silu(Wg[e] @ xq[t]) * (Wu[e] @ xq[t])) @ Wd[e].T)
    got = o.expert_ffn_q8(x, idx, w, *_tensors(layer), F=shape.F, E=shape.E)
    _close(got, ref.astype(np.float32), 1e-6, "int8-activation block")
    prev = (x * 2.0).astype(np.float32)
    acc = o.expert_ffn_q8(x, idx, w, *_tensors(layer), F=shape.F, E=shape.E, out=prev,
                          accumulate=True)
    _close(acc, prev.astype(np.float64) + ref, 1e-6, "int8-activation block, accumulate")


def pin_rmsnorm_closed_form(o):
    """With unit gain, RMS(y)^2 = ms / (ms + eps); gains multiply
    elementwise; with eps = 0 the result is scale invariant."""
    g = gen.make_generator(41)
    x = gen.normal_f32((5, 128), 1e-3, g).numpy()
    eps = 1e-6
    y = o.rmsnorm(x, np.ones(128, np.float32), eps).astype(np.float64)
    ms = (x.astype(np.float64) ** 2).mean(1)
    assert np.allclose((y ** 2).mean(1), ms / (ms + eps), rtol=1e-6)
    gain = gen.uniform_f32((128,), 0.5, 1.5, g).numpy()
    yg = o.rmsnorm(x, gain, eps).astype(np.float64)
    assert np.allclose(yg, y * gain, rtol=3e-7, atol=0)
    y0 = o.rmsnorm(x, np.ones(128, np.float32), 0.0)
    y1 = o.rmsnorm(x * np.float32(1024.0), np.ones(128, np.float32), 0.0)
    assert np.allclose(y0, y1, rtol=1e-6, atol=0)


def _onehot_heads(D, i):
    v = np.zeros((1, 1, D), np.float32)
    v[0, 0, i] = 1.0
    return v


def pin_rope_neox_pairs(o):
    """NEOX pairing: unit vector e_i at position p lands on (cos t, sin t) at
    indices (i, i + D/2) with t = p * base^(-2i/D).  For i = 0, t = p; for
    i = D/4, base^(-1/2) = 1/sqrt(base).  Interleaved RoPE would move e_0
    into index 1 instead."""
    D, base = 128, 1e7
    for i, p, theta in ((0, 1, 1.0), (0, 7, 7.0), (32, 4095, 4095 / math.sqrt(base))):
        r = o.rope_neox(_onehot_heads(D, i), np.array([p]), base)[0, 0].astype(np.float64)
        exp = np.zeros(D)
        exp[i] = math.cos(theta)
        exp[i + D // 2] = math.sin(theta)
        assert np.allclose(r, exp, atol=1e-7), (i, p)


def pin_rope_invariants(o):
    """Rotation keeps each head's norm, p = 0 is the identity, rotating by
    -p undoes p, and <R_m q, R_n k> depends only on m - n."""
    g = gen.make_generator(42)
    D, base = 128, 1e7
    x = gen.normal_f32((3, 4, D), 1.0, g).numpy()
    pos = np.array([0, 17, 4095])
    r = o.rope_neox(x, pos, base)
    assert np.allclose(np.linalg.norm(r.astype(np.float64), axis=2),
                       np.linalg.norm(x.astype(np.float64), axis=2), rtol=1e-6)
    assert np.array_equal(r[0], x[0])
    back = o.rope_neox(r, -pos, base)
    assert np.allclose(back, x, atol=2e-6)
    q = gen.normal_f32((1, 1, D), 1.0, g).numpy()
    k = gen.normal_f32((1, 1, D), 1.0, g).numpy()
    d1 = np.dot(o.rope_neox(q, np.array([900]), base).ravel().astype(np.float64),
                o.rope_neox(k, np.array([100]), base).ravel())
    d2 = np.dot(o.rope_neox(q, np.array([800]), base).ravel().astype(np.float64), k.ravel())
    assert abs(d1 - d2) <= 1e-5 * (abs(d2) + 1)


def pin_prologue(o):
    """Per-head QK-norm then RoPE: (a) head_dim 128 with 32 q heads (q_dim
    4096 != hidden 2048) normalises each 128-slice as a whole, so a head
    whose first half is 10x its second half keeps that 10:1 ratio; (b) at
    position 0 the result is the per-head RMSNorm alone with the q gain for
    q and the k gain for k; (c) the result equals RoPE applied after
    RMSNorm and differs from RMSNorm after RoPE when the gain is not flat."""
    g = gen.make_generator(43)
    D, nq, nkv, eps, base = 128, 32, 4, 1e-6, 1e7
    q = gen.normal_f32((2, nq, D), 1.0, g).numpy()
    k = gen.normal_f32((2, nkv, D), 1.0, g).numpy()
    q[:, :, :64] *= 10.0
    ones = np.ones(D, np.float32)
    qn = gen.uniform_f32((D,), 0.5, 1.5, g).numpy()
    kn = gen.uniform_f32((D,), 0.5, 1.5, g).numpy()
    zero = np.zeros(2, np.int32)
    q1, _ = o.attn_prologue(q, k, ones, ones, zero, eps, base)
    ratio = np.sqrt((q1[:, :, :64].astype(np.float64) ** 2).mean(2) /
                    (q1[:, :, 64:].astype(np.float64) ** 2).mean(2))
    ref_ratio = np.sqrt((q[:, :, :64].astype(np.float64) ** 2).mean(2) /
                        (q[:, :, 64:].astype(np.float64) ** 2).mean(2))
    assert np.allclose(ratio, ref_ratio, rtol=1e-5)
    assert np.allclose((q1.astype(np.float64) ** 2).mean(2), 1.0, rtol=1e-5)
    qa, ka = o.attn_prologue(q, k, qn, kn, zero, eps, base)
    assert np.allclose(qa, o.rmsnorm(q.reshape(-1, D), qn, eps).reshape(q.shape), rtol=1e-6)
    assert np.allclose(ka, o.rmsnorm(k.reshape(-1, D), kn, eps).reshape(k.shape), rtol=1e-6)
    pos = np.array([5, 4095], np.int32)
    qb, kb = o.attn_prologue(q, k, qn, kn, pos, eps, base)
    qr = o.rope_neox(o.rmsnorm(q.reshape(-1, D), qn, eps).reshape(q.shape), pos, base)
    assert np.allclose(qb, qr, atol=1e-5)
    qw = o.rmsnorm(o.rope_neox(q, pos, base).reshape(-1, D), qn, eps).reshape(q.shape)
    assert not np.allclose(qb, qw, atol=1e-2)


# ------------------------------------------------- token -> expert grouping --

def pin_group_hand_example(o):
    """A worked example: 3 tokens, k = 2, E = 4.
    Pairs (p = t*k + slot): 0->2, 1->0, 2->2, 3->3, 4->0, 5->2.
    Expert 0: pairs 1, 4; expert 1: none; expert 2: pairs 0, 2, 5; expert 3: pair 3."""
    idx = np.array([[2, 0], [2, 3], [0, 2]], np.int32)
    counts, offsets, pairs = o.group_by_expert(idx, 4)
    assert counts.tolist() == [2, 0, 3, 1]
    assert offsets.tolist() == [0, 2, 2, 5, 6]
    assert pairs.tolist() == [1, 4, 0, 2, 5, 3]


def pin_group_library_sort(o):
    """Random routings (incl. out-of-range indices) against a library sort of
    the valid pairs by (expert, pair), and the count / offset invariants."""
    rng = np.random.default_rng(31)
    for T, k, E in [(1, 8, 128), (13, 8, 128), (512, 8, 128), (40, 3, 5), (9, 32, 1024), (0, 4, 7)]:
        idx = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
        counts, offsets, pairs = o.group_by_expert(idx, E)
        flat = idx.reshape(-1)
        valid = [p for p in range(flat.size) if 0 <= flat[p] < E]
        expect = sorted(valid, key=lambda p: (int(flat[p]), p))
        assert pairs.tolist() == expect
        assert offsets[0] == 0 and offsets[E] == len(valid)
        assert np.array_equal(np.diff(offsets), counts)
        assert counts.tolist() == [int(np.sum(flat == e)) for e in range(E)]


def pin_group_skewed_routing(o):
    """Half of 64 tokens pick the same 4 experts: their pairs come first
    within those experts' lists in token order, every pair exactly once."""
    T, k, E = 64, 8, 128
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[::2, :4] = [3, 17, 64, 101]
    counts, offsets, pairs = o.group_by_expert(idx, E)
    assert sorted(pairs.tolist()) == list(range(T * k))
    for e in (3, 17, 64, 101):
        seg = pairs[offsets[e]:offsets[e + 1]]
        assert list(seg) == sorted(seg) and all(idx.reshape(-1)[seg] == e)
        assert counts[e] >= T // 2


# ------------------------------------------------- decoder-layer pieces --

def _torch_bf16_bits(a) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(b) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def pin_bf16_all_patterns(o):
    """All 65,536 bfloat16 patterns against torch's own bfloat16 widening."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _bits_to_f64(bits)
    got = np.array([o.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_float_to_bf16_rounding(o):
    """Round to nearest even against torch.bfloat16 on random values, exact
    ties (odd and even), values that round up into the next binade, and
    signed zeros / infinities."""
    rng = np.random.default_rng(41)
    vals = list(rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 2000))
    for base in (1.0, 1.5, 3.0, -2.25, 1e-3, 6e4):
        b = np.float32(base).view(np.uint32)
        for low in (0x7fff, 0x8000, 0x8001, 0x18000, 0xffff):
            vals.append(np.uint32((int(b) & 0xffff0000) | low).view(np.float32))
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(np.inf), np.float32(-np.inf)]
    vals = np.array(vals, np.float32)
    got = np.array([o.float_to_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, _torch_bf16_bits(vals))


def pin_bf16_gemv_dense(o):
    """Random bf16 weights against a dense NumPy product; one-hot probes pin
    the orientation (y[t][n] reads row n of W and x[t]); accumulate adds."""
    rng = np.random.default_rng(42)
    N, K, T = 48, 96, 3
    W = _torch_bf16_bits(rng.standard_normal((N, K)).astype(np.float32) * 0.05)
    x = rng.standard_normal((T, K)).astype(np.float32)
    _close(o.bf16_gemv(W, x), x.astype(np.float64) @ _bits_to_f64(W).T, 1e-7, "bf16 gemv")
    one = np.zeros((N, K), np.uint16)
    one[7, 30] = _torch_bf16_bits(np.array([1.0]))[0]
    y = o.bf16_gemv(one, x)
    assert np.array_equal(y[:, 7], x[:, 30]) and np.count_nonzero(y) == np.count_nonzero(x[:, 30])
    prev = rng.standard_normal((T, N)).astype(np.float32)
    _close(o.bf16_gemv(W, x, prev, accumulate=True),
           prev + x.astype(np.float64) @ _bits_to_f64(W).T, 1e-7, "bf16 gemv accumulate")


def pin_kv_write(o):
    """The new k, v land at each sequence's position as torch.bfloat16 bits;
    every other slot is untouched."""
    rng = np.random.default_rng(43)
    B, nkv, S, D = 3, 2, 7, 8
    kc = rng.integers(0, 65535, (B, nkv, S, D)).astype(np.uint16)
    vc = rng.integers(0, 65535, (B, nkv, S, D)).astype(np.uint16)
    kn = rng.standard_normal((B, nkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, nkv, D)).astype(np.float32)
    pos = np.array([0, 6, 3], np.int32)
    k2, v2 = o.kv_write(kn, vn, pos, kc, vc)
    for b in range(B):
        assert np.array_equal(k2[b, :, pos[b]], _torch_bf16_bits(kn[b]))
        assert np.array_equal(v2[b, :, pos[b]], _torch_bf16_bits(vn[b]))
    mask = np.ones((B, nkv, S), bool)
    mask[np.arange(B), :, pos] = False
    assert np.array_equal(k2[mask], kc[mask]) and np.array_equal(v2[mask], vc[mask])


def _attention_numpy(q, kc, vc, lengths, scale):
    B, nq, D = q.shape
    nkv = kc.shape[1]
    K, V = _bits_to_f64(kc), _bits_to_f64(vc)
    out = np.empty((B, nq, D))
    for b in range(B):
        for h in range(nq):
            g = h // (nq // nkv)
            L = lengths[b]
            sc = scale * (K[b, g, :L] @ q[b, h].astype(np.float64))
            p = scipy.special.softmax(sc)
            out[b, h] = p @ V[b, g, :L]
    return out


def pin_attention_bruteforce(o):
    rng = np.random.default_rng(44)
    B, nq, nkv, D, S = 2, 8, 2, 16, 12
    q = rng.standard_normal((B, nq, D)).astype(np.float32)
    kc = _torch_bf16_bits(rng.standard_normal((B, nkv, S, D)).astype(np.float32))
    vc = _torch_bf16_bits(rng.standard_normal((B, nkv, S, D)).astype(np.float32))
    lengths = np.array([5, 12], np.int32)
    scale = 1.0 / math.sqrt(D)
    _close(o.gqa_attention(q, kc, vc, lengths, scale), _attention_numpy(q, kc, vc, lengths, scale),
           1e-7, "gqa attention")


def pin_attention_closed_forms(o):
    """One position: the output is that position's v.  Equal keys: uniform
    weights, the mean of v over the positions."""
    rng = np.random.default_rng(45)
    B, nq, nkv, D, S = 1, 4, 1, 8, 6
    q = rng.standard_normal((B, nq, D)).astype(np.float32)
    kc = _torch_bf16_bits(rng.standard_normal((B, nkv, S, D)).astype(np.float32))
    vc = _torch_bf16_bits(rng.standard_normal((B, nkv, S, D)).astype(np.float32))
    out1 = o.gqa_attention(q, kc, vc, np.array([1], np.int32), 0.3)
    assert np.array_equal(out1[0], np.broadcast_to(_bits_to_f64(vc[0, 0, 0]).astype(np.float32), (nq, D)))
    kc_eq = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    outm = o.gqa_attention(q, kc_eq, vc, np.array([S], np.int32), 0.3)
    _close(outm[0], np.broadcast_to(_bits_to_f64(vc[0, 0]).mean(0), (nq, D)), 1e-7, "equal keys")


def pin_attention_gqa_mapping(o):
    """v of kv head g is the constant g: query head h must read g = h / (n_q / n_kv)."""
    B, nq, nkv, D, S = 1, 8, 4, 4, 3
    rng = np.random.default_rng(46)
    q = rng.standard_normal((B, nq, D)).astype(np.float32)
    kc = _torch_bf16_bits(rng.standard_normal((B, nkv, S, D)).astype(np.float32))
    vc = np.zeros((B, nkv, S, D), np.float32)
    for g in range(nkv):
        vc[0, g] = g
    out = o.gqa_attention(q, kc, _torch_bf16_bits(vc), np.array([S], np.int32), 0.5)
    assert np.allclose(out[0, :, 0], np.arange(nq) // (nq // nkv))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
