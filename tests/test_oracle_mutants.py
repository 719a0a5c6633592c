"""Plant plausible mistakes in copies of the oracle and show the pins catch
every one (the oracle's pins "bite").  Each mutant is a one-site textual
edit of oracle/q3moe_oracle.c compiled to a private library; the real
oracle source is never modified."""
import re
import tempfile
from pathlib import Path

import pytest

import oracle
import pins

SRC = Path(oracle.__file__).resolve().parent / "q3moe_oracle.c"

# (name, exact source text, replacement)
MUTANTS = [
    ("q4k_min_sign", "w[32 * j + l] = d * sc * q - dmin * m;", "w[32 * j + l] = d * sc * q + dmin * m;"),
    ("q4k_nibble_swap", "(Q[32 * c + l] >> (4 * h)) & 15", "(Q[32 * c + l] >> (4 * (1 - h))) & 15"),
    ("q4k_scale_high_bits_dropped", "sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);", "sc = (S[j + 4] & 15);"),
    ("q4k_min_high_bits_wrong_byte", "m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);", "m = (S[j + 4] >> 4) | ((S[j - 4] >> 6) << 4);"),
    ("q4k_low_min_from_scale_byte", "m = S[j + 4] & 63;", "m = S[j] & 63;"),
    ("q4k_dmin_as_d", "double dmin = orc_half_to_double(rd16(blk + 2));", "double dmin = orc_half_to_double(rd16(blk));"),
    ("q6k_nibble_by_parity", "int low = (r < 2) ? (byte & 15) : (byte >> 4);", "int low = (r & 1) ? (byte >> 4) : (byte & 15);"),
    ("q6k_high_bits_reversed", "(Hb[32 * n + l] >> (2 * r)) & 3", "(Hb[32 * n + l] >> (2 * (3 - r))) & 3"),
    ("q6k_scale_index", "s[8 * n + 2 * r + l / 16]", "s[8 * n + r + l / 16]"),
    ("q6k_offset", "(q - 32);", "(q - 31);"),
    ("q6k_low_byte_index", "L[64 * n + 32 * (r & 1) + l]", "L[64 * n + 16 * (r & 1) + l]"),
    ("half_exponent_bias", "expo - 25", "expo - 24"),
    ("half_subnormal", "ldexp((double)mant, -24)", "ldexp((double)mant, -25)"),
    ("row_stride", "const uint8_t *row = mat + r * nb * bb;", "const uint8_t *row = mat + r * bb;"),
    ("gemv_transposed_x", "acc += wrow[c] * x[c];", "acc += wrow[c] * x[(c + 1) % cols];"),
    ("router_transposed", "(double)R[(int64_t)e * H + h]", "(double)R[(int64_t)h * E + e]"),
    ("tie_to_higher_index", "(best < 0 || l[e] > l[best])", "(best < 0 || l[e] >= l[best])"),
    ("uniform_weights", "w[t * k + j] = exp(l[idx[t * k + j]] - top) / den;", "w[t * k + j] = 1.0 / k;"),
    ("weights_not_renormalised", "den += exp(l[idx[t * k + j]] - top);", "den += 0.5 * exp(l[idx[t * k + j]] - top);"),
    ("wrong_expert", "int64_t e = idx[t * k + s];", "int64_t e = (idx[t * k + s] + 1) % E;"),
    ("drop_top_expert", "for (int32_t s = 0; s < k; s++) {", "for (int32_t s = 1; s < k; s++) {"),
    ("silu_sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    ("swiglu_swapped", "h[f] = silu(g[f]) * u[f];", "h[f] = g[f] * silu(u[f]);"),
    ("down_stride", "down + e * down_stride", "down + e * gate_stride"),
    ("accumulate_ignored", "(accumulate ? (double)out[i] : 0.0)", "0.0"),
    ("rms_eps_outside", "sqrt(ss / (double)n + eps)", "(sqrt(ss / (double)n) + eps)"),
    ("rms_mean_n_minus_1", "ss / (double)n + eps", "ss / (double)(n - 1) + eps"),
    ("rms_gain_dropped", "y[i] = (double)g[i] * x[i] * inv;", "y[i] = x[i] * inv;"),
    ("rope_sign", "v[i] = a * cos(theta) - b * sin(theta);", "v[i] = a * cos(theta) + b * sin(theta);"),
    ("rope_frequency", "pow(base, -2.0 * i / (double)D)", "pow(base, -1.0 * i / (double)D)"),
    ("rope_pair_adjacent", "int32_t half = D / 2;", "int32_t half = 1;"),
    ("prologue_rope_before_norm",
     "rmsnorm_vec(v, D, g, (double)eps, y);\n                rope_neox_head(y, D, (double)pos[t], (double)rope_base);",
     "rope_neox_head(v, D, (double)pos[t], (double)rope_base);\n                rmsnorm_vec(v, D, g, (double)eps, y);"),
    ("prologue_k_gain_for_q", "const float *g = pass == 0 ? q_norm : k_norm;", "const float *g = k_norm;"),
    ("group_offsets_off_by_one", "offsets[e] = (int32_t)pos;", "offsets[e] = (int32_t)(pos + 1);"),
    ("group_keeps_last_pair_out", "for (int64_t p = 0; p < n; p++)\n            if (idx[p] == e)", "for (int64_t p = 0; p + 1 < n; p++)\n            if (idx[p] == e)"),
    ("group_token_not_pair", "if (idx[p] == e) pairs[pos++] = (int32_t)p;", "if (idx[p] == e) pairs[pos++] = (int32_t)(p / k);"),
    ("group_reverse_order", "for (int64_t p = 0; p < n; p++)\n            if (idx[p] == e)", "for (int64_t p = n - 1; p >= 0; p--)\n            if (idx[p] == e)"),
    ("bf16_round_truncates", "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;", "if (rest > 0x8000u) keep += 1;"),
    ("bf16_widen_wrong_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("gemv_column_major", "orc_bf16_to_double(W[n * K + k])", "orc_bf16_to_double(W[k * N + n])"),
    ("gemv_accumulate_ignored", "(accumulate ? (double)y[t * N + n] : 0.0)", "0.0"),
    ("kv_write_wrong_slot", "int64_t dst = ((b * n_kv + g) * S_max + pos[b]) * (int64_t)D + i;", "int64_t dst = ((b * n_kv + g) * S_max + pos[b] - (pos[b] > 0)) * (int64_t)D + i;"),
    ("gqa_interleaved_heads", "int32_t g = h / group;", "int32_t g = h % n_kv;"),
    ("attention_scale_dropped", "sc[j] = scale * d;", "sc[j] = d;"),
    ("attention_one_past_length", "int64_t L = len[b];", "int64_t L = len[b] < S_max ? len[b] + 1 : len[b];"),
    ("attention_k_as_v", "acc += sc[j] * orc_bf16_to_double(V[j * D + i]);", "acc += sc[j] * orc_bf16_to_double(K[j * D + i]);"),
    ("prefill_window_one_short", "int32_t len = pos[t] + 1;", "int32_t len = pos[t] > 0 ? pos[t] : 1;"),
    ("prefill_rows_into_one_slot", "pos + t, kcache, vcache, S_max))", "pos, kcache, vcache, S_max))"),
    ("embed_row_off_by_one", "orc_dequant_row(qtype, table, v, H, row);", "orc_dequant_row(qtype, table, v > 0 ? v - 1 : v, H, row);"),
    ("embed_out_of_range_clamped", "for (int64_t i = 0; i < H; i++) out[t * H + i] = NAN;\n            continue;", "v = v < 0 ? 0 : V - 1;"),
    ("head_logit_transposed", "for (int64_t v = 0; v < V; v++) logits[t * V + v] = (float)y[v];", "for (int64_t v = 0; v < V; v++) logits[t * V + v] = (float)y[V - 1 - v];"),
    ("q8_round_half_away", "rintf(v[i] / dg)", "roundf(v[i] / dg)"),
    ("q8_scale_128", "amax / 127.0f", "amax / 128.0f"),
    ("q8_output_scaled", "expert_ffn_on(xq, T, H, F, E, k, idx, w, gate, gate_qt, gate_stride,\n                           up, up_qt, up_stride, down, down_qt, down_stride, o);",
     "expert_ffn_on(xq, T, H, F, E, k, idx, w, gate, gate_qt, gate_stride,\n                           up, up_qt, up_stride, down, down_qt, down_stride, o);\n    for (int64_t i = 0; i < T * H; i++) o[i] = (double)(float)o[i] * 1.0001;"),
    ("prologue_head_dim_halved", "rmsnorm_vec(v, D, g, (double)eps, y);", "rmsnorm_vec(v, D / 2, g, (double)eps, y); rmsnorm_vec(v + D / 2, D / 2, g, (double)eps, y + D / 2);"),
]


def _interleaved_rope(src: str) -> str:
    """Whole-function mutant: LLaMA-style interleaved pairs (2i, 2i+1)."""
    start = src.index("static void rope_neox_head")
    end = src.index("}\n}", start) + 3
    body = src[start:end]
    body = body.replace("double a = v[i], b = v[i + half];", "double a = v[2 * i], b = v[2 * i + 1];")
    body = body.replace("v[i] = a * cos", "v[2 * i] = a * cos").replace("v[i + half] = a * sin", "v[2 * i + 1] = a * sin")
    return src[:start] + body + src[end:]


@pytest.fixture(scope="module")
def source():
    return SRC.read_text()


def _caught(lib_path, want: str | None = None) -> list[str]:
    """Names of the pins the library fails; stops at the first one (or at
    ``want`` when given)."""
    o = oracle.Oracle(oracle.load(lib_path))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as exc:       # a crash inside a pin also counts as caught
            failed.append(f"{pin.__name__}:{type(exc).__name__}")
        if failed and (want is None or want in failed):
            break
    return failed


def _build_mutant(text: str, tmp: Path, name: str) -> Path:
    src = tmp / f"{name}.c"
    src.write_text(text)
    return oracle.build(src, tmp / f"lib_{name}.so")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new, tmp_path):
    assert source.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_mutant(source.replace(old, new), tmp_path, name)
    assert _caught(lib), f"mutant {name} passed every pin"


def test_interleaved_rope_is_caught(source, tmp_path):
    text = _interleaved_rope(source)
    assert text != source
    lib = _build_mutant(text, tmp_path, "interleaved")
    assert "pin_rope_neox_pairs" in _caught(lib, want="pin_rope_neox_pairs")
