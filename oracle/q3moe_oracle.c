/*
 * CPU oracle for the Qwen3-MoE sparse FFN block -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain scalar C, every dot product accumulated in double.  It is the
 * definition of what the block computes, written out so a reader can check
 * it against the pages by eye: no blocking, no fusion, no reordering beyond
 * what the definitions state.  It shares no code with the HIP library and is
 * only ever loaded by the tests, by the package's smoke check and by the
 * benchmark's CPU-baseline leg.  Results are rounded to f32 only at the
 * outputs a caller sees.
 *
 * Sources (all statements restated, not quoted):
 *  - aprender issue #3714 "qwen3moe has NO working CUDA path", section
 *    "File facts": the layer shape, the f32 router [128 x 2048], expert
 *    tensors in Q4_K / Q6_K with expert e at base + e*stride, and the byte
 *    counts 884,736 / 1,290,240 per expert; gap G3: router GEMV, expert
 *    GEMVs, SwiGLU, the weighted sum of expert outputs, and softmax, top-8
 *    and renormalisation of the routing weights; "Risk to track": near-tie
 *    top-8 flips from accumulation order.
 *  - aprender PR #1228 "apply per-head Q/K RMSNorm in forward_qwen3_moe",
 *    section "The fix": RMSNorm over each head slice of q and k with one gain
 *    vector per projection, after the bias and before RoPE.
 *  - aprender issue #479 "Qwen3 GPU inference produces garbage output",
 *    "Fix Applied": head_dim is explicit (128) and differs from
 *    hidden / heads.
 *  - SharpInference issue #6 "Forward-pass divergence on Qwen3-Coder
 *    30B-A3B", closing comment: Qwen3 uses NEOX-style RoPE, pairing element
 *    i with element i + head_dim/2.
 *
 * Readings where the pages are silent:
 *  - k-quant bit layout: the GGUF k-quant super-block layout (the pages name
 *    the formats and their byte counts only).  Q4_K: fp16 d, fp16 dmin,
 *    12 bytes of packed 6-bit scales/mins for 8 sub-blocks of 32, 128 bytes
 *    of 4-bit quants; Q6_K: 128 bytes of low nibbles, 64 bytes of high
 *    2-bit pairs, 16 int8 scales, fp16 d.
 *  - matrix orientation: a matrix with N output rows and K inputs stores
 *    row r as K/256 consecutive super-blocks; rows are consecutive.
 *  - router: logits accumulated in double; experts selected on logits
 *    (softmax is monotone), ties to the lower expert index; weights are the
 *    softmax over the selected logits (= probabilities renormalised over
 *    the selected set), in double, rounded to f32.
 *  - RMSNorm: y = g * x / sqrt(mean(x^2) + eps).
 *  - RoPE frequencies: theta_i = pos * base^(-2i/D), i < D/2, all D dims
 *    rotated.
 *  - Decoder-layer pieces (the projections and the attention around the MoE
 *    block): bf16 weights of N output rows x K inputs stored row-major; no
 *    projection bias; the KV cache of a sequence holds bf16 k and v
 *    [n_kv][S_max][D]; a decode step writes the new token's k and v at its
 *    position p (round to nearest even) and attends over positions 0..p;
 *    query head h reads kv head h / (n_q / n_kv); scores are scaled by the
 *    given scale (1/sqrt(D) in the layer).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q4_K 1
#define ORC_Q6_K 2
#define ORC_QK 256

/* Threads the OpenMP loops below may use: infrastructure for timing the
 * oracle (single-threaded and on every host core); no result depends on it,
 * since every output element is computed by one thread in a fixed order. */
int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { if (n >= 1) omp_set_num_threads(n); }

/* IEEE 754 binary16 -> double, from the format definition. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int mant = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)mant, -24);                 /* subnormal or zero */
    else if (expo == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + mant), expo - 25);  /* (1 + m/1024) 2^(e-15) */
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

int orc_block_bytes(int qtype)
{
    if (qtype == ORC_Q4_K) return 144;
    if (qtype == ORC_Q6_K) return 210;
    return 0;
}

/* Q4_K super-block (144 bytes) -> 256 weights.
 * Sub-block j (32 weights) has a 6-bit scale sc_j and a 6-bit min m_j:
 *   j < 4 : sc_j = S[j] & 63,               m_j = S[j+4] & 63
 *   j >= 4: sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
 *           m_j  = (S[j+4] >> 4) | (S[j]   >> 6) << 4
 * Quant byte Q[32c + l] holds weight 64c + l in its low nibble and weight
 * 64c + 32 + l in its high nibble, so sub-block j = 2c + h for nibble h.
 * Weight value: d * sc_j * q - dmin * m_j. */
void orc_dequant_q4k_block(const uint8_t *blk, double *w)
{
    double d = orc_half_to_double(rd16(blk));
    double dmin = orc_half_to_double(rd16(blk + 2));
    const uint8_t *S = blk + 4;
    const uint8_t *Q = blk + 16;
    for (int j = 0; j < 8; j++) {
        int sc, m;
        if (j < 4) {
            sc = S[j] & 63;
            m = S[j + 4] & 63;
        } else {
            sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
            m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
        }
        int c = j / 2, h = j % 2;
        for (int l = 0; l < 32; l++) {
            int q = (Q[32 * c + l] >> (4 * h)) & 15;
            w[32 * j + l] = d * sc * q - dmin * m;
        }
    }
}

/* Q6_K super-block (210 bytes) -> 256 weights.
 * Weight i = 128n + 32r + l (n in {0,1}, r in 0..3, l in 0..31):
 *   low 4 bits: byte L[64n + 32(r&1) + l], low nibble for r < 2, high for r >= 2
 *   high 2 bits: (Hb[32n + l] >> 2r) & 3
 *   q = low | high << 4 in [0, 63]
 *   scale s[8n + 2r + l/16] (int8), value d * s * (q - 32). */
void orc_dequant_q6k_block(const uint8_t *blk, double *w)
{
    const uint8_t *L = blk;
    const uint8_t *Hb = blk + 128;
    const int8_t *s = (const int8_t *)(blk + 192);
    double d = orc_half_to_double(rd16(blk + 208));
    for (int n = 0; n < 2; n++)
        for (int r = 0; r < 4; r++)
            for (int l = 0; l < 32; l++) {
                int byte = L[64 * n + 32 * (r & 1) + l];
                int low = (r < 2) ? (byte & 15) : (byte >> 4);
                int high = (Hb[32 * n + l] >> (2 * r)) & 3;
                int q = low | (high << 4);
                w[128 * n + 32 * r + l] = d * s[8 * n + 2 * r + l / 16] * (q - 32);
            }
}

int orc_dequant_block(int qtype, const uint8_t *blk, double *w)
{
    if (qtype == ORC_Q4_K) orc_dequant_q4k_block(blk, w);
    else if (qtype == ORC_Q6_K) orc_dequant_q6k_block(blk, w);
    else return -1;
    return 0;
}

/* Row r of a rows x cols matrix: cols/256 consecutive super-blocks. */
int orc_dequant_row(int qtype, const uint8_t *mat, int64_t r, int64_t cols, double *out)
{
    int bb = orc_block_bytes(qtype);
    if (!bb || cols % ORC_QK) return -1;
    int64_t nb = cols / ORC_QK;
    const uint8_t *row = mat + r * nb * bb;
    for (int64_t b = 0; b < nb; b++)
        orc_dequant_block(qtype, row + b * bb, out + b * ORC_QK);
    return 0;
}

int orc_dequant_matrix(int qtype, const uint8_t *mat, int64_t rows, int64_t cols, double *out)
{
    for (int64_t r = 0; r < rows; r++)
        if (orc_dequant_row(qtype, mat, r, cols, out + r * cols)) return -1;
    return 0;
}

/* y[r] = sum_c W[r][c] x[c] with W dequantised row by row. */
int orc_qgemv(int qtype, const uint8_t *mat, int64_t rows, int64_t cols,
              const double *x, double *y)
{
    if (!orc_block_bytes(qtype) || cols % ORC_QK) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        double *wrow = (double *)malloc(sizeof(double) * cols);
        orc_dequant_row(qtype, mat, r, cols, wrow);
        double acc = 0.0;
        for (int64_t c = 0; c < cols; c++) acc += wrow[c] * x[c];
        y[r] = acc;
        free(wrow);
    }
    return 0;
}

/* Router GEMV: logit[t][e] = sum_h R[e][h] x[t][h], products exact in double. */
void orc_router_logits(const float *x, int64_t T, int64_t H, const float *R, int32_t E,
                       double *logits)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int32_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t h = 0; h < H; h++)
                acc += (double)R[(int64_t)e * H + h] * (double)x[t * H + h];
            logits[t * E + e] = acc;
        }
}

/* Top-k over one token's logits, largest first, ties to the lower index;
 * weights = softmax over the selected logits. */
int orc_topk_softmax(const double *logits, int64_t T, int32_t E, int32_t k,
                     int32_t *idx, double *w)
{
    if (k < 1 || k > E) return -1;
    char *taken = (char *)malloc((size_t)E);
    for (int64_t t = 0; t < T; t++) {
        const double *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; j++) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; e++)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            idx[t * k + j] = best;
        }
        double top = l[idx[t * k]];
        double den = 0.0;
        for (int32_t j = 0; j < k; j++) den += exp(l[idx[t * k + j]] - top);
        for (int32_t j = 0; j < k; j++) w[t * k + j] = exp(l[idx[t * k + j]] - top) / den;
    }
    free(taken);
    return 0;
}

int orc_route(const float *x, int64_t T, int64_t H, const float *R, int32_t E, int32_t k,
              int32_t *idx, float *w, double *logits_out)
{
    if (k < 1 || k > E) return -1;
    double *lg = logits_out ? logits_out : (double *)malloc(sizeof(double) * T * E);
    double *wd = (double *)malloc(sizeof(double) * T * k);
    orc_router_logits(x, T, H, R, E, lg);
    orc_topk_softmax(lg, T, E, k, idx, wd);
    for (int64_t i = 0; i < T * k; i++) w[i] = (float)wd[i];
    free(wd);
    if (!logits_out) free(lg);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Sparse expert FFN for T tokens (gap G3 of issue #3714):
 *   for each selected slot: g = Wg[e] x, u = Wu[e] x, h = silu(g) * u,
 *   y = Wd[e] h; out[t] = sum over slots (in slot order) of w * y.
 * Expert e's matrices start at base + e * stride.  out is double here.
 * The gate/up input is taken from xin (double [T x H]); see the two entry
 * points below. */
static int expert_ffn_on(const double *xin, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k,
                         const int32_t *idx, const float *w,
                         const uint8_t *gate, int gate_qt, int64_t gate_stride,
                         const uint8_t *up, int up_qt, int64_t up_stride,
                         const uint8_t *down, int down_qt, int64_t down_stride,
                         double *out)
{
    if (H % ORC_QK || F % ORC_QK) return -1;
    for (int64_t i = 0; i < T * k; i++)
        if (idx[i] < 0 || idx[i] >= E) return -2;
    double *g = (double *)malloc(sizeof(double) * F);
    double *u = (double *)malloc(sizeof(double) * F);
    double *h = (double *)malloc(sizeof(double) * F);
    double *y = (double *)malloc(sizeof(double) * H);
    for (int64_t t = 0; t < T; t++) {
        const double *xd = xin + t * H;
        for (int64_t c = 0; c < H; c++) out[t * H + c] = 0.0;
        for (int32_t s = 0; s < k; s++) {
            int64_t e = idx[t * k + s];
            orc_qgemv(gate_qt, gate + e * gate_stride, F, H, xd, g);
            orc_qgemv(up_qt, up + e * up_stride, F, H, xd, u);
            for (int64_t f = 0; f < F; f++) h[f] = silu(g[f]) * u[f];
            orc_qgemv(down_qt, down + e * down_stride, H, F, h, y);
            double ws = w[t * k + s];
            for (int64_t c = 0; c < H; c++) out[t * H + c] += ws * y[c];
        }
    }
    free(g); free(u); free(h); free(y);
    return 0;
}

/* The block on the f32 activations as given (each exact in double). */
int orc_expert_ffn_f64(const float *x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k,
                       const int32_t *idx, const float *w,
                       const uint8_t *gate, int gate_qt, int64_t gate_stride,
                       const uint8_t *up, int up_qt, int64_t up_stride,
                       const uint8_t *down, int down_qt, int64_t down_stride,
                       double *out)
{
    double *xd = (double *)malloc(sizeof(double) * (T * H > 0 ? T * H : 1));
    for (int64_t i = 0; i < T * H; i++) xd[i] = x[i];
    int rc = expert_ffn_on(xd, T, H, F, E, k, idx, w, gate, gate_qt, gate_stride,
                           up, up_qt, up_stride, down, down_qt, down_stride, out);
    free(xd);
    return rc;
}

/* Activations as one int8 value per element, the int8-activation route of
 * the expert GEMVs (issue #3714, G8: the expert GEMVs stay on DP4A; R1
 * receipt: the Q8_K point).  Reading: for every group of 32 consecutive
 * values of a row (one Q4_K sub-block), amax = max |x| in f32, the group
 * scale d = amax / 127 (one f32 division, rounded to nearest), and
 * p = rintf(x / d) (an f32 quotient, rounded to the nearest integer with
 * ties to even), so |p| <= 127; the GEMV then sees d * p, exact in double.
 * A group of zeros gets d = 0 and p = 0; a group holding a NaN or an
 * infinity gets d = NaN (every value of the group NaN).  Outputs: p [T x H],
 * d [T x H/32] and the values d * p [T x H]; H % 32 == 0. */
int orc_quantize_act_q8(const float *x, int64_t T, int64_t H, int8_t *p, float *d, double *xq)
{
    if (H % 32) return -1;
    for (int64_t t = 0; t < T; t++)
        for (int64_t g0 = 0; g0 < H; g0 += 32) {
            const float *v = x + t * H + g0;
            float amax = 0.0f;
            int finite = 1;
            for (int i = 0; i < 32; i++) {
                if (!isfinite(v[i])) finite = 0;
                else if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
            }
            float dg = finite ? amax / 127.0f : NAN;
            d[t * (H / 32) + g0 / 32] = dg;
            for (int i = 0; i < 32; i++) {
                float q = (finite && amax > 0.0f) ? rintf(v[i] / dg) : 0.0f;
                p[t * H + g0 + i] = (int8_t)q;
                xq[t * H + g0 + i] = finite ? (double)dg * (double)q : NAN;
            }
        }
    return 0;
}

/* The block with the gate/up activations taken in the int8 form above; the
 * down projection reads h as computed (f32 activations only enter gate/up).
 * accumulate as for orc_expert_ffn; out f32. */
int orc_expert_ffn_q8(const float *x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k,
                      const int32_t *idx, const float *w,
                      const uint8_t *gate, int gate_qt, int64_t gate_stride,
                      const uint8_t *up, int up_qt, int64_t up_stride,
                      const uint8_t *down, int down_qt, int64_t down_stride,
                      float *out, int accumulate)
{
    int64_t n = T * H > 0 ? T * H : 1;
    int8_t *p = (int8_t *)malloc((size_t)n);
    float *dg = (float *)malloc(sizeof(float) * (n / 32 + 1));
    double *xq = (double *)malloc(sizeof(double) * n);
    double *o = (double *)malloc(sizeof(double) * n);
    int rc = orc_quantize_act_q8(x, T, H, p, dg, xq);
    if (rc == 0)
        rc = expert_ffn_on(xq, T, H, F, E, k, idx, w, gate, gate_qt, gate_stride,
                           up, up_qt, up_stride, down, down_qt, down_stride, o);
    if (rc == 0)
        for (int64_t i = 0; i < T * H; i++)
            out[i] = (float)(o[i] + (accumulate != 0 ? (double)out[i] : 0.0));
    free(p); free(dg); free(xq); free(o);
    return rc;
}

/* As above with the f32 output a caller sees; accumulate = 1 adds the
 * block's output to what `out` holds (the residual add), rounding once. */
int orc_expert_ffn(const float *x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k,
                   const int32_t *idx, const float *w,
                   const uint8_t *gate, int gate_qt, int64_t gate_stride,
                   const uint8_t *up, int up_qt, int64_t up_stride,
                   const uint8_t *down, int down_qt, int64_t down_stride,
                   float *out, int accumulate)
{
    double *o = (double *)malloc(sizeof(double) * T * H);
    int rc = orc_expert_ffn_f64(x, T, H, F, E, k, idx, w, gate, gate_qt, gate_stride,
                                up, up_qt, up_stride, down, down_qt, down_stride, o);
    if (rc == 0)
        for (int64_t i = 0; i < T * H; i++)
            out[i] = (float)((accumulate ? (double)out[i] : 0.0) + o[i]);
    free(o);
    return rc;
}

/* The attention side of batched prefill (issue #3714, 0.70.3 gap list:
 * prefill runs token by token; the fix batches the projections, the RoPE
 * rows and the attention of the prompt).  T new tokens of ONE sequence sit
 * at positions pos[t] of its caches [n_kv][S_max][D]:
 *   - their k and v rows are written as the decode step writes one token's,
 *     row t into slot pos[t];
 *   - query t then attends to positions 0..pos[t] of the cache (causal), as
 *     the decode attention of one token whose length is pos[t] + 1.
 * So a prefill of T tokens equals T decode steps over the same cache. */
int orc_kv_write(const float *k_new, const float *v_new, int64_t B, int32_t n_kv, int32_t D,
                 const int32_t *pos, uint16_t *kcache, uint16_t *vcache, int64_t S_max);
int orc_gqa_attention(const float *q, int64_t B, int32_t n_q, int32_t n_kv, int32_t D,
                      const uint16_t *kcache, const uint16_t *vcache, int64_t S_max,
                      const int32_t *len, double scale, float *out);

int orc_kv_write_rows(const float *k_new, const float *v_new, int64_t T, int32_t n_kv, int32_t D,
                      const int32_t *pos, uint16_t *kcache, uint16_t *vcache, int64_t S_max)
{
    for (int64_t t = 0; t < T; t++)
        if (orc_kv_write(k_new + t * n_kv * (int64_t)D, v_new + t * n_kv * (int64_t)D, 1, n_kv, D,
                         pos + t, kcache, vcache, S_max))
            return -1;
    return 0;
}

int orc_prefill_attention(const float *q, int64_t T, int32_t n_q, int32_t n_kv, int32_t D,
                          const uint16_t *kcache, const uint16_t *vcache, int64_t S_max,
                          const int32_t *pos, double scale, float *out)
{
    for (int64_t t = 0; t < T; t++) {
        int32_t len = pos[t] + 1;
        if (orc_gqa_attention(q + t * n_q * (int64_t)D, 1, n_q, n_kv, D, kcache, vcache, S_max, &len,
                              scale, out + t * n_q * (int64_t)D))
            return -1;
    }
    return 0;
}

/* Whole-model ends of the decode step (the token embedding and the output
 * head around the 48 layers; issue #3714 "File facts": the output matrix is
 * Q6_K; the embedding rows and the head rows are k-quant rows of H inputs).
 * Embedding: out[t] = row tokens[t] of the table [V x H], dequantised and
 * rounded once to f32; a token outside [0, V) gives a row of NaN. */
int orc_embed(const int32_t *tokens, int64_t T, const uint8_t *table, int qtype, int64_t V,
              int64_t H, float *out)
{
    if (!orc_block_bytes(qtype) || H % ORC_QK) return -1;
    double *row = (double *)malloc(sizeof(double) * H);
    for (int64_t t = 0; t < T; t++) {
        int64_t v = tokens[t];
        if (v < 0 || v >= V) {
            for (int64_t i = 0; i < H; i++) out[t * H + i] = NAN;
            continue;
        }
        orc_dequant_row(qtype, table, v, H, row);
        for (int64_t i = 0; i < H; i++) out[t * H + i] = (float)row[i];
    }
    free(row);
    return 0;
}

/* Output head: logits[t][v] = sum_h W[v][h] x[t][h] for the V rows of W
 * (the k-quant GEMV above over the vocabulary), each logit rounded once to
 * f32. */
int orc_output_head(const float *x, int64_t T, const uint8_t *W, int qtype, int64_t V, int64_t H,
                    float *logits)
{
    if (!orc_block_bytes(qtype) || H % ORC_QK) return -1;
    double *xd = (double *)malloc(sizeof(double) * H);
    double *y = (double *)malloc(sizeof(double) * (V > 0 ? V : 1));
    for (int64_t t = 0; t < T; t++) {
        for (int64_t i = 0; i < H; i++) xd[i] = x[t * H + i];
        orc_qgemv(qtype, W, V, H, xd, y);
        for (int64_t v = 0; v < V; v++) logits[t * V + v] = (float)y[v];
    }
    free(xd); free(y);
    return 0;
}

/* Token -> expert grouping of the routed (token, slot) pairs (the pages'
 * plan groups tokens by expert for batched prefill: aprender issue #3714,
 * gap list).  Pair p = t*k + slot with expert idx[p].  For every expert e in
 * order, the pairs routed to it in increasing p: counts[e] of them starting
 * at offsets[e]; offsets[E] is the number of grouped pairs.  A pair whose
 * index is outside [0, E) is not grouped. */
int orc_group_by_expert(const int32_t *idx, int64_t T, int32_t k, int32_t E,
                        int32_t *counts, int32_t *offsets, int32_t *pairs)
{
    int64_t n = T * k, pos = 0;
    for (int32_t e = 0; e < E; e++) {
        offsets[e] = (int32_t)pos;
        for (int64_t p = 0; p < n; p++)
            if (idx[p] == e) pairs[pos++] = (int32_t)p;
        counts[e] = (int32_t)(pos - offsets[e]);
    }
    offsets[E] = (int32_t)pos;
    return 0;
}

/* IEEE 754 bfloat16 (the top 16 bits of a binary32) -> double, and binary32
 * -> bfloat16 rounding to nearest, ties to even, both from the format. */
double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

uint16_t orc_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x40);                 /* NaN stays NaN */
    uint32_t rest = u & 0xffffu, keep = u >> 16;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;
    return (uint16_t)keep;
}

/* y[t][n] = sum_k W[n][k] x[t][k] with W bf16 [N][K] (the attention
 * projections of the decoder layer), in double, rounded to f32; with
 * accumulate the product is added to y (the residual add after O). */
int orc_bf16_gemv(const uint16_t *W, int64_t N, int64_t K, const float *x, int64_t T,
                  float *y, int accumulate)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t t = 0; t < T; t++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++)
                acc += orc_bf16_to_double(W[n * K + k]) * (double)x[t * K + k];
            y[t * N + n] = (float)((accumulate ? (double)y[t * N + n] : 0.0) + acc);
        }
    return 0;
}

/* Write the new token's k and v (f32 [B][n_kv][D]) into each sequence's
 * bf16 cache [B][n_kv][S_max][D] at position pos[b]. */
int orc_kv_write(const float *k_new, const float *v_new, int64_t B, int32_t n_kv, int32_t D,
                 const int32_t *pos, uint16_t *kcache, uint16_t *vcache, int64_t S_max)
{
    for (int64_t b = 0; b < B; b++) {
        if (pos[b] < 0 || pos[b] >= S_max) return -1;
        for (int32_t g = 0; g < n_kv; g++)
            for (int32_t i = 0; i < D; i++) {
                int64_t src = (b * n_kv + g) * (int64_t)D + i;
                int64_t dst = ((b * n_kv + g) * S_max + pos[b]) * (int64_t)D + i;
                kcache[dst] = orc_float_to_bf16(k_new[src]);
                vcache[dst] = orc_float_to_bf16(v_new[src]);
            }
    }
    return 0;
}

/* Grouped-query decode attention: for sequence b and query head h (kv head
 * g = h / (n_q / n_kv)), over positions j < len[b]:
 *   s_j = scale * q . k_j,  p = softmax(s),  out = sum_j p_j v_j,
 * all in double (max subtracted), rounded to f32. */
int orc_gqa_attention(const float *q, int64_t B, int32_t n_q, int32_t n_kv, int32_t D,
                      const uint16_t *kcache, const uint16_t *vcache, int64_t S_max,
                      const int32_t *len, double scale, float *out)
{
    if (n_q % n_kv) return -1;
    int32_t group = n_q / n_kv;
    for (int64_t b = 0; b < B; b++)
        if (len[b] < 1 || len[b] > S_max) return -1;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; b++)
        for (int32_t h = 0; h < n_q; h++) {
            int32_t g = h / group;
            int64_t L = len[b];
            const float *qh = q + (b * n_q + h) * (int64_t)D;
            const uint16_t *K = kcache + (b * n_kv + g) * S_max * (int64_t)D;
            const uint16_t *V = vcache + (b * n_kv + g) * S_max * (int64_t)D;
            double *sc = (double *)malloc(sizeof(double) * L);
            double mx = -INFINITY;
            for (int64_t j = 0; j < L; j++) {
                double d = 0.0;
                for (int32_t i = 0; i < D; i++) d += (double)qh[i] * orc_bf16_to_double(K[j * D + i]);
                sc[j] = scale * d;
                if (sc[j] > mx) mx = sc[j];
            }
            double den = 0.0;
            for (int64_t j = 0; j < L; j++) { sc[j] = exp(sc[j] - mx); den += sc[j]; }
            for (int32_t i = 0; i < D; i++) {
                double acc = 0.0;
                for (int64_t j = 0; j < L; j++) acc += sc[j] * orc_bf16_to_double(V[j * D + i]);
                out[(b * n_q + h) * (int64_t)D + i] = (float)(acc / den);
            }
            free(sc);
        }
    return 0;
}

/* RMSNorm of one vector: y = g * x / sqrt(mean(x^2) + eps). */
static void rmsnorm_vec(const double *x, int64_t n, const float *g, double eps, double *y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++) y[i] = (double)g[i] * x[i] * inv;
}

int orc_rmsnorm(const float *x, int64_t T, int64_t n, const float *gain, float eps, float *out)
{
    double *xv = (double *)malloc(sizeof(double) * n);
    double *yv = (double *)malloc(sizeof(double) * n);
    for (int64_t t = 0; t < T; t++) {
        for (int64_t i = 0; i < n; i++) xv[i] = x[t * n + i];
        rmsnorm_vec(xv, n, gain, (double)eps, yv);
        for (int64_t i = 0; i < n; i++) out[t * n + i] = (float)yv[i];
    }
    free(xv); free(yv);
    return 0;
}

/* NEOX rotation of one head in place: element i pairs with i + D/2,
 * angle pos * base^(-2i/D). */
static void rope_neox_head(double *v, int32_t D, double pos, double base)
{
    int32_t half = D / 2;
    for (int32_t i = 0; i < half; i++) {
        double theta = pos * pow(base, -2.0 * i / (double)D);
        double a = v[i], b = v[i + half];
        v[i] = a * cos(theta) - b * sin(theta);
        v[i + half] = a * sin(theta) + b * cos(theta);
    }
}

/* RoPE alone on x [T][n_heads][D] (for the rotation's own pins). */
int orc_rope_neox(float *x, int64_t T, int32_t n_heads, int32_t D, const int32_t *pos,
                  double base)
{
    if (D % 2) return -1;
    double *v = (double *)malloc(sizeof(double) * D);
    for (int64_t t = 0; t < T; t++)
        for (int32_t hd = 0; hd < n_heads; hd++) {
            float *p = x + (t * n_heads + hd) * (int64_t)D;
            for (int32_t i = 0; i < D; i++) v[i] = p[i];
            rope_neox_head(v, D, (double)pos[t], base);
            for (int32_t i = 0; i < D; i++) p[i] = (float)v[i];
        }
    free(v);
    return 0;
}

/* Attention prologue (PR #1228 "The fix"; issue #6 closing comment): for every
 * head slice of q [T][n_q][D] and k [T][n_kv][D], RMSNorm with the shared gain
 * (q_norm or k_norm, length D), then NEOX RoPE at positions[t].  In place. */
int orc_attn_prologue(float *q, float *k, int64_t T, int32_t n_q, int32_t n_kv, int32_t D,
                      const float *q_norm, const float *k_norm, const int32_t *pos,
                      float eps, float rope_base)
{
    if (D % 2) return -1;
    double *v = (double *)malloc(sizeof(double) * D);
    double *y = (double *)malloc(sizeof(double) * D);
    for (int64_t t = 0; t < T; t++) {
        for (int pass = 0; pass < 2; pass++) {
            float *base = pass == 0 ? q + t * n_q * (int64_t)D : k + t * n_kv * (int64_t)D;
            int32_t nh = pass == 0 ? n_q : n_kv;
            const float *g = pass == 0 ? q_norm : k_norm;
            for (int32_t hd = 0; hd < nh; hd++) {
                float *p = base + hd * (int64_t)D;
                for (int32_t i = 0; i < D; i++) v[i] = p[i];
                rmsnorm_vec(v, D, g, (double)eps, y);
                rope_neox_head(y, D, (double)pos[t], (double)rope_base);
                for (int32_t i = 0; i < D; i++) p[i] = (float)y[i];
            }
        }
    }
    free(v); free(y);
    return 0;
}
