/*
 * q3moe -- the Qwen3-MoE sparse FFN block for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Unless a comment says otherwise every tensor pointer is a DEVICE
 * pointer (HBM) owned by the caller, and every `stream` argument is a
 * hipStream_t handle passed as void* (NULL selects the null stream).
 *
 * Common contract of every entry point:
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    failed check returns a status code and enqueues nothing.
 *  - On success the call only enqueues kernels on `stream` and returns; it
 *    never synchronises with the host and never allocates memory.  Buffers
 *    must stay alive until the stream has passed the work.
 *  - The library keeps no pointer after a call returns and holds no mutable
 *    global state; concurrent calls on different streams with disjoint
 *    buffers are safe, with one exception: two calls that each run as the
 *    persistent kernel (q3moe_persistent_path returns 1) must not overlap in
 *    time on one device.  That kernel's workgroups wait on each other, so
 *    all of them must be resident at once; two such launches could each
 *    hold part of the compute units and wait for workgroups that cannot
 *    start.  Their waits are bounded, so neither hangs, but the output is
 *    then invalid and the status word of the workspace says so.  Issue
 *    such calls on one stream (or otherwise ordered).
 *  - T = 0 (no tokens) is valid and enqueues nothing.
 *  - Q3MOE_E_HIP reports a failed kernel launch (hipGetLastError).
 *
 * The block (aprender issue #3714 "qwen3moe has NO working CUDA path",
 * "File facts" and gap G3): an f32 router GEMV over E experts, softmax,
 * top-k with renormalised weights, per selected expert the gate and up
 * GEMVs, SwiGLU and the down GEMV on k-quant weights read in place at
 * base + e*stride, and the routing-weighted sum of the expert outputs.
 * The optional attention prologue applies per-head Q/K RMSNorm (aprender
 * PR #1228, "The fix") and NEOX RoPE (SharpInference issue #6, closing
 * comment) with an explicit head_dim (aprender issue #479, "Fix Applied").
 */
#ifndef Q3MOE_H
#define Q3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t q3moe_status;
enum {
    Q3MOE_OK = 0,
    Q3MOE_E_NULL = 1,       /* a required pointer is NULL                       */
    Q3MOE_E_SHAPE = 2,      /* a size is out of range or inconsistent           */
    Q3MOE_E_QTYPE = 3,      /* unknown or unsupported quantisation type         */
    Q3MOE_E_ALIGN = 4,      /* a pointer or stride is not 16-byte aligned       */
    Q3MOE_E_WORKSPACE = 5,  /* workspace NULL or smaller than the size query    */
    Q3MOE_E_HIP = 6,        /* the HIP runtime rejected a launch                */
    Q3MOE_E_ALIAS = 7       /* an output overlaps an input it must not overlap  */
};

/* k-quant super-block formats (256 weights each).  The GGUF k-quant layout:
 *  Q3MOE_Q4_K, 144 bytes: fp16 d, fp16 dmin, 12 bytes of packed 6-bit
 *    scales and mins for 8 sub-blocks of 32, 128 bytes of 4-bit quants;
 *    weight = d*scale*q - dmin*min.
 *  Q3MOE_Q6_K, 210 bytes: 128 bytes of low nibbles, 64 bytes of 2-bit high
 *    parts, 16 int8 scales (one per 16 weights), fp16 d;
 *    weight = d*scale*(q - 32). */
enum { Q3MOE_Q4_K = 1, Q3MOE_Q6_K = 2 };

/* One 3-D expert tensor: E matrices of `rows` x `cols` weights.  Matrix e
 * starts at (const char*)base + e*expert_stride_bytes; inside it, row r is
 * cols/256 consecutive super-blocks (the super-blocks run along the
 * reduction dimension).  base must be 16-byte aligned; the stride must be a
 * multiple of 16 and at least rows*(cols/256)*block_bytes.  The tensor is
 * read in place (no repacking), as the per-expert pointer base + e*stride
 * in "File facts" of issue #3714 allows. */
typedef struct q3moe_experts {
    const void *base;
    int32_t qtype;
    int32_t reserved;               /* must be 0 */
    int64_t expert_stride_bytes;
} q3moe_experts;

/* Human-readable name of a status code (static storage). */
const char *q3moe_status_string(q3moe_status s);

/* Bytes per 256-weight super-block: 144 (Q4_K), 210 (Q6_K), 0 otherwise. */
int32_t q3moe_qtype_block_bytes(int32_t qtype);

/* rows*(cols/256)*block_bytes, or -1 when cols % 256 != 0 or qtype unknown.
 * For the Qwen3-30B-A3B layer this is 884,736 (Q4_K 768x2048) and
 * 1,290,240 (Q6_K 2048x768), the per-expert sizes of "File facts". */
int64_t q3moe_expert_matrix_bytes(int32_t qtype, int64_t rows, int64_t cols);

/* ---------------------------------------------------------------- route --
 * Router GEMV, softmax, top-k and renormalisation (issue #3714, gap G3; the
 * on-device form planned as kernel K1 under G8).
 *   hidden   [T x H] f32, row-major, 16-byte aligned, H % 4 == 0
 *   router   [E x H] f32, row-major (the ffn_gate_inp matrix), 16-byte aligned
 *   topk_idx [T x k] int32 out: the k experts with the largest logits, in
 *            descending logit order, equal logits broken by the lower index
 *   topk_w   [T x k] f32 out: softmax over the k selected logits (equal to
 *            the full softmax renormalised over the selected set); sums to 1
 * Logits are accumulated in double, which keeps the top-k choice stable
 * against summation order (the near-tie risk named in "Risk to track").
 * Limits: 1 <= k <= 32, k <= E <= 1024, 1 <= H.
 * workspace: device memory of at least q3moe_route_workspace_bytes(T, E)
 * bytes, 16-byte aligned.  Its first 4 KiB hold completion counters and
 * must be zero before the first call that uses the workspace (e.g. one
 * hipMemset after allocation); every call leaves them zero again, so the
 * workspace can be reused by later calls of any size on the same stream.
 * Calls that overlap in time (different streams) need different workspaces.
 * For T <= 8 the whole route is one kernel: each workgroup computes one
 * expert's logits and the last one to finish selects the top-k (nothing
 * waits on another workgroup).
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_HIP. */
size_t q3moe_route_workspace_bytes(int64_t T, int32_t E);
q3moe_status q3moe_route(const float *hidden, int64_t T, int64_t H,
                         const float *router, int32_t E, int32_t top_k,
                         int32_t *topk_idx, float *topk_w,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------ token -> expert grouping --
 * The routed (token, slot) pairs grouped by expert, for the batched expert
 * FFN (the pages' plan groups prefill tokens by expert: issue #3714, gap
 * list).  Pair p = t*top_k + slot has expert topk_idx[p].
 *   counts  [E] int32 out: pairs routed to each expert
 *   offsets [E+1] int32 out: exclusive prefix of counts; offsets[E] is the
 *           number of grouped pairs
 *   pairs   [T*top_k] int32 out: pair indices ordered by (expert, pair),
 *           i.e. stable in token and slot order; entries from offsets[E]
 *           on are left untouched
 * A pair whose index is outside [0, E) is not grouped.  Runs as one
 * workgroup; unlike the other entry points it also launches for T = 0
 * (writing zero counts and offsets).
 * Limits: 1 <= top_k <= 32, 1 <= E <= 1024, T*top_k < 2^31.
 * Errors: E_NULL, E_SHAPE, E_ALIAS (an output overlaps topk_idx or another
 * output), E_HIP. */
q3moe_status q3moe_group_by_expert(const int32_t *topk_idx, int64_t T, int32_t top_k,
                                   int32_t E, int32_t *counts, int32_t *offsets,
                                   int32_t *pairs, void *stream);

/* ----------------------------------------------------------- expert FFN --
 * For each token t and slot s with e = topk_idx[t*k+s] (issue #3714, gap G3;
 * the device-side expert-pointer gather and weighted accumulate planned as
 * K3 and K2 under G8):
 *   g = Wg[e] x_t, u = Wu[e] x_t         (F values each; gate/up are F x H)
 *   h = silu(g) * u, silu(z) = z / (1 + exp(-z))
 *   y = Wd[e] h                          (H values; down is H x F)
 *   out[t] = [out[t] +] sum over s of topk_w[t*k+s] * y
 *            (summed in a fixed order, so results are deterministic)
 *   hidden   [T x H] f32, 16-byte aligned (the FFN input)
 *   topk_idx [T x k] int32, each in [0, E); an index outside that range
 *            makes that slot contribute zero (caller error, not reported)
 *   topk_w   [T x k] f32
 *   gate, up Q4_K expert tensors of F x H matrices
 *   down     Q4_K or Q6_K expert tensor of H x F matrices (the qtype may
 *            differ per layer, as ffn_down_exps does in the 30B-A3B files)
 *   out      [T x H] f32, 16-byte aligned, must not overlap hidden.
 *            accumulate = 0: out = block output; 1: out += block output
 *            (the residual add fused).
 * Limits: H % 256 == 0, F % 256 == 0, 256 <= H <= 4096, 256 <= F <= 1536,
 * 1 <= k <= 32, k <= E.
 * workspace: at least q3moe_expert_ffn_workspace_bytes(T, H, F, E, k)
 * bytes, 16-byte aligned, all of it zero before the first call that uses
 * it (e.g. one hipMemset after allocation).  Its first 8 KiB hold
 * synchronisation words (counters that every call leaves at zero again, and
 * a call counter); the rest holds the intermediate h, which the batch-1..4
 * kernel publishes as 64-bit words tagged with the call counter.  A
 * workspace can be reused by later calls of any size on the same stream.
 * Calls that overlap in time (different streams) need different workspaces.
 * For small T the library runs the whole FFN as one persistent kernel with
 * at most one workgroup per compute unit, whose down-projection threads wait
 * for h words carrying the current tag; each wait is bounded.  Its
 * workgroups must all be resident at once: the grid is sized from the
 * compute-unit count and the occupancy calculator, and a device that cannot
 * hold one workgroup per unit gets the separate kernels instead; overlapping
 * persistent calls are excluded by the common contract above.  The int32 at
 * byte offset q3moe_expert_ffn_status_offset(...) of the workspace is a
 * sticky status word: it stays 0 unless a bounded wait ran out, in which
 * case that call's output is invalid.
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_WORKSPACE, E_ALIAS, E_HIP. */
size_t q3moe_expert_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F,
                                        int32_t E, int32_t top_k);
size_t q3moe_expert_ffn_status_offset(int64_t T, int64_t H, int64_t F,
                                      int32_t E, int32_t top_k);
q3moe_status q3moe_expert_ffn(const float *hidden, int64_t T, int64_t H, int64_t F,
                              int32_t E, int32_t top_k,
                              const int32_t *topk_idx, const float *topk_w,
                              q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                              float *out, int32_t accumulate,
                              void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------ MoE block --
 * The whole sparse MoE block of the tokens in one call: q3moe_route on
 * (hidden, router), then q3moe_expert_ffn with that routing (issue #3714,
 * gap G3 and the fused decode plan K1-K3 under G8).  topk_idx, topk_w and out
 * receive what the two calls produce, except that the router logits are
 * summed in another order (still in double, so the selection differs only
 * at logits equal to about 1e-16 relative).  Arguments as for the two calls;
 * topk_idx and topk_w are outputs here and must not overlap hidden, out or
 * each other.  Router input is the FFN input (hidden).
 * For T <= 4, H = 2048, top_k <= 8 and E <= 256 this is one persistent
 * kernel: each workgroup computes a slice of the router dot products and
 * publishes it as tagged words, every workgroup selects the top-k from all
 * slices and goes on into the expert FFN.  Other shapes run the route and
 * expert-FFN kernels back to back.
 * workspace: at least q3moe_moe_ffn_workspace_bytes(T, H, F, E, k) bytes,
 * 16-byte aligned, all of it zero before the first call that uses it; it can
 * be reused by later calls of any size on the same stream.  Its first bytes
 * are an expert-FFN workspace, so the status word is at
 * q3moe_expert_ffn_status_offset(...) (bit 2 set: the in-kernel routing
 * waited in vain).
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_WORKSPACE, E_ALIAS, E_HIP. */
size_t q3moe_moe_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E,
                                     int32_t top_k);
q3moe_status q3moe_moe_ffn(const float *hidden, int64_t T, int64_t H, int64_t F,
                           int32_t E, int32_t top_k, const float *router,
                           q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                           int32_t *topk_idx, float *topk_w, float *out, int32_t accumulate,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------- MoE block, int8 activations --
 * q3moe_moe_ffn with the gate/up GEMVs on int8 activations, the DP4A-style
 * route the pages keep for the expert GEMVs (issue #3714, gap G8: an
 * alternative Q4_K GEMV measured about 4x slower than the DP4A one) and
 * judge against FP32 activations (R1 receipt, "The Q8_K point").  Routing
 * is the f32/double routing of q3moe_moe_ffn (identical indices and
 * weights); the down projection reads h in f32.  For every group of 32
 * consecutive input values (one Q4_K sub-block) d = max|x| / 127 (f32) and
 * p = rint(x / d) (f32 quotient, ties to even): the gate and up GEMVs see
 * d * p, each sub-block's dot product an exact int32 sum of 4-bit quant x
 * int8 products (v_dot4), one piece per value instead of the three of the
 * f32 block.  Error budget against the f32 block: each input value moves by
 * at most d/2 (at most 0.4 % of its group's largest value), which gives
 * about 0.5-1 % relative L2 on the block output over a batch of tokens
 * (bound held by the tests: 2e-2 over a batch, 0.25 for a single token,
 * whose output can nearly cancel); against a reference that quantises the
 * same way, the f32 rounding of the rest only (1e-4).
 * Available for the one-kernel shapes of q3moe_moe_ffn only
 * (q3moe_persistent_path(..., 1) == 1 on this device); other shapes return
 * Q3MOE_E_SHAPE.  Arguments, workspace and errors as for q3moe_moe_ffn. */
q3moe_status q3moe_moe_ffn_q8(const float *hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                              int32_t top_k, const float *router,
                              q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                              int32_t *topk_idx, float *topk_w, float *out, int32_t accumulate,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Which form q3moe_moe_ffn / q3moe_moe_ffn_prenorm (with_route = 1) or
 * q3moe_expert_ffn (with_route = 0) takes for this shape on the CURRENT
 * device: 1 = the one persistent kernel (its workgroups wait on each other
 * and must all be resident at once; see the common contract), 0 = separate
 * kernels that never wait on each other (also for T = 0), -1 = arguments
 * the calls would reject (down_qtype is Q3MOE_Q4_K or Q3MOE_Q6_K).  The
 * answer depends on the device's compute-unit count and on how many
 * workgroups of the kernel one unit holds (registers, waves, LDS). */
int32_t q3moe_persistent_path(int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k,
                              int32_t down_qtype, int32_t with_route);

/* ------------------------------------------------------ MoE block, no-alloc --
 * For callers that cannot allocate device memory or hold a workspace of their
 * own (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): exactly q3moe_moe_ffn, with the workspace taken from a
 * file-scope device array of Q3MOE_NOALLOC_SCRATCH_BYTES (4 MiB) inside the
 * library instead of an argument.  Each GPU the library runs on holds its own
 * copy of the array until the process ends; the call allocates nothing (no
 * hipMalloc, no allocating library routine).  The caller still passes every
 * input and output.
 *  - Sizes: a shape whose q3moe_moe_ffn_workspace_bytes(T, H, F, E, k)
 *    exceeds Q3MOE_NOALLOC_SCRATCH_BYTES returns Q3MOE_E_WORKSPACE and
 *    enqueues nothing (at the 30B-A3B layer shape that admits up to 31 tokens).
 *  - State: every call on a device shares that device's array and leaves its
 *    counters at zero; the first calls on a device also enqueue a zero fill
 *    of the array ahead of the block (until one call made outside graph
 *    capture has done so; a graph captured before then replays the fill).
 *  - Calls that overlap in time on one device (different streams, threads or
 *    graphs) race on the array and give wrong results: order them.
 * Errors: those of q3moe_moe_ffn, and E_HIP if the array's device address
 * cannot be obtained. */
#define Q3MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
q3moe_status q3moe_moe_ffn_noalloc(const float *hidden, int64_t T, int64_t H, int64_t F,
                                   int32_t E, int32_t top_k, const float *router,
                                   q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                                   int32_t *topk_idx, float *topk_w, float *out,
                                   int32_t accumulate, void *stream);

/* ------------------------------------------------- MoE block after RMSNorm --
 * The MoE block of a pre-norm decoder layer: its input is the token's hidden
 * row x normalised as
 *   xn = norm_gain * x / sqrt(mean(x^2) + eps)
 * (the post-attention RMSNorm that feeds the sparse MoE FFN in the Qwen3-MoE
 * layer of aprender issue #3714, "File facts" and gap G3, and the norm between
 * stacked layers), then exactly q3moe_moe_ffn on xn: out = [out +] MoE(xn),
 * routing outputs in topk_idx / topk_w.  out may be hidden itself: with
 * accumulate = 1 that is the residual update x += MoE(RMSNorm(x)) in one
 * call.  Any other overlap of out with hidden, topk_idx, topk_w or norm_gain
 * is E_ALIAS.  The squares are summed in double and each xn value formed in
 * double and rounded once to f32, as q3moe_rmsnorm does.
 * For the one-kernel shapes of q3moe_moe_ffn the norm runs inside that
 * kernel (every workgroup normalises the rows it reads); other shapes run
 * q3moe_rmsnorm into the workspace first.
 * norm_gain: H f32 values, 16-byte aligned; eps >= 0 and finite.
 * workspace: as for q3moe_moe_ffn (the same size query).
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_WORKSPACE, E_ALIAS, E_HIP. */
q3moe_status q3moe_moe_ffn_prenorm(const float *hidden, int64_t T, int64_t H, int64_t F,
                                   int32_t E, int32_t top_k, const float *norm_gain, float eps,
                                   const float *router, q3moe_experts gate, q3moe_experts up,
                                   q3moe_experts down, int32_t *topk_idx, float *topk_w,
                                   float *out, int32_t accumulate, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* ------------------------------------------------------ stacked MoE blocks --
 * n_layers MoE blocks applied one after another to the residual stream x,
 * in place:
 *   for l = 0 .. n_layers-1:  x = x + MoE_l(RMSNorm_l(x))
 * exactly as n_layers calls of q3moe_moe_ffn_prenorm with out = hidden = x
 * and accumulate = 1 would (same arithmetic and rounding per layer; the
 * stream is f32 between layers).  This is the stack of the Qwen3-30B-A3B
 * decoder's 48 MoE layers with the attention taken out (aprender issue
 * #3714, "File facts": 48 layers, down Q6_K in some and Q4_K in others),
 * the post-attention RMSNorm of each layer kept between blocks.
 * layers: HOST array of n_layers descriptors (read during the call only);
 * each names device memory: norm_gain [H] f32 and router [E x H] f32, both
 * 16-byte aligned, and the layer's expert tensors as for q3moe_moe_ffn
 * (gate/up Q4_K, down Q4_K or Q6_K, may differ from layer to layer).  All
 * layers share T, H, F, E and top_k.
 * topk_idx / topk_w: device arrays [n_layers x T x top_k]: layer l's
 * routing at offset l*T*top_k.
 * For the one-kernel shapes of q3moe_moe_ffn (q3moe_persistent_path(..., 1)
 * == 1) the whole stack runs as one persistent kernel per 48 layers: each
 * workgroup hands the rows of x it produced to the next layer as tagged
 * words, so the launch's ramp and drain are paid once per 48 layers instead
 * of once per layer.  Other shapes run q3moe_moe_ffn_prenorm per layer.
 * workspace: at least q3moe_moe_stack_workspace_bytes(T, H, F, E, k) bytes,
 * 16-byte aligned, all zero before the first call that uses it, reusable by
 * later calls of any size on the same stream; its first bytes are a
 * q3moe_moe_ffn workspace (status word at q3moe_expert_ffn_status_offset;
 * bit 8: a layer's input stream was waited for in vain).
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_WORKSPACE, E_ALIAS (x overlaps
 * the routing outputs or a layer's norm_gain or router, or the two routing
 * outputs overlap), E_HIP.  n_layers = 0 or T = 0 does nothing. */
typedef struct q3moe_moe_layer {
    const float *norm_gain;
    const float *router;
    q3moe_experts gate, up, down;
} q3moe_moe_layer;
size_t q3moe_moe_stack_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E,
                                       int32_t top_k);
q3moe_status q3moe_moe_stack(float *x, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t top_k, float eps, const q3moe_moe_layer *layers,
                             int32_t n_layers, int32_t *topk_idx, float *topk_w,
                             void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------ attention prologue --
 * In place on q [T x n_q_heads x head_dim] and k [T x n_kv_heads x head_dim]
 * (f32, row-major): for every head slice, RMSNorm with the gain vector shared
 * by all heads of that projection (q_norm or k_norm, head_dim values),
 *   y = gain * x / sqrt(mean(x^2) + eps),
 * applied after the projection and its bias and before RoPE (aprender
 * PR #1228, "The fix"); then NEOX RoPE at positions[t]: element i pairs with
 * element i + head_dim/2 (SharpInference issue #6) and rotates by
 * positions[t] * rope_base^(-2i/head_dim), all head_dim elements rotated.
 * head_dim is explicit and need not equal hidden/heads (aprender issue #479:
 * 128 for Qwen3 where hidden/heads is 64 or 80).  Angles are formed in
 * double precision.
 * Limits: head_dim even, 2 <= head_dim <= 512; n_q_heads >= 1,
 * n_kv_heads >= 1, n_q_heads % n_kv_heads == 0; eps >= 0; rope_base > 0.
 * Errors: E_NULL, E_SHAPE, E_ALIAS (q and k overlap), E_HIP. */
q3moe_status q3moe_attn_prologue(float *q, float *k, int64_t T, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 const float *q_norm, const float *k_norm,
                                 const int32_t *positions, float eps, float rope_base,
                                 void *stream);

/* The attention prologue and the KV write of the decode step in one launch:
 * q3moe_attn_prologue on q and k (in place), then, for sequence t (one new
 * token each, t < T = B), the rotated k and the untouched v rounded to bf16
 * into cache slot positions[t], exactly as q3moe_kv_write stores them
 * (a position outside [0, S_max) writes nothing).  Arguments as for those
 * two calls; v [T x n_kv_heads x head_dim] f32.
 * Limits: those of both calls; n_q_heads + 2 n_kv_heads <= 65535.
 * Errors: E_NULL, E_SHAPE, E_ALIAS (any two of q, k, v, the caches and
 * positions overlap), E_HIP. */
q3moe_status q3moe_attn_prologue_kv(float *q, float *k, const float *v, int64_t T,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    const float *q_norm, const float *k_norm,
                                    const int32_t *positions, float eps, float rope_base,
                                    uint16_t *k_cache, uint16_t *v_cache, int64_t S_max,
                                    void *stream);

/* ------------------------------------------------ model ends: embedding --
 * The ends of a whole-model decode step around the decoder layers: token
 * embedding, final RMSNorm (q3moe_rmsnorm) and the output head (the Qwen3
 * weight loader of the atlas docs, spark_model/weight_loader/qwen3.rs, loads
 * these three; issue #3714 "File facts": the output matrix is Q6_K).
 *
 * out[t] = row tokens[t] of the embedding table, dequantised:
 *   tokens [T] int32 (device); table: V rows of H/256 k-quant super-blocks
 *   (Q4_K or Q6_K, the row layout of the expert matrices), read in place;
 *   out [T x H] f32.  Each value is the block formula rounded once to f32
 *   (bit-identical to a dequantisation in exact arithmetic).  A token outside
 *   [0, V) gives a row of NaN.
 * Limits: H % 256 == 0, 256 <= H <= 65536, 1 <= V < 2^31.
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIAS (out overlaps tokens or table),
 * E_HIP. */
q3moe_status q3moe_embed(const int32_t *tokens, int64_t T, const void *table, int32_t qtype,
                         int64_t V, int64_t H, float *out, void *stream);

/* ----------------------------------------------- model ends: output head --
 * logits[t][v] = sum_h W[v][h] x[t][h] over the V rows of a Q6_K matrix (the
 * lm_head / output.weight of the model, read in place as one stream):
 *   x [T x H] f32, 16-byte aligned (the final-norm output); W: V rows of
 *   H/256 Q6_K super-blocks, 16-byte aligned; logits [T x V] f32, 4-byte
 *   aligned.  The activations enter as three int8 pieces with a power-of-two
 *   scale per 32 values (exact to 2^-15 of the group's largest value), each
 *   16-weight group's dot product is an exact int32 sum, scales apply in f32.
 *   The matrix is read once per two tokens.
 * Limits: H = 2048, qtype Q3MOE_Q6_K, 1 <= V < 2^31.
 * Errors: E_NULL, E_SHAPE, E_QTYPE, E_ALIGN, E_ALIAS (logits overlap x or W),
 * E_HIP. */
q3moe_status q3moe_output_head(const float *x, int64_t T, const void *W, int32_t qtype, int64_t V,
                               int64_t H, float *logits, void *stream);

/* --------------------------------------------------------------- RMSNorm --
 * out[t] = gain * x[t] / sqrt(mean(x[t]^2) + eps) for x [T x n] f32; the
 * per-layer input / post-attention norm of the decoder layer.  The squares
 * are summed in double and each output formed in double and rounded once to
 * f32.  out may equal x (in place) but must not partially overlap it.
 * Limits: 1 <= n <= 65536, eps >= 0.
 * Errors: E_NULL, E_SHAPE, E_ALIAS, E_HIP. */
q3moe_status q3moe_rmsnorm(const float *x, int64_t T, int64_t n, const float *gain,
                           float eps, float *out, void *stream);

/* ------------------------------------------------- decoder layer: attention --
 * The attention side of the full Qwen3-MoE decoder layer that the MoE block
 * sits in (aprender issue #3714: "File facts" gives 32 query heads, 4 kv
 * heads, head_dim 128, hidden 2048; gap G3 asks for a device-resident model
 * with a per-layer KV cache and Qwen3 attention).  One decode step of a
 * layer, per sequence b at position p = pos[b]:
 *   xn = rmsnorm(x); q = Wq xn; k = Wk xn; v = Wv xn      (q3moe_bf16_gemv)
 *   per-head Q/K RMSNorm + NEOX RoPE at p                  (q3moe_attn_prologue)
 *   k, v -> cache slot p                                   (q3moe_kv_write)
 *   a = attention(q, cache[0..p])                          (q3moe_gqa_attention)
 *   x += Wo a                                              (q3moe_bf16_gemv, accumulate)
 *   then rmsnorm, route and the expert FFN with accumulate.
 * The projections have no bias. */

/* y[t][n] = (accumulate ? y[t][n] : 0) + sum_k W[n][k] * x[t][k].
 *   W [N x K] bf16 (raw bits, row-major), 16-byte aligned; x [T x K] f32,
 *   16-byte aligned; y [T x N] f32 (must not overlap W or x).
 * Up to 8 tokens (and for K not a multiple of 256 or above 4096, up to 63):
 * products and sums are formed in f32 (each bf16 weight is exact in f32),
 * the weights read once per 16 tokens.  From 9 tokens with K % 256 == 0 and
 * K <= 4096, a matrix-core GEMV in passes of 16 tokens, and from 64 tokens
 * on (K % 64 == 0) a matrix-core GEMM: x enters as two bf16 pieces (x to
 * 2^-17 relative), products exact, sums in f32.
 * Limits: K % 8 == 0, 8 <= K <= 2^30, 1 <= N <= 2^30, accumulate 0 or 1.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_ALIAS, E_HIP. */
q3moe_status q3moe_bf16_gemv(const uint16_t *W, int64_t N, int64_t K, const float *x, int64_t T,
                             float *y, int32_t accumulate, void *stream);

/* The Q, K and V projections of the decoder layer in one launch, after the
 * layer's input RMSNorm (the first two steps of the layer above):
 *   xn = norm_gain ? norm_gain * x / sqrt(mean(x^2) + eps) : x
 *   y0 = W0 xn [T x N0], y1 = W1 xn [T x N1], y2 = W2 xn [T x N2]
 * (no accumulate).  N1 or N2 may be 0 (that matrix and output are then not
 * used and may be null).  The norm is formed as q3moe_rmsnorm forms it
 * (squares summed in double, each value formed in double and rounded once
 * to f32) on the way into the projections; products and sums as for
 * q3moe_bf16_gemv.  W0..W2, x and norm_gain 16-byte aligned; outputs 4-byte
 * aligned and overlapping no input or each other.
 * Without the norm, 64 tokens or more take the matrix-core GEMM of
 * q3moe_bf16_gemv, all matrices in one launch.  From 9 tokens with
 * K % 256 == 0 and K <= 4096 (with the norm also beyond 63 tokens) the
 * matrix-core GEMV of q3moe_bf16_gemv runs all matrices in one launch per
 * 16 tokens; with the norm it splits gain * x (rounded once to f32) into
 * the two pieces and scales each token's sums by its 1 / rms (squares summed
 * in double) in double, which agrees with normalising first to the pieces'
 * 2^-17.
 * Limits: as q3moe_bf16_gemv for each matrix; with the norm, K <= 16384 and
 * eps >= 0 and finite.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_ALIAS, E_HIP. */
q3moe_status q3moe_bf16_gemv3(const uint16_t *W0, int64_t N0, const uint16_t *W1, int64_t N1,
                              const uint16_t *W2, int64_t N2, int64_t K, const float *x, int64_t T,
                              const float *norm_gain, float eps, float *y0, float *y1, float *y2,
                              void *stream);

/* Store the new token's keys and values in the bf16 KV caches:
 *   k_cache[b][g][pos[b]][i] = bf16(k_new[b][g][i]), likewise v,
 * for b < B, g < n_kv_heads, i < head_dim.  Caches are
 * [B x n_kv_heads x S_max x head_dim] bf16 (raw bits); conversion rounds to
 * nearest, ties to even (NaN stays NaN).  positions is a device array; an
 * entry outside [0, S_max) writes nothing for that sequence.
 * Limits: n_kv_heads * head_dim <= 65536, S_max >= 1.
 * Errors: E_NULL, E_SHAPE, E_ALIAS (caches overlap each other or an input),
 * E_HIP. */
q3moe_status q3moe_kv_write(const float *k_new, const float *v_new, int64_t B,
                            int32_t n_kv_heads, int32_t head_dim, const int32_t *positions,
                            uint16_t *k_cache, uint16_t *v_cache, int64_t S_max, void *stream);

/* ------------------------------------------- prefill: the attention side --
 * The prompt of one sequence, T tokens at once (aprender issue #3714, 0.70.3
 * gap list: token-by-token prefill is the bottleneck; the fix batches the
 * projections, the RoPE rows and the attention, head_dim 128).  A prefill
 * step of a layer for positions pos[t]:
 *   xn = rmsnorm(x)                         (q3moe_rmsnorm, T rows)
 *   q, k, v = Wq xn, Wk xn, Wv xn           (q3moe_bf16_gemv / _gemv3; matrix cores for T >= 64)
 *   QK-norm + RoPE at pos[t]                (q3moe_attn_prologue, T rows)
 *   k, v -> cache slots pos[t]              (q3moe_kv_write_rows)
 *   a = causal attention                    (q3moe_prefill_attention)
 *   x += Wo a                               (q3moe_bf16_gemv, accumulate)
 *   then the MoE block (q3moe_moe_ffn_prenorm; grouped prefill kernels for T >= 32).
 *
 * q3moe_kv_write_rows: row t of k_new and v_new ([T x n_kv x head_dim] f32),
 * rounded to bf16 (nearest even), into slot positions[t] of ONE sequence's
 * caches [n_kv x S_max x head_dim] (the decode write of one token, for T
 * tokens; a position outside [0, S_max) writes nothing; two rows with one
 * position leave either row).
 * Limits: n_kv * head_dim <= 65536, S_max >= 1.
 * Errors: E_NULL, E_SHAPE, E_ALIAS, E_HIP. */
q3moe_status q3moe_kv_write_rows(const float *k_new, const float *v_new, int64_t T, int32_t n_kv,
                                 int32_t head_dim, const int32_t *positions, uint16_t *k_cache,
                                 uint16_t *v_cache, int64_t S_max, void *stream);

/* Causal grouped-query attention of T queries of ONE sequence over its cache:
 * query t (head h, kv head h / (n_q / n_kv)) attends to positions
 * 0 .. positions[t] (its own row must already be in the cache), scores
 * scale * q . k, softmax with the max subtracted, out = sum p v / sum p.  The
 * same as q3moe_gqa_attention run for each token with length positions[t] + 1.
 *   q [T x n_q x head_dim] f32, 16-byte aligned; caches [n_kv x S_max x
 *   head_dim] bf16, 16-byte aligned; positions [T] int32 device array (any
 *   order); out like q, 4-byte aligned.
 * On the matrix cores: q and the probabilities enter as two bf16 pieces each
 * (to 2^-17 relative), K and V as stored; sums, max and normaliser in f32.
 * A position outside [0, S_max) gives NaN outputs for that token.
 * Limits: head_dim = 128; n_q % n_kv == 0 and (n_q / n_kv) divides 64.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_ALIAS, E_HIP. */
q3moe_status q3moe_prefill_attention(const float *q, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, const uint16_t *k_cache, const uint16_t *v_cache,
                                     int64_t S_max, const int32_t *positions, float scale, float *out,
                                     void *stream);

/* Grouped-query decode attention.  For sequence b and query head h, with
 * kv head g = h / (n_q_heads / n_kv_heads) and L = lengths[b]:
 *   s_j = scale * q[b][h] . k_cache[b][g][j],  j < L
 *   out[b][h] = sum_j softmax(s)_j * v_cache[b][g][j]
 *   q [B x n_q_heads x head_dim] f32, 16-byte aligned; caches as for
 *   q3moe_kv_write, 16-byte aligned; out like q, 4-byte aligned.
 * Scores, the softmax and the sums are f32.  lengths is a device array; a
 * length outside [1, S_max] gives NaN outputs for that sequence and reads no
 * cache row.  No mask beyond the length (decode attends to every cached
 * position); the usual scale is 1/sqrt(head_dim).
 * workspace: at least q3moe_gqa_attention_workspace_bytes(...) bytes,
 * 16-byte aligned, for per-chunk partial results; no state survives a call.
 * Limits: head_dim in {64, 128, 256}; n_q_heads % n_kv_heads == 0;
 * n_q_heads / n_kv_heads <= 16; B <= 65535; scale finite.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ALIAS, E_HIP. */
size_t q3moe_gqa_attention_workspace_bytes(int64_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int64_t S_max);
q3moe_status q3moe_gqa_attention(const float *q, int64_t B, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, const uint16_t *k_cache,
                                 const uint16_t *v_cache, int64_t S_max, const int32_t *lengths,
                                 float scale, float *out, void *workspace,
                                 size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3MOE_H */
