// C-ABI entry points: host-side validation, then kernel launches on the
// caller's stream.  The contract is documented in include/q3moe.h.
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/q3moe.h"
#include "device_common.h"
#include "internal.h"

using q3moe::ExpertTensor;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

q3moe_status from_hip(hipError_t e) { return e == hipSuccess ? Q3MOE_OK : Q3MOE_E_HIP; }

q3moe_status check_experts(const q3moe_experts& x, int64_t rows, int64_t cols, bool allow_q6,
                           ExpertTensor& out) {
    if (!x.base) return Q3MOE_E_NULL;
    if (x.reserved != 0) return Q3MOE_E_SHAPE;
    if (x.qtype != Q3MOE_Q4_K && !(allow_q6 && x.qtype == Q3MOE_Q6_K)) return Q3MOE_E_QTYPE;
    if (!aligned16(x.base) || (x.expert_stride_bytes & 15) != 0) return Q3MOE_E_ALIGN;
    if (x.expert_stride_bytes < q3moe_expert_matrix_bytes(x.qtype, rows, cols)) return Q3MOE_E_SHAPE;
    out.base = static_cast<const uint8_t*>(x.base);
    out.qtype = x.qtype;
    out.stride = x.expert_stride_bytes;
    return Q3MOE_OK;
}

}  // namespace

extern "C" {

const char* q3moe_status_string(q3moe_status s) {
    switch (s) {
        case Q3MOE_OK: return "ok";
        case Q3MOE_E_NULL: return "a required pointer is NULL";
        case Q3MOE_E_SHAPE: return "a size is out of range or inconsistent";
        case Q3MOE_E_QTYPE: return "unknown or unsupported quantisation type";
        case Q3MOE_E_ALIGN: return "a pointer or stride is not 16-byte aligned";
        case Q3MOE_E_WORKSPACE: return "workspace missing or smaller than the size query";
        case Q3MOE_E_HIP: return "the HIP runtime rejected a launch";
        case Q3MOE_E_ALIAS: return "an output overlaps an input it must not overlap";
        default: return "unknown status";
    }
}

int32_t q3moe_qtype_block_bytes(int32_t qtype) {
    return qtype == Q3MOE_Q4_K ? q3moe::kQ4KBytes : qtype == Q3MOE_Q6_K ? q3moe::kQ6KBytes : 0;
}

int64_t q3moe_expert_matrix_bytes(int32_t qtype, int64_t rows, int64_t cols) {
    const int32_t bb = q3moe_qtype_block_bytes(qtype);
    if (!bb || rows < 0 || cols < 0 || cols % 256) return -1;
    return rows * (cols / 256) * bb;
}

size_t q3moe_route_workspace_bytes(int64_t T, int32_t E) {
    return q3moe::route_workspace_bytes(T, E);
}

q3moe_status q3moe_route(const float* hidden, int64_t T, int64_t H, const float* router,
                         int32_t E, int32_t top_k, int32_t* topk_idx, float* topk_w,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (T < 0 || H < 1 || E < 1 || E > q3moe::kMaxExperts || top_k < 1 ||
        top_k > q3moe::kMaxTopK || top_k > E || (H & 3) != 0 || T > 0x7fffffff)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!hidden || !router || !topk_idx || !topk_w) return Q3MOE_E_NULL;
    if (!aligned16(hidden) || !aligned16(router)) return Q3MOE_E_ALIGN;
    if (!workspace || workspace_bytes < q3moe_route_workspace_bytes(T, E))
        return Q3MOE_E_WORKSPACE;
    if (!aligned16(workspace)) return Q3MOE_E_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    return from_hip(q3moe::launch_route(hidden, T, H, router, E, top_k, topk_idx, topk_w,
                                        reinterpret_cast<int32_t*>(ws),
                                        reinterpret_cast<double*>(ws + q3moe::kRouteSyncBytes),
                                        as_stream(stream)));
}

q3moe_status q3moe_group_by_expert(const int32_t* topk_idx, int64_t T, int32_t top_k,
                                   int32_t E, int32_t* counts, int32_t* offsets,
                                   int32_t* pairs, void* stream) {
    if (T < 0 || top_k < 1 || top_k > q3moe::kMaxTopK || E < 1 || E > q3moe::kMaxExperts ||
        T * (int64_t)top_k > 0x7fffffff)
        return Q3MOE_E_SHAPE;
    if (!counts || !offsets || (T > 0 && (!topk_idx || !pairs))) return Q3MOE_E_NULL;
    const int64_t n = T * top_k;
    if (n > 0 && (overlaps(pairs, n * 4, topk_idx, n * 4) || overlaps(counts, E * 4, topk_idx, n * 4) ||
                  overlaps(offsets, (E + 1) * 4, topk_idx, n * 4)))
        return Q3MOE_E_ALIAS;
    if (overlaps(counts, E * 4, offsets, (E + 1) * 4) ||
        (n > 0 && (overlaps(pairs, n * 4, counts, E * 4) || overlaps(pairs, n * 4, offsets, (E + 1) * 4))))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_group_by_expert(topk_idx, n, E, counts, offsets, pairs,
                                                  as_stream(stream)));
}

size_t q3moe_expert_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E,
                                        int32_t top_k) {
    return q3moe::expert_ffn_workspace_bytes(T, H, F, E, top_k);
}

size_t q3moe_expert_ffn_status_offset(int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k) {
    return q3moe::expert_ffn_status_offset(T, H, F, E, top_k);
}

q3moe_status q3moe_expert_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                              int32_t top_k, const int32_t* topk_idx, const float* topk_w,
                              q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                              float* out, int32_t accumulate, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (T < 0 || H % 256 || F % 256 || H < 256 || H > 4096 || F < 256 || F > 1536 || E < 1 ||
        top_k < 1 || top_k > q3moe::kMaxTopK || top_k > E || (accumulate != 0 && accumulate != 1) ||
        T * top_k > 0x7fffffff)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!hidden || !topk_idx || !topk_w || !out) return Q3MOE_E_NULL;
    ExpertTensor g, u, d;
    q3moe_status st;
    if ((st = check_experts(gate, F, H, false, g)) != Q3MOE_OK) return st;
    if ((st = check_experts(up, F, H, false, u)) != Q3MOE_OK) return st;
    if ((st = check_experts(down, H, F, true, d)) != Q3MOE_OK) return st;
    if (!aligned16(hidden) || !aligned16(out)) return Q3MOE_E_ALIGN;
    const size_t act = (size_t)T * (size_t)H * sizeof(float);
    if (overlaps(hidden, act, out, act)) return Q3MOE_E_ALIAS;
    if (!workspace || workspace_bytes < q3moe_expert_ffn_workspace_bytes(T, H, F, E, top_k))
        return Q3MOE_E_WORKSPACE;
    if (!aligned16(workspace)) return Q3MOE_E_ALIGN;
    return from_hip(q3moe::launch_expert_ffn(hidden, T, H, F, E, top_k, topk_idx, topk_w, g, u,
                                             d, out, accumulate, workspace, as_stream(stream)));
}

namespace {
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace

size_t q3moe_moe_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k) {
    // expert-FFN workspace, route workspace, the fused kernel's tagged
    // router words, and (for the pre-norm form on the multi-kernel path) the
    // normalised input rows
    return round256(q3moe::expert_ffn_workspace_bytes(T, H, F, E, top_k)) +
           round256(q3moe::route_workspace_bytes(T, E)) + round256(q3moe::moe_route_words_bytes(T, E)) +
           (size_t)(T > 0 ? T : 0) * (size_t)(H > 0 ? H : 0) * sizeof(float);
}

namespace {

// The MoE block, with (norm_gain != null) or without the input RMSNorm.
// With the norm, out may be hidden itself; any other overlap is rejected.
q3moe_status moe_ffn_impl(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                          int32_t top_k, bool want_norm, const float* norm_gain, float eps,
                          const float* router,
                          q3moe_experts gate, q3moe_experts up, q3moe_experts down,
                          int32_t* topk_idx, float* topk_w, float* out, int32_t accumulate,
                          void* workspace, size_t workspace_bytes, void* stream,
                          int act_pieces = 3) {
    if (T < 0 || H % 256 || F % 256 || H < 256 || H > 4096 || F < 256 || F > 1536 || E < 1 ||
        E > q3moe::kMaxExperts || top_k < 1 || top_k > q3moe::kMaxTopK || top_k > E ||
        (accumulate != 0 && accumulate != 1) || T * top_k > 0x7fffffff || !(eps >= 0.0f) ||
        !(eps <= 3.4028235e38f))
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!hidden || !router || !topk_idx || !topk_w || !out || (want_norm && !norm_gain))
        return Q3MOE_E_NULL;
    ExpertTensor g, u, d;
    q3moe_status st;
    if ((st = check_experts(gate, F, H, false, g)) != Q3MOE_OK) return st;
    if ((st = check_experts(up, F, H, false, u)) != Q3MOE_OK) return st;
    if ((st = check_experts(down, H, F, true, d)) != Q3MOE_OK) return st;
    if (!aligned16(hidden) || !aligned16(router) || !aligned16(out) ||
        (norm_gain && !aligned16(norm_gain)))
        return Q3MOE_E_ALIGN;
    const size_t act = (size_t)T * (size_t)H * sizeof(float);
    const size_t rt = (size_t)T * (size_t)top_k * 4;
    const bool in_place = norm_gain && static_cast<const void*>(hidden) == static_cast<const void*>(out);
    if ((!in_place && overlaps(hidden, act, out, act)) || overlaps(topk_idx, rt, out, act) ||
        overlaps(topk_w, rt, out, act) || overlaps(topk_idx, rt, topk_w, rt) ||
        overlaps(topk_idx, rt, hidden, act) || overlaps(topk_w, rt, hidden, act) ||
        (norm_gain && overlaps(norm_gain, (size_t)H * sizeof(float), out, act)))
        return Q3MOE_E_ALIAS;
    if (!workspace || workspace_bytes < q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k))
        return Q3MOE_E_WORKSPACE;
    if (!aligned16(workspace)) return Q3MOE_E_ALIGN;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* ws_route = ws + round256(q3moe::expert_ffn_workspace_bytes(T, H, F, E, top_k));
    uint8_t* ws_words = ws_route + round256(q3moe::route_workspace_bytes(T, E));
    float* ws_norm = reinterpret_cast<float*>(ws_words + round256(q3moe::moe_route_words_bytes(T, E)));
    const hipStream_t s = as_stream(stream);
    if (q3moe::moe_decode_fused(T, H, F, E, top_k, d.qtype, act_pieces))
        return from_hip(q3moe::launch_moe_decode(hidden, T, H, F, E, top_k, router, topk_idx, topk_w,
                                                 g, u, d, out, accumulate, ws, ws_words, norm_gain,
                                                 eps, s, act_pieces));
    if (act_pieces != 3) return Q3MOE_E_SHAPE;      // the int8 mode has only the one-kernel form
    const float* x = hidden;
    if (norm_gain) {                          // normalised rows into the workspace first
        hipError_t e = q3moe::launch_rmsnorm(hidden, T, H, norm_gain, eps, ws_norm, s);
        if (e != hipSuccess) return from_hip(e);
        x = ws_norm;
    }
    // The route's arrival counters live in the expert-FFN header at a fixed
    // offset: ws_route moves with T, H, F and k, and a region that a larger
    // call filled with data must never serve as counters that have to be zero.
    hipError_t e = q3moe::launch_route(x, T, H, router, E, top_k, topk_idx, topk_w,
                                       reinterpret_cast<int32_t*>(ws + q3moe::kFfnRouteSyncOffset),
                                       reinterpret_cast<double*>(ws_route + q3moe::kRouteSyncBytes), s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(q3moe::launch_expert_ffn(x, T, H, F, E, top_k, topk_idx, topk_w, g, u, d,
                                             out, accumulate, ws, s));
}

}  // namespace

q3moe_status q3moe_moe_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                           int32_t top_k, const float* router, q3moe_experts gate,
                           q3moe_experts up, q3moe_experts down, int32_t* topk_idx,
                           float* topk_w, float* out, int32_t accumulate, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return moe_ffn_impl(hidden, T, H, F, E, top_k, false, nullptr, 0.0f, router, gate, up, down, topk_idx,
                        topk_w, out, accumulate, workspace, workspace_bytes, stream);
}

q3moe_status q3moe_moe_ffn_q8(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                              int32_t top_k, const float* router, q3moe_experts gate,
                              q3moe_experts up, q3moe_experts down, int32_t* topk_idx,
                              float* topk_w, float* out, int32_t accumulate, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return moe_ffn_impl(hidden, T, H, F, E, top_k, false, nullptr, 0.0f, router, gate, up, down, topk_idx,
                        topk_w, out, accumulate, workspace, workspace_bytes, stream, 1);
}

q3moe_status q3moe_moe_ffn_prenorm(const float* hidden, int64_t T, int64_t H, int64_t F,
                                   int32_t E, int32_t top_k, const float* norm_gain, float eps,
                                   const float* router, q3moe_experts gate, q3moe_experts up,
                                   q3moe_experts down, int32_t* topk_idx, float* topk_w,
                                   float* out, int32_t accumulate, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return moe_ffn_impl(hidden, T, H, F, E, top_k, true, norm_gain, eps, router, gate, up, down, topk_idx,
                        topk_w, out, accumulate, workspace, workspace_bytes, stream);
}

size_t q3moe_moe_stack_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k) {
    // a q3moe_moe_ffn workspace, then the residual stream's tagged words
    return round256(q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k)) + q3moe::moe_stack_xbuf_bytes(T, H);
}

q3moe_status q3moe_moe_stack(float* x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k,
                             float eps, const q3moe_moe_layer* layers, int32_t n_layers,
                             int32_t* topk_idx, float* topk_w, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (T < 0 || H % 256 || F % 256 || H < 256 || H > 4096 || F < 256 || F > 1536 || E < 1 ||
        E > q3moe::kMaxExperts || top_k < 1 || top_k > q3moe::kMaxTopK || top_k > E || n_layers < 0 ||
        T * top_k > 0x7fffffff / (n_layers > 0 ? n_layers : 1) || !(eps >= 0.0f) || !(eps <= 3.4028235e38f))
        return Q3MOE_E_SHAPE;
    if (T == 0 || n_layers == 0) return Q3MOE_OK;
    if (!x || !layers || !topk_idx || !topk_w) return Q3MOE_E_NULL;
    if (!aligned16(x)) return Q3MOE_E_ALIGN;
    const size_t act = (size_t)T * (size_t)H * sizeof(float);
    const size_t rt = (size_t)n_layers * (size_t)T * (size_t)top_k * 4;
    if (overlaps(topk_idx, rt, x, act) || overlaps(topk_w, rt, x, act) || overlaps(topk_idx, rt, topk_w, rt))
        return Q3MOE_E_ALIAS;
    std::vector<q3moe::MoeLayerTensors> ly((size_t)n_layers);
    for (int32_t l = 0; l < n_layers; ++l) {
        const q3moe_moe_layer& d = layers[l];
        if (!d.norm_gain || !d.router) return Q3MOE_E_NULL;
        q3moe_status st;
        if ((st = check_experts(d.gate, F, H, false, ly[l].gate)) != Q3MOE_OK) return st;
        if ((st = check_experts(d.up, F, H, false, ly[l].up)) != Q3MOE_OK) return st;
        if ((st = check_experts(d.down, H, F, true, ly[l].down)) != Q3MOE_OK) return st;
        if (!aligned16(d.norm_gain) || !aligned16(d.router)) return Q3MOE_E_ALIGN;
        if (overlaps(d.norm_gain, (size_t)H * sizeof(float), x, act) ||
            overlaps(d.router, (size_t)E * (size_t)H * sizeof(float), x, act) ||
            overlaps(d.norm_gain, (size_t)H * sizeof(float), topk_idx, rt) ||
            overlaps(d.norm_gain, (size_t)H * sizeof(float), topk_w, rt))
            return Q3MOE_E_ALIAS;
        ly[l].router = d.router;
        ly[l].gain = d.norm_gain;
    }
    if (!workspace || workspace_bytes < q3moe_moe_stack_workspace_bytes(T, H, F, E, top_k))
        return Q3MOE_E_WORKSPACE;
    if (!aligned16(workspace)) return Q3MOE_E_ALIGN;
    const hipStream_t s = as_stream(stream);
    if (q3moe::moe_stack_fused(T, H, F, E, top_k, ly.data(), n_layers)) {
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        uint8_t* ws_words = ws + round256(q3moe::expert_ffn_workspace_bytes(T, H, F, E, top_k)) +
                            round256(q3moe::route_workspace_bytes(T, E));
        uint8_t* ws_x = ws + round256(q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k));
        return from_hip(q3moe::launch_moe_stack(x, T, H, F, E, top_k, eps, ly.data(), n_layers, topk_idx,
                                                topk_w, ws, ws_words, ws_x, s));
    }
    const int64_t nr = T * top_k;
    for (int32_t l = 0; l < n_layers; ++l) {
        const q3moe_status st = moe_ffn_impl(x, T, H, F, E, top_k, true, layers[l].norm_gain, eps,
                                             layers[l].router, layers[l].gate, layers[l].up, layers[l].down,
                                             topk_idx + l * nr, topk_w + l * nr, x, 1, workspace,
                                             workspace_bytes, stream);
        if (st != Q3MOE_OK) return st;
    }
    return Q3MOE_OK;
}

int32_t q3moe_persistent_path(int64_t T, int64_t H, int64_t F, int32_t E, int32_t top_k,
                              int32_t down_qtype, int32_t with_route) {
    if (T < 0 || H % 256 || F % 256 || H < 256 || H > 4096 || F < 256 || F > 1536 || E < 1 ||
        E > q3moe::kMaxExperts || top_k < 1 || top_k > q3moe::kMaxTopK || top_k > E ||
        (down_qtype != Q3MOE_Q4_K && down_qtype != Q3MOE_Q6_K) || (with_route != 0 && with_route != 1))
        return -1;
    if (T == 0) return 0;
    return with_route ? (q3moe::moe_decode_fused(T, H, F, E, top_k, down_qtype, 3) ? 1 : 0)
                      : (q3moe::expert_ffn_fused(T, H, F, top_k, down_qtype) ? 1 : 0);
}

q3moe_status q3moe_attn_prologue(float* q, float* k, int64_t T, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, const float* q_norm,
                                 const float* k_norm, const int32_t* positions, float eps,
                                 float rope_base, void* stream) {
    if (T < 0 || T > 0x7fffffff || n_q_heads < 1 || n_kv_heads < 1 ||
        n_q_heads % n_kv_heads != 0 || head_dim < 2 || head_dim > 512 || (head_dim & 1) ||
        !(eps >= 0.0f) || !(rope_base > 0.0f) || n_q_heads + n_kv_heads > 65535)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!q || !k || !q_norm || !k_norm || !positions) return Q3MOE_E_NULL;
    if (overlaps(q, (size_t)T * n_q_heads * head_dim * sizeof(float), k,
                 (size_t)T * n_kv_heads * head_dim * sizeof(float)))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_attn_prologue(q, k, T, n_q_heads, n_kv_heads, head_dim, q_norm,
                                                k_norm, positions, eps, rope_base,
                                                as_stream(stream)));
}

q3moe_status q3moe_attn_prologue_kv(float* q, float* k, const float* v, int64_t T,
                                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    const float* q_norm, const float* k_norm,
                                    const int32_t* positions, float eps, float rope_base,
                                    uint16_t* k_cache, uint16_t* v_cache, int64_t S_max,
                                    void* stream) {
    if (T < 0 || T > 0x7fffffff || n_q_heads < 1 || n_kv_heads < 1 ||
        n_q_heads % n_kv_heads != 0 || head_dim < 2 || head_dim > 512 || (head_dim & 1) ||
        !(eps >= 0.0f) || !(rope_base > 0.0f) || (int64_t)n_q_heads + 2 * (int64_t)n_kv_heads > 65535 ||
        S_max < 1)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!q || !k || !v || !q_norm || !k_norm || !positions || !k_cache || !v_cache) return Q3MOE_E_NULL;
    const size_t nqb = (size_t)T * n_q_heads * head_dim * sizeof(float);
    const size_t nkb = (size_t)T * n_kv_heads * head_dim * sizeof(float);
    const size_t nc = (size_t)T * n_kv_heads * (size_t)S_max * head_dim * 2;
    if (overlaps(q, nqb, k, nkb) || overlaps(q, nqb, v, nkb) || overlaps(k, nkb, v, nkb) ||
        overlaps(k_cache, nc, v_cache, nc) || overlaps(k_cache, nc, q, nqb) ||
        overlaps(k_cache, nc, k, nkb) || overlaps(k_cache, nc, v, nkb) ||
        overlaps(v_cache, nc, q, nqb) || overlaps(v_cache, nc, k, nkb) ||
        overlaps(v_cache, nc, v, nkb) || overlaps(k_cache, nc, positions, (size_t)T * 4) ||
        overlaps(v_cache, nc, positions, (size_t)T * 4))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_attn_prologue_kv(q, k, v, T, n_q_heads, n_kv_heads, head_dim, q_norm,
                                                   k_norm, positions, eps, rope_base, k_cache, v_cache,
                                                   S_max, as_stream(stream)));
}

q3moe_status q3moe_embed(const int32_t* tokens, int64_t T, const void* table, int32_t qtype,
                         int64_t V, int64_t H, float* out, void* stream) {
    if (T < 0 || T > 0x7fffffff || V < 1 || V > 0x7fffffff || H < 256 || H > 65536 || H % 256)
        return Q3MOE_E_SHAPE;
    if (qtype != Q3MOE_Q4_K && qtype != Q3MOE_Q6_K) return Q3MOE_E_QTYPE;
    if (T == 0) return Q3MOE_OK;
    if (!tokens || !table || !out) return Q3MOE_E_NULL;
    const size_t no = (size_t)T * (size_t)H * sizeof(float);
    const size_t nt = (size_t)V * (size_t)q3moe_expert_matrix_bytes(qtype, 1, H);
    if (overlaps(out, no, table, nt) || overlaps(out, no, tokens, (size_t)T * 4)) return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_embed(tokens, T, static_cast<const uint8_t*>(table), qtype, V, H, out,
                                        as_stream(stream)));
}

q3moe_status q3moe_output_head(const float* x, int64_t T, const void* W, int32_t qtype, int64_t V,
                               int64_t H, float* logits, void* stream) {
    if (T < 0 || T > 0x7fffffff || V < 1 || V > 0x7fffffff || H < 256 || H % 256 ||
        (int64_t)T * V > ((int64_t)1 << 40))
        return Q3MOE_E_SHAPE;
    if (qtype != Q3MOE_Q6_K) return Q3MOE_E_QTYPE;
    if (!q3moe::output_head_supported(H, qtype)) return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!x || !W || !logits) return Q3MOE_E_NULL;
    if (!aligned16(x) || !aligned16(W) || (reinterpret_cast<uintptr_t>(logits) & 3u)) return Q3MOE_E_ALIGN;
    const size_t nl = (size_t)T * (size_t)V * sizeof(float);
    if (overlaps(logits, nl, x, (size_t)T * (size_t)H * sizeof(float)) ||
        overlaps(logits, nl, W, (size_t)V * (size_t)q3moe_expert_matrix_bytes(qtype, 1, H)))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_output_head(x, T, static_cast<const uint8_t*>(W), V, logits,
                                              as_stream(stream)));
}

q3moe_status q3moe_rmsnorm(const float* x, int64_t T, int64_t n, const float* gain, float eps,
                           float* out, void* stream) {
    if (T < 0 || T > 0x7fffffff || n < 1 || n > 65536 || !(eps >= 0.0f)) return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!x || !gain || !out) return Q3MOE_E_NULL;
    const size_t nb = (size_t)T * (size_t)n * sizeof(float);
    if (x != out && overlaps(x, nb, out, nb)) return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_rmsnorm(x, T, n, gain, eps, out, as_stream(stream)));
}

q3moe_status q3moe_bf16_gemv(const uint16_t* W, int64_t N, int64_t K, const float* x, int64_t T,
                             float* y, int32_t accumulate, void* stream) {
    if (T < 0 || T > 0x7fffffff || N < 1 || N > ((int64_t)1 << 30) || K < 8 || (K & 7) ||
        K > ((int64_t)1 << 30) || (accumulate != 0 && accumulate != 1))
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!W || !x || !y) return Q3MOE_E_NULL;
    if (!aligned16(W) || !aligned16(x) || (reinterpret_cast<uintptr_t>(y) & 3u)) return Q3MOE_E_ALIGN;
    const size_t ny = (size_t)T * (size_t)N * sizeof(float);
    if (overlaps(y, ny, W, (size_t)N * (size_t)K * 2) || overlaps(y, ny, x, (size_t)T * (size_t)K * sizeof(float)))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_bf16_gemv(W, N, K, x, T, y, accumulate, as_stream(stream)));
}

q3moe_status q3moe_bf16_gemv3(const uint16_t* W0, int64_t N0, const uint16_t* W1, int64_t N1,
                              const uint16_t* W2, int64_t N2, int64_t K, const float* x, int64_t T,
                              const float* norm_gain, float eps, float* y0, float* y1, float* y2,
                              void* stream) {
    const int64_t lim = (int64_t)1 << 30;
    if (T < 0 || T > 0x7fffffff || N0 < 1 || N0 > lim || N1 < 0 || N1 > lim || N2 < 0 || N2 > lim ||
        K < 8 || (K & 7) || K > lim || (norm_gain && (K > q3moe::kGemvNormMaxK || !(eps >= 0.0f) ||
                                                       !(eps <= 3.4028235e38f))))
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!W0 || !x || !y0 || (N1 && (!W1 || !y1)) || (N2 && (!W2 || !y2))) return Q3MOE_E_NULL;
    if (!aligned16(W0) || (N1 && !aligned16(W1)) || (N2 && !aligned16(W2)) || !aligned16(x) ||
        (norm_gain && !aligned16(norm_gain)) || (reinterpret_cast<uintptr_t>(y0) & 3u) ||
        (N1 && (reinterpret_cast<uintptr_t>(y1) & 3u)) || (N2 && (reinterpret_cast<uintptr_t>(y2) & 3u)))
        return Q3MOE_E_ALIGN;
    const uint16_t* Ws[3] = {W0, W1, W2};
    float* ys[3] = {y0, y1, y2};
    const int64_t Ns[3] = {N0, N1, N2};
    const size_t nx = (size_t)T * (size_t)K * sizeof(float);
    for (int i = 0; i < 3; ++i) {
        if (!Ns[i]) continue;
        const size_t ny = (size_t)T * (size_t)Ns[i] * sizeof(float);
        if (overlaps(ys[i], ny, x, nx) || (norm_gain && overlaps(ys[i], ny, norm_gain, (size_t)K * 4)))
            return Q3MOE_E_ALIAS;
        for (int j = 0; j < 3; ++j) {
            if (!Ns[j]) continue;
            if (overlaps(ys[i], ny, Ws[j], (size_t)Ns[j] * (size_t)K * 2)) return Q3MOE_E_ALIAS;
            if (j != i && overlaps(ys[i], ny, ys[j], (size_t)T * (size_t)Ns[j] * sizeof(float)))
                return Q3MOE_E_ALIAS;
        }
    }
    return from_hip(q3moe::launch_bf16_gemv3(W0, N0, N1 ? W1 : nullptr, N1, N2 ? W2 : nullptr, N2, K,
                                             x, T, norm_gain, eps, y0, N1 ? y1 : nullptr,
                                             N2 ? y2 : nullptr, as_stream(stream)));
}

q3moe_status q3moe_kv_write(const float* k_new, const float* v_new, int64_t B, int32_t n_kv_heads,
                            int32_t head_dim, const int32_t* positions, uint16_t* k_cache,
                            uint16_t* v_cache, int64_t S_max, void* stream) {
    if (B < 0 || B > 0x7fffffff || n_kv_heads < 1 || head_dim < 1 ||
        (int64_t)n_kv_heads * head_dim > 65536 || S_max < 1)
        return Q3MOE_E_SHAPE;
    if (B == 0) return Q3MOE_OK;
    if (!k_new || !v_new || !positions || !k_cache || !v_cache) return Q3MOE_E_NULL;
    const size_t nc = (size_t)B * n_kv_heads * (size_t)S_max * head_dim * 2;
    const size_t nn = (size_t)B * n_kv_heads * head_dim * sizeof(float);
    if (overlaps(k_cache, nc, v_cache, nc) || overlaps(k_cache, nc, k_new, nn) ||
        overlaps(k_cache, nc, v_new, nn) || overlaps(v_cache, nc, k_new, nn) ||
        overlaps(v_cache, nc, v_new, nn) || overlaps(k_cache, nc, positions, (size_t)B * 4) ||
        overlaps(v_cache, nc, positions, (size_t)B * 4))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_kv_write(k_new, v_new, B, n_kv_heads, head_dim, positions, k_cache,
                                           v_cache, S_max, as_stream(stream)));
}

q3moe_status q3moe_kv_write_rows(const float* k_new, const float* v_new, int64_t T, int32_t n_kv,
                                 int32_t head_dim, const int32_t* positions, uint16_t* k_cache,
                                 uint16_t* v_cache, int64_t S_max, void* stream) {
    if (T < 0 || T > 0x7fffffff || n_kv < 1 || head_dim < 1 || (int64_t)n_kv * head_dim > 65536 ||
        S_max < 1)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!k_new || !v_new || !positions || !k_cache || !v_cache) return Q3MOE_E_NULL;
    const size_t nc = (size_t)n_kv * (size_t)S_max * head_dim * 2;
    const size_t nn = (size_t)T * n_kv * head_dim * sizeof(float);
    if (overlaps(k_cache, nc, v_cache, nc) || overlaps(k_cache, nc, k_new, nn) ||
        overlaps(k_cache, nc, v_new, nn) || overlaps(v_cache, nc, k_new, nn) ||
        overlaps(v_cache, nc, v_new, nn) || overlaps(k_cache, nc, positions, (size_t)T * 4) ||
        overlaps(v_cache, nc, positions, (size_t)T * 4))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_kv_write_rows(k_new, v_new, T, n_kv, head_dim, positions, k_cache,
                                                v_cache, S_max, as_stream(stream)));
}

q3moe_status q3moe_prefill_attention(const float* q, int64_t T, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, const uint16_t* k_cache, const uint16_t* v_cache,
                                     int64_t S_max, const int32_t* positions, float scale, float* out,
                                     void* stream) {
    if (T < 0 || T > 0x7fffffff || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads > 65535 ||
        S_max < 1 || S_max > 0x7fffffff ||
        !q3moe::prefill_attention_supported(n_q_heads, n_kv_heads, head_dim) || !(scale == scale) ||
        scale == __builtin_inff() || scale == -__builtin_inff())
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    if (!q || !k_cache || !v_cache || !positions || !out) return Q3MOE_E_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(out) & 3u))
        return Q3MOE_E_ALIGN;
    const size_t nq = (size_t)T * n_q_heads * head_dim * sizeof(float);
    const size_t nc = (size_t)n_kv_heads * (size_t)S_max * head_dim * 2;
    if (overlaps(out, nq, q, nq) || overlaps(out, nq, k_cache, nc) || overlaps(out, nq, v_cache, nc) ||
        overlaps(out, nq, positions, (size_t)T * 4))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_prefill_attention(q, T, n_q_heads, n_kv_heads, head_dim, k_cache,
                                                    v_cache, S_max, positions, scale, out,
                                                    as_stream(stream)));
}

size_t q3moe_gqa_attention_workspace_bytes(int64_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                           int32_t head_dim, int64_t S_max) {
    if (B < 0 || n_q_heads < 1 || S_max < 1 || !q3moe::gqa_attention_supported(n_q_heads, n_kv_heads, head_dim))
        return 0;
    return q3moe::gqa_attention_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, S_max);
}

q3moe_status q3moe_gqa_attention(const float* q, int64_t B, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const uint16_t* k_cache, const uint16_t* v_cache,
                                 int64_t S_max, const int32_t* lengths, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || B > 65535 || S_max < 1 || S_max > 0x7fffffff ||
        !q3moe::gqa_attention_supported(n_q_heads, n_kv_heads, head_dim) || !(scale == scale) ||
        scale == __builtin_inff() || scale == -__builtin_inff())
        return Q3MOE_E_SHAPE;
    if (B == 0) return Q3MOE_OK;
    if (!q || !k_cache || !v_cache || !lengths || !out) return Q3MOE_E_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(q) & 15u) || (reinterpret_cast<uintptr_t>(out) & 3u))
        return Q3MOE_E_ALIGN;
    const size_t need = q3moe::gqa_attention_workspace_bytes(B, n_q_heads, n_kv_heads, head_dim, S_max);
    if (!workspace || workspace_bytes < need) return Q3MOE_E_WORKSPACE;
    const size_t nq = (size_t)B * n_q_heads * head_dim * sizeof(float);
    const size_t nc = (size_t)B * n_kv_heads * (size_t)S_max * head_dim * 2;
    if (overlaps(out, nq, q, nq) || overlaps(out, nq, workspace, need) || overlaps(out, nq, k_cache, nc) ||
        overlaps(out, nq, v_cache, nc) || overlaps(workspace, need, q, nq) ||
        overlaps(workspace, need, k_cache, nc) || overlaps(workspace, need, v_cache, nc) ||
        overlaps(workspace, need, lengths, (size_t)B * 4) || overlaps(out, nq, lengths, (size_t)B * 4))
        return Q3MOE_E_ALIAS;
    return from_hip(q3moe::launch_gqa_attention(q, B, n_q_heads, n_kv_heads, head_dim, k_cache, v_cache,
                                                S_max, lengths, scale, out, workspace, as_stream(stream)));
}

}  // extern "C"
