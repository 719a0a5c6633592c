// Internal launchers shared between the C-ABI layer and the kernel files.
// Every launcher assumes its arguments were validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace q3moe {

struct ExpertTensor {
    const uint8_t* base;
    int32_t qtype;
    int64_t stride;
};

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 1024;

// Raise a kernel's dynamic-LDS limit once per (kernel, device, size) instead
// of on every launch, so launches inside a captured graph make no attribute
// call.  One LdsLimit per kernel (a function-local static at the launch site).
constexpr int kMaxDevices = 64;
struct LdsLimit {
    std::atomic<int> set[kMaxDevices];
};

inline hipError_t ensure_lds(const void* fn, LdsLimit& lim, int bytes) {
    if (bytes <= 65536) return hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached && bytes <= lim.set[dev].load(std::memory_order_relaxed)) return hipSuccess;
    const hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (err == hipSuccess && cached) lim.set[dev].store(bytes, std::memory_order_relaxed);
    return err;
}

// group.hip: counts [E], offsets [E+1] and the pair list ordered by (expert,
// pair) of idx [n] (pairs outside [0, E) are not grouped); optionally also
// tile_off [E+1], the exclusive prefix of ceil(counts / tile_rows).
hipError_t launch_group_by_expert(const int32_t* idx, int64_t n, int32_t E, int32_t* counts,
                                  int32_t* offsets, int32_t* pairs, hipStream_t stream,
                                  int32_t* tile_off = nullptr, int32_t tile_rows = 1);

// prefill.hip: the batched expert FFN for larger T (tokens grouped by
// expert, matrix-core tiles).  Workspace layout in prefill_workspace_bytes.
constexpr int64_t kPrefillMinTokens = 32;
size_t prefill_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k);
hipError_t launch_prefill_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                              int32_t k, const int32_t* idx, const float* w,
                              const ExpertTensor& gate, const ExpertTensor& up,
                              const ExpertTensor& down, float* out, int accumulate, void* ws,
                              hipStream_t stream);

// route.hip.  The route workspace starts with kRouteSyncBytes of completion
// counters (zero before the first call; every call leaves them zero), then
// holds the logits.  launch_route takes the counter and the logits apart, so
// a caller that embeds the route in a larger workspace can keep the counter
// at an offset that does not depend on the call's sizes.
constexpr size_t kRouteSyncBytes = 4096;
// The counters use the first kRouteCounterBytes of that (a top counter and
// 8 stripe counters, 128 bytes apart).
constexpr size_t kRouteCounterBytes = 9 * 128;
size_t route_workspace_bytes(int64_t T, int32_t E);
hipError_t launch_route(const float* hidden, int64_t T, int64_t H, const float* router,
                        int32_t E, int32_t k, int32_t* idx, float* w, int32_t* sync,
                        double* logits, hipStream_t stream);

// ffn_decode.hip: the decode-batch path (H/256 in {1, 2, 4, 8, 16})
bool decode_ffn_supported(int64_t H, int64_t F, int32_t k);
// The expert-FFN workspace starts with kFfnSyncBytes of synchronisation
// words (the status word, then line-spaced completion counters of the fused
// kernel), then holds the intermediate h from that offset on.
constexpr size_t kFfnSyncBytes = 8192;
// Byte offset, inside that header, of the route kernel's arrival counters when
// the route runs as part of the MoE block (the header's first half holds the
// expert FFN's own words; the counters take kRouteCounterBytes, below the
// fused kernel's presence words).  Fixed, so the counters sit at one address
// for calls of every size through one workspace.
constexpr size_t kFfnRouteSyncOffset = 4096;
hipError_t launch_decode_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const int32_t* idx, const float* w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ws,
                             hipStream_t stream);

// Route + expert FFN of a few tokens in one launch (H = 2048, T <= 4, k <= 8,
// E <= 256): moe_decode_fused tells whether the shape qualifies.  ffn_ws is
// an expert-FFN workspace, route_words moe_route_words_bytes(T, E) of zeroed
// memory that the kernel's routing step uses for its tagged partial logits;
// norm_gain (or null) applies the input RMSNorm inside the kernel, and then
// hidden may equal out.
// act_pieces: 3 = the gate/up activations as three exact int8 pieces (the
// f32 block), 1 = one int8 piece per value (the int8-activation mode).
bool moe_decode_fused(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, int32_t dqtype,
                      int act_pieces = 3);
// Whether launch_expert_ffn runs this shape as the one persistent kernel.
bool expert_ffn_fused(int64_t T, int64_t H, int64_t F, int32_t k, int32_t dqtype);
size_t moe_route_words_bytes(int64_t T, int32_t E);
hipError_t launch_moe_decode(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const float* router, int32_t* topk_idx, float* topk_w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ffn_ws,
                             void* route_words, const float* norm_gain, float eps,
                             hipStream_t stream, int act_pieces = 3);

// Several stacked MoE blocks, x <- x + MoE_l(RMSNorm_l(x)) for l = 0..n-1,
// in one persistent launch per 48 layers (shape limits of launch_moe_decode;
// each layer its own router, gain and experts, down Q4_K or Q6_K) when
// moe_stack_fused says so.
// ffn_ws and route_words as for launch_moe_decode, xbuf
// moe_stack_xbuf_bytes(T, H) of memory for the residual stream between
// layers; topk_idx / topk_w receive [n_layers][T][k].
struct MoeLayerTensors {
    const float* router;
    const float* gain;
    ExpertTensor gate, up, down;
};
// (and whether every layer's expert strides fit the kernel's 32-bit fields)
bool moe_stack_fused(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, const MoeLayerTensors* layers,
                     int32_t n_layers);
size_t moe_stack_xbuf_bytes(int64_t T, int64_t H);
hipError_t launch_moe_stack(float* x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, float eps,
                            const MoeLayerTensors* layers, int32_t n_layers, int32_t* topk_idx,
                            float* topk_w, void* ffn_ws, void* route_words, void* xbuf,
                            hipStream_t stream);

// ffn.hip: dispatch, and the generic path for any H, F multiple of 256
size_t expert_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k);
size_t expert_ffn_status_offset(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k);
hipError_t launch_expert_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const int32_t* idx, const float* w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ws,
                             hipStream_t stream);

// layer.hip: the attention side of the decoder layer
hipError_t launch_bf16_gemv(const uint16_t* W, int64_t N, int64_t K, const float* x, int64_t T,
                            float* y, int accumulate, hipStream_t stream);
// Up to three matrices on one input in one launch (N1 or N2 may be 0), with
// the input RMSNorm inside when gain is not null (K <= kGemvNormMaxK).
constexpr int64_t kGemvNormMaxK = 16384;
hipError_t launch_bf16_gemv3(const uint16_t* W0, int64_t N0, const uint16_t* W1, int64_t N1,
                             const uint16_t* W2, int64_t N2, int64_t K, const float* x, int64_t T,
                             const float* gain, float eps, float* y0, float* y1, float* y2,
                             hipStream_t stream);
hipError_t launch_kv_write(const float* k_new, const float* v_new, int64_t B, int32_t n_kv,
                           int32_t D, const int32_t* pos, uint16_t* kcache, uint16_t* vcache,
                           int64_t S_max, hipStream_t stream);
bool gqa_attention_supported(int32_t n_q, int32_t n_kv, int32_t D);
size_t gqa_attention_workspace_bytes(int64_t B, int32_t n_q, int32_t n_kv, int32_t D, int64_t S_max);
hipError_t launch_gqa_attention(const float* q, int64_t B, int32_t n_q, int32_t n_kv, int32_t D,
                                const uint16_t* kcache, const uint16_t* vcache, int64_t S_max,
                                const int32_t* len, float scale, float* out, void* ws,
                                hipStream_t stream);

// attn_prefill.hip: the attention side of batched prefill.  launch_bf16_gemm
// serves q3moe_bf16_gemv for T >= kGemmMinTokens (K % 64 == 0) on the
// matrix cores.
constexpr int64_t kGemmMinTokens = 64;
bool gemm_path(int64_t T, int64_t K);
hipError_t launch_bf16_gemm(const uint16_t* W, int64_t N, int64_t K, const float* x, int64_t T,
                            float* y, int accumulate, hipStream_t stream);
hipError_t launch_bf16_gemm_multi(const uint16_t* const* Ws, float* const* ys, const int64_t* Ns,
                                  int nmat, int64_t K, const float* x, int64_t T, int accumulate,
                                  hipStream_t stream);
hipError_t launch_kv_write_rows(const float* k_new, const float* v_new, int64_t T, int32_t nkv,
                                int32_t D, const int32_t* pos, uint16_t* kc, uint16_t* vc,
                                int64_t S_max, hipStream_t stream);
bool prefill_attention_supported(int32_t nq, int32_t nkv, int32_t D);
hipError_t launch_prefill_attention(const float* q, int64_t T, int32_t nq, int32_t nkv, int32_t D,
                                    const uint16_t* kc, const uint16_t* vc, int64_t S_max,
                                    const int32_t* pos, float scale, float* out, hipStream_t stream);

// model.hip: the token embedding gather and the Q6_K output head
hipError_t launch_embed(const int32_t* tokens, int64_t T, const uint8_t* table, int32_t qtype,
                        int64_t V, int64_t H, float* out, hipStream_t stream);
bool output_head_supported(int64_t H, int32_t qtype);
hipError_t launch_output_head(const float* x, int64_t T, const uint8_t* W, int64_t V, float* logits,
                              hipStream_t stream);

// norm.hip
hipError_t launch_rmsnorm(const float* x, int64_t T, int64_t n, const float* gain, float eps,
                          float* out, hipStream_t stream);
hipError_t launch_attn_prologue(float* q, float* k, int64_t T, int32_t nq, int32_t nkv,
                                int32_t D, const float* qn, const float* kn,
                                const int32_t* pos, float eps, float base, hipStream_t stream);
hipError_t launch_attn_prologue_kv(float* q, float* k, const float* v, int64_t T, int32_t nq,
                                   int32_t nkv, int32_t D, const float* qn, const float* kn,
                                   const int32_t* pos, float eps, float base, uint16_t* kc,
                                   uint16_t* vc, int64_t S_max, hipStream_t stream);

}  // namespace q3moe
