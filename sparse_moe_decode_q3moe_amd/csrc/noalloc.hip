// q3moe_moe_ffn_noalloc: the MoE block with its workspace in a file-scope
// device array, for callers that cannot allocate.  The contract is in
// include/q3moe.h.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/q3moe.h"
#include "internal.h"

// ---------------------------------------------------------------- no-alloc --
// q3moe_moe_ffn_noalloc takes its workspace from this file-scope device array
// instead of an argument.  In host code `scratch` names a host-side stand-in,
// never the device memory: the device address comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// passed to kernels.
namespace {

constexpr size_t kNoAllocScratchBytes = Q3MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Zero n16 16-byte words (the fill runs as a kernel, not a memset node, so a
// graph that captures it replays a plain kernel).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchState {
    std::atomic<void*> ptr[q3moe::kMaxDevices];
    std::atomic<int> cleared[q3moe::kMaxDevices];   // an uncaptured call enqueued the fill
};
ScratchState g_scratch;

// This device's copy of `scratch` (looked up on its first use); nullptr on
// failure.  The first calls on a device also enqueue a zero fill of the whole
// array on `stream` ahead of the block, until one that is not being captured
// into a graph has done so (a captured fill only runs when the graph runs).
void* device_scratch(hipStream_t stream, hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= q3moe::kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* p = g_scratch.ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch.ptr[dev].store(p, std::memory_order_release);
    }
    if (!g_scratch.cleared[dev].load(std::memory_order_acquire)) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        *err = hipStreamIsCapturing(stream, &cs);
        if (*err != hipSuccess) return nullptr;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(p),
                           kNoAllocScratchBytes / 16);
        *err = hipGetLastError();
        if (*err != hipSuccess) return nullptr;
        if (cs == hipStreamCaptureStatusNone) g_scratch.cleared[dev].store(1, std::memory_order_release);
    }
    *err = hipSuccess;
    return p;
}

}  // namespace

extern "C" {

q3moe_status q3moe_moe_ffn_noalloc(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                                   int32_t top_k, const float* router, q3moe_experts gate,
                                   q3moe_experts up, q3moe_experts down, int32_t* topk_idx,
                                   float* topk_w, float* out, int32_t accumulate, void* stream) {
    // the size checks of q3moe_moe_ffn first, so a shape error is reported as
    // one and the workspace query below only sees valid shapes
    if (T < 0 || H % 256 || F % 256 || H < 256 || H > 4096 || F < 256 || F > 1536 || E < 1 ||
        E > q3moe::kMaxExperts || top_k < 1 || top_k > q3moe::kMaxTopK || top_k > E ||
        (accumulate != 0 && accumulate != 1) || T * top_k > 0x7fffffff)
        return Q3MOE_E_SHAPE;
    if (T == 0) return Q3MOE_OK;
    const size_t need = q3moe_moe_ffn_workspace_bytes(T, H, F, E, top_k);
    if (need > kNoAllocScratchBytes) return Q3MOE_E_WORKSPACE;
    if (!hidden || !router || !topk_idx || !topk_w || !out) return Q3MOE_E_NULL;
    hipError_t e = hipSuccess;
    void* ws = device_scratch(static_cast<hipStream_t>(stream), &e);
    if (!ws) return Q3MOE_E_HIP;
    return q3moe_moe_ffn(hidden, T, H, F, E, top_k, router, gate, up, down, topk_idx, topk_w, out,
                         accumulate, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
