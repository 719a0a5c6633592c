// Router GEMV + softmax / top-k / renormalisation on the device
// (aprender issue #3714, gap G3 "router: f32_gemv_into" and the on-device
// top-8 planned as K1 under G8).  Logits are accumulated in double: the
// f32 x f32 products are exact in double and summation-order noise drops
// to ~1e-16, which keeps the top-k choice identical to any other double
// evaluation except at genuine ties ("Risk to track" in the same issue).
//
// Decode-sized batches (T <= 8) run as ONE kernel: workgroup e computes
// expert e's logits for every token, and the last workgroup to finish
// (found with striped completion counters, no waiting) selects the top-k of
// every token.  Larger batches run a logits kernel over (4-expert, 16-token)
// tiles and a top-k kernel with one wave per token.
//
// Selection (both paths, topk_wave): k rounds of a wave-wide argmax over the
// token's logits, larger value first and equal values broken by the lower
// expert index, each round screened in f32 and decided exactly; weights are
// the softmax over the selected logits in double (the first selected logit
// subtracted), normalised by their sum taken in rank order, then rounded to
// f32.
#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace q3moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteTokTile = 8;
constexpr int kRouteChunk = 4;                         // float4 per thread and pass

// Workspace: kRouteSyncBytes holding the arrival counter (zero between
// calls), then the logits [T x E] doubles.

// This thread's share of row e of the router dotted with tokens t0..t0+ntok-1
// (ntok <= 8), accumulated in double.  Loads use clamped indices and a zero
// mask instead of branches so they are not serialised behind one another.
__device__ __forceinline__ void router_row_dots(const float* __restrict__ hidden, int64_t t0,
                                                int ntok, int64_t H,
                                                const float* __restrict__ row, int tid,
                                                double acc[kRouteTokTile]) {
    const int64_t n4 = H / 4;
    const float4* r4 = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int j = 0; j < kRouteTokTile; ++j) acc[j] = 0.0;
    for (int64_t base = 0; base < n4; base += kRouteChunk * kRouteThreads) {
        float4 rv[kRouteChunk];
        float keep[kRouteChunk];
        int64_t ii[kRouteChunk];
#pragma unroll
        for (int c = 0; c < kRouteChunk; ++c) {
            const int64_t i = base + c * kRouteThreads + tid;
            keep[c] = i < n4 ? 1.0f : 0.0f;
            ii[c] = i < n4 ? i : n4 - 1;
            rv[c] = r4[ii[c]];
        }
        for (int j = 0; j < ntok; ++j) {
            const float4* x4 = reinterpret_cast<const float4*>(hidden + (t0 + j) * H);
            float4 xv[kRouteChunk];
#pragma unroll
            for (int c = 0; c < kRouteChunk; ++c) xv[c] = x4[ii[c]];
            double a = acc[j];
#pragma unroll
            for (int c = 0; c < kRouteChunk; ++c) {
                const double kc = (double)keep[c];
                a = fma((double)rv[c].x * kc, (double)xv[c].x, a);
                a = fma((double)rv[c].y * kc, (double)xv[c].y, a);
                a = fma((double)rv[c].z * kc, (double)xv[c].z, a);
                a = fma((double)rv[c].w * kc, (double)xv[c].w, a);
            }
            acc[j] = a;
        }
    }
}

// Workgroup-wide sums of acc[0..ntok); thread j < ntok receives token j's sum.
__device__ __forceinline__ double workgroup_token_sums(double acc[kRouteTokTile], int ntok,
                                                       int tid) {
    __shared__ double part[kRouteTokTile][kRouteWaves];
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int j = 0; j < kRouteTokTile; ++j) {
        if (j < ntok) {
            const double s = wave_sum_dpp_f64(acc[j]);
            if (lane == 0) part[j][wave] = s;
        }
    }
    __syncthreads();
    double s = 0.0;
    if (tid < ntok) {
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) s += part[tid][w];
    }
    return s;
}

// ------------------------------------------------------------ T <= 8 --
// grid: E workgroups; workgroup e computes logits[t][e] for every token and
// stores them with device-scope stores; after they complete it counts itself
// on one device-scope counter, and the workgroup that completes the count
// (every logit is then visible at device scope) selects the top-k of all
// tokens, one wave per token, reading the logits with device-scope loads.
// It finally zeroes the counter for the next call.  Nothing waits on
// another workgroup.

template <int NPER>
__global__ __launch_bounds__(kRouteThreads) void route_small_kernel(
    const float* __restrict__ hidden, int32_t T, int64_t H, const float* __restrict__ router,
    int32_t E, int32_t k, int32_t* __restrict__ idx, float* __restrict__ w,
    int32_t* __restrict__ sync, double* __restrict__ logits) {
    const int e = blockIdx.x, grid = (int)gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int last;
    double acc[kRouteTokTile];
    router_row_dots(hidden, 0, T, H, router + (int64_t)e * H, tid, acc);
    const double s = workgroup_token_sums(acc, T, tid);
    if (tid < T)
        __hip_atomic_store(logits + (int64_t)tid * E + e, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_all_loads();                         // the logit stores have completed
    __syncthreads();
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = done == grid - 1;
    }
    __syncthreads();
    if (!last) return;
    for (int t = wave; t < T; t += kRouteWaves) {
        double v[NPER];
#pragma unroll
        for (int j = 0; j < NPER; ++j) {
            const int ee = lane + kWave * j;
            v[j] = ee < E ? __hip_atomic_load(logits + (int64_t)t * E + ee, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT)
                          : 0.0;
        }
        topk_wave<NPER>(v, E, k, lane, idx + (int64_t)t * k, w + (int64_t)t * k);
    }
    if (tid == 0) __hip_atomic_store(sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- T > 8 --
// grid: (ceil(E / 4), ceil(T / 8)).  A workgroup computes the logits of 4
// experts x 8 tokens: each thread takes float4 columns i = tid, tid + 256,
// ... of the 4 router rows and the 8 token rows and accumulates the 32
// exact f32 x f32 products per column in double (32 independent sums); the
// wave then folds its 32 sums over its 64 lanes with a transposed butterfly
// (lanes 2v, 2v + 1 end with sum v), and the 4 waves' results are added in
// a fixed order.  Each router row is read once per 8 tokens and each token
// row once per 4 experts (an expert x 8-token tile read the token rows once
// per expert: ~590 MB of L2 reads at 512 tokens instead of ~200 MB).
constexpr int kRtExp = 4, kRtTok = 8;
constexpr int kRtV = kRtExp * kRtTok;          // 32 sums per thread

// Sum of v[0..32) over the 64 lanes, transposed: lanes 2j and 2j + 1 end
// with the total of value j.
__device__ __forceinline__ double transposed_sum32_f64(double (&v)[kRtV], int lane) {
#pragma unroll
    for (int lev = 0; lev < 5; ++lev) {
        const int half = kRtV >> (lev + 1);
        const int bit = 5 - lev;
        const bool up = (lane >> bit) & 1;
        const uint64_t m = up ? ~0ull : 0ull;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            // the selects act on the values' bits: a select between two
            // array elements would become a select between their addresses
            // and keep the array out of registers
            const uint64_t a = __builtin_bit_cast(uint64_t, v[i]);
            const uint64_t b = __builtin_bit_cast(uint64_t, v[i + half]);
            const double send = __builtin_bit_cast(double, (a & m) | (b & ~m));
            const double keep = __builtin_bit_cast(double, (b & m) | (a & ~m));
            v[i] = keep + __shfl_xor(send, 1 << bit, kWave);
        }
    }
    return v[0] + __shfl_xor(v[0], 1, kWave);
}

__global__ __launch_bounds__(kRouteThreads) void router_tile_kernel(
    const float* __restrict__ hidden, int64_t T, int64_t H, const float* __restrict__ router,
    int32_t E, double* __restrict__ logits) {
    const int64_t e0 = (int64_t)blockIdx.x * kRtExp, t0 = (int64_t)blockIdx.y * kRtTok;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n4 = H / 4;
    const float4* r4 = reinterpret_cast<const float4*>(router);
    const float4* x4 = reinterpret_cast<const float4*>(hidden);
    // rows past E or T read the last valid row and are multiplied by zero
    double rkeep[kRtExp], xkeep[kRtTok];
    int64_t rrow[kRtExp], xrow[kRtTok];
#pragma unroll
    for (int e = 0; e < kRtExp; ++e) {
        rkeep[e] = e0 + e < E ? 1.0 : 0.0;
        rrow[e] = (e0 + e < E ? e0 + e : E - 1) * n4;
    }
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) {
        xkeep[t] = t0 + t < T ? 1.0 : 0.0;
        xrow[t] = (t0 + t < T ? t0 + t : T - 1) * n4;
    }
    double acc[kRtV];
#pragma unroll
    for (int i = 0; i < kRtV; ++i) acc[i] = 0.0;
    for (int64_t i = tid; i < n4; i += kRouteThreads) {
        float4 rv[kRtExp], xv[kRtTok];
#pragma unroll
        for (int e = 0; e < kRtExp; ++e) rv[e] = r4[rrow[e] + i];
#pragma unroll
        for (int t = 0; t < kRtTok; ++t) xv[t] = x4[xrow[t] + i];
#pragma unroll
        for (int e = 0; e < kRtExp; ++e) {
            const double rx = (double)rv[e].x * rkeep[e], ry = (double)rv[e].y * rkeep[e];
            const double rz = (double)rv[e].z * rkeep[e], rw = (double)rv[e].w * rkeep[e];
#pragma unroll
            for (int t = 0; t < kRtTok; ++t) {
                double a = fma(rx, (double)xv[t].x * xkeep[t], acc[e * kRtTok + t]);
                a = fma(ry, (double)xv[t].y * xkeep[t], a);
                a = fma(rz, (double)xv[t].z * xkeep[t], a);
                acc[e * kRtTok + t] = fma(rw, (double)xv[t].w * xkeep[t], a);
            }
        }
    }
    __shared__ double part[kRouteWaves][kRtV];
    const double ws = transposed_sum32_f64(acc, lane);
    if ((lane & 1) == 0) part[wave][lane >> 1] = ws;
    __syncthreads();
    if (tid < kRtV) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) s += part[w][tid];
        const int64_t e = e0 + tid / kRtTok, t = t0 + tid % kRtTok;
        if (e < E && t < T) logits[t * E + e] = s;
    }
}

// grid: ceil(T / 4) workgroups, one wave per token.
template <int NPER>
__global__ __launch_bounds__(kRouteThreads) void topk_kernel(const double* __restrict__ logits,
                                                             int64_t T, int32_t E, int32_t k,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T) return;
    double v[NPER];
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
        const int ee = lane + kWave * j;
        v[j] = ee < E ? logits[t * E + ee] : 0.0;
    }
    topk_wave<NPER>(v, E, k, lane, idx + t * k, w + t * k);
}

template <int NPER>
hipError_t launch_route_nper(const float* hidden, int64_t T, int64_t H, const float* router,
                             int32_t E, int32_t k, int32_t* idx, float* w, int32_t* sync,
                             double* logits, hipStream_t stream) {
    if (T <= kRouteTokTile) {
        hipLaunchKernelGGL(route_small_kernel<NPER>, dim3((unsigned)E), dim3(kRouteThreads), 0,
                           stream, hidden, (int32_t)T, H, router, E, k, idx, w, sync, logits);
        return hipGetLastError();
    }
    dim3 g1((unsigned)((E + kRtExp - 1) / kRtExp), (unsigned)((T + kRtTok - 1) / kRtTok));
    hipLaunchKernelGGL(router_tile_kernel, g1, dim3(kRouteThreads), 0, stream, hidden, T, H,
                       router, E, logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(topk_kernel<NPER>, dim3((unsigned)((T + kRouteWaves - 1) / kRouteWaves)),
                       dim3(kRouteThreads), 0, stream, logits, T, E, k, idx, w);
    return hipGetLastError();
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int32_t E) {
    return kRouteSyncBytes + (size_t)(T > 0 ? T : 0) * (size_t)E * sizeof(double);
}

hipError_t launch_route(const float* hidden, int64_t T, int64_t H, const float* router,
                        int32_t E, int32_t k, int32_t* idx, float* w, int32_t* sync,
                        double* logits, hipStream_t stream) {
    if (E <= 64) return launch_route_nper<1>(hidden, T, H, router, E, k, idx, w, sync, logits, stream);
    if (E <= 128) return launch_route_nper<2>(hidden, T, H, router, E, k, idx, w, sync, logits, stream);
    if (E <= 256) return launch_route_nper<4>(hidden, T, H, router, E, k, idx, w, sync, logits, stream);
    if (E <= 512) return launch_route_nper<8>(hidden, T, H, router, E, k, idx, w, sync, logits, stream);
    return launch_route_nper<16>(hidden, T, H, router, E, k, idx, w, sync, logits, stream);
}

}  // namespace q3moe
