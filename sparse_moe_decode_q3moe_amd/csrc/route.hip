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
constexpr int kRouteStripes = 8;                       // completion counter stripes
constexpr int kRouteStripeWords = 32;                  // 128 bytes apart
static_assert((kRouteStripes + 1) * kRouteStripeWords * 4 <= (int)kRouteCounterBytes, "route counters");

// Workspace: kRouteSyncBytes holding the arrival counters (a top counter
// and 8 stripe counters 128 bytes apart, all zero between calls, in the
// first kRouteCounterBytes), then the logits [T x E] doubles.

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
// on stripe counter e % 8, the workgroup that completes a stripe counts the
// stripe on the top counter, and the workgroup that completes the top count
// (every logit is then visible at device scope) selects the top-k of all
// tokens, one wave per token, reading the logits with device-scope loads.
// It finally zeroes the counters for the next call.  Nothing waits on
// another workgroup.  (One counter for all 128 workgroups serialised their
// atomics: the two-call step took 18.5 against 18.0 us striped.)

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
        // workgroup e counts itself on stripe e % S; the last of a stripe
        // counts the stripe on the top counter (fewer atomics on any one word)
        const int S = grid < kRouteStripes ? grid : kRouteStripes, st = e % S;
        const int members = grid / S + (st < grid % S ? 1 : 0);
        const int done = __hip_atomic_fetch_add(sync + kRouteStripeWords * (1 + st), 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        last = 0;
        if (done == members - 1)
            last = __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
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
    if (tid <= kRouteStripes)                 // the top counter and the stripes, zero for the next call
        __hip_atomic_store(sync + kRouteStripeWords * tid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- T > 8 --
// grid: (ceil(E / 16), ceil(T / 16)), 16 waves.  A workgroup computes the
// logits of 16 tokens x 16 experts on the matrix cores in double:
// v_mfma_f64_16x16x4_f64 with the token rows as A and the router rows as B,
// both converted from f32 (each product of two f32 values is exact in
// double and the matrix unit accumulates in double).  The H columns go in
// 16-column chunks, chunk c to wave c % 16; a wave requests its chunks 8 at
// a time and feeds them to 4 independent accumulator chains (chain j % 4
// for the j-th of the 8), so the loads are in flight together and no step
// waits for the previous one; the chains, then the 16 waves, are added in
// a fixed order.  Per chunk a lane loads one float4 of its token row and one
// of its router row (lane l: row l % 16, columns 4 (l / 16) .. + 3 of the
// chunk) and feeds them to 4 matrix steps, step s taking column 4 (l / 16)
// + s: A and B use the same lane-to-k pairing, so every product pairs
// x[t][c] with R[e][c].  Columns past H (a last partial chunk, H % 16 != 0)
// and chunks past the end read column 0 and enter as zeros; rows past T or
// E read the last valid row and their sums are not stored.
// f64 16x16x4 layout (checked on the device): A lane l holds row l % 16 at
// k = l / 16, B lane l column l % 16 at the same k, and result value i of
// lane l is row 4 i + l / 16, column l % 16.
constexpr int kRtTile = 16;
constexpr int kRtWaves = 16;
constexpr int kRtThreads = kRtWaves * kWave;
constexpr int kRtBatch = 8;
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kRtThreads) void router_tile_kernel(
    const float* __restrict__ hidden, int64_t T, int64_t H, const float* __restrict__ router,
    int32_t E, double* __restrict__ logits) {
    const int64_t e0 = (int64_t)blockIdx.x * kRtTile, t0 = (int64_t)blockIdx.y * kRtTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int64_t t = t0 + r < T ? t0 + r : T - 1, e = e0 + r < E ? e0 + r : E - 1;
    const float* xrow = hidden + t * H;
    const float* rrow = router + e * H;
    const int64_t nch = (H + 15) / 16;
    f64x4_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    for (int64_t c0 = wave; c0 < nch; c0 += (int64_t)kRtWaves * kRtBatch) {
        float4 xv[kRtBatch], rv[kRtBatch];
        bool in[kRtBatch];
#pragma unroll
        for (int j = 0; j < kRtBatch; ++j) {
            const int64_t c = c0 + (int64_t)j * kRtWaves;
            in[j] = c < nch && 16 * c + 4 * q < H;
            const int64_t col = in[j] ? 16 * c + 4 * q : 0;
            xv[j] = *reinterpret_cast<const float4*>(xrow + col);
            rv[j] = *reinterpret_cast<const float4*>(rrow + col);
        }
#pragma unroll
        for (int j = 0; j < kRtBatch; ++j) {
            const float4 x = in[j] ? xv[j] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 w = in[j] ? rv[j] : make_float4(0.f, 0.f, 0.f, 0.f);
            acc[j & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x.x, (double)w.x, acc[j & 3], 0, 0, 0);
            acc[j & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x.y, (double)w.y, acc[j & 3], 0, 0, 0);
            acc[j & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x.z, (double)w.z, acc[j & 3], 0, 0, 0);
            acc[j & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x.w, (double)w.w, acc[j & 3], 0, 0, 0);
        }
    }
    const f64x4_t tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __shared__ double part[kRtWaves][4][kWave];
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][i][lane] = tot[i];
    __syncthreads();
    if (tid < 4 * kWave) {                                    // value i = tid / 64 of lane tid % 64
        const int i = tid >> 6, l = tid & 63;
        double sum = 0.0;
#pragma unroll
        for (int w = 0; w < kRtWaves; ++w) sum += part[w][i][l];
        const int64_t tt = t0 + 4 * i + (l >> 4), ee = e0 + (l & 15);
        if (tt < T && ee < E) logits[tt * E + ee] = sum;
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
    dim3 g1((unsigned)((E + kRtTile - 1) / kRtTile), (unsigned)((T + kRtTile - 1) / kRtTile));
    hipLaunchKernelGGL(router_tile_kernel, g1, dim3(kRtThreads), 0, stream, hidden, T, H,
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
