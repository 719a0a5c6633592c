// Router GEMV + softmax / top-k / renormalisation on the device
// (aprender issue #3714, gap G3 "router: f32_gemv_into" and the on-device
// top-8 planned as K1 under G8).  Logits are accumulated in double: the
// f32 x f32 products are exact in double and summation-order noise drops
// to ~1e-16, which keeps the top-k choice identical to any other double
// evaluation except at genuine ties ("Risk to track" in the same issue).
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteTokTile = 8;

// One workgroup per (expert e, tile of up to 8 tokens).  Threads stride the
// router row in float4 units; the row stays in registers across the token
// tile while each token's hidden vector streams from L2.
__global__ __launch_bounds__(kRouteThreads) void router_logits_kernel(
    const float* __restrict__ hidden, int64_t T, int64_t H, const float* __restrict__ router,
    int32_t E, double* __restrict__ logits) {
    const int e = blockIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * kRouteTokTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n4 = H / 4;
    const float4* r4 = reinterpret_cast<const float4*>(router + (int64_t)e * H);
    __shared__ double part[kRouteTokTile][kRouteThreads / kWave];

    const int ntok = (int)((T - t0) < kRouteTokTile ? (T - t0) : kRouteTokTile);
    double acc[kRouteTokTile];
#pragma unroll
    for (int j = 0; j < kRouteTokTile; ++j) acc[j] = 0.0;
    for (int64_t i = tid; i < n4; i += kRouteThreads) {
        const float4 rv = r4[i];
#pragma unroll
        for (int j = 0; j < kRouteTokTile; ++j) {
            if (j < ntok) {
                const float4 xv = reinterpret_cast<const float4*>(hidden + (t0 + j) * H)[i];
                double a = acc[j];
                a = fma((double)rv.x, (double)xv.x, a);
                a = fma((double)rv.y, (double)xv.y, a);
                a = fma((double)rv.z, (double)xv.z, a);
                a = fma((double)rv.w, (double)xv.w, a);
                acc[j] = a;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kRouteTokTile; ++j) {
        const double s = wave_sum_f64(acc[j]);
        if (lane == 0) part[j][wave] = s;
    }
    __syncthreads();
    if (tid < ntok) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kRouteThreads / kWave; ++w) s += part[tid][w];
        logits[(t0 + tid) * E + e] = s;
    }
}

// One wave per token: k rounds of a wave-wide argmax over the token's E
// logits (larger value first, lower index on equal values), then the
// softmax over the k selected logits in double, rounded to f32.
__global__ __launch_bounds__(kWave) void topk_softmax_kernel(const double* __restrict__ logits,
                                                             int32_t E, int32_t k,
                                                             int32_t* __restrict__ idx,
                                                             float* __restrict__ w) {
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x;
    constexpr int kPer = kMaxExperts / kWave;
    double v[kPer];
    const double* lt = logits + t * E;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = lane + kWave * j;
        v[j] = (e < E) ? lt[e] : -INFINITY;
    }
    bool taken[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) taken[j] = (lane + kWave * j) >= E;

    double sel_val = 0.0;   // lane s < k keeps the s-th selected logit
    int sel_idx = 0;
    for (int s = 0; s < k; ++s) {
        double bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int e = lane + kWave * j;
            if (!taken[j] && (v[j] > bv || (v[j] == bv && e < bi))) {
                bv = v[j];
                bi = e;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const double ov = __shfl_xor(bv, m, kWave);
            const int oi = __shfl_xor(bi, m, kWave);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        // bi is now the same in every lane; mark it taken in its owner lane.
        if ((bi & (kWave - 1)) == lane) {
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                if (lane + kWave * j == bi) taken[j] = true;
        }
        if (lane == s) {
            sel_val = bv;
            sel_idx = bi;
        }
    }
    const double top = __shfl(sel_val, 0, kWave);
    const double ex = (lane < k) ? exp(sel_val - top) : 0.0;
    const double den = wave_sum_f64(ex);
    if (lane < k) {
        idx[t * k + lane] = sel_idx;
        w[t * k + lane] = (float)(ex / den);
    }
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int32_t E) {
    return (size_t)(T > 0 ? T : 0) * (size_t)E * sizeof(double);
}

hipError_t launch_route(const float* hidden, int64_t T, int64_t H, const float* router,
                        int32_t E, int32_t k, int32_t* idx, float* w, void* ws,
                        hipStream_t stream) {
    double* logits = static_cast<double*>(ws);
    dim3 g1(E, (unsigned)((T + kRouteTokTile - 1) / kRouteTokTile));
    hipLaunchKernelGGL(router_logits_kernel, g1, dim3(kRouteThreads), 0, stream, hidden, T, H,
                       router, E, logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)T), dim3(kWave), 0, stream, logits, E,
                       k, idx, w);
    return hipGetLastError();
}

}  // namespace q3moe
