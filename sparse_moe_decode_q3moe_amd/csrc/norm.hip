// RMSNorm and the fused attention prologue (per-head Q/K RMSNorm, then NEOX
// RoPE, optionally followed by the token's KV-cache write).  Sources: aprender PR #1228 "The fix" (per-head norm with one gain
// vector per projection, after the bias and before RoPE); SharpInference
// issue #6 closing comment (NEOX pairing i <-> i + head_dim/2); aprender
// issue #479 "Fix Applied" (head_dim explicit, not hidden/heads).
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

constexpr int kNormThreads = 256;

// One workgroup per row: out = gain * x / sqrt(mean(x^2) + eps), the
// squares summed in double (f32 squares are exact there) and each output
// formed in double and rounded once to f32.  x and out may be the same row:
// after the barrier each thread reads and writes only its own elements.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float* x, int64_t n,
                                                               const float* __restrict__ gain,
                                                               float eps, float* out) {
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const float* xr = x + t * n;
    __shared__ double part[kNormThreads / kWave];
    double ss = 0.0;
    for (int64_t i = tid; i < n; i += kNormThreads) ss = fma((double)xr[i], (double)xr[i], ss);
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const double tot = (part[0] + part[1]) + (part[2] + part[3]);
    const double inv = 1.0 / sqrt(tot / (double)n + (double)eps);
    for (int64_t i = tid; i < n; i += kNormThreads)
        out[t * n + i] = (float)((double)gain[i] * (double)xr[i] * inv);
}

// One wave per (token, head): lane i owns the NEOX pair (i, i + D/2) for
// i = lane, lane + 64, ... < D/2.  RMSNorm over the whole head, then the
// rotation by pos * base^(-2i/D), with the angle and its sine/cosine in
// double precision (at position 4095 an f32 angle would carry ~2e-4 rad of
// rounding error).  With caches (kc not null) the kernel also does the KV
// write of the token: heads nq..nq+nkv-1 store their rotated k, rounded to
// bf16, at cache slot pos[t] of sequence t, and nkv more waves (heads
// nq+nkv..) store v there; a position outside [0, S_max) writes nothing.
constexpr int kMaxPairsPerLane = 4;   // head_dim <= 512

__global__ __launch_bounds__(kWave) void attn_prologue_kernel(
    float* q, float* k, const float* __restrict__ v, int32_t nq, int32_t nkv, int32_t D,
    const float* __restrict__ qn, const float* __restrict__ kn, const int32_t* __restrict__ pos,
    float eps, float base, uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int64_t S_max) {
    const int h = blockIdx.y;
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x;
    const int slot = kc ? pos[t] : -1;
    const bool write_kv = kc && slot >= 0 && slot < S_max;
    if (h >= nq + nkv) {                      // v head: the cache write alone
        const int64_t g = h - nq - nkv;
        if (write_kv)
            for (int i = lane; i < D; i += kWave)
                vc[((t * nkv + g) * S_max + slot) * D + i] = float_to_bf16_rne(v[(t * nkv + g) * D + i]);
        return;
    }
    const bool isq = h < nq;
    float* p = isq ? q + (t * nq + h) * (int64_t)D : k + (t * nkv + (h - nq)) * (int64_t)D;
    const float* g = isq ? qn : kn;
    const int half = D / 2;
    float a[kMaxPairsPerLane], b[kMaxPairsPerLane];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPairsPerLane; ++j) {
        const int i = lane + kWave * j;
        a[j] = (i < half) ? p[i] : 0.f;
        b[j] = (i < half) ? p[i + half] : 0.f;
        ss = fmaf(a[j], a[j], fmaf(b[j], b[j], ss));
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    const double pd = (double)pos[t];
    const double lb = log((double)base);
#pragma unroll
    for (int j = 0; j < kMaxPairsPerLane; ++j) {
        const int i = lane + kWave * j;
        if (i < half) {
            const float ya = g[i] * (a[j] * inv);
            const float yb = g[i + half] * (b[j] * inv);
            const double theta = pd * exp(-2.0 * (double)i / (double)D * lb);
            double sd, cd;
            sincos(theta, &sd, &cd);
            const float c = (float)cd, s = (float)sd;
            const float ra = ya * c - yb * s, rb = ya * s + yb * c;
            p[i] = ra;
            p[i + half] = rb;
            if (!isq && write_kv) {
                uint16_t* dst = kc + ((t * nkv + (h - nq)) * S_max + slot) * (int64_t)D;
                dst[i] = float_to_bf16_rne(ra);
                dst[i + half] = float_to_bf16_rne(rb);
            }
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, int64_t T, int64_t n, const float* gain, float eps,
                          float* out, hipStream_t stream) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)T), dim3(kNormThreads), 0, stream, x, n,
                       gain, eps, out);
    return hipGetLastError();
}

hipError_t launch_attn_prologue(float* q, float* k, int64_t T, int32_t nq, int32_t nkv,
                                int32_t D, const float* qn, const float* kn, const int32_t* pos,
                                float eps, float base, hipStream_t stream) {
    hipLaunchKernelGGL(attn_prologue_kernel, dim3((unsigned)T, (unsigned)(nq + nkv)), dim3(kWave),
                       0, stream, q, k, nullptr, nq, nkv, D, qn, kn, pos, eps, base, nullptr, nullptr,
                       (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_attn_prologue_kv(float* q, float* k, const float* v, int64_t T, int32_t nq,
                                   int32_t nkv, int32_t D, const float* qn, const float* kn,
                                   const int32_t* pos, float eps, float base, uint16_t* kc,
                                   uint16_t* vc, int64_t S_max, hipStream_t stream) {
    hipLaunchKernelGGL(attn_prologue_kernel, dim3((unsigned)T, (unsigned)(nq + 2 * nkv)), dim3(kWave),
                       0, stream, q, k, v, nq, nkv, D, qn, kn, pos, eps, base, kc, vc, S_max);
    return hipGetLastError();
}

}  // namespace q3moe
