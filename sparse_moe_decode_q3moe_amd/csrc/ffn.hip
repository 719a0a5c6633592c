// Sparse expert FFN on k-quant weights read in place (aprender issue #3714,
// gap G3 and "File facts": expert e at base + e*stride, gate/up Q4_K, down
// Q6_K or Q4_K per layer).  launch_expert_ffn sends hidden sizes that are a
// power-of-two number of super-blocks (up to 16) to the decode kernels in
// ffn_decode.hip; every other shape runs the generic pair of kernels here:
//   gateup: per (token, slot) pair and 8-row tile, g = Wg[e] x and u = Wu[e] x
//           for the same 8 rows, then h = silu(g) * u into the workspace;
//   down:   per (token, 8 output rows), y_s = Wd[e_s] h_s for every slot and
//           out = [out +] sum_s w_s y_s in slot order (no float atomics, so the
//           result is bitwise reproducible).
// Weights are dequantised in registers; nothing is repacked.  Each tile of
// contiguous rows is staged HBM -> LDS with 16-byte coalesced loads, then
// every lane parses its quant chunk from LDS.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRowTile = 8;   // rows per tile; 8 Q6_K rows of 3 blocks = 5040 B (16-B aligned)

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void copy16(uint8_t* dst, const uint8_t* __restrict__ src, int nbytes,
                                       int tid, int nthreads) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (int i = tid; i < nbytes / 16; i += nthreads) d4[i] = s4[i];
}

// Row dot of a Q4_K row (nb blocks) in LDS with x (nb*256 values in LDS);
// lanes walk the row's 8*nb quant chunks; result reduced over the wave.
__device__ __forceinline__ float q4k_row_dot(const uint8_t* row, int nb, const float* x, int lane) {
    float acc = 0.f;
    for (int c = lane; c < 8 * nb; c += kWave)
        acc += q4k_chunk_dot(row + (c >> 3) * kQ4KBytes, c & 7, x + (c >> 3) * kQK);
    return wave_sum(acc);
}

__device__ __forceinline__ float q6k_row_dot(const uint8_t* tile, int row_off, int nb,
                                             const float* x, int lane) {
    float acc = 0.f;
    for (int u = lane; u < 16 * nb; u += kWave)
        acc += q6k_unit_dot(tile, row_off + (u >> 4) * kQ6KBytes, u & 15, x + (u >> 4) * kQK);
    return wave_sum(acc);
}

// grid: (T*k pairs, F/8 row tiles); dynamic LDS: H*4 + 2*8*(H/256)*144 bytes.
__global__ __launch_bounds__(kThreads) void gateup_q4k_kernel(
    const float* __restrict__ hidden, int64_t H, int64_t F, int32_t E, int32_t k,
    const int32_t* __restrict__ idx, const uint8_t* __restrict__ gbase, int64_t gstride,
    const uint8_t* __restrict__ ubase, int64_t ustride, float* __restrict__ hbuf) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = (int)(H / kQK);
    const int rowb = nb * kQ4KBytes;
    float* xs = reinterpret_cast<float*>(smem);
    uint8_t* tg = smem + H * 4;
    uint8_t* tu = tg + kRowTile * rowb;

    const int64_t p = blockIdx.x;
    const int64_t t = p / k;
    const int64_t r0 = (int64_t)blockIdx.y * kRowTile;
    float* hout = hbuf + p * F + r0;
    const int e = idx[p];
    if (e < 0 || e >= E) {
        if (tid < kRowTile) hout[tid] = 0.f;
        return;
    }
    copy16(smem, reinterpret_cast<const uint8_t*>(hidden + t * H), (int)(H * 4), tid, kThreads);
    copy16(tg, gbase + (int64_t)e * gstride + r0 * rowb, kRowTile * rowb, tid, kThreads);
    copy16(tu, ubase + (int64_t)e * ustride + r0 * rowb, kRowTile * rowb, tid, kThreads);
    __syncthreads();
    for (int rr = wave; rr < kRowTile; rr += kWaves) {
        const float g = q4k_row_dot(tg + rr * rowb, nb, xs, lane);
        const float u = q4k_row_dot(tu + rr * rowb, nb, xs, lane);
        if (lane == 0) hout[rr] = silu(g) * u;
    }
}

// grid: (T, H/8); dynamic LDS: 4 waves x (F*4 + tile + 16) + 32*8*4 bytes.
__global__ __launch_bounds__(kThreads) void down_combine_kernel(
    int64_t H, int64_t F, int32_t E, int32_t k, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const uint8_t* __restrict__ dbase, int32_t qtype,
    int64_t dstride, const float* __restrict__ hbuf, float* __restrict__ out, int accumulate) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = (int)(F / kQK);
    const bool q6 = qtype == 2;
    const int rowb = nb * (q6 ? kQ6KBytes : kQ4KBytes);
    const int tile = kRowTile * rowb;
    const int region = (int)(F * 4) + tile + 16;
    float* hs = reinterpret_cast<float*>(smem + wave * region);
    uint8_t* wt = smem + wave * region + F * 4;
    float* ys = reinterpret_cast<float*>(smem + kWaves * region);

    const int64_t t = blockIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kRowTile;
    for (int s0 = 0; s0 < k; s0 += kWaves) {
        const int s = s0 + wave;
        const bool active = s < k;
        int e = -1;
        float ws = 0.f;
        if (active) {
            e = idx[t * k + s];
            ws = w[t * k + s];
        }
        const bool valid = active && e >= 0 && e < E;
        if (valid) {
            copy16(reinterpret_cast<uint8_t*>(hs),
                   reinterpret_cast<const uint8_t*>(hbuf + (t * k + s) * F), (int)(F * 4), lane,
                   kWave);
            copy16(wt, dbase + (int64_t)e * dstride + r0 * rowb, tile, lane, kWave);
        }
        __syncthreads();
        if (active) {
            for (int rr = 0; rr < kRowTile; ++rr) {
                float y = 0.f;
                if (valid)
                    y = q6 ? q6k_row_dot(wt, rr * rowb, nb, hs, lane)
                           : q4k_row_dot(wt + rr * rowb, nb, hs, lane);
                if (lane == 0) ys[s * kRowTile + rr] = valid ? ws * y : 0.f;
            }
        }
        __syncthreads();
    }
    if (tid < kRowTile) {
        float acc = 0.f;
        for (int s = 0; s < k; ++s) acc += ys[s * kRowTile + tid];
        float* o = out + t * H + r0 + tid;
        *o = accumulate ? *o + acc : acc;
    }
}

size_t gateup_lds(int64_t H) { return (size_t)(H * 4 + 2 * kRowTile * (H / kQK) * kQ4KBytes); }

size_t down_lds(int64_t F, int32_t qtype) {
    const int64_t rowb = (F / kQK) * (qtype == 2 ? kQ6KBytes : kQ4KBytes);
    return (size_t)(kWaves * (F * 4 + kRowTile * rowb + 16) + kMaxTopK * kRowTile * 4);
}

}  // namespace

size_t expert_ffn_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k) {
    const int64_t t = T > 0 ? T : 0;
    if (t >= kPrefillMinTokens) return prefill_workspace_bytes(t, H, F, E, k);
    // synchronisation words, then h: 8 bytes per value (the fused decode
    // kernel's tagged words; the other decode kernels use 4)
    const size_t h = (size_t)t * (size_t)k * (size_t)F * sizeof(uint64_t);
    return kFfnSyncBytes + ((h + 255) & ~(size_t)255);
}

size_t expert_ffn_status_offset(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k) {
    (void)T;
    (void)H;
    (void)F;
    (void)E;
    (void)k;
    return 0;
}

hipError_t launch_expert_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const int32_t* idx, const float* w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ws,
                             hipStream_t stream) {
    if (T >= kPrefillMinTokens)
        return launch_prefill_ffn(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, ws,
                                  stream);
    if (decode_ffn_supported(H, F, k))
        return launch_decode_ffn(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, ws,
                                 stream);
    float* hbuf = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kFfnSyncBytes);
    const size_t l1 = gateup_lds(H), l2 = down_lds(F, down.qtype);
    static LdsLimit lim1, lim2;
    hipError_t err;
    if ((err = ensure_lds(reinterpret_cast<const void*>(gateup_q4k_kernel), lim1, (int)l1)) != hipSuccess)
        return err;
    if ((err = ensure_lds(reinterpret_cast<const void*>(down_combine_kernel), lim2, (int)l2)) != hipSuccess)
        return err;
    hipLaunchKernelGGL(gateup_q4k_kernel, dim3((unsigned)(T * k), (unsigned)(F / kRowTile)),
                       dim3(kThreads), l1, stream, hidden, H, F, E, k, idx, gate.base, gate.stride,
                       up.base, up.stride, hbuf);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(down_combine_kernel, dim3((unsigned)T, (unsigned)(H / kRowTile)),
                       dim3(kThreads), l2, stream, H, F, E, k, idx, w, down.base, down.qtype,
                       down.stride, hbuf, out, accumulate);
    return hipGetLastError();
}

}  // namespace q3moe
