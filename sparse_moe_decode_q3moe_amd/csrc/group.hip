// Token -> expert grouping of the routed (token, slot) pairs: per-expert
// counts, offsets and the pair list ordered by (expert, pair), i.e. stable
// in token and slot order.  The batched (prefill) expert FFN reads each
// expert's tokens through this list (the pages' plan groups prefill tokens by
// expert: aprender issue #3714, gap list).
//
// One workgroup of 16 waves.  Wave w owns a contiguous segment of the pairs.
//   1. Every wave counts its segment into its own LDS histogram row.
//   2. Thread e turns column e into per-wave start positions, and a block
//      scan over experts adds the expert's offset.
//   3. Every wave scatters its segment in order, 64 pairs at a time.  Lanes
//      holding the same expert find each other with ten ballots (one per
//      index bit), take their rank among the lower lanes, and the group's
//      first lane advances that expert's position.  The order is stable
//      without any sort.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

constexpr int kGrpThreads = 1024;
constexpr int kGrpWaves = kGrpThreads / kWave;
constexpr int kGrpIndexBits = 10;                       // E <= 1024

// Inclusive scan of v over the workgroup's threads in thread order: each
// wave scans its 64 values with shuffles, wave 0 scans the wave totals
// (wsum, kGrpWaves ints of LDS), every wave adds the totals before it.  Two
// barriers; every thread of the workgroup must call it.
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* wsum, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    if (lane == kWave - 1) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int32_t w = lane < kGrpWaves ? wsum[lane] : 0;
#pragma unroll
        for (int off = 1; off < kGrpWaves; off <<= 1) {
            const int32_t t = __shfl_up(w, off, kWave);
            if (lane >= off) w += t;
        }
        if (lane < kGrpWaves) wsum[lane] = w;
    }
    __syncthreads();
    return wave > 0 ? v + wsum[wave - 1] : v;
}

__global__ __launch_bounds__(kGrpThreads) void group_by_expert_kernel(
    const int32_t* __restrict__ idx, int64_t n, int32_t E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pairs, int32_t* __restrict__ tile_off,
    int32_t tile_rows) {
    extern __shared__ int32_t lds_i32[];
    int32_t* hist = lds_i32;                            // [wave][E]
    int32_t* scan = lds_i32 + kGrpWaves * E;            // [kGrpThreads]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int i = tid; i < kGrpWaves * E; i += kGrpThreads) hist[i] = 0;
    __syncthreads();
    const int64_t seg = (n + kGrpWaves - 1) / kGrpWaves;
    const int64_t b0 = wave * seg;
    const int64_t b1 = b0 + seg < n ? b0 + seg : n;
    int32_t* my_hist = hist + wave * E;
    for (int64_t p = b0 + lane; p < b1; p += kWave) {
        const int32_t e = idx[p];
        if (e >= 0 && e < E) atomicAdd(my_hist + e, 1);
    }
    __syncthreads();

    int32_t total = 0;
    if (tid < E) {
        int32_t run = 0;
        for (int w = 0; w < kGrpWaves; ++w) {
            const int32_t c = hist[w * E + tid];
            hist[w * E + tid] = run;
            run += c;
        }
        total = run;
    }
    const int32_t incl = block_inclusive_scan(total, scan, tid);   // over experts
    if (tid < E) {
        const int32_t excl = incl - total;
        counts[tid] = total;
        offsets[tid] = excl;
        for (int w = 0; w < kGrpWaves; ++w) hist[w * E + tid] += excl;
    }
    if (tid == kGrpThreads - 1) offsets[E] = incl;
    __syncthreads();                                    // wsum is reused below
    if (tile_off) {                                     // tiles of tile_rows pairs per expert
        const int32_t tiles = (total + tile_rows - 1) / tile_rows;
        const int32_t tincl = block_inclusive_scan(tiles, scan, tid);
        if (tid < E) tile_off[tid] = tincl - tiles;
        if (tid == kGrpThreads - 1) tile_off[E] = tincl;
    }

    const uint64_t lower = (1ull << lane) - 1ull;
    for (int64_t c0 = b0; c0 < b1; c0 += kWave) {
        const int64_t p = c0 + lane;
        const int32_t e = p < b1 ? idx[p] : -1;
        const bool valid = e >= 0 && e < E;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < kGrpIndexBits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t set = __ballot(valid && bit);
            peers &= bit ? set : ~set;
        }
        const int rank = __popcll(peers & lower);
        int32_t base = 0;
        if (valid) {
            base = my_hist[e];
            pairs[base + rank] = (int32_t)p;
        }
        if (valid && rank == 0) my_hist[e] = base + __popcll(peers);
    }
}

}  // namespace

hipError_t launch_group_by_expert(const int32_t* idx, int64_t n, int32_t E, int32_t* counts,
                                  int32_t* offsets, int32_t* pairs, hipStream_t stream,
                                  int32_t* tile_off, int32_t tile_rows) {
    const size_t lds = ((size_t)kGrpWaves * E + kGrpThreads) * sizeof(int32_t);
    static LdsLimit lds_set;
    const hipError_t err = ensure_lds(reinterpret_cast<const void*>(group_by_expert_kernel), lds_set, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(group_by_expert_kernel, dim3(1), dim3(kGrpThreads), lds, stream, idx, n, E,
                       counts, offsets, pairs, tile_off, tile_rows);
    return hipGetLastError();
}

}  // namespace q3moe
