// Decoder-layer pieces around the MoE block at decode batch sizes: the bf16
// attention projections, the KV-cache write and grouped-query decode
// attention.  The layer of the pages runs input RMSNorm, the Q/K/V
// projections, per-head Q/K RMSNorm then NEOX RoPE (aprender PR #1228, "The
// fix"), attention over the cached positions, the O projection with the
// residual, post-attention RMSNorm, the MoE block and its residual; head_dim
// is 128 although hidden / heads is 64 (aprender issue #479, "Fix Applied").
//
//   bf16_gemv_kernel<TT, R>: y[t][n] = [y +] sum_k W[n][k] x[t][k] for up to
//       TT <= 16 tokens per pass, W bf16 [N][K].  A wave owns R rows and the
//       lanes split k in 16-byte pieces (8 weights), so every load is a
//       1 KiB coalesced row segment.  x is staged in LDS in chunks and shared
//       by the workgroup's 4 waves; the next chunk's weights and activations
//       are loaded into registers while the current one is multiplied.  One
//       transposed butterfly finally gives every lane group one (row, token)
//       total.  One launch can serve up to three matrices on the same input
//       (workgroups split by matrix) and apply the input RMSNorm on the way
//       into LDS (the Q/K/V projections after the layer's input norm).
//   kv_write_kernel: the new token's k and v, rounded to bf16 (nearest even),
//       into each sequence's cache at its position.
//   attn_partial_kernel<D, HPW>: flash-decode.  A workgroup per (position
//       chunk, kv head, sequence) stages the chunk's K and V rows in LDS in
//       tiles of 64 positions; its 4 waves share them and split the group's
//       query heads (HPW each).  For each tile: lane j scores position j,
//       the wave updates the running max and exp sum, and the lanes (now one
//       per d-range) accumulate the p-weighted V rows.  K rows are stored
//       with their 16-byte pieces XOR-swizzled by row, so that lane j reading
//       row j hits distinct banks.
//   attn_combine_kernel: merges the chunk records with the log-sum-exp rule.
#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace q3moe {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ GEMV --
constexpr int kGvThreads = 256;
constexpr int kGvWaves = kGvThreads / kWave;
constexpr int kGvStep = 8 * kWave;                  // k values per wave-wide load
constexpr int kGvLdsFloats = 16384;                 // 64 KiB of staged activations

constexpr int ilog2c(int v) { return v <= 1 ? 0 : 1 + ilog2c(v >> 1); }

// Sum of v[0..V) over the 64 lanes, transposed: the result in lane l is the
// total of value index l >> (6 - log2 V).  V is a power of two <= 64.
template <int V>
__device__ __forceinline__ float transposed_sum(float (&v)[V], int lane) {
    constexpr int LV = ilog2c(V);
    static_assert((1 << LV) == V && V <= 64, "V must be a power of two <= 64");
#pragma unroll
    for (int lev = 0; lev < LV; ++lev) {
        const int half = V >> (lev + 1);
        const int bit = 5 - lev;
        const bool up = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = up ? v[i] : v[i + half];
            const float keep = up ? v[i + half] : v[i];
            v[i] = keep + __shfl_xor(send, 1 << bit, kWave);
        }
    }
    float r = v[0];
#pragma unroll
    for (int bit = 5 - LV; bit >= 0; --bit) r += __shfl_xor(r, 1 << bit, kWave);
    return r;
}

template <int TT, int R>
struct GvShape {
    static constexpr int kc_w = 8192 / R;                          // 16 loads per lane per chunk
    static constexpr int kc_x = kGvLdsFloats / TT;
    static constexpr int KC = kc_w < kc_x ? kc_w : kc_x;           // k per chunk
    static constexpr int S = KC / kGvStep;                         // wave-wide steps per chunk
};

template <int S, int R>
__device__ __forceinline__ void gv_load_chunk(uint4 (&wb)[S][R], const uint16_t* W, int64_t N, int64_t K,
                                              int64_t n0, int64_t k0, int lane) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t k = k0 + s * kGvStep + 8 * lane;
        const bool kin = k < K;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = n0 + r < N ? n0 + r : N - 1;        // clamped; result dropped
            wb[s][r] = kin ? load_nt16(W + row * K + k) : make_uint4(0, 0, 0, 0);
        }
    }
}

// The activation chunk [TT][KC] moves through registers: each thread loads
// NX float4 of the next chunk while the current one is multiplied, then
// stores them to LDS after the barrier.
template <int TT, int R>
struct GvX {
    static constexpr int KC = GvShape<TT, R>::KC;
    static constexpr int NX = TT * KC / 4 / kGvThreads;
    static_assert(NX * 4 * kGvThreads == TT * KC, "chunk must split evenly over the threads");
};

template <int TT, int R, int NX>
__device__ __forceinline__ void gv_load_x(float4 (&xr)[NX], const float* x, int64_t K, int64_t T,
                                          int64_t t0, int64_t k0, int tid) {
    constexpr int KC = GvShape<TT, R>::KC;
#pragma unroll
    for (int u = 0; u < NX; ++u) {
        const int i = tid + u * kGvThreads;
        const int t = i / (KC / 4), c = i % (KC / 4);
        const int64_t k = k0 + 4 * c;
        xr[u] = (t0 + t < T && k < K) ? *reinterpret_cast<const float4*>(x + (t0 + t) * K + k)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int NX>
__device__ __forceinline__ void gv_store_x(float* xs, const float4 (&xr)[NX], int tid) {
#pragma unroll
    for (int u = 0; u < NX; ++u) *reinterpret_cast<float4*>(xs + 4 * (tid + u * kGvThreads)) = xr[u];
}

// The same with the input RMSNorm applied on the way into LDS: value k of
// token t becomes gain[k] * x * inv[t], formed in double and rounded once to
// f32 (gs: the gain in LDS, inv: the tokens' 1 / rms in LDS).
template <int TT, int R, int NX>
__device__ __forceinline__ void gv_store_x_norm(float* xs, const float4 (&xr)[NX], int tid, int64_t k0,
                                                const float* gs, const double* inv, int64_t K) {
    constexpr int KC = GvShape<TT, R>::KC;
#pragma unroll
    for (int u = 0; u < NX; ++u) {
        const int i = tid + u * kGvThreads;
        const int t = i / (KC / 4), c = i % (KC / 4);
        const int64_t k = k0 + 4 * c;
        float4 v = xr[u];
        if (k < K) {
            const double s = inv[t];
            const float4 g = *reinterpret_cast<const float4*>(gs + k);
            v = make_float4((float)((double)g.x * v.x * s), (float)((double)g.y * v.y * s),
                            (float)((double)g.z * v.z * s), (float)((double)g.w * v.w * s));
        }
        *reinterpret_cast<float4*>(xs + 4 * i) = v;
    }
}

template <int TT, int R, int S>
__device__ __forceinline__ void gv_mul_chunk(float (&acc)[R * TT], const uint4 (&wb)[S][R], const float* xs,
                                             int lane) {
    constexpr int KC = GvShape<TT, R>::KC;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float wf[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            wf[r][0] = bf16_lo(wb[s][r].x); wf[r][1] = bf16_hi(wb[s][r].x);
            wf[r][2] = bf16_lo(wb[s][r].y); wf[r][3] = bf16_hi(wb[s][r].y);
            wf[r][4] = bf16_lo(wb[s][r].z); wf[r][5] = bf16_hi(wb[s][r].z);
            wf[r][6] = bf16_lo(wb[s][r].w); wf[r][7] = bf16_hi(wb[s][r].w);
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float* xp = xs + t * KC + s * kGvStep + 8 * lane;
            const float4 xa = *reinterpret_cast<const float4*>(xp);
            const float4 xb = *reinterpret_cast<const float4*>(xp + 4);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float a = acc[r * TT + t];
                a = fmaf(wf[r][0], xa.x, a); a = fmaf(wf[r][1], xa.y, a);
                a = fmaf(wf[r][2], xa.z, a); a = fmaf(wf[r][3], xa.w, a);
                a = fmaf(wf[r][4], xb.x, a); a = fmaf(wf[r][5], xb.y, a);
                a = fmaf(wf[r][6], xb.z, a); a = fmaf(wf[r][7], xb.w, a);
                acc[r * TT + t] = a;
            }
        }
    }
}

// Up to three matrices sharing one input: workgroups [0, b1) work on
// matrix 0, [b1, b2) on matrix 1, the rest on matrix 2.  gain (or null) is
// the input RMSNorm's gain.
struct GvJob {
    const uint16_t* W0;
    const uint16_t* W1;
    const uint16_t* W2;
    float* y0;
    float* y1;
    float* y2;
    int64_t N0, N1, N2;
    int64_t b1, b2;
    const float* gain;
    float eps;
};

template <int TT, int R>
__global__ __launch_bounds__(kGvThreads) void bf16_gemv_kernel(GvJob job, int64_t K,
                                                               const float* __restrict__ x, int64_t T,
                                                               int64_t t0, int accumulate) {
    constexpr int KC = GvShape<TT, R>::KC, S = GvShape<TT, R>::S;
    constexpr int V = R * TT;
    __shared__ __align__(16) float xs[TT * KC];
    __shared__ double inv[TT];
    __shared__ double part[kGvWaves][TT];
    extern __shared__ __align__(16) float gs[];              // the gain, K values (norm only)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bx = blockIdx.x;
    const int m = bx < job.b1 ? 0 : (bx < job.b2 ? 1 : 2);
    const uint16_t* __restrict__ W = m == 0 ? job.W0 : (m == 1 ? job.W1 : job.W2);
    float* __restrict__ y = m == 0 ? job.y0 : (m == 1 ? job.y1 : job.y2);
    const int64_t N = m == 0 ? job.N0 : (m == 1 ? job.N1 : job.N2);
    const int64_t blk = bx - (m == 0 ? 0 : (m == 1 ? job.b1 : job.b2));
    const int64_t n0 = (blk * kGvWaves + wave) * R;
    const bool norm = job.gain != nullptr;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;

    uint4 wa[S][R], wb[S][R];
    constexpr int NX = GvX<TT, R>::NX;
    float4 xr[NX];
    gv_load_chunk<S, R>(wa, W, N, K, n0, 0, lane);
    if (norm) {
        // the gain into LDS and each token's 1 / rms: squares summed in
        // double (exact f32 squares) over the whole row, in a fixed order
        for (int64_t kk = tid; kk < K; kk += kGvThreads) gs[kk] = job.gain[kk];
        // every token's float4 of a chunk in flight together
        double ss[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) ss[t] = 0.0;
        for (int64_t c = tid; c < K / 4; c += kGvThreads) {
            float4 v[TT];
#pragma unroll
            for (int t = 0; t < TT; ++t)
                v[t] = t0 + t < T ? reinterpret_cast<const float4*>(x + (t0 + t) * K)[c]
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                double a = fma((double)v[t].x, (double)v[t].x, ss[t]);
                a = fma((double)v[t].y, (double)v[t].y, a);
                a = fma((double)v[t].z, (double)v[t].z, a);
                ss[t] = fma((double)v[t].w, (double)v[t].w, a);
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const double w = wave_sum_dpp_f64(ss[t]);
            if (lane == 0) part[wave][t] = w;
        }
        __syncthreads();
        if (tid < TT) {
            double tot = 0.0;
#pragma unroll
            for (int w = 0; w < kGvWaves; ++w) tot += part[w][tid];
            // slots past T (a partial last pass) are zeros and stay zeros
            inv[tid] = t0 + tid < T ? 1.0 / sqrt(tot / (double)K + (double)job.eps) : 0.0;
        }
    }
    gv_load_x<TT, R, NX>(xr, x, K, T, t0, 0, tid);
    for (int64_t k0 = 0; k0 < K; k0 += 2 * KC) {
        __syncthreads();
        if (norm) gv_store_x_norm<TT, R, NX>(xs, xr, tid, k0, gs, inv, K);
        else gv_store_x<NX>(xs, xr, tid);
        __syncthreads();
        if (k0 + KC < K) {
            gv_load_chunk<S, R>(wb, W, N, K, n0, k0 + KC, lane);
            gv_load_x<TT, R, NX>(xr, x, K, T, t0, k0 + KC, tid);
        }
        gv_mul_chunk<TT, R, S>(acc, wa, xs, lane);
        if (k0 + KC >= K) break;
        __syncthreads();
        if (norm) gv_store_x_norm<TT, R, NX>(xs, xr, tid, k0 + KC, gs, inv, K);
        else gv_store_x<NX>(xs, xr, tid);
        __syncthreads();
        if (k0 + 2 * KC < K) {
            gv_load_chunk<S, R>(wa, W, N, K, n0, k0 + 2 * KC, lane);
            gv_load_x<TT, R, NX>(xr, x, K, T, t0, k0 + 2 * KC, tid);
        }
        gv_mul_chunk<TT, R, S>(acc, wb, xs, lane);
    }

    const float s = transposed_sum<V>(acc, lane);
    constexpr int LV = ilog2c(V);
    if ((lane & ((1 << (6 - LV)) - 1)) == 0) {
        const int vi = lane >> (6 - LV);
        const int r = vi / TT, t = vi % TT;
        const int64_t row = n0 + r;
        if (row < N && t0 + t < T) {
            float* o = y + (t0 + t) * N + row;
            *o = accumulate ? *o + s : s;
        }
    }
}

template <int TT, int R>
hipError_t launch_gemv_rt(GvJob job, int64_t K, const float* x, int64_t T, int accumulate,
                          hipStream_t stream) {
    const int64_t rows_per_wg = (int64_t)kGvWaves * R;
    auto blocks = [&](int64_t n) { return (n + rows_per_wg - 1) / rows_per_wg; };
    job.b1 = blocks(job.N0);
    job.b2 = job.b1 + blocks(job.N1);
    const unsigned grid = (unsigned)(job.b2 + blocks(job.N2));
    const size_t lds = job.gain ? (size_t)K * sizeof(float) : 0;
    if (lds) {
        static LdsLimit lds_set;
        const hipError_t e = ensure_lds(reinterpret_cast<const void*>(bf16_gemv_kernel<TT, R>), lds_set,
                                        (int)lds);
        if (e != hipSuccess) return e;
    }
    for (int64_t t0 = 0; t0 < T; t0 += TT) {
        hipLaunchKernelGGL((bf16_gemv_kernel<TT, R>), dim3(grid), dim3(kGvThreads), lds, stream, job, K, x,
                           T, t0, accumulate);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

template <int TT>
hipError_t launch_gemv_tt(const GvJob& job, int64_t K, const float* x, int64_t T, int accumulate,
                          hipStream_t stream) {
    // rows per wave: keep about 1024 waves or more in flight
    const int64_t N = job.N0 + job.N1 + job.N2;
    if (N >= 4096) return launch_gemv_rt<TT, 4>(job, K, x, T, accumulate, stream);
    if (N >= 2048) return launch_gemv_rt<TT, 2>(job, K, x, T, accumulate, stream);
    return launch_gemv_rt<TT, 1>(job, K, x, T, accumulate, stream);
}

hipError_t launch_gemv_job(const GvJob& job, int64_t K, const float* x, int64_t T, int accumulate,
                           hipStream_t stream) {
    if (T <= 1) return launch_gemv_tt<1>(job, K, x, T, accumulate, stream);
    if (T <= 2) return launch_gemv_tt<2>(job, K, x, T, accumulate, stream);
    if (T <= 4) return launch_gemv_tt<4>(job, K, x, T, accumulate, stream);
    if (T <= 8) return launch_gemv_tt<8>(job, K, x, T, accumulate, stream);
    return launch_gemv_tt<16>(job, K, x, T, accumulate, stream);
}

// ------------------------------------------------- GEMV, matrix cores --
// bf16_gemv_mt_kernel: the same product for 9 or more tokens, 16 per pass,
// on v_mfma_f32_16x16x32_bf16, for K a multiple of 256 up to 4096.  A
// workgroup owns one block of 16 rows and all of k: K / 256 waves, each
// taking 256 consecutive k as 8 steps of 32.  The weights are the A operand
// straight from memory (lane l: row l % 16, the 8 weights at
// k = 32 s + 8 (l / 16) of step s; all 8 steps requested at once, after the
// activations); the activations are the B operand (lane l: token l % 16 at
// the same k), read as f32 and split in registers into two bf16 pieces,
// hi = bf16(v), lo = bf16(v - hi) (|v - hi - lo| <= 2^-17 |v|), so each
// product pair is exact and the sums run in f32.  With the input RMSNorm
// v = gain * x (rounded once to f32), and each token's 1 / rms (squares of
// x summed in double as the values arrive) scales that token's sums at the
// end, in double.  The waves' 16 x 16 partial tiles meet in LDS and are
// added in wave order.
constexpr int kMtSteps = 8;                          // 32-k steps per wave
constexpr int kMtWaveK = kMtSteps * 32;              // 256
constexpr int kMtMaxWaves = 16;                      // K <= 4096
constexpr int64_t kMtMinTokens = 9;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct MtJob {
    const uint16_t* W[3];
    float* y[3];
    int64_t N[3];
    int tile_end[3];            // cumulative 16-row tile counts
    const float* gain;          // the input RMSNorm's gain, or null
    float eps;
};

// two f32 values -> (hi, lo) bf16 pairs, round to nearest even
__device__ __forceinline__ void mt_split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const f32x2_t v = {a, b};
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    const f32x2_t r = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
}

// grid: the matrices' 16-row tiles; block: K / 256 waves.  x, W, gain
// 16-byte aligned; tokens t0 .. min(t0 + 16, T) - 1.
__global__ __launch_bounds__(kMtMaxWaves * kWave) void bf16_gemv_mt_kernel(MtJob job, int64_t K,
                                                                          const float* __restrict__ x,
                                                                          int64_t T, int64_t t0,
                                                                          int accumulate) {
    __shared__ __align__(16) float red[kMtMaxWaves][4][kWave];
    __shared__ double ssw[kMtMaxWaves][16];
    extern __shared__ __align__(16) float gs[];                 // the gain's K values (norm only)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int bx = blockIdx.x;
    const int mi = bx < job.tile_end[0] ? 0 : bx < job.tile_end[1] ? 1 : 2;
    const int tile = bx - (mi == 0 ? 0 : job.tile_end[mi - 1]);
    const uint16_t* __restrict__ W = job.W[mi];
    float* __restrict__ y = job.y[mi];
    const int64_t N = job.N[mi];
    const int64_t n0 = (int64_t)tile * 16;
    const bool norm = job.gain != nullptr;
    const int c = lane & 15, kb = lane >> 4;                    // A row / B column, k block
    const int64_t kw = (int64_t)wave * kMtWaveK + 8 * kb;
    const int64_t wrow = n0 + c < N ? n0 + c : N - 1;           // clamped; its sums are dropped
    const int64_t tok = t0 + c < T ? t0 + c : t0;               // clamped; its column is dropped

    if (norm) {
        for (int i = tid; i < K / 4; i += blockDim.x)
            reinterpret_cast<float4*>(gs)[i] = reinterpret_cast<const float4*>(job.gain)[i];
    }
    float4 xa[kMtSteps], xb[kMtSteps];
    const float* xp = x + tok * K + kw;
#pragma unroll
    for (int s = 0; s < kMtSteps; ++s) {
        xa[s] = *reinterpret_cast<const float4*>(xp + 32 * s);
        xb[s] = *reinterpret_cast<const float4*>(xp + 32 * s + 4);
    }
    u32x4_t wv[kMtSteps];
    const uint16_t* wp = W + wrow * K + kw;
#pragma unroll
    for (int s = 0; s < kMtSteps; ++s)
        wv[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(wp + 32 * s));

    double ss = 0.0;
    if (norm) {
#pragma unroll
        for (int s = 0; s < kMtSteps; ++s) {
            const float v[8] = {xa[s].x, xa[s].y, xa[s].z, xa[s].w, xb[s].x, xb[s].y, xb[s].z, xb[s].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fma((double)v[i], (double)v[i], ss);
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        if (kb == 0) ssw[wave][c] = ss;
        __syncthreads();                                        // gs and ssw written
#pragma unroll
        for (int s = 0; s < kMtSteps; ++s) {
            const float4 ga = *reinterpret_cast<const float4*>(gs + kw + 32 * s);
            const float4 gb = *reinterpret_cast<const float4*>(gs + kw + 32 * s + 4);
            xa[s] = make_float4(ga.x * xa[s].x, ga.y * xa[s].y, ga.z * xa[s].z, ga.w * xa[s].w);
            xb[s] = make_float4(gb.x * xb[s].x, gb.y * xb[s].y, gb.z * xb[s].z, gb.w * xb[s].w);
        }
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMtSteps; ++s) {
        uint32_t h[4], l[4];
        mt_split2(xa[s].x, xa[s].y, h[0], l[0]);
        mt_split2(xa[s].z, xa[s].w, h[1], l[1]);
        mt_split2(xb[s].x, xb[s].y, h[2], l[2]);
        mt_split2(xb[s].z, xb[s].w, h[3], l[3]);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, wv[s]);
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, u32x4_t{h[0], h[1], h[2], h[3]});
        const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, u32x4_t{l[0], l[1], l[2], l[3]});
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
        float sum[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum[i] += red[w][i][lane];
        const int64_t t = t0 + c;
        double inv = 1.0;
        if (norm) {
            double tot = 0.0;
            for (int w = 0; w < nw; ++w) tot += ssw[w][c];
            inv = 1.0 / sqrt(tot / (double)K + (double)job.eps);
        }
        if (t < T) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = n0 + 4 * kb + i;
                if (n < N) {
                    const float v = norm ? (float)((double)sum[i] * inv) : sum[i];
                    float* o = y + t * N + n;
                    *o = accumulate ? *o + v : v;
                }
            }
        }
    }
}

bool mt_path(int64_t T, int64_t K) {
    return T >= kMtMinTokens && K % kMtWaveK == 0 && K <= (int64_t)kMtMaxWaves * kMtWaveK;
}

hipError_t launch_gemv_mt(MtJob job, int64_t K, const float* x, int64_t T, int accumulate,
                          hipStream_t stream) {
    int tiles = 0;
    for (int i = 0; i < 3; ++i) {
        tiles += (int)((job.N[i] + 15) / 16);
        job.tile_end[i] = tiles;
    }
    const int threads = (int)(K / kMtWaveK) * kWave;
    const size_t lds = job.gain ? (size_t)K * sizeof(float) : 0;
    for (int64_t t0 = 0; t0 < T; t0 += 16) {
        hipLaunchKernelGGL(bf16_gemv_mt_kernel, dim3((unsigned)tiles), dim3(threads), lds, stream, job, K, x, T,
                           t0, accumulate);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// ------------------------------------------------------------- KV write --

// grid: B workgroups.  A position outside [0, S_max) writes nothing.
__global__ void kv_write_kernel(const float* __restrict__ k_new, const float* __restrict__ v_new,
                                int32_t n_kv, int32_t D, const int32_t* __restrict__ pos,
                                uint16_t* __restrict__ kcache, uint16_t* __restrict__ vcache,
                                int64_t S_max) {
    const int64_t b = blockIdx.x;
    const int p = pos[b];
    if (p < 0 || p >= S_max) return;
    for (int i = threadIdx.x; i < n_kv * D; i += blockDim.x) {
        const int g = i / D, d = i % D;
        const int64_t src = (b * n_kv + g) * (int64_t)D + d;
        const int64_t dst = ((b * n_kv + g) * S_max + p) * (int64_t)D + d;
        kcache[dst] = float_to_bf16_rne(k_new[src]);
        vcache[dst] = float_to_bf16_rne(v_new[src]);
    }
}

// ------------------------------------------------------------- attention --
constexpr int kAtTile = 64;                // positions per LDS tile (one per lane)
constexpr int kAtThreads = 256;
constexpr int kAtWaves = kAtThreads / kWave;
constexpr int kAtMaxGroup = 16;            // query heads per kv head
constexpr int kAtMaxD = 256;
constexpr int kDppQuadXor1 = 0xb1, kDppQuadXor2 = 0x4e, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float readlane_f32(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor4>(v));
    v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f32<kDppQuadXor1>(v);
    v += dpp_f32<kDppQuadXor2>(v);
    v += dpp_f32<kDppRowRor4>(v);
    v += dpp_f32<kDppRowRor8>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// LDS bytes: K tile, V tile (bf16 [64][D] each), q [group][D] f32 and the
// per-wave probabilities [4][64][HPW] f32.
inline int at_lds_bytes(int D, int group, int hpw) {
    return 2 * kAtTile * D * 2 + group * D * 4 + kAtWaves * kAtTile * hpw * 4;
}

// Per (sequence, query head, chunk) record of D + 2 floats: running max m,
// exp sum l, then the D accumulated values (all relative to m).
template <int D, int HPW>
__global__ __launch_bounds__(kAtThreads) void attn_partial_kernel(
    const float* __restrict__ q, int32_t n_q, int32_t n_kv, const uint16_t* __restrict__ kcache,
    const uint16_t* __restrict__ vcache, int64_t S_max, const int32_t* __restrict__ len,
    float scale, float* __restrict__ part, int nchunks, int nsub) {
    constexpr int CPR = D / 8;                       // 16-byte pieces per row
    constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;   // swizzle mask
    constexpr int DPL = D / kWave;                   // V values per lane
    constexpr int REC = D + 2;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* lk = smem;
    uint8_t* lv = smem + kAtTile * D * 2;
    const int group = n_q / n_kv;
    float* lq = reinterpret_cast<float*>(smem + 2 * kAtTile * D * 2);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* lp = lq + group * D + wave * kAtTile * HPW;

    const int c = blockIdx.x, g = blockIdx.y;
    const int64_t b = blockIdx.z;
    int L = len[b];
    if (L < 1 || L > S_max) L = 0;                   // invalid length: every record stays empty
    const int64_t kv_row0 = (b * n_kv + g) * S_max;
    const int h0 = wave * HPW;                       // first head of this wave within the group

    for (int i = tid; i < group * D; i += kAtThreads) lq[i] = q[(b * n_q + g * group) * (int64_t)D + i];

    float m[HPW], l[HPW], acc[HPW][DPL];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        m[h] = -__builtin_inff();
        l[h] = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[h][d] = 0.f;
    }

    for (int sub = 0; sub < nsub; ++sub) {
        const int j0 = (c * nsub + sub) * kAtTile;
        const int nj = L - j0 < kAtTile ? L - j0 : kAtTile;
        if (nj <= 0) break;
        __syncthreads();                             // the previous tile is fully read
        {
            // K rows swizzled (slot s of row r holds piece s ^ (r & SWM)), V rows plain
            const uint8_t* kg = reinterpret_cast<const uint8_t*>(kcache + (kv_row0 + j0) * D);
            const uint8_t* vg = reinterpret_cast<const uint8_t*>(vcache + (kv_row0 + j0) * D);
            const int n16 = nj * CPR;
            for (int base = wave * kWave; base < n16; base += kAtThreads) {
                const int i = base + lane;
                if (i < n16) {
                    const int r = i / CPR, s = i % CPR;
                    const int piece = s ^ (r & SWM);
                    __builtin_amdgcn_global_load_lds(kg + (int64_t)(r * CPR + piece) * 16,
                                                     (lds_ptr_t)(lk + base * 16), 16, 0, kCachePolicyNt);
                    __builtin_amdgcn_global_load_lds(vg + (int64_t)i * 16, (lds_ptr_t)(lv + base * 16), 16, 0,
                                                     kCachePolicyNt);
                }
            }
        }
        wait_all_loads();
        __syncthreads();

        // scores: lane j <-> position j0 + j
        float s[HPW];
#pragma unroll
        for (int h = 0; h < HPW; ++h) s[h] = 0.f;
        const uint8_t* krow = lk + lane * D * 2;
#pragma unroll 4
        for (int cc = 0; cc < CPR; ++cc) {
            const uint4 kw = *reinterpret_cast<const uint4*>(krow + ((cc ^ (lane & SWM)) * 16));
            const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                                 bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
#pragma unroll
            for (int h = 0; h < HPW; ++h) {
                const int hh = h0 + h < group ? h0 + h : 0;
                const float4 qa = *reinterpret_cast<const float4*>(lq + hh * D + cc * 8);
                const float4 qb = *reinterpret_cast<const float4*>(lq + hh * D + cc * 8 + 4);
                float a = s[h];
                a = fmaf(qa.x, kf[0], a); a = fmaf(qa.y, kf[1], a);
                a = fmaf(qa.z, kf[2], a); a = fmaf(qa.w, kf[3], a);
                a = fmaf(qb.x, kf[4], a); a = fmaf(qb.y, kf[5], a);
                a = fmaf(qb.z, kf[6], a); a = fmaf(qb.w, kf[7], a);
                s[h] = a;
            }
        }
        const bool valid = lane < nj;
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
            const float sc = valid ? scale * s[h] : -__builtin_inff();
            const float mn = fmaxf(m[h], wave_max_dpp(sc));
            const float p = valid ? expf(sc - mn) : 0.f;
            const float corr = expf(m[h] - mn);      // 0 on the first tile (m = -inf)
            l[h] = l[h] * corr + wave_sum_dpp(p);
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[h][d] *= corr;
            m[h] = mn;
            lp[lane * HPW + h] = p;
        }
        // p-weighted V rows: lane owns d = DPL*lane .. +DPL
#pragma unroll 8
        for (int j = 0; j < nj; ++j) {
            float pj[HPW];
#pragma unroll
            for (int h = 0; h < HPW; ++h) pj[h] = lp[j * HPW + h];
            float vf[DPL];
            if constexpr (DPL == 1) {
                vf[0] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(lv + j * D * 2 + lane * 2)) << 16);
            } else if constexpr (DPL == 2) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(lv + j * D * 2 + lane * 4);
                vf[0] = bf16_lo(w);
                vf[1] = bf16_hi(w);
            } else {
                const uint2 w = *reinterpret_cast<const uint2*>(lv + j * D * 2 + lane * 8);
                vf[0] = bf16_lo(w.x); vf[1] = bf16_hi(w.x);
                vf[2] = bf16_lo(w.y); vf[3] = bf16_hi(w.y);
            }
#pragma unroll
            for (int h = 0; h < HPW; ++h)
#pragma unroll
                for (int d = 0; d < DPL; ++d) acc[h][d] = fmaf(pj[h], vf[d], acc[h][d]);
        }
    }

#pragma unroll
    for (int h = 0; h < HPW; ++h) {
        if (h0 + h >= group) break;
        float* pr = part + ((b * n_q + g * group + h0 + h) * (int64_t)nchunks + c) * REC;
        if (lane == 0) {
            pr[0] = m[h];
            pr[1] = l[h];
        }
#pragma unroll
        for (int d = 0; d < DPL; ++d) pr[2 + DPL * lane + d] = acc[h][d];
    }
}

// grid: (n_q, B); one thread per output value, with the chunk weights
// exp(m_c - M) and the denominator formed once in LDS.  A record with
// m = -inf (a chunk past the sequence end) adds nothing; a sequence without
// any valid record yields 0 / 0.
constexpr int kCbChunks = 256;             // chunk weights held in LDS per pass

__global__ void attn_combine_kernel(const float* __restrict__ part, int32_t n_q, int32_t D,
                                    int nchunks, float* __restrict__ out) {
    __shared__ float fw[kCbChunks];
    __shared__ float red[kAtMaxD / kWave];
    __shared__ float sM;
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t b = blockIdx.y;
    const int rec = D + 2;
    const float* pr = part + (b * n_q + h) * (int64_t)nchunks * rec;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    float M = -__builtin_inff();
    for (int c = tid; c < nchunks; c += blockDim.x) M = fmaxf(M, pr[c * rec]);
    M = wave_max_dpp(M);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    if (tid == 0) {
        float m = red[0];
        for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
        sM = m;
    }
    __syncthreads();
    M = sM;
    float Ls = 0.f, a = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += kCbChunks) {
        const int nc = nchunks - c0 < kCbChunks ? nchunks - c0 : kCbChunks;
        __syncthreads();
        for (int c = tid; c < nc; c += blockDim.x) {
            const float mc = pr[(c0 + c) * rec];
            fw[c] = mc == -__builtin_inff() ? 0.f : expf(mc - M);
        }
        __syncthreads();
        if (tid < D) {
#pragma unroll 8
            for (int c = 0; c < nc; ++c) {
                const float f = fw[c];
                Ls = fmaf(pr[(c0 + c) * rec + 1], f, Ls);
                a = fmaf(pr[(c0 + c) * rec + 2 + tid], f, a);
            }
        }
    }
    if (tid < D) out[(b * n_q + h) * (int64_t)D + tid] = a / Ls;
}

// Tiles per workgroup: one while the (sequence, kv head, tile) triples do
// not fill the chip, more once they do, which keeps the records a small
// fraction of the K/V bytes.
int at_nsub(int64_t B, int32_t n_kv, int64_t S_max) {
    const int64_t tiles = B * n_kv * ((S_max + kAtTile - 1) / kAtTile);
    int nsub = 1;
    while (nsub < 8 && tiles / (2 * nsub) >= 1024) nsub *= 2;
    return nsub;
}

int at_nchunks(int64_t S_max, int nsub) {
    const int64_t per = (int64_t)nsub * kAtTile;
    return (int)((S_max + per - 1) / per);
}

template <int D, int HPW>
hipError_t launch_attn_dh(const float* q, int64_t B, int32_t n_q, int32_t n_kv,
                          const uint16_t* kcache, const uint16_t* vcache, int64_t S_max,
                          const int32_t* len, float scale, float* out, void* ws, hipStream_t stream) {
    const int nsub = at_nsub(B, n_kv, S_max);
    const int nchunks = at_nchunks(S_max, nsub);
    const int lds = at_lds_bytes(D, n_q / n_kv, HPW);
    static LdsLimit lim;
    hipError_t err = ensure_lds(reinterpret_cast<const void*>(attn_partial_kernel<D, HPW>), lim, lds);
    if (err != hipSuccess) return err;
    float* part = static_cast<float*>(ws);
    hipLaunchKernelGGL((attn_partial_kernel<D, HPW>), dim3((unsigned)nchunks, (unsigned)n_kv, (unsigned)B),
                       dim3(kAtThreads), lds, stream, q, n_q, n_kv, kcache, vcache, S_max, len, scale, part,
                       nchunks, nsub);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)n_q, (unsigned)B), dim3(D), 0, stream, part, n_q, D,
                       nchunks, out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_attn_d(const float* q, int64_t B, int32_t n_q, int32_t n_kv, const uint16_t* kcache,
                         const uint16_t* vcache, int64_t S_max, const int32_t* len, float scale,
                         float* out, void* ws, hipStream_t stream) {
    const int group = n_q / n_kv;
    if (group <= kAtWaves)
        return launch_attn_dh<D, 1>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
    if (group <= 2 * kAtWaves)
        return launch_attn_dh<D, 2>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
    return launch_attn_dh<D, 4>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
}

}  // namespace

hipError_t launch_bf16_gemv(const uint16_t* W, int64_t N, int64_t K, const float* x, int64_t T,
                            float* y, int accumulate, hipStream_t stream) {
    if (gemm_path(T, K)) return launch_bf16_gemm(W, N, K, x, T, y, accumulate, stream);
    if (mt_path(T, K)) {
        MtJob mj{{W, nullptr, nullptr}, {y, nullptr, nullptr}, {N, 0, 0}, {0, 0, 0}, nullptr, 0.f};
        return launch_gemv_mt(mj, K, x, T, accumulate, stream);
    }
    GvJob job{W, nullptr, nullptr, y, nullptr, nullptr, N, 0, 0, 0, 0, nullptr, 0.f};
    return launch_gemv_job(job, K, x, T, accumulate, stream);
}

hipError_t launch_bf16_gemv3(const uint16_t* W0, int64_t N0, const uint16_t* W1, int64_t N1,
                             const uint16_t* W2, int64_t N2, int64_t K, const float* x, int64_t T,
                             const float* gain, float eps, float* y0, float* y1, float* y2,
                             hipStream_t stream) {
    if (!gain && gemm_path(T, K)) {          // many tokens: one matrix-core GEMM launch
        const uint16_t* Ws[3];
        float* ys[3];
        int64_t Ns[3];
        int n = 0;
        const uint16_t* W_in[3] = {W0, W1, W2};
        float* y_in[3] = {y0, y1, y2};
        const int64_t N_in[3] = {N0, N1, N2};
        for (int i = 0; i < 3; ++i)
            if (N_in[i]) {
                Ws[n] = W_in[i];
                ys[n] = y_in[i];
                Ns[n++] = N_in[i];
            }
        return launch_bf16_gemm_multi(Ws, ys, Ns, n, K, x, T, 0, stream);
    }
    if (mt_path(T, K)) {                       // 9+ tokens (with the norm also 64+)
        MtJob mj{{W0, W1, W2}, {y0, y1, y2}, {N0, N1, N2}, {0, 0, 0}, gain, eps};
        return launch_gemv_mt(mj, K, x, T, 0, stream);
    }
    GvJob job{W0, W1, W2, y0, y1, y2, N0, N1, N2, 0, 0, gain, eps};
    return launch_gemv_job(job, K, x, T, 0, stream);
}

hipError_t launch_kv_write(const float* k_new, const float* v_new, int64_t B, int32_t n_kv,
                           int32_t D, const int32_t* pos, uint16_t* kcache, uint16_t* vcache,
                           int64_t S_max, hipStream_t stream) {
    const int n = n_kv * D;
    const int threads = n < 1024 ? ((n + kWave - 1) / kWave) * kWave : 1024;
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)B), dim3(threads), 0, stream, k_new, v_new, n_kv, D, pos,
                       kcache, vcache, S_max);
    return hipGetLastError();
}

bool gqa_attention_supported(int32_t n_q, int32_t n_kv, int32_t D) {
    return n_kv >= 1 && n_q >= n_kv && n_q % n_kv == 0 && n_q / n_kv <= kAtMaxGroup &&
           (D == 64 || D == 128 || D == 256);
}

size_t gqa_attention_workspace_bytes(int64_t B, int32_t n_q, int32_t n_kv, int32_t D, int64_t S_max) {
    if (B <= 0 || S_max <= 0) return 0;
    const int nchunks = at_nchunks(S_max, at_nsub(B, n_kv, S_max));
    return (size_t)B * n_q * nchunks * (D + 2) * sizeof(float);
}

hipError_t launch_gqa_attention(const float* q, int64_t B, int32_t n_q, int32_t n_kv, int32_t D,
                                const uint16_t* kcache, const uint16_t* vcache, int64_t S_max,
                                const int32_t* len, float scale, float* out, void* ws,
                                hipStream_t stream) {
    switch (D) {
        case 64: return launch_attn_d<64>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
        case 128: return launch_attn_d<128>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
        default: return launch_attn_d<256>(q, B, n_q, n_kv, kcache, vcache, S_max, len, scale, out, ws, stream);
    }
}

}  // namespace q3moe
