// The attention side of batched prefill (aprender issue #3714, 0.70.3 gap
// list: prefill runs token by token; the fix batches the Q/K/V projections,
// the RoPE rows and the attention of the prompt, head_dim 128).  Three
// kernels; the per-row QK-norm + RoPE is attn_prologue_kernel (norm.hip),
// which already takes T rows.
//
// bf16_gemm_kernel: Y[T x N] (+)= X[T x K] W[N x K]^T for the projections of
//   many tokens, on the matrix cores.  W is bf16 (exact in the products); X
//   is f32, split on its way into LDS into two bf16 pieces hi = bf16(x),
//   lo = bf16(x - hi) (|x - hi - lo| <= 2^-17 |x|), so each product pair is
//   exact and the sums run in f32.  Workgroup tile 64 tokens x 128 rows (64
//   when that leaves the device short of workgroups), k in stages of 64
//   staged through LDS one stage ahead (double buffer, one barrier per
//   stage); each of the 4 waves owns 32 tokens x 64 (32) rows as blocks of
//   v_mfma_f32_16x16x32_bf16, two per block and 32 k (hi, lo).  Up to three
//   matrices on one input share one launch (the Q, K and V projections).
//
// kv_rows_kernel: row t of the new keys and values, rounded to bf16, into
//   slot pos[t] of one sequence's caches.
//
// prefill_attn_kernel: causal attention of T queries of one sequence over
//   its cache (query t sees positions 0 .. pos[t]), GQA.  A workgroup of 12
//   waves takes 64 query rows = (64 / G tokens) x (the G query heads of one
//   kv head): 4 row waves of 16 rows each, times 3 key splits that take every
//   third K/V tile of 64 positions, each split streaming its tiles through its
//   own LDS buffer (V transposed on the way in: each thread packs one value
//   of 4 keys into an 8-byte store); at the end the splits' O,
//   running maximum and sum meet in LDS and are merged with the log-sum-exp
//   rule.  Per tile each wave forms S^T = K Q^T for its
//   16 rows (K as the A operand, the query pieces, held in registers, as B),
//   so a lane holds 16 scores of ONE query row and the row's online softmax
//   needs two cross-lane steps; P = exp(S - m) (f32) is split into two bf16
//   pieces and O += P V uses the same lane's 8 keys per 32-key step as its
//   A operand (the k order inside a product does not matter), with the
//   matching 8 rows of V^T as B.  O, the running max and the sum stay in
//   f32; the output is O / sum.
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16, as in prefill.hip): A lane
// l holds row l % 16, k = 8 (l / 16) .. + 7; B lane l holds column l % 16 at
// the same k; C lane l holds rows 4 (l / 16) + r (r = 0..3), column l % 16.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// hi = bf16(x), lo = bf16(x - hi), both round to nearest even.
__device__ __forceinline__ void split2(float x, uint32_t& hi, uint32_t& lo) {
    hi = bf16_rne_bits(x);
    lo = bf16_rne_bits(x - bf16_bits_to_float(hi));
}

// ----------------------------------------------------------------- GEMM --

constexpr int kGmThreads = 256;
constexpr int kGmBM = 64;                      // tokens per workgroup tile
constexpr int kGmBK = 64;                      // k per stage
constexpr int kGmStride = kGmBK * 2 + 16;      // bytes per LDS row (144: 16 bytes of padding)
constexpr int kGmArrA = kGmBM * kGmStride;     // one [64][64] bf16 array

template <int BN>
struct GmGeom {
    static constexpr int BUF = 2 * kGmArrA + BN * kGmStride;   // A hi, A lo, B
    static constexpr int LDS = 2 * BUF;                         // double buffer
    static constexpr int NB = BN / 32;                          // 16-row blocks per wave
    static constexpr int BLOADS = BN / 32;                      // 16-byte W loads per thread and stage
};

// Up to three matrices on one input: workgroup x indexes the concatenated
// row tiles of the matrices.
struct GemmJob {
    const uint16_t* W[3];
    float* y[3];
    int64_t N[3];
    int tile_end[3];            // cumulative row-tile counts
};

// grid: (total row tiles, ceil(T / 64)).  K % 64 == 0; x, W 16-byte aligned.
// Wave w owns tokens 32 (w / 2) .. + 31 and rows (BN / 2)(w % 2) .. of the tile.
template <int BN>
__global__ __launch_bounds__(kGmThreads) void bf16_gemm_kernel(GemmJob job, int64_t K,
                                                               const float* __restrict__ x, int64_t T,
                                                               int accumulate) {
    using Gm = GmGeom<BN>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bx = blockIdx.x;
    const int mi = bx < job.tile_end[0] ? 0 : bx < job.tile_end[1] ? 1 : 2;
    const int tile = bx - (mi == 0 ? 0 : job.tile_end[mi - 1]);
    const uint16_t* __restrict__ W = job.W[mi];
    float* __restrict__ y = job.y[mi];
    const int64_t N = job.N[mi];
    const int64_t n0 = (int64_t)tile * BN, t0 = (int64_t)blockIdx.y * kGmBM;
    const int wm = wave >> 1, wn = wave & 1;

    float4 ax[4];
    uint4 bw[Gm::BLOADS];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = tid + j * kGmThreads, tok = f >> 4, k4 = f & 15;
            const int64_t t = t0 + tok < T ? t0 + tok : T - 1;
            ax[j] = *reinterpret_cast<const float4*>(x + t * K + k0 + 4 * k4);
        }
#pragma unroll
        for (int j = 0; j < Gm::BLOADS; ++j) {
            const int f = tid + j * kGmThreads, row = f >> 3, k8 = f & 7;
            const int64_t n = n0 + row < N ? n0 + row : N - 1;
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W + n * K + k0 + 8 * k8));
            bw[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store = [&](uint8_t* buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int f = tid + j * kGmThreads, tok = f >> 4, k4 = f & 15;
            const float v[4] = {ax[j].x, ax[j].y, ax[j].z, ax[j].w};
            uint32_t h[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) split2(v[i], h[i], l[i]);
            const int off = tok * kGmStride + 8 * k4;
            *reinterpret_cast<uint2*>(buf + off) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            *reinterpret_cast<uint2*>(buf + kGmArrA + off) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
        }
#pragma unroll
        for (int j = 0; j < Gm::BLOADS; ++j) {
            const int f = tid + j * kGmThreads, row = f >> 3, k8 = f & 7;
            *reinterpret_cast<uint4*>(buf + 2 * kGmArrA + row * kGmStride + 16 * k8) = bw[j];
        }
    };

    f32x4_t acc[2][Gm::NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < Gm::NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int stages = (int)(K / kGmBK);
    load(0);
    store(smem);
    __syncthreads();
    const int fr = lane & 15, fk = 16 * (lane >> 4);          // fragment row, byte offset of k
    for (int s = 0; s < stages; ++s) {
        const uint8_t* cur = smem + (s & 1) * Gm::BUF;
        if (s + 1 < stages) load((int64_t)(s + 1) * kGmBK);
#pragma unroll
        for (int kk = 0; kk < kGmBK / 32; ++kk) {
            bf16x8_t bfr[Gm::NB];
#pragma unroll
            for (int j = 0; j < Gm::NB; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(
                    cur + 2 * kGmArrA + ((BN / 2) * wn + 16 * j + fr) * kGmStride + 64 * kk + fk);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ro = (32 * wm + 16 * i + fr) * kGmStride + 64 * kk + fk;
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(cur + ro);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(cur + kGmArrA + ro);
#pragma unroll
                for (int j = 0; j < Gm::NB; ++j) {
                    acc[i][j] = mfma32(ah, bfr[j], acc[i][j]);
                    acc[i][j] = mfma32(al, bfr[j], acc[i][j]);
                }
            }
        }
        if (s + 1 < stages) store(smem + ((s + 1) & 1) * Gm::BUF);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < Gm::NB; ++j) {
            const int64_t n = n0 + (BN / 2) * wn + 16 * j + fr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + 32 * wm + 16 * i + 4 * (lane >> 4) + r;
                if (t < T && n < N) {
                    float* dst = y + t * N + n;
                    *dst = accumulate ? *dst + acc[i][j][r] : acc[i][j][r];
                }
            }
        }
}

// ---------------------------------------------------------------- KV rows --

// grid: T workgroups of 256 threads; row t of k_new / v_new ([n_kv][D] f32)
// into slot pos[t] of the caches [n_kv][S_max][D] (nothing for a position
// outside [0, S_max)).
__global__ __launch_bounds__(256) void kv_rows_kernel(const float* __restrict__ k_new,
                                                      const float* __restrict__ v_new, int32_t nkv,
                                                      int32_t D, const int32_t* __restrict__ pos,
                                                      uint16_t* __restrict__ kc,
                                                      uint16_t* __restrict__ vc, int64_t S_max) {
    const int64_t t = blockIdx.x;
    const int64_t p = pos[t];
    if (p < 0 || p >= S_max) return;
    const int n = nkv * D;
    for (int i = threadIdx.x; i < n; i += 256) {
        const int g = i / D, d = i % D;
        const int64_t dst = ((int64_t)g * S_max + p) * D + d;
        kc[dst] = float_to_bf16_rne(k_new[t * n + i]);
        vc[dst] = float_to_bf16_rne(v_new[t * n + i]);
    }
}

// ------------------------------------------------------- prefill attention --

constexpr int kPaD = 128;                      // head_dim
constexpr int kPaBlk = 1;                      // 16-row blocks per wave
constexpr int kPaRowWaves = 4;                 // waves across the query rows
constexpr int kPaSplit = 3;                    // wave groups across the key tiles
constexpr int kPaWaves = kPaRowWaves * kPaSplit;
constexpr int kPaRows = 16 * kPaBlk * kPaRowWaves;   // query rows per workgroup
constexpr int kPaKeys = 64;                    // positions per K/V tile
constexpr int kPaKStride = kPaD * 2 + 16;      // K tile row: 272 bytes
constexpr int kPaVStride = kPaKeys * 2 + 16;   // V^T tile row: 144 bytes
constexpr int kPaKBytes = kPaKeys * kPaKStride;
constexpr int kPaTileLds = kPaKBytes + kPaD * kPaVStride;   // 17,408 + 18,432: one split's tile
constexpr int kPaLds = kPaSplit * kPaTileLds;
constexpr int kPaRecF = 34 * kPaBlk;           // merge record per lane: 32 O values, m, sum per block
static_assert((kPaSplit - 1) * kPaRowWaves * kPaRecF * 64 * 4 <= kPaLds, "merge records exceed the tiles");

// K/V staging of one split: thread ts loads K chunks ts + 256 u (key c / 16,
// 8 values at 8 (c % 16)) and the 16-byte rows of keys 4 kq .. 4 kq + 3 at
// chunk d8v of V, for the tile starting at position jt (keys past kmax as
// zeros); pa_store_tile writes them to the split's LDS tile (V transposed).
constexpr int kPaKu = kPaKeys * 16 / (kPaRowWaves * 64);           // K chunks per thread
__device__ __forceinline__ void pa_load_tile(u32x4_t (&kr)[kPaKu], u32x4_t (&vq)[4], const uint16_t* K,
                                             const uint16_t* V, int64_t jt, int64_t kmax, int ts, int kq,
                                             int d8v) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < kPaKu; ++u) {
        const int c = ts + u * kPaRowWaves * 64, key = c >> 4, d8 = c & 15;
        const bool live = jt + key <= kmax;
        const int64_t j = live ? jt + key : 0;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(K + j * kPaD + 8 * d8);
        kr[u] = live ? v : z;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int key = 4 * kq + r;
        const bool live = jt + key <= kmax;
        const int64_t j = live ? jt + key : 0;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(V + j * kPaD + 8 * d8v);
        vq[r] = live ? v : z;
    }
}

__device__ __forceinline__ void pa_store_tile(const u32x4_t (&kr)[kPaKu], const u32x4_t (&vq)[4], uint8_t* ks,
                                              uint8_t* vs, int ts, int kq, int d8v) {
#pragma unroll
    for (int u = 0; u < kPaKu; ++u) {
        const int c = ts + u * kPaRowWaves * 64, key = c >> 4, d8 = c & 15;
        *reinterpret_cast<u32x4_t*>(ks + key * kPaKStride + 16 * d8) = kr[u];
    }
    // V^T: value i of chunk d8v for keys 4 kq .. 4 kq + 3 is one 8-byte
    // store in row 8 d8v + i
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = vq[0][w], a1 = vq[1][w], a2 = vq[2][w], a3 = vq[3][w];
        // value 2w: the low halves of the four keys' word w; 2w + 1: the high halves
        const uint2 lo = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                                    __builtin_amdgcn_perm(a3, a2, 0x05040100u));
        const uint2 hi = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                                    __builtin_amdgcn_perm(a3, a2, 0x07060302u));
        *reinterpret_cast<uint2*>(vs + (8 * d8v + 2 * w) * kPaVStride + 8 * kq) = lo;
        *reinterpret_cast<uint2*>(vs + (8 * d8v + 2 * w + 1) * kPaVStride + 8 * kq) = hi;
    }
}

// grid: (ceil(T / (64 / G)), n_kv); G = n_q / n_kv divides 64.  q [T][n_q][128]
// f32 (16-byte aligned), caches [n_kv][S_max][128] bf16 of the one sequence,
// out like q.
__global__ __launch_bounds__(kPaWaves * 64) void prefill_attn_kernel(
    const float* __restrict__ q, int64_t T, int32_t nq, int32_t G, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, int64_t S_max, const int32_t* __restrict__ pos, float scale,
    float* __restrict__ out) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rw = wave % kPaRowWaves, sp = wave / kPaRowWaves;    // row wave, key split
    uint8_t* ks = smem + sp * kPaTileLds;
    uint8_t* vs = ks + kPaKBytes;
    const int ts = rw * 64 + lane;                                 // thread within the split's waves
    const int tpw = kPaRows / G;                                   // tokens per workgroup
    // heavier tiles (later tokens) first
    const int64_t tile = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t t0 = tile * tpw;
    const int g = blockIdx.y;
    const uint16_t* K = kc + (int64_t)g * S_max * kPaD;
    const uint16_t* V = vc + (int64_t)g * S_max * kPaD;

    // the workgroup's key range: positions 0 .. (largest valid position) of its tokens
    int64_t kmax = -1;
    for (int i = 0; i < tpw; ++i) {
        const int64_t t = t0 + i;
        if (t < T) {
            const int64_t p = pos[t];
            if (p >= 0 && p < S_max && p > kmax) kmax = p;
        }
    }

    // this lane's query row in each of its two row blocks, its position
    // (-1 when invalid: no key passes the mask) and its query pieces
    const int fr = lane & 15, fg = lane >> 4;
    int64_t prow[kPaBlk];
    bf16x8_t qh[kPaBlk][4], ql[kPaBlk][4];
#pragma unroll
    for (int b = 0; b < kPaBlk; ++b) {
        const int row = 16 * kPaBlk * rw + 16 * b + fr;
        const int64_t t = t0 + row / G;
        const int h = g * G + row % G;
        const int64_t tc = t < T ? t : T - 1;
        const int64_t p = t < T ? pos[tc] : -1;
        prow[b] = p >= 0 && p < S_max ? p : -1;
        const float* qr = q + (tc * nq + h) * kPaD;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
            const float4 a = *reinterpret_cast<const float4*>(qr + 32 * ds + 8 * fg);
            const float4 c = *reinterpret_cast<const float4*>(qr + 32 * ds + 8 * fg + 4);
            const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t h0, l0, h1, l1;
                split2(v[2 * i], h0, l0);
                split2(v[2 * i + 1], h1, l1);
                hw[i] = h0 | (h1 << 16);
                lw[i] = l0 | (l1 << 16);
            }
            qh[b][ds] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            ql[b][ds] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
    }

    f32x4_t o[kPaBlk][8];
#pragma unroll
    for (int b = 0; b < kPaBlk; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[b][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[kPaBlk], lsum[kPaBlk];
#pragma unroll
    for (int b = 0; b < kPaBlk; ++b) {
        m[b] = -__builtin_inff();
        lsum[b] = 0.f;
    }

    const int64_t ntiles = (kmax + kPaKeys) / kPaKeys;             // 0 when no valid row
    const float scale2 = scale * 1.4426950408889634f;
    // split sp takes tiles sp, sp + kPaSplit, ...; every wave runs the same
    // number of rounds (a split without a tile in a round only meets the
    // barriers).  Staging: 64 keys x 16 chunks of 8 values for K and for V
    // over the split's 256 threads, the next round's tile loaded into
    // registers while this round's is multiplied.  Rows past the
    // workgroup's last position are never attended to: they enter as
    // zeros, since a masked probability (0) times whatever such a row holds
    // (NaN included) must contribute nothing.
    static_assert(kPaRowWaves * 64 == kPaKeys / 4 * 16, "one V key quad per thread");
    const int kq = ts >> 4, d8v = ts & 15;                         // V: 16 lanes read a key's 256 bytes
    u32x4_t kr[kPaKu], vq[4];
    // the loads are unconditional (a tile past the last one reads row 0 and
    // enters as zeros), so the staged rows never live in scratch
    pa_load_tile(kr, vq, K, V, (int64_t)sp * kPaKeys, kmax, ts, kq, d8v);
    for (int64_t base = 0; base < ntiles; base += kPaSplit) {
        const int64_t it = base + sp;
        const bool tl = it < ntiles;
        const int64_t j0 = it * kPaKeys;
        __syncthreads();                                           // the previous tile is consumed
        if (tl) pa_store_tile(kr, vq, ks, vs, ts, kq, d8v);
        __syncthreads();
        pa_load_tile(kr, vq, K, V, j0 + (int64_t)kPaSplit * kPaKeys, kmax, ts, kq, d8v);
        if (!tl) continue;
        // S^T = K Q^T: s[b][kb] lane l holds keys 16 kb + 4 fg + r of query row fr of block b
        f32x4_t s[kPaBlk][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            bf16x8_t kf[4];
#pragma unroll
            for (int ds = 0; ds < 4; ++ds)
                kf[ds] = *reinterpret_cast<const bf16x8_t*>(ks + (16 * kb + fr) * kPaKStride + 64 * ds + 16 * fg);
#pragma unroll
            for (int b = 0; b < kPaBlk; ++b) {
                f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < 4; ++ds) {
                    a = mfma32(kf[ds], qh[b][ds], a);
                    a = mfma32(kf[ds], ql[b][ds], a);
                }
                s[b][kb] = a;
            }
        }
        // online softmax per query row (the row's 64 scores sit in the 4
        // lanes fr, fr + 16, fr + 32, fr + 48, 16 each)
#pragma unroll
        for (int b = 0; b < kPaBlk; ++b) {
            // scores in base-2 units: exp(scale s - m) = 2^(scale log2(e) s - m')
            float tmax = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t j = j0 + 16 * kb + 4 * fg + r;
                    const float v = j <= prow[b] ? s[b][kb][r] * scale2 : -__builtin_inff();
                    s[b][kb][r] = v;
                    tmax = fmaxf(tmax, v);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mnew = fmaxf(m[b], tmax);
            const bool live = mnew > -__builtin_inff();
            const float corr = live ? exp2f(m[b] - mnew) : 1.f;
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = live ? exp2f(s[b][kb][r] - mnew) : 0.f;
                    s[b][kb][r] = p;
                    psum += p;
                }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            lsum[b] = lsum[b] * corr + psum;
            m[b] = mnew;
            // rescale O: lane l holds rows 4 fg + r of the block, whose
            // factor sits in lane (4 fg + r) (query row = lane % 16)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float cr = __shfl(corr, 4 * fg + r, 64);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[b][j][r] *= cr;
            }
        }
        // O += P V: per 32-key step (blocks kb, kb + 1) this lane's 8 keys
        // are 16 kb + 4 fg + r and 16 (kb + 1) + 4 fg + r
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
            const int kb = 2 * ks2;
            bf16x8_t ph[kPaBlk], pl[kPaBlk];
#pragma unroll
            for (int b = 0; b < kPaBlk; ++b) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = i < 2 ? s[b][kb][2 * i] : s[b][kb + 1][2 * i - 4];
                    const float p1 = i < 2 ? s[b][kb][2 * i + 1] : s[b][kb + 1][2 * i - 3];
                    uint32_t h0, l0, h1, l1;
                    split2(p0, h0, l0);
                    split2(p1, h1, l1);
                    hw[i] = h0 | (h1 << 16);
                    lw[i] = l0 | (l1 << 16);
                }
                ph[b] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                pl[b] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint8_t* vrow = vs + (16 * j + fr) * kPaVStride;
                const uint2 va = *reinterpret_cast<const uint2*>(vrow + 2 * (16 * kb + 4 * fg));
                const uint2 vb = *reinterpret_cast<const uint2*>(vrow + 2 * (16 * (kb + 1) + 4 * fg));
                const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
#pragma unroll
                for (int b = 0; b < kPaBlk; ++b) {
                    o[b][j] = mfma32(ph[b], vf, o[b][j]);
                    o[b][j] = mfma32(pl[b], vf, o[b][j]);
                }
            }
        }
    }
    // the splits meet in LDS (over the tiles): splits 1.. store O, m and the
    // sum of every lane, split 0 adds them in split order with the
    // log-sum-exp rule
    __syncthreads();
    float* rec = reinterpret_cast<float*>(smem);
    if (sp > 0) {
        float* rr = rec + ((sp - 1) * kPaRowWaves + rw) * kPaRecF * 64;
#pragma unroll
        for (int b = 0; b < kPaBlk; ++b) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) rr[((b * 8 + j) * 4 + r) * 64 + lane] = o[b][j][r];
            rr[(32 * kPaBlk + b) * 64 + lane] = m[b];
            rr[(33 * kPaBlk + b) * 64 + lane] = lsum[b];
        }
    }
    __syncthreads();
    if (sp > 0) return;
    for (int i = 1; i < kPaSplit; ++i) {
        const float* rr = rec + ((i - 1) * kPaRowWaves + rw) * kPaRecF * 64;
#pragma unroll
        for (int b = 0; b < kPaBlk; ++b) {
            const float mi = rr[(32 * kPaBlk + b) * 64 + lane], li = rr[(33 * kPaBlk + b) * 64 + lane];
            const float mn = fmaxf(m[b], mi);
            const bool lv = mn > -__builtin_inff();
            const float ca = lv ? exp2f(m[b] - mn) : 1.f;
            const float cb = lv ? exp2f(mi - mn) : 1.f;
            lsum[b] = lsum[b] * ca + li * cb;
            m[b] = mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float fa = __shfl(ca, 4 * fg + r, 64), fb = __shfl(cb, 4 * fg + r, 64);
#pragma unroll
                for (int j = 0; j < 8; ++j) o[b][j][r] = o[b][j][r] * fa + rr[((b * 8 + j) * 4 + r) * 64 + lane] * fb;
            }
        }
    }
    // out = O / sum: lane l holds rows 4 fg + r of each block, column 16 j + fr
#pragma unroll
    for (int b = 0; b < kPaBlk; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 4 * fg + r;
            const float den = __shfl(lsum[b], rl, 64);
            const bool valid = __shfl((int)(prow[b] >= 0), rl, 64) != 0;
            const int row = 16 * kPaBlk * rw + 16 * b + rl;
            const int64_t t = t0 + row / G;
            const int h = g * G + row % G;
            if (t < T) {
                float* dst = out + (t * nq + h) * kPaD;
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[16 * j + fr] = valid ? o[b][j][r] / den : __builtin_nanf("");
            }
        }
}

}  // namespace

bool gemm_path(int64_t T, int64_t K) { return T >= kGemmMinTokens && K % kGmBK == 0; }

hipError_t launch_bf16_gemm_multi(const uint16_t* const* Ws, float* const* ys, const int64_t* Ns, int nmat,
                                  int64_t K, const float* x, int64_t T, int accumulate,
                                  hipStream_t stream) {
    // 128-row tiles unless that leaves the device short of workgroups
    int64_t t128 = 0;
    for (int i = 0; i < nmat; ++i) t128 += (Ns[i] + 127) / 128;
    const int64_t ttiles = (T + kGmBM - 1) / kGmBM;
    const bool wide = t128 * ttiles >= 256;
    const int BN = wide ? 128 : 64;
    GemmJob job{};
    int acc_tiles = 0;
    for (int i = 0; i < 3; ++i) {
        if (i < nmat) {
            job.W[i] = Ws[i];
            job.y[i] = ys[i];
            job.N[i] = Ns[i];
            acc_tiles += (int)((Ns[i] + BN - 1) / BN);
        }
        job.tile_end[i] = acc_tiles;
    }
    dim3 grid((unsigned)acc_tiles, (unsigned)ttiles);
    if (wide)
        hipLaunchKernelGGL(bf16_gemm_kernel<128>, grid, dim3(kGmThreads), GmGeom<128>::LDS, stream, job,
                           K, x, T, accumulate);
    else
        hipLaunchKernelGGL(bf16_gemm_kernel<64>, grid, dim3(kGmThreads), GmGeom<64>::LDS, stream, job,
                           K, x, T, accumulate);
    return hipGetLastError();
}

hipError_t launch_bf16_gemm(const uint16_t* W, int64_t N, int64_t K, const float* x, int64_t T,
                            float* y, int accumulate, hipStream_t stream) {
    return launch_bf16_gemm_multi(&W, &y, &N, 1, K, x, T, accumulate, stream);
}

hipError_t launch_kv_write_rows(const float* k_new, const float* v_new, int64_t T, int32_t nkv,
                                int32_t D, const int32_t* pos, uint16_t* kc, uint16_t* vc,
                                int64_t S_max, hipStream_t stream) {
    hipLaunchKernelGGL(kv_rows_kernel, dim3((unsigned)T), dim3(256), 0, stream, k_new, v_new, nkv, D,
                       pos, kc, vc, S_max);
    return hipGetLastError();
}

bool prefill_attention_supported(int32_t nq, int32_t nkv, int32_t D) {
    return D == kPaD && nkv >= 1 && nq % nkv == 0 && kPaRows % (nq / nkv) == 0;
}

hipError_t launch_prefill_attention(const float* q, int64_t T, int32_t nq, int32_t nkv, int32_t D,
                                    const uint16_t* kc, const uint16_t* vc, int64_t S_max,
                                    const int32_t* pos, float scale, float* out, hipStream_t stream) {
    (void)D;
    const int G = nq / nkv;
    const int tpw = kPaRows / G;
    dim3 grid((unsigned)((T + tpw - 1) / tpw), (unsigned)nkv);
    static LdsLimit lds_set;
    const hipError_t e = ensure_lds(reinterpret_cast<const void*>(prefill_attn_kernel), lds_set, kPaLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_attn_kernel, grid, dim3(kPaWaves * 64), kPaLds, stream, q, T, nq, G,
                       kc, vc, S_max, pos, scale, out);
    return hipGetLastError();
}

}  // namespace q3moe
