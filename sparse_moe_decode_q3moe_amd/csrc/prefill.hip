// Batched expert FFN for larger T (prefill): tokens grouped by expert, each
// expert's token tile multiplied by its weight tiles on the matrix cores.
// The pages name token-by-token prefill as the bottleneck and plan grouped
// expert GEMMs for it (aprender issue #3714, gap list); the weights are the
// same Q4_K / Q6_K tensors the decode path reads, in place at base + e*stride.
//
// Pipeline (all on the caller's stream, all grids fixed at launch):
//   1. group: (token, slot) pairs ordered by (expert, pair), per-expert
//      offsets and tile offsets for tiles of 64 pairs (so an expert with up
//      to 64 pairs reads its weights once);
//   2. pieces of the hidden rows: bf16 hi + mid + lo (x to 2^-27; the
//      gate/up outputs amplify the input's rounding most) and the f32 sum of
//      every 16 values;
//   3. gate/up: one workgroup per (128 h features, pair tile), k in stages
//      of 128 staged through LDS one stage ahead; v_mfma_f32_16x16x32_bf16
//      per Q4_K sub-block on exact bf16 weights 128 + 8q with each piece;
//      h = silu(g) * u goes to the workspace in grouped row order;
//   4. pieces of h (hi + lo);
//   5. down: one workgroup per (64 output rows, pair tile), Q6_K or Q4_K,
//      the row tile of the expert's down matrix resident in LDS, h staged per
//      128-wide stage; v_mfma_f32_16x16x16bf16_1k per 16-wide scale group;
//      rows go to Y indexed by pair;
//   6. combine: out[t] = [out +] sum over slots in slot order of w * Y.
// In both matrix kernels the weights' offset (and the Q4_K min) times the
// activation sums leaves once per stage as v_mfma_f32_16x16x4_f32 rank-4
// steps.  Workgroups are mapped so that the ones sharing a pair tile run on
// one XCD (one L2).
// MFMA operand layouts (checked on the device): A lane l holds row l % 16,
// k = K (l / 16) .. + K - 1 (K = 4, 8 or 1 values for the 16-, 32-wide bf16
// and the f32 forms); B lane l holds column l % 16 at the same k; C lane l
// holds rows 4 (l / 16) + r, r = 0..3, column l % 16.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 64;                 // grouped pairs per tile (four 16-row MFMA blocks)
constexpr uint32_t kPfBias8 = 0x43434343u;

__device__ __forceinline__ float pf_silu(float z) { return z / (1.0f + expf(-z)); }

// Four weight bytes (each < 128) as the bf16 pair operand (128 + q0, 128 + q1),
// (128 + q2, 128 + q3), in k order.
__device__ __forceinline__ s16x4_t pf_bf16x4(uint32_t q) {
    const uint32_t a = __builtin_amdgcn_perm(kPfBias8, q, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(kPfBias8, q, 0x04030402u);
    s16x4_t r;
    r[0] = (short)(a & 0xffffu);
    r[1] = (short)(a >> 16);
    r[2] = (short)(b & 0xffffu);
    r[3] = (short)(b >> 16);
    return r;
}

__device__ __forceinline__ f32x4_t pf_mfma(s16x4_t a, s16x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pf_lds_u32_a2(const uint8_t* lds, int off) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (off & ~3));
    return __builtin_amdgcn_alignbyte(p[1], p[0], (uint32_t)(off & 3));
}

// Q4_K scale factors of one block header (d, dmin, 12 packed bytes) for
// the 8 sub-blocks, for weights encoded as bf16 128 + 8q: s[j] = d*sc_j/8,
// b[j] = 128*s[j] + dmin*m_j (removes the offset and applies the min).
__device__ __forceinline__ void pf_q4k_factors_hdr(uint4 hdr, float s[8], float b[8]) {
    const float d = half_bits_to_float(hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    const uint32_t s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;        // packed bytes 0-3, 4-7, 8-11
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int sc, m;
        if (j < 4) {
            sc = (s0 >> (8 * j)) & 63;
            m = (s1 >> (8 * j)) & 63;
        } else {
            const int jj = j - 4;
            sc = ((s2 >> (8 * jj)) & 15) | (((s0 >> (8 * jj + 6)) & 3) << 4);
            m = ((s2 >> (8 * jj + 4)) & 15) | (((s1 >> (8 * jj + 6)) & 3) << 4);
        }
        s[j] = 0.125f * d * (float)sc;                        // weights enter as 128 + 8q
        b[j] = 128.f * s[j] + dmin * (float)m;
    }
}

// ---------------------------------------------------------------- pieces --
// rows x cols f32 (cols % 16 == 0) -> NP bf16 piece arrays [rows][cols]
// (each round-to-nearest-even of what the previous leave: |x - sum| <=
// 2^-18 |x| for two pieces, 2^-27 |x| for three) and s16 f32 [rows][cols/16],
// the sums of the pieces per 16 values.  One float4 per thread per step; 4
// neighbouring threads make one 16-value group.
template <int NP>
__global__ __launch_bounds__(256) void pf_pieces_kernel(const float* __restrict__ src, int64_t n4,
                                                        uint32_t* __restrict__ p0,
                                                        uint32_t* __restrict__ p1,
                                                        uint32_t* __restrict__ p2,
                                                        float* __restrict__ s16) {
    const int64_t step = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += step) {
        const float4 v = reinterpret_cast<const float4*>(src)[i];
        const float x[4] = {v.x, v.y, v.z, v.w};
        uint32_t b[NP][4];
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = x[j], part = 0.f;
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                b[q][j] = bf16_rne_bits(r);
                const float f = bf16_bits_to_float(b[q][j]);
                r -= f;
                part += f;
            }
            sum += part;
        }
        float g = sum + __shfl_xor(sum, 1, kWave);           // n4 % 4 == 0: quads stay together
        g += __shfl_xor(g, 2, kWave);
        uint32_t* dst[3] = {p0, p1, p2};
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            dst[q][2 * i] = b[q][0] | (b[q][1] << 16);
            dst[q][2 * i + 1] = b[q][2] | (b[q][3] << 16);
        }
        if ((i & 3) == 0) s16[i >> 2] = g;
    }
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8), each with its own L2.  Tile slot s goes to XCD s % 8 and all
// its column tiles to consecutive workgroups there, so the workgroups that
// share a token tile's activations meet in one L2, and the used slots (a
// prefix of the slot range) spread evenly over the XCDs.  The grid is
// ctiles * nslots workgroups with nslots a multiple of 8.
constexpr int kXcds = 8;
__device__ __forceinline__ void pf_xcd_tile(int w, int ctiles, int& slot, int& ctile) {
    const int x = w % kXcds, local = w / kXcds;
    slot = (local / ctiles) * kXcds + x;
    ctile = local % ctiles;
}

// The expert and tile index of tile slot `slot` (tile_off: exclusive prefix
// of per-expert tile counts, tile_off[E] = total): the last e with
// tile_off[e] <= slot.
__device__ __forceinline__ int pf_tile_expert(const int32_t* tile_off, int32_t E, int slot) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] <= slot) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------- staged operands --
// Both matrix kernels work on a tile of up to 64 grouped pairs (four 16-row
// MFMA blocks) and walk k in stages of 128 (half a super-block).  Every
// operand of a stage is loaded by plain coalesced 16-byte loads into
// registers one stage ahead and stored into LDS after the barrier, so the
// next stage's memory traffic overlaps this stage's matrix work.  Activation
// rows sit in LDS row-major with 16 bytes of padding (272 bytes per row and
// piece), which makes the 16 rows an MFMA operand read start in 16 distinct
// bank quads.
constexpr int kStageK = 128;
constexpr int kXRowB = kStageK * 2 + 16;                      // 272
constexpr int kXPieceB = kPfRows * kXRowB;                    // 17408

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x4_f32: A lane l holds row l % 16, k = l / 16; B lane l
// holds column l % 16 at the same k; C as for the bf16 forms.
__device__ __forceinline__ f32x4_t pf_mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t pf_mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight Q4_K nibbles (sub-block half h of 8 quant bytes) as bf16 128 + 8q.
__device__ __forceinline__ bf16x8_t pf_q4k_b8(uint2 w, int h) {
    const uint32_t v0 = (h ? (w.x >> 1) : (w.x << 3)) & 0x78787878u;
    const uint32_t v1 = (h ? (w.y >> 1) : (w.y << 3)) & 0x78787878u;
    const u32x4v_t r = {__builtin_amdgcn_perm(kPfBias8, v0, 0x04010400u),
                        __builtin_amdgcn_perm(kPfBias8, v0, 0x04030402u),
                        __builtin_amdgcn_perm(kPfBias8, v1, 0x04010400u),
                        __builtin_amdgcn_perm(kPfBias8, v1, 0x04030402u)};
    return __builtin_bit_cast(bf16x8_t, r);
}

// ---------------------------------------------------------------- gate/up --
// One workgroup per (128 h features, pair tile): 256 weight rows, gate rows
// f0.. then up rows f0..  8 waves: wave w owns token blocks w >> 2 and
// (w >> 2) + 2 (interleaved, so that waves w and w + 4, which share a SIMD,
// both have work when a tile holds 32 pairs or fewer; blocks with no pairs
// are skipped) and features 32 (w & 3)..+31 of both matrices, so
// silu(g) * u is formed in registers and each wave reads half the tile's
// activations per step.  Each k step covers one Q4_K sub-block
// (v_mfma_f32_16x16x32_bf16 on exact bf16 weights 128 + 8q with each of the
// three activation pieces) and is scaled by that sub-block's d*sc/8.  The 128
// offset and the min, (128 s + dmin m) times each sub-block's activation sum
// S, leave once per stage as one f32 rank-4 matrix step per tile.
// LDS per stage: pieces hi/mid/lo [64 rows][272]; weight quant bytes as
// planes of 8-byte pieces [chunk 2][group 4][256 rows] (each plane padded by
// 128 bytes, so the two groups a half-wave reads land in different banks);
// the (s, b) factors [4 sub-blocks][256 rows]; the sums S [4][64].
constexpr int kGuFeat = 128;
constexpr int kGuWRows = 2 * kGuFeat;                         // 256
constexpr int kGuThreads = 512;
constexpr int kGuPlaneB = kGuWRows * 8 + 128;                 // 2176
constexpr int kGuWOff = 3 * kXPieceB;                         // 52224
constexpr int kGuFacOff = kGuWOff + 8 * kGuPlaneB;            // 69632
constexpr int kGuSOff = kGuFacOff + 4 * kGuWRows * 8;         // 77824
constexpr int kGuLds = kGuSOff + 4 * kPfRows * 4;             // 78848

__global__ __launch_bounds__(kGuThreads) void pf_gateup_kernel(
    const uint16_t* __restrict__ xhi, const uint16_t* __restrict__ xmid,
    const uint16_t* __restrict__ xlo, const float* __restrict__ xs16, int64_t H,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ pairs, int32_t E, int32_t k, const uint8_t* __restrict__ gbase,
    int64_t gstride, const uint8_t* __restrict__ ubase, int64_t ustride, int64_t F,
    float* __restrict__ hbuf) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int slot, ftile;
    pf_xcd_tile((int)blockIdx.x, (int)(F / kGuFeat), slot, ftile);
    if (slot >= tile_off[E]) return;                          // uniform: an unused tile slot
    const int e = pf_tile_expert(tile_off, E, slot);
    const int64_t row0 = offsets[e] + (int64_t)(slot - tile_off[e]) * kPfRows;
    const int nrows = (int)min((int64_t)kPfRows, (int64_t)offsets[e + 1] - row0);
    const int64_t f0 = (int64_t)ftile * kGuFeat;
    const int64_t rowb = (H / kQK) * kQ4KBytes;               // bytes per gate/up row
    const uint8_t* gexp = gbase + (int64_t)e * gstride + f0 * rowb;
    const uint8_t* uexp = ubase + (int64_t)e * ustride + f0 * rowb;
    const int nst = (int)(H / kStageK);

    // staging roles.  Activations: 3 pieces x 64 rows x 16 chunks of 16 B,
    // item q = u * 512 + tid (u < 6): piece u >> 1, row tid/16 (u even) or
    // 32 + tid/16 (u odd), chunk tid & 15.  Weights: 256 rows x 4 parts of
    // 16 B (q = u * 512 + tid, u < 2: row q >> 2, part q & 3); headers:
    // thread tid < 256 reads row tid's.  Sums: thread tid < 256 reads the S
    // of row tid >> 2, sub-block tid & 3.
    const int ra = tid >> 4, rb2 = 32 + (tid >> 4), xc = tid & 15;
    const int64_t toka = ra < nrows ? pairs[row0 + ra] / k : -1;
    const int64_t tokb = rb2 < nrows ? pairs[row0 + rb2] / k : -1;
    const int64_t toks = tid < 4 * kPfRows && (tid >> 2) < nrows ? pairs[row0 + (tid >> 2)] / k : -1;
    uint4 rx[6], rw[2], rh;
    float2 rs = make_float2(0.f, 0.f);
    auto wrow = [&](int r) -> const uint8_t* { return r < kGuFeat ? gexp + r * rowb : uexp + (r - kGuFeat) * rowb; };
    auto load_stage = [&](int st) {
        const int64_t k0 = (int64_t)st * kStageK;
        const int64_t sb = st >> 1;
        const int half = st & 1;
#pragma unroll
        for (int u = 0; u < 6; ++u) {
            const int64_t tok = (u & 1) ? tokb : toka;
            const uint16_t* xs = u < 2 ? xhi : u < 4 ? xmid : xlo;
            rx[u] = tok >= 0 ? *reinterpret_cast<const uint4*>(xs + tok * H + k0 + 8 * xc)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = u * kGuThreads + tid;
            rw[u] = *reinterpret_cast<const uint4*>(wrow(q >> 2) + sb * kQ4KBytes + 16 + 64 * half + 16 * (q & 3));
        }
        if (tid < kGuWRows) rh = *reinterpret_cast<const uint4*>(wrow(tid) + sb * kQ4KBytes);
        // the sub-block's two 16-value sums, from a clamped row and added
        // only when stored: an add here would wait for this stage's loads at
        // once and leave nothing to overlap with the matrix work
        const int64_t g16 = (k0 >> 4) + 2 * (tid & 3);
        rs = *reinterpret_cast<const float2*>(xs16 + (toks >= 0 ? toks : 0) * (H / 16) + g16);
    };
    auto store_stage = [&](int half) {
#pragma unroll
        for (int u = 0; u < 6; ++u) {
            const int r = (u & 1) ? rb2 : ra;
            *reinterpret_cast<uint4*>(smem + (u >> 1) * kXPieceB + r * kXRowB + xc * 16) = rx[u];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = u * kGuThreads + tid, r = q >> 2, part = q & 3;
            const int c = part >> 1, g0 = 2 * (part & 1);         // 16 B = groups g0, g0 + 1 of chunk c
            *reinterpret_cast<uint2*>(smem + kGuWOff + (c * 4 + g0) * kGuPlaneB + r * 8) = make_uint2(rw[u].x, rw[u].y);
            *reinterpret_cast<uint2*>(smem + kGuWOff + (c * 4 + g0 + 1) * kGuPlaneB + r * 8) = make_uint2(rw[u].z, rw[u].w);
        }
        if (tid < kGuWRows) {
            float sj[8], bj[8];
            pf_q4k_factors_hdr(rh, sj, bj);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                reinterpret_cast<float2*>(smem + kGuFacOff)[j * kGuWRows + tid] =
                    half ? make_float2(sj[4 + j], bj[4 + j]) : make_float2(sj[j], bj[j]);
        }
        if (tid < 4 * kPfRows)
            reinterpret_cast<float*>(smem + kGuSOff)[(tid & 3) * kPfRows + (tid >> 2)] = toks >= 0 ? rs.x + rs.y : 0.f;
    };

    const int col = lane & 15, g = lane >> 4;
    const int th = wave >> 2, fq = wave & 3;
    const int frow0 = 32 * fq + col;                          // gate rows frow0, frow0 + 16; up rows + 128
    f32x4_t acc[2][2][2];                                     // [token block][feature block][gate, up]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
            acc[i][fb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc[i][fb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    load_stage(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();                                      // the previous stage is consumed
        store_stage(st & 1);
        __syncthreads();
        if (st + 1 < nst) load_stage(st + 1);
        if (16 * th >= nrows) continue;                       // both of this wave's token blocks empty
#pragma unroll
        for (int j = 0; j < 4; ++j) {                         // one sub-block per k step
            const int c = j >> 1, h = j & 1;
            const uint8_t* plane = smem + kGuWOff + (c * 4 + g) * kGuPlaneB;
            bf16x8_t B[2][2];
            float fs[2][2];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                const int gr = frow0 + 16 * fb, ur = kGuFeat + gr;
                B[fb][0] = pf_q4k_b8(*reinterpret_cast<const uint2*>(plane + gr * 8), h);
                B[fb][1] = pf_q4k_b8(*reinterpret_cast<const uint2*>(plane + ur * 8), h);
                fs[fb][0] = reinterpret_cast<const float2*>(smem + kGuFacOff)[j * kGuWRows + gr].x;
                fs[fb][1] = reinterpret_cast<const float2*>(smem + kGuFacOff)[j * kGuWRows + ur].x;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tb = th + 2 * i;
                if (16 * tb >= nrows) continue;               // no pairs in this token block
                const int xo = (16 * tb + col) * kXRowB + (32 * j + 8 * g) * 2;
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(smem + xo);
                const bf16x8_t am = *reinterpret_cast<const bf16x8_t*>(smem + kXPieceB + xo);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(smem + 2 * kXPieceB + xo);
#pragma unroll
                for (int fb = 0; fb < 2; ++fb)
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        f32x4_t t = pf_mfma32(ah, B[fb][m], f32x4_t{0.f, 0.f, 0.f, 0.f});
                        t = pf_mfma32(am, B[fb][m], t);
                        t = pf_mfma32(al, B[fb][m], t);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][fb][m][r] += fs[fb][m] * t[r];
                    }
            }
        }
        // offset and min of the stage's 4 sub-blocks: acc -= S . b, a rank-4
        // product per tile, as one f32 matrix step (k = sub-block = lane / 16)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (16 * (th + 2 * i) >= nrows) continue;
            const float sa = reinterpret_cast<const float*>(smem + kGuSOff)[g * kPfRows + 16 * (th + 2 * i) + col];
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                const int gr = frow0 + 16 * fb;
                const float nbg = -reinterpret_cast<const float2*>(smem + kGuFacOff)[g * kGuWRows + gr].y;
                const float nbu = -reinterpret_cast<const float2*>(smem + kGuFacOff)[g * kGuWRows + kGuFeat + gr].y;
                acc[i][fb][0] = pf_mfma_f32(sa, nbg, acc[i][fb][0]);
                acc[i][fb][1] = pf_mfma_f32(sa, nbu, acc[i][fb][1]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * (th + 2 * i) + 4 * g + r;
                if (t < nrows)
                    hbuf[(row0 + t) * F + f0 + frow0 + 16 * fb] = pf_silu(acc[i][fb][0][r]) * acc[i][fb][1][r];
            }
}

// ------------------------------------------------------------------- down --
// One workgroup per (64 output rows, pair tile).  The expert's 64-row tile
// of the down matrix (all F/256 blocks, contiguous in HBM) is staged once
// with the first stage; the h pieces (hi, lo) and their 16-value sums are
// staged per 128-wide k stage.  8 waves: wave w owns output rows
// 16 (w & 3).. and token blocks w >> 2, (w >> 2) + 2 (interleaved as in the
// gate/up kernel; empty ones skipped).  Each k step is
// one 16-wide scale group (v_mfma_f32_16x16x16bf16_1k on exact bf16 weights
// 128 + q (Q6_K) or 128 + 8q (Q4_K) with each h piece), scaled by the
// group's factor; the offset (and the Q4_K min) times each group's h sum
// leaves once per stage as f32 rank-4 matrix steps.
constexpr int kDnOut = 64;
constexpr int kDnThreads = 512;
constexpr int kDnMaxW16 = 10;                                 // F <= 1536: <= 5040 16-byte pieces
__host__ __device__ inline int pf_down_wbytes(int64_t F, int32_t qtype) {
    return (int)(kDnOut * (F / kQK) * (qtype == 2 ? kQ6KBytes : kQ4KBytes));
}
__host__ __device__ inline int pf_down_hoff(int64_t F, int32_t qtype) {
    return (pf_down_wbytes(F, qtype) + 16 + 15) & ~15;       // + padding for the unaligned Q6_K reads
}
// h rows in LDS: 264 bytes (66 dwords), so the 8-byte operand reads of the
// 16 rows of a block land on 16 distinct bank pairs (a 272-byte row put rows
// r and r + 8 on the same banks)
constexpr int kDnRowB = kStageK * 2 + 8;                      // 264
constexpr int kDnPieceB = kPfRows * kDnRowB;                  // 16896
__host__ __device__ inline int pf_down_lds(int64_t F, int32_t qtype) {
    return pf_down_hoff(F, qtype) + 2 * kDnPieceB + 8 * kPfRows * 4;
}

template <bool Q6>
__global__ __launch_bounds__(kDnThreads) void pf_down_kernel(
    const uint16_t* __restrict__ hhi, const uint16_t* __restrict__ hlo,
    const float* __restrict__ hs16, int64_t F, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ pairs, int32_t E,
    const uint8_t* __restrict__ dbase, int32_t qtype, int64_t dstride, int64_t H,
    float* __restrict__ Y) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int slot, htile;
    pf_xcd_tile((int)blockIdx.x, (int)(H / kDnOut), slot, htile);
    if (slot >= tile_off[E]) return;
    const int e = pf_tile_expert(tile_off, E, slot);
    const int64_t row0 = offsets[e] + (int64_t)(slot - tile_off[e]) * kPfRows;
    const int nrows = (int)min((int64_t)kPfRows, (int64_t)offsets[e + 1] - row0);
    const int64_t h0 = (int64_t)htile * kDnOut;
    constexpr bool q6 = Q6;                                   // the down type, fixed per instantiation
    const int bb = q6 ? kQ6KBytes : kQ4KBytes;
    const int nb = (int)(F / kQK);
    const int rowb = nb * bb;
    const int wbytes = kDnOut * rowb;                         // a multiple of 16
    const int hoff = pf_down_hoff(F, qtype);
    const int soff = hoff + 2 * kDnPieceB;
    const int nst = (int)(F / kStageK);

    // staging roles: the weight tile (n16 pieces of 16 B over 512 threads,
    // with the first stage); h pieces 2 x 64 rows x 16 chunks (u < 4: piece
    // u >> 1, rows tid/16 and 32 + tid/16); sums 8 groups x 64 rows (one per
    // thread: row tid >> 3, group tid & 7).
    const u32x4v_t* wsrc = reinterpret_cast<const u32x4v_t*>(dbase + (int64_t)e * dstride + h0 * rowb);
    const int n16 = wbytes >> 4;
    u32x4v_t rwt[kDnMaxW16];                                  // the weight tile, with stage 0
#pragma unroll
    for (int u = 0; u < kDnMaxW16; ++u) {
        const int q = u * kDnThreads + tid;
        if (q < n16) rwt[u] = __builtin_nontemporal_load(wsrc + q);
    }
    const int ra = tid >> 4, rb2 = 32 + (tid >> 4), hc = tid & 15;
    const int64_t pa = ra < nrows ? row0 + ra : -1;
    const int64_t pb = rb2 < nrows ? row0 + rb2 : -1;
    const int srow = tid >> 3, sgrp = tid & 7;
    const int64_t ps = srow < nrows ? row0 + srow : -1;
    const uint16_t* hsrc[2] = {hhi, hlo};
    uint4 rx[4];
    float rs = 0.f;
    auto load_stage = [&](int st) {
        const int64_t k0 = (int64_t)st * kStageK;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t pr = (u & 1) ? pb : pa;
            rx[u] = pr >= 0 ? *reinterpret_cast<const uint4*>(hsrc[u >> 1] + pr * F + k0 + 8 * hc)
                            : make_uint4(0, 0, 0, 0);
        }
        rs = ps >= 0 ? hs16[ps * (F / 16) + (k0 >> 4) + sgrp] : 0.f;
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = (u & 1) ? rb2 : ra;
            uint8_t* d = smem + hoff + (u >> 1) * kDnPieceB + r * kDnRowB + hc * 16;   // 8-byte aligned
            *reinterpret_cast<uint2*>(d) = make_uint2(rx[u].x, rx[u].y);
            *reinterpret_cast<uint2*>(d + 8) = make_uint2(rx[u].z, rx[u].w);
        }
        reinterpret_cast<float*>(smem + soff)[sgrp * kPfRows + srow] = rs;
    };

    const int col = lane & 15, g = lane >> 4;
    const int orow = 16 * (wave & 3) + col;                   // this lane's output row in the tile
    const int tb0 = wave >> 2;                                // token blocks tb0, tb0 + 2
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    // the pair index of each output row this lane stores, read now (reading
    // it at the store would put a memory round trip before each of them)
    int32_t opair[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * (tb0 + 2 * i) + 4 * g + r;
            opair[i][r] = pairs[row0 + (t < nrows ? t : 0)];
        }

    load_stage(0);
#pragma unroll
    for (int u = 0; u < kDnMaxW16; ++u) {
        const int q = u * kDnThreads + tid;
        if (q < n16) *reinterpret_cast<u32x4v_t*>(smem + 16 * q) = rwt[u];
    }
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
        store_stage();
        __syncthreads();
        if (st + 1 < nst) load_stage(st + 1);
        if (16 * tb0 >= nrows) continue;                      // both of this wave's token blocks empty
        const int sb = st >> 1, half = st & 1;
        const int boff = orow * rowb + sb * bb;               // this lane's block in the tile
        const uint8_t* blk = smem + boff;
        float dq = 0.f, dm = 0.f;
        uint4 hdr = make_uint4(0, 0, 0, 0);
        if (q6) {
            dq = half_bits_to_float(blk[208] | (blk[209] << 8));
        } else {
            hdr = *reinterpret_cast<const uint4*>(blk);
            dq = 0.125f * half_bits_to_float(hdr.x & 0xffffu);   // weights enter as 128 + 8q
            dm = half_bits_to_float(hdr.x >> 16);
        }
#pragma unroll
        for (int G = 0; G < 8; ++G) {                         // one 16-wide group per k step
            const int gi = 8 * half + G;                      // group within the super-block
            uint32_t q;
            float sc;
            if (q6) {
                const int r = (gi >> 1) & 3, lp = 16 * (gi & 1) + 4 * g;
                const uint32_t ql = pf_lds_u32_a2(smem, boff + 64 * half + 32 * (r & 1) + lp);
                const uint32_t qh = pf_lds_u32_a2(smem, boff + 128 + 32 * half + lp);
                q = ((ql >> (4 * (r >> 1))) & 0x0f0f0f0fu) | (((qh >> (2 * r)) & 0x03030303u) << 4);
                sc = dq * (float)(int8_t)blk[192 + gi];
            } else {
                const int J = gi >> 1, c = J >> 1, h = J & 1, lp = 16 * (gi & 1) + 4 * g;
                q = ((*reinterpret_cast<const uint32_t*>(blk + 16 + 32 * c + lp) >> (4 * h)) << 3) & 0x78787878u;
                int scj, mj;
                q4k_scale_min(blk + 4, J, scj, mj);
                sc = dq * (float)scj;
            }
            const s16x4_t bw = pf_bf16x4(q);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tb = tb0 + 2 * i;
                if (16 * tb >= nrows) continue;               // no pairs in this token block
                const int xo = hoff + (16 * tb + col) * kDnRowB + (16 * G + 4 * g) * 2;
                f32x4_t t = pf_mfma(*reinterpret_cast<const s16x4_t*>(smem + xo), bw, f32x4_t{0.f, 0.f, 0.f, 0.f});
                t = pf_mfma(*reinterpret_cast<const s16x4_t*>(smem + kDnPieceB + xo), bw, t);
                acc[i][0] += sc * t[0];
                acc[i][1] += sc * t[1];
                acc[i][2] += sc * t[2];
                acc[i][3] += sc * t[3];
            }
        }
        // the offset (and the Q4_K min) of the stage's 8 groups: acc -= S . off,
        // two f32 rank-4 matrix steps per tile (k = group = 4 * p + lane / 16)
#pragma unroll
        for (int pq = 0; pq < 2; ++pq) {
            const int gi = 8 * half + 4 * pq + g;             // this lane's group (its k slot)
            float off;
            if (q6) {
                off = 160.f * dq * (float)(int8_t)blk[192 + gi];   // (128 + q) - 160 = q - 32
            } else {
                int scj, mj;
                q4k_scale_min(blk + 4, gi >> 1, scj, mj);
                off = 128.f * dq * (float)scj + dm * (float)mj;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (16 * (tb0 + 2 * i) >= nrows) continue;
                const float sa = reinterpret_cast<const float*>(smem + soff)[(4 * pq + g) * kPfRows + 16 * (tb0 + 2 * i) + col];
                acc[i] = pf_mfma_f32(sa, -off, acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * (tb0 + 2 * i) + 4 * g + r;
            if (t < nrows) Y[(int64_t)opair[i][r] * H + h0 + orow] = acc[i][r];
        }
}

// ---------------------------------------------------------------- combine --
// grid: (T, H / 1024); thread: 4 consecutive outputs of one token.
__global__ __launch_bounds__(256) void pf_combine_kernel(const float* __restrict__ Y,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w, int32_t k,
                                                         int32_t E, int64_t H,
                                                         float* __restrict__ out, int accumulate) {
    const int64_t t = blockIdx.x;
    const int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; ++s) {
        const int e = idx[t * k + s];
        if (e < 0 || e >= E) continue;
        const float ws = w[t * k + s];
        const float4 y = *reinterpret_cast<const float4*>(Y + (t * k + s) * H + c);
        acc.x += ws * y.x;
        acc.y += ws * y.y;
        acc.z += ws * y.z;
        acc.w += ws * y.w;
    }
    float4* o = reinterpret_cast<float4*>(out + t * H + c);
    if (accumulate) {
        const float4 p = *o;
        acc.x += p.x;
        acc.y += p.y;
        acc.z += p.z;
        acc.w += p.w;
    }
    *o = acc;
}

struct PfLayout {
    size_t counts, offsets, tile_off, pairs, xhi, xmid, xlo, xs16, h, hhi, hlo, hs16, y, total;
};

inline size_t pf_align(size_t x) { return (x + 255) & ~(size_t)255; }

PfLayout pf_layout(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k) {
    const size_t n = (size_t)T * (size_t)k;
    PfLayout L;
    size_t o = kFfnSyncBytes;
    L.counts = o;   o += pf_align((size_t)E * 4);
    L.offsets = o;  o += pf_align((size_t)(E + 1) * 4);
    L.tile_off = o; o += pf_align((size_t)(E + 1) * 4);
    L.pairs = o;    o += pf_align(n * 4);
    L.xhi = o;      o += pf_align((size_t)T * H * 2);
    L.xmid = o;     o += pf_align((size_t)T * H * 2);
    L.xlo = o;      o += pf_align((size_t)T * H * 2);
    L.xs16 = o;     o += pf_align((size_t)T * (H / 16) * 4);
    L.h = o;        o += pf_align(n * F * 4);
    L.hhi = o;      o += pf_align(n * F * 2);
    L.hlo = o;      o += pf_align(n * F * 2);
    L.hs16 = o;     o += pf_align(n * (F / 16) * 4);
    L.y = o;        o += pf_align(n * H * 4);
    L.total = o;
    return L;
}

unsigned pf_pieces_grid(int64_t n4) {
    const int64_t blocks = (n4 + 255) / 256;
    return (unsigned)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

}  // namespace

size_t prefill_workspace_bytes(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k) {
    return pf_layout(T, H, F, E, k).total;
}

hipError_t launch_prefill_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                              int32_t k, const int32_t* idx, const float* w,
                              const ExpertTensor& gate, const ExpertTensor& up,
                              const ExpertTensor& down, float* out, int accumulate, void* ws,
                              hipStream_t stream) {
    const PfLayout L = pf_layout(T, H, F, E, k);
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(base + L.tile_off);
    int32_t* pairs = reinterpret_cast<int32_t*>(base + L.pairs);
    const int64_t n = T * k;
    hipError_t err = launch_group_by_expert(idx, n, E, counts, offsets, pairs, stream, tile_off, kPfRows);
    if (err != hipSuccess) return err;

    const int64_t xq = T * H / 4;
    hipLaunchKernelGGL(pf_pieces_kernel<3>, dim3(pf_pieces_grid(xq)), dim3(256), 0, stream, hidden, xq,
                       reinterpret_cast<uint32_t*>(base + L.xhi), reinterpret_cast<uint32_t*>(base + L.xmid),
                       reinterpret_cast<uint32_t*>(base + L.xlo), reinterpret_cast<float*>(base + L.xs16));
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const unsigned slots = (unsigned)(((n + kPfRows - 1) / kPfRows + E + 7) / 8 * 8);
    static LdsLimit gu_lds;
    if ((err = ensure_lds(reinterpret_cast<const void*>(pf_gateup_kernel), gu_lds, kGuLds)) != hipSuccess)
        return err;
    hipLaunchKernelGGL(pf_gateup_kernel, dim3((unsigned)(F / kGuFeat) * slots), dim3(kGuThreads), kGuLds,
                       stream, reinterpret_cast<const uint16_t*>(base + L.xhi),
                       reinterpret_cast<const uint16_t*>(base + L.xmid),
                       reinterpret_cast<const uint16_t*>(base + L.xlo),
                       reinterpret_cast<const float*>(base + L.xs16), H, offsets, tile_off, pairs, E, k,
                       gate.base, gate.stride, up.base, up.stride, F, reinterpret_cast<float*>(base + L.h));
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const int64_t hq = n * F / 4;
    hipLaunchKernelGGL(pf_pieces_kernel<2>, dim3(pf_pieces_grid(hq)), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(base + L.h), hq,
                       reinterpret_cast<uint32_t*>(base + L.hhi), reinterpret_cast<uint32_t*>(base + L.hlo),
                       nullptr, reinterpret_cast<float*>(base + L.hs16));
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const int dl = pf_down_lds(F, down.qtype);
    const void* dfn = down.qtype == 2 ? reinterpret_cast<const void*>(pf_down_kernel<true>)
                                      : reinterpret_cast<const void*>(pf_down_kernel<false>);
    static LdsLimit down_lds6, down_lds4;
    if ((err = ensure_lds(dfn, down.qtype == 2 ? down_lds6 : down_lds4, dl)) != hipSuccess) return err;
    float* Y = reinterpret_cast<float*>(base + L.y);
    auto dk = down.qtype == 2 ? pf_down_kernel<true> : pf_down_kernel<false>;
    hipLaunchKernelGGL(dk, dim3((unsigned)(H / kDnOut) * slots), dim3(kDnThreads), dl, stream,
                       reinterpret_cast<const uint16_t*>(base + L.hhi),
                       reinterpret_cast<const uint16_t*>(base + L.hlo),
                       reinterpret_cast<const float*>(base + L.hs16), F, offsets, tile_off, pairs, E,
                       down.base, down.qtype, down.stride, H, Y);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    hipLaunchKernelGGL(pf_combine_kernel, dim3((unsigned)T, (unsigned)((H + 1023) / 1024)), dim3(256), 0,
                       stream, Y, idx, w, k, E, H, out, accumulate);
    return hipGetLastError();
}

}  // namespace q3moe
