// Batched expert FFN for larger T (prefill): tokens grouped by expert, each
// expert's token tile multiplied by its weight tiles on the matrix cores.
// The pages name token-by-token prefill as the bottleneck and plan grouped
// expert GEMMs for it (aprender issue #3714, gap list); the weights are the
// same Q4_K / Q6_K tensors the decode path reads, in place at base + e*stride.
//
// Pipeline (all on the caller's stream, all grids fixed at launch):
//   1. group: (token, slot) pairs ordered by (expert, pair), per-expert
//      offsets and tile offsets for tiles of kPfRows pairs;
//   2. pieces of the hidden rows: bf16 hi + mid + lo (x to 2^-27; the
//      gate/up outputs amplify the input's rounding most) and the f32 sum of
//      every 16 values;
//   3. gate/up: one workgroup per (64 features, expert tile).  Per super-block
//      the tile's activation pieces and both weight tiles are gathered into
//      LDS with direct-to-LDS loads.  Each 16-wide k step runs
//      v_mfma_f32_16x16x16 on exact bf16 weights (128 + q) with each
//      activation piece.  Each step's result is scaled per (feature, group), and
//      the 128 offset and the Q4_K min are removed through the group sums.
//      h = silu(g) * u goes to the workspace in grouped row order;
//   4. pieces of h (hi + lo);
//   5. down: one workgroup per (64 output rows, expert tile), Q6_K or Q4_K,
//      the whole row tile of the expert's down matrix resident in LDS;
//      rows go to Y indexed by pair;
//   6. combine: out[t] = [out +] sum over slots in slot order of w * Y.
// MFMA operand layouts (checked on the device): A lane l holds row l % 16,
// k = 4 (l / 16) .. + 3; B lane l holds column l % 16 at the same k;
// C lane l holds rows 4 (l / 16) + r, r = 0..3, column l % 16.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRows = 32;                 // grouped pairs per tile (two 16-row MFMA blocks)
constexpr int kPfCols = 64;                 // output features per workgroup (16 per wave)
constexpr int kPfThreads = 256;
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
__device__ __forceinline__ void pf_q4k_factors(const uint8_t* blk, float s[8], float b[8]) {
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    const float d = half_bits_to_float(hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    const uint8_t* S = blk + 4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int sc, m;
        if (j < 4) {
            sc = S[j] & 63;
            m = S[j + 4] & 63;
        } else {
            sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
            m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
        }
        s[j] = 0.125f * d * (float)sc;                    // weights enter as 128 + 8q
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

// ---------------------------------------------------------------- gate/up --
// LDS: activation pieces hi, mid, lo of the 32 rows x 256 values (k-major:
// 16-byte chunk c of row i at (c * 32 + i) * 16), group sums [16][32] f32,
// gate and up weight tiles [64 rows][144 B] of the current super-block.
constexpr int kGuXBytes = kPfRows * kQK * 2;                  // 16 KiB per piece array
constexpr int kGuSBytes = kPfRows * 16 * 4;
constexpr int kGuWBytes = kPfCols * kQ4KBytes;                // 9216
constexpr int kGuLds = 3 * kGuXBytes + kGuSBytes + 2 * kGuWBytes;

__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void pf_gateup_kernel(
    const uint16_t* __restrict__ xhi, const uint16_t* __restrict__ xmid,
    const uint16_t* __restrict__ xlo, const float* __restrict__ xs16, int64_t H, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ pairs, int32_t E, int32_t k,
    const uint8_t* __restrict__ gbase, int64_t gstride, const uint8_t* __restrict__ ubase,
    int64_t ustride, int64_t F, float* __restrict__ hbuf) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* lx_hi = smem;
    uint8_t* lx_mid = smem + kGuXBytes;
    uint8_t* lx_lo = smem + 2 * kGuXBytes;
    const float* ls16 = reinterpret_cast<const float*>(smem + 3 * kGuXBytes);
    uint8_t* lwg = smem + 3 * kGuXBytes + kGuSBytes;
    uint8_t* lwu = lwg + kGuWBytes;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int slot, ftile;
    pf_xcd_tile((int)blockIdx.x, (int)(F / kPfCols), slot, ftile);
    if (slot >= tile_off[E]) return;                          // uniform: an unused tile slot
    const int e = pf_tile_expert(tile_off, E, slot);
    const int64_t row0 = offsets[e] + (int64_t)(slot - tile_off[e]) * kPfRows;
    const int nrows = (int)min((int64_t)kPfRows, (int64_t)offsets[e + 1] - row0);
    const int64_t f0 = (int64_t)ftile * kPfCols;
    const int64_t nsb = H / kQK;
    const int64_t rowb = nsb * kQ4KBytes;                     // bytes per gate/up row
    const uint8_t* gexp = gbase + (int64_t)e * gstride + f0 * rowb;
    const uint8_t* uexp = ubase + (int64_t)e * ustride + f0 * rowb;

    // activation pieces are staged k-major: 16-byte chunk c (8 values) of row
    // i at LDS (c * 32 + i) * 16, so the 16 rows an MFMA operand read touches
    // are 16 consecutive chunks (no bank conflicts); thread tid stages row
    // tid % 32.  Group sums are staged as [group][row] with 4-byte loads.
    const int my_row = tid & 31;
    const int64_t my_tok = my_row < nrows ? pairs[row0 + my_row] / k : -1;
    const int col = lane & 15, kq = lane >> 4;               // MFMA column / k quarter
    const int frow = wave * 16 + col;                        // this lane's weight row in the tile
    f32x4_t acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
        for (int m = 0; m < 2; ++m) acc[rb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int64_t sb = 0; sb < nsb; ++sb) {
        __syncthreads();                                      // the previous stage is consumed
        if (my_tok >= 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {                     // 32 chunks x 32 rows of 16 B
                const int c = (j * kPfThreads + tid) >> 5;
                const int64_t off = (my_tok * H + sb * kQK) * 2 + c * 16;
                const int lo16 = (j * kPfThreads + wave * kWave) * 16;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(xhi) + off,
                                                 (lds_ptr_t)(lx_hi + lo16), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(xmid) + off,
                                                 (lds_ptr_t)(lx_mid + lo16), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(xlo) + off,
                                                 (lds_ptr_t)(lx_lo + lo16), 16, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {                     // 16 groups x 32 rows of 4 B
                const int g = (j * kPfThreads + tid) >> 5;
                __builtin_amdgcn_global_load_lds(xs16 + my_tok * (H / 16) + sb * 16 + g,
                                                 (lds_ptr_t)(smem + 3 * kGuXBytes + (j * kPfThreads + wave * kWave) * 4),
                                                 4, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {                         // 64 rows x 9 pieces per matrix
            const int q = j * kPfThreads + tid;
            if (q < kPfCols * 9) {
                const int64_t off = (int64_t)(q / 9) * rowb + sb * kQ4KBytes + (q % 9) * 16;
                __builtin_amdgcn_global_load_lds(gexp + off, (lds_ptr_t)(lwg + (j * kPfThreads + wave * kWave) * 16),
                                                 16, 0, kCachePolicyNt);
                __builtin_amdgcn_global_load_lds(uexp + off, (lds_ptr_t)(lwu + (j * kPfThreads + wave * kWave) * 16),
                                                 16, 0, kCachePolicyNt);
            }
        }
        wait_all_loads();
        __syncthreads();

        float gs[8], gb[8], us[8], ub[8];
        pf_q4k_factors(lwg + frow * kQ4KBytes, gs, gb);
        pf_q4k_factors(lwu + frow * kQ4KBytes, us, ub);
#pragma unroll
        for (int s = 0; s < 16; ++s) {                        // 16-wide k steps
            const int kk = 16 * s + 4 * kq;                   // this lane's first k in the block
            const int c = kk >> 6, h = (kk >> 5) & 1, lp = kk & 31, j = s >> 1;
            const int qoff = frow * kQ4KBytes + 16 + 32 * c + lp;
            const s16x4_t bg = pf_bf16x4(((*reinterpret_cast<const uint32_t*>(lwg + qoff) >> (4 * h)) << 3) & 0x78787878u);
            const s16x4_t bu = pf_bf16x4(((*reinterpret_cast<const uint32_t*>(lwu + qoff) >> (4 * h)) << 3) & 0x78787878u);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int xoff = ((kk >> 3) * kPfRows + rb * 16 + col) * 16 + (kk & 7) * 2;
                const s16x4_t ah = *reinterpret_cast<const s16x4_t*>(lx_hi + xoff);
                const s16x4_t am = *reinterpret_cast<const s16x4_t*>(lx_mid + xoff);
                const s16x4_t al = *reinterpret_cast<const s16x4_t*>(lx_lo + xoff);
                const float4 S4 = *reinterpret_cast<const float4*>(ls16 + s * kPfRows + rb * 16 + 4 * kq);
                const float Sv[4] = {S4.x, S4.y, S4.z, S4.w};
                f32x4_t tg = pf_mfma(ah, bg, f32x4_t{0.f, 0.f, 0.f, 0.f});
                tg = pf_mfma(am, bg, tg);
                tg = pf_mfma(al, bg, tg);
                f32x4_t tu = pf_mfma(ah, bu, f32x4_t{0.f, 0.f, 0.f, 0.f});
                tu = pf_mfma(am, bu, tu);
                tu = pf_mfma(al, bu, tu);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[rb][0][r] += gs[j] * tg[r] - gb[j] * Sv[r];
                    acc[rb][1][r] += us[j] * tu[r] - ub[j] * Sv[r];
                }
            }
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rb * 16 + 4 * kq + r;
            if (i < nrows) hbuf[(row0 + i) * F + f0 + frow] = pf_silu(acc[rb][0][r]) * acc[rb][1][r];
        }
}

// ------------------------------------------------------------------- down --
// LDS: the expert's down rows h0..h0+63 (all F/256 blocks, contiguous in HBM,
// + 16 bytes of padding for the unaligned Q6_K reads), then the h pieces of
// the tile for the current super-block (k-major), their group sums [16][32],
// and the (scale, offset) of every (row, 16-wide group) of the super-block.
__host__ __device__ inline int pf_down_wbytes(int64_t F, int32_t qtype) {
    return (int)(kPfCols * (F / kQK) * (qtype == 2 ? kQ6KBytes : kQ4KBytes));
}
constexpr int kDnFacBytes = kPfCols * 16 * 8;                 // (scale, offset) per row and group
__host__ __device__ inline int pf_down_lds(int64_t F, int32_t qtype) {
    return pf_down_wbytes(F, qtype) + 16 + 2 * kGuXBytes + kGuSBytes + kDnFacBytes;
}

__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void pf_down_kernel(
    const uint16_t* __restrict__ hhi, const uint16_t* __restrict__ hlo,
    const float* __restrict__ hs16, int64_t F, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ pairs, int32_t E,
    const uint8_t* __restrict__ dbase, int32_t qtype, int64_t dstride, int64_t H,
    float* __restrict__ Y) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int slot, htile;
    pf_xcd_tile((int)blockIdx.x, (int)(H / kPfCols), slot, htile);
    if (slot >= tile_off[E]) return;
    const int e = pf_tile_expert(tile_off, E, slot);
    const int64_t row0 = offsets[e] + (int64_t)(slot - tile_off[e]) * kPfRows;
    const int nrows = (int)min((int64_t)kPfRows, (int64_t)offsets[e + 1] - row0);
    const int64_t h0 = (int64_t)htile * kPfCols;
    const bool q6 = qtype == 2;
    const int bb = q6 ? kQ6KBytes : kQ4KBytes;
    const int64_t nsb = F / kQK;
    const int rowb = (int)(nsb * bb);
    const int wbytes = kPfCols * rowb;
    uint8_t* lw = smem;
    uint8_t* lx_hi = smem + wbytes + 16;
    uint8_t* lx_lo = lx_hi + kGuXBytes;
    const float* ls16 = reinterpret_cast<const float*>(lx_lo + kGuXBytes);
    float2* lfac = reinterpret_cast<float2*>(lx_lo + kGuXBytes + kGuSBytes);   // [group][row]

    // the whole row tile of the down matrix, once
    {
        const uint8_t* src = dbase + (int64_t)e * dstride + h0 * rowb;
        const int n16 = wbytes >> 4;
        for (int base = wave * kWave; base < n16; base += kPfThreads)
            if (base + lane < n16)
                __builtin_amdgcn_global_load_lds(src + (int64_t)(base + lane) * 16, (lds_ptr_t)(lw + base * 16), 16, 0,
                                                 kCachePolicyNt);
    }

    const int my_row = tid & 31;
    const int col = lane & 15, kq = lane >> 4;
    const int frow = wave * 16 + col;
    const uint8_t* wrow = lw + frow * rowb;
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};

    for (int64_t sb = 0; sb < nsb; ++sb) {
        __syncthreads();
        if (my_row < nrows) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {                     // 32 chunks x 32 rows of 16 B, k-major
                const int c = (j * kPfThreads + tid) >> 5;
                const int64_t off = ((row0 + my_row) * F + sb * kQK) * 2 + c * 16;
                const int lo16 = (j * kPfThreads + wave * kWave) * 16;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(hhi) + off,
                                                 (lds_ptr_t)(lx_hi + lo16), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(hlo) + off,
                                                 (lds_ptr_t)(lx_lo + lo16), 16, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {                     // 16 groups x 32 rows of 4 B
                const int g = (j * kPfThreads + tid) >> 5;
                __builtin_amdgcn_global_load_lds(hs16 + (row0 + my_row) * (F / 16) + sb * 16 + g,
                                                 (lds_ptr_t)(lx_lo + kGuXBytes + (j * kPfThreads + wave * kWave) * 4),
                                                 4, 0, 0);
            }
        }
        wait_all_loads();
        __syncthreads();

        // (scale, offset) of every (row, 16-wide group) of this super-block
        for (int f = tid; f < kPfCols * 16; f += kPfThreads) {
            const int r = f >> 4, g = f & 15;
            const uint8_t* b = lw + r * rowb + sb * bb;
            float sc, off;
            if (q6) {
                sc = half_bits_to_float(b[208] | (b[209] << 8)) * (float)(int8_t)b[192 + g];
                off = 160.f * sc;                             // (128 + q) - 160 = q - 32
            } else {
                const uint4 hdr = *reinterpret_cast<const uint4*>(b);
                int scj, mj;
                const int j = g >> 1;
                const uint32_t s0 = hdr.y, s1 = hdr.z, s2 = hdr.w;
                if (j < 4) {
                    scj = (s0 >> (8 * j)) & 63;
                    mj = (s1 >> (8 * j)) & 63;
                } else {
                    const int jj = j - 4;
                    scj = ((s2 >> (8 * jj)) & 15) | (((s0 >> (8 * jj + 6)) & 3) << 4);
                    mj = ((s2 >> (8 * jj + 4)) & 15) | (((s1 >> (8 * jj + 6)) & 3) << 4);
                }
                sc = 0.125f * half_bits_to_float(hdr.x & 0xffffu) * (float)scj;   // 128 + 8q
                off = 128.f * sc + half_bits_to_float(hdr.x >> 16) * (float)mj;
            }
            lfac[g * kPfCols + r] = make_float2(sc, off);
        }
        __syncthreads();

        const uint8_t* blk = wrow + sb * bb;
#pragma unroll 4
        for (int s = 0; s < 16; ++s) {
            const int kk = 16 * s + 4 * kq;
            const float2 fac = lfac[s * kPfCols + frow];
            uint32_t q;
            if (q6) {
                const int n = kk >> 7, r = (kk >> 5) & 3, lp = kk & 31;
                const uint32_t ql = pf_lds_u32_a2(blk, 64 * n + 32 * (r & 1) + lp);
                const uint32_t qh = pf_lds_u32_a2(blk, 128 + 32 * n + lp);
                q = ((ql >> (4 * (r >> 1))) & 0x0f0f0f0fu) | (((qh >> (2 * r)) & 0x03030303u) << 4);
            } else {
                const int c = kk >> 6, h = (kk >> 5) & 1, lp = kk & 31;
                q = ((*reinterpret_cast<const uint32_t*>(blk + 16 + 32 * c + lp) >> (4 * h)) << 3) & 0x78787878u;
            }
            const s16x4_t bw = pf_bf16x4(q);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int xoff = ((kk >> 3) * kPfRows + rb * 16 + col) * 16 + (kk & 7) * 2;
                f32x4_t t = pf_mfma(*reinterpret_cast<const s16x4_t*>(lx_hi + xoff), bw, f32x4_t{0.f, 0.f, 0.f, 0.f});
                t = pf_mfma(*reinterpret_cast<const s16x4_t*>(lx_lo + xoff), bw, t);
                const float4 S4 = *reinterpret_cast<const float4*>(ls16 + s * kPfRows + rb * 16 + 4 * kq);
                acc[rb][0] += fac.x * t[0] - fac.y * S4.x;
                acc[rb][1] += fac.x * t[1] - fac.y * S4.y;
                acc[rb][2] += fac.x * t[2] - fac.y * S4.z;
                acc[rb][3] += fac.x * t[3] - fac.y * S4.w;
            }
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rb * 16 + 4 * kq + r;
            if (i < nrows) Y[(int64_t)pairs[row0 + i] * H + h0 + frow] = acc[rb][r];
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
    hipLaunchKernelGGL(pf_gateup_kernel, dim3((unsigned)(F / kPfCols) * slots), dim3(kPfThreads), kGuLds,
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
    static LdsLimit down_lds;
    if ((err = ensure_lds(reinterpret_cast<const void*>(pf_down_kernel), down_lds, dl)) != hipSuccess)
        return err;
    float* Y = reinterpret_cast<float*>(base + L.y);
    hipLaunchKernelGGL(pf_down_kernel, dim3((unsigned)(H / kPfCols) * slots), dim3(kPfThreads), dl, stream,
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
