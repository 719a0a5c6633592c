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
//   2. pieces of the hidden rows: each row scaled by a power of two and
//      split into fp16 hi + lo (x to 2^-22), with the f32 sum of every 32
//      values and the row's 2^-s;
//   3. gate/up: one workgroup per (128 h features, pair tile), k in stages
//      of 128 through two LDS stage buffers (one barrier per stage);
//      v_mfma_f32_16x16x32_f16 per Q4_K sub-block on the exact fp16 weights
//      1024 + sc q (the sub-block scale folded in), accumulated over the
//      super-block and scaled by its d once; h = silu(g) * u goes to the
//      workspace in grouped row order as two bf16 pieces (hi + lo) with the
//      f32 sum of every 16 values;
//   4. down: one workgroup per (64 output rows, pair tile), Q6_K or Q4_K,
//      the row tile of the expert's down matrix resident in LDS, h staged per
//      128-wide stage; v_mfma_f32_16x16x16bf16_1k per 16-wide scale group;
//      rows go to Y indexed by pair;
//   5. combine: out[t] = [out +] sum over slots in slot order of w * Y.
// In both matrix kernels the weights' offset (and the Q4_K min) times the
// activation sums leaves once per stage as v_mfma_f32_16x16x4_f32 rank-4
// steps.  Workgroups are mapped so that the ones sharing a pair tile run on
// one XCD (one L2).
// MFMA operand layouts (checked on the device): A lane l holds row l % 16,
// k = K (l / 16) .. + K - 1 (K = 4, 8 or 1 values for the 16- and 32-wide
// 16-bit and the f32 forms); B lane l holds column l % 16 at the same k;
// C lane l holds rows 4 (l / 16) + r, r = 0..3, column l % 16.
#include <type_traits>

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

// Q4_K 6-bit scale and min of sub-block j (0..7) from the header's 12 packed
// bytes held as three words (bytes 0-3, 4-7, 8-11).
__device__ __forceinline__ void pf_q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, int& sc, int& m) {
    if (j < 4) {
        sc = (s0 >> (8 * j)) & 63;
        m = (s1 >> (8 * j)) & 63;
    } else {
        const int jj = j - 4;
        sc = ((s2 >> (8 * jj)) & 15) | (((s0 >> (8 * jj + 6)) & 3) << 4);
        m = ((s2 >> (8 * jj + 4)) & 15) | (((s1 >> (8 * jj + 6)) & 3) << 4);
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

// Issue priority of this wave (wave-uniform condition).  In the gate/up
// loop the two waves that share a SIMD alternate in the raised priority from
// stage to stage: the SIMD otherwise serves the older wave first and the
// other one reaches each barrier late (measured 2-3 % faster; the same in
// the down loop measured slower).
__device__ __forceinline__ void wave_prio(bool high) {
    if (high) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
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

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x4_f32: A lane l holds row l % 16, k = l / 16; B lane l
// holds column l % 16 at the same k; C as for the 16-bit forms.
__device__ __forceinline__ f32x4_t pf_mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------ activation pieces --
// One workgroup per hidden row t: the row scaled by a power of two 2^s_t
// (max |x| * 2^s_t < 2^15, so no fp16 piece overflows and the low pieces of
// small values keep their absolute precision), then split into two fp16
// pieces, x' = hi + lo + r with |r| <= 2^-22 |x'| (hi = fp16(x'),
// lo = fp16(x' - hi), both round to nearest even; x' - hi is exact in f32).
// Within every 4 values the order is 0, 2, 1, 3 (the order the gate/up
// kernel's weight operand takes from the packed nibbles).  s32: the f32 sum
// of hi + lo over every 32 values (a Q4_K sub-block); tinv[t] = 2^-s_t.
constexpr int kPfXThreads = 256;
__device__ __forceinline__ uint32_t pf_f16_bits(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__global__ __launch_bounds__(kPfXThreads) void pf_xpieces_kernel(const float* __restrict__ src, int64_t H,
                                                                 uint32_t* __restrict__ phi,
                                                                 uint32_t* __restrict__ plo,
                                                                 float* __restrict__ s32,
                                                                 float* __restrict__ tinv) {
    __shared__ float wmax[kPfXThreads / kWave];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const float4* row = reinterpret_cast<const float4*>(src + t * H);
    const int n4 = (int)(H / 4);                              // a multiple of 64
    float m = 0.f;
    for (int i = tid; i < n4; i += kPfXThreads) {
        const float4 v = row[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if ((tid & (kWave - 1)) == 0) wmax[tid / kWave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPfXThreads / kWave; ++w) m = fmaxf(m, wmax[w]);
    int e = 0;
    if (m > 0.f && m <= 3.4028235e38f) (void)frexpf(m, &e);  // m < 2^e
    const int sh = m > 0.f && m <= 3.4028235e38f ? min(max(15 - e, -126), 126) : 0;
    const float scale = ldexpf(1.f, sh);
    if (tid == 0) tinv[t] = ldexpf(1.f, -sh);
    for (int i = tid; i < n4; i += kPfXThreads) {
        const float4 v = row[i];
        const float x[4] = {v.x * scale, v.z * scale, v.y * scale, v.w * scale};   // order 0, 2, 1, 3
        uint32_t hb[4], lb[4];
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hb[j] = pf_f16_bits(x[j]);
            const float hf = half_bits_to_float(hb[j]);
            lb[j] = pf_f16_bits(x[j] - hf);
            sum += hf + half_bits_to_float(lb[j]);
        }
        phi[2 * (int64_t)t * (n4) + 2 * i] = hb[0] | (hb[1] << 16);
        phi[2 * (int64_t)t * (n4) + 2 * i + 1] = hb[2] | (hb[3] << 16);
        plo[2 * (int64_t)t * (n4) + 2 * i] = lb[0] | (lb[1] << 16);
        plo[2 * (int64_t)t * (n4) + 2 * i + 1] = lb[2] | (lb[3] << 16);
        sum += __shfl_xor(sum, 1, kWave);                     // 8 neighbouring threads: 32 values
        sum += __shfl_xor(sum, 2, kWave);
        sum += __shfl_xor(sum, 4, kWave);
        if ((i & 7) == 0) s32[t * (H / 32) + (i >> 3)] = sum;
    }
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t pf_mfma16h(f16x8_t a, f16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight Q4_K nibbles of one sub-block (nibble h of 8 quant bytes) times the
// sub-block's 6-bit scale sc, as the fp16 values 1024 + sc q (sc q <= 945,
// exact): two nibbles 16 bits apart times sc in one 24-bit multiply-add whose
// addend 0x6400 is the fp16 pattern of 1024.  k order 0, 2, 1, 3 per 4.
__device__ __forceinline__ f16x8_t pf_q4k_f16(uint2 w, int h, uint32_t sc) {
    constexpr uint32_t kM = 0x000f000fu, kBias = 0x64006400u;
    const uint32_t x = h ? (w.x >> 4) : w.x, y = h ? (w.y >> 4) : w.y;
    const u32x4v_t r = {(x & kM) * sc + kBias, ((x >> 8) & kM) * sc + kBias,
                        (y & kM) * sc + kBias, ((y >> 8) & kM) * sc + kBias};
    return __builtin_bit_cast(f16x8_t, r);
}

// ---------------------------------------------------------------- gate/up --
// One workgroup per (128 h features, pair tile): 256 weight rows, gate rows
// f0.. then up rows f0..  8 waves: wave w owns features 16 w..16 w + 15 of
// both matrices and all four 16-pair token blocks (blocks with no pairs are
// skipped), so every weight operand is built once per workgroup and
// silu(g) * u is formed in registers.  Each k step is one Q4_K sub-block:
// v_mfma_f32_16x16x32_f16 of the two activation pieces with the exact fp16
// weights 1024 + sc q, accumulated over the whole super-block and scaled by
// its d once; the 1024 offset and the min, (1024 d + dmin m) times each
// sub-block's activation sum, leave once per stage as one f32 rank-4 matrix
// step per tile.  Results are in the rows' 2^s scale until the epilogue.
// The weights never pass through LDS: each lane loads its row's quant words
// and block header in the matrix operand layout and decodes the scales
// itself (an LDS copy of the weights measured 1.6 % slower).  LDS per stage:
// pieces hi/lo [64 rows][272], the sums [4][64]; then the rows' 2^-s.
constexpr int kGuFeat = 128;
constexpr int kGuThreads = 512;
constexpr int kGuSOff = 2 * kXPieceB;                         // 34816
constexpr int kGuBufB = kGuSOff + 4 * kPfRows * 4;            // 35840: one stage buffer
constexpr int kGuInvOff = 2 * kGuBufB;                        // 71680
constexpr int kGuLds = kGuInvOff + kPfRows * 4;               // 71936

__global__ __launch_bounds__(kGuThreads) void pf_gateup_kernel(
    const uint16_t* __restrict__ xhi, const uint16_t* __restrict__ xlo,
    const float* __restrict__ xs32, const float* __restrict__ tinv, int64_t H,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off,
    const int32_t* __restrict__ pairs, int32_t E, int32_t k, const uint8_t* __restrict__ gbase,
    int64_t gstride, const uint8_t* __restrict__ ubase, int64_t ustride, int64_t F,
    uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo, float* __restrict__ hs16) {
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
    const int nst = (int)(H / kStageK);                       // even (H % 256 == 0)

    // staging roles.  Activations: 2 pieces x 64 rows x 16 chunks of 16 B,
    // item u < 4: piece u >> 1, row tid/16 (u even) or 32 + tid/16 (u odd),
    // chunk tid & 15; sums: thread tid < 256 reads the sum of row tid >> 2,
    // sub-block tid & 3.  Weights go straight into registers in the matrix
    // operand layout: lane (col, g) of wave w holds, per stage, the 8 quant
    // bytes 64 half + 32 c + 8 g (c = 0, 1) of gate row f0 + 16 w + col and of
    // the same up row, and both rows' 16-byte block headers.  Every load is
    // unconditional (rows past the tile read token 0's and are zeroed when
    // stored), so the loop is straight-line code.
    const int ra = tid >> 4, rb2 = 32 + (tid >> 4), xc = tid & 15;
    const bool va = ra < nrows, vb = rb2 < nrows, vs = tid < 4 * kPfRows && (tid >> 2) < nrows;
    const int64_t toka = va ? pairs[row0 + ra] / k : 0;
    const int64_t tokb = vb ? pairs[row0 + rb2] / k : 0;
    const int64_t toks = vs ? pairs[row0 + (tid >> 2)] / k : 0;
    if (tid < kPfRows)
        reinterpret_cast<float*>(smem + kGuInvOff)[tid] = tid < nrows ? tinv[pairs[row0 + tid] / k] : 0.f;
    const int col = lane & 15, g = lane >> 4;
    const int frow = 16 * wave + col;                         // gate row frow, up row frow of uexp
    const uint8_t* grow = gexp + frow * rowb;
    const uint8_t* urow = uexp + frow * rowb;
    // a stage's activation operands in registers: chunks and the sub-block sum
    auto load_x = [&](uint4 (&rx)[4], float& rs, int st) __attribute__((always_inline)) {
        const int64_t k0 = (int64_t)st * kStageK;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t tok = (u & 1) ? tokb : toka;
            const uint16_t* xs = u < 2 ? xhi : xlo;
            rx[u] = *reinterpret_cast<const uint4*>(xs + tok * H + k0 + 8 * xc);
        }
        rs = xs32[toks * (H / 32) + 4 * st + (tid & 3)];
    };
    // this lane's weight operands of stage st: quant words (gate c0, c1, up
    // c0, c1) and the two block headers
    auto load_w = [&](uint2 (&rw)[4], uint4 (&rh)[2], int st) __attribute__((always_inline)) {
        const int64_t off = (int64_t)(st >> 1) * kQ4KBytes;
        const int q0 = 16 + 64 * (st & 1) + 8 * g;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            rw[c] = *reinterpret_cast<const uint2*>(grow + off + q0 + 32 * c);
            rw[2 + c] = *reinterpret_cast<const uint2*>(urow + off + q0 + 32 * c);
        }
        rh[0] = *reinterpret_cast<const uint4*>(grow + off);
        rh[1] = *reinterpret_cast<const uint4*>(urow + off);
    };
    auto store_x = [&](const uint4 (&rx)[4], const float& rs, int half) __attribute__((always_inline)) {
        uint8_t* const sbuf = smem + (half ? kGuBufB : 0);   // stage st goes to buffer st & 1
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = (u & 1) ? rb2 : ra;
            const uint32_t mk = ((u & 1) ? vb : va) ? ~0u : 0u;   // (a mask, not a select of values)
            *reinterpret_cast<uint4*>(sbuf + (u >> 1) * kXPieceB + r * kXRowB + xc * 16) =
                make_uint4(rx[u].x & mk, rx[u].y & mk, rx[u].z & mk, rx[u].w & mk);
        }
        if (tid < 4 * kPfRows)
            reinterpret_cast<float*>(sbuf + kGuSOff)[(tid & 3) * kPfRows + (tid >> 2)] = vs ? rs : 0.f;
    };

    f32x4_t acc[4][2], sbk[4][2];                             // [token block][gate, up]: total, this super-block
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            acc[i][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            sbk[i][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }

    // the matrix work of the stage in LDS for the tile's first NTB token
    // blocks (the rest hold no pairs; NTB is fixed per instantiation so the
    // body has no branches and the LDS reads of later steps can be issued
    // ahead of the matrix work); half: which half of its super-block; rw, rh:
    // this lane's weight words and headers of the stage
    auto compute = [&](auto ntb_c, int half, const uint2 (&rw)[4], const uint4 (&rh)[2])
                       __attribute__((always_inline)) {
        constexpr int NTB = decltype(ntb_c)::value;
        const uint8_t* const sbuf = smem + (half ? kGuBufB : 0);
        // the stage's four 6-bit scales of each row, d, and the offset
        // 1024 d + dmin m of the lane's k slot (sub-block 4 half + g)
        uint32_t scg = 0, scu = 0;
        float nog, nou;
        {
            int sc, m;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                pf_q4k_scale_min(rh[0].y, rh[0].z, rh[0].w, 4 * half + jj, sc, m);
                scg |= (uint32_t)sc << (8 * jj);
                pf_q4k_scale_min(rh[1].y, rh[1].z, rh[1].w, 4 * half + jj, sc, m);
                scu |= (uint32_t)sc << (8 * jj);
            }
            pf_q4k_scale_min(rh[0].y, rh[0].z, rh[0].w, 4 * half + g, sc, m);
            nog = -(1024.f * half_bits_to_float(rh[0].x & 0xffffu) + half_bits_to_float(rh[0].x >> 16) * (float)m);
            pf_q4k_scale_min(rh[1].y, rh[1].z, rh[1].w, 4 * half + g, sc, m);
            nou = -(1024.f * half_bits_to_float(rh[1].x & 0xffffu) + half_bits_to_float(rh[1].x >> 16) * (float)m);
        }
        // the NTB activation blocks' two pieces of sub-block j, read one
        // sub-block ahead of its matrix steps
        f16x8_t ah[2][NTB], al[2][NTB];
        auto read = [&](int j) __attribute__((always_inline)) {
            const int b = j & 1;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int xo = (16 * tb + col) * kXRowB + (32 * j + 8 * g) * 2;
                ah[b][tb] = *reinterpret_cast<const f16x8_t*>(sbuf + xo);
                al[b][tb] = *reinterpret_cast<const f16x8_t*>(sbuf + kXPieceB + xo);
            }
        };
        read(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {                         // one sub-block per k step
            const int b = j & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (j + 1 < 4) read(j + 1);
            const f16x8_t bg = pf_q4k_f16(rw[j >> 1], j & 1, (scg >> (8 * j)) & 0xffu);
            const f16x8_t bu = pf_q4k_f16(rw[2 + (j >> 1)], j & 1, (scu >> (8 * j)) & 0xffu);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                sbk[tb][0] = pf_mfma16h(ah[b][tb], bg, sbk[tb][0]);
                sbk[tb][1] = pf_mfma16h(ah[b][tb], bu, sbk[tb][1]);
            }
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                sbk[tb][0] = pf_mfma16h(al[b][tb], bg, sbk[tb][0]);
                sbk[tb][1] = pf_mfma16h(al[b][tb], bu, sbk[tb][1]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // offset and min of the stage's 4 sub-blocks: acc -= S . off, a rank-4
        // product per tile, as one f32 matrix step (k = sub-block = lane / 16)
        const float dg = half_bits_to_float(rh[0].x & 0xffffu);
        const float du = half_bits_to_float(rh[1].x & 0xffffu);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const float sa = reinterpret_cast<const float*>(sbuf + kGuSOff)[g * kPfRows + 16 * tb + col];
            acc[tb][0] = pf_mfma_f32(sa, nog, acc[tb][0]);
            acc[tb][1] = pf_mfma_f32(sa, nou, acc[tb][1]);
            if (half) {                                       // the super-block is complete
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[tb][0][r] += dg * sbk[tb][0][r];
                    acc[tb][1][r] += du * sbk[tb][1][r];
                }
                sbk[tb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                sbk[tb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    const int ntb = (nrows + 15) >> 4;                        // 1..4, uniform
    // Two LDS stage buffers for the activations (stage st in buffer st & 1),
    // one barrier per stage and two stages in flight in registers (odd
    // stages in set A, even ones in set B): after the barrier before stage
    // st's matrix work, stage st is in its buffer and every wave is done with
    // stage st - 1; stage st + 1 (loaded two stages earlier) goes into the
    // other buffer, stage st + 3 is requested into the registers that held
    // it, and stage st is multiplied.  The weights go into two register sets
    // by stage parity, each requested right after the stage that used it.
    // Past the end the requests repeat the last stage and the stores fill the
    // free buffer (not read), so every trip issues the same loads and stores.
    auto run = [&](auto ntb_c) __attribute__((always_inline)) {
        uint4 rxA[4], rxB[4];
        float rsA, rsB;
        uint2 wA[4], wB[4];
        uint4 hA[2], hB[2];
        load_x(rxA, rsA, 0);
        store_x(rxA, rsA, 0);
        load_x(rxA, rsA, min(1, nst - 1));
        load_x(rxB, rsB, min(2, nst - 1));
        load_w(wA, hA, 0);
        load_w(wB, hB, min(1, nst - 1));
        __syncthreads();
        store_x(rxA, rsA, 1);
        for (int st = 0; st < nst; st += 2) {
            load_x(rxA, rsA, min(st + 3, nst - 1));
            wave_prio(wave >= 4);
            compute(ntb_c, 0, wA, hA);
            load_w(wA, hA, min(st + 2, nst - 1));
            __syncthreads();
            store_x(rxB, rsB, 0);
            load_x(rxB, rsB, min(st + 4, nst - 1));
            wave_prio(wave < 4);
            compute(ntb_c, 1, wB, hB);
            load_w(wB, hB, min(st + 3, nst - 1));
            __syncthreads();
            store_x(rxA, rsA, 1);
        }
    };
    if (ntb == 1) run(std::integral_constant<int, 1>{});
    else if (ntb == 2) run(std::integral_constant<int, 2>{});
    else if (ntb == 3) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 4>{});
    // h = silu(g) * u of the tile's rows, leaving as the down kernel's input:
    // two bf16 pieces (hi = bf16(h), lo = bf16(h - hi)) and the f32 sum of
    // hi + lo over each 16 consecutive features (this wave's 16, held by the
    // 16 lanes of a lane row)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        if (16 * tb >= nrows) continue;                       // uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * g + r;
            float hv = 0.f;
            if (t < nrows) {
                const float inv = reinterpret_cast<const float*>(smem + kGuInvOff)[t];
                hv = pf_silu(acc[tb][0][r] * inv) * (acc[tb][1][r] * inv);
            }
            const uint32_t hb = bf16_rne_bits(hv);
            const uint32_t lb = bf16_rne_bits(hv - bf16_bits_to_float(hb));
            float sp = bf16_bits_to_float(hb) + bf16_bits_to_float(lb);
            sp += __shfl_xor(sp, 1, kWave);
            sp += __shfl_xor(sp, 2, kWave);
            sp += __shfl_xor(sp, 4, kWave);
            sp += __shfl_xor(sp, 8, kWave);
            if (t < nrows) {
                const int64_t o = (row0 + t) * F + f0 + frow;
                hhi[o] = (uint16_t)hb;
                hlo[o] = (uint16_t)lb;
                if (col == 0) hs16[(row0 + t) * (F / 16) + (f0 >> 4) + wave] = sp;
            }
        }
    }
}

// ------------------------------------------------------------------- down --
// One workgroup per (64 output rows, pair tile).  The expert's 64-row tile
// of the down matrix (all F/256 blocks, contiguous in HBM) is staged once
// with the first stage; the h pieces (hi, lo) and their 16-value sums are
// staged per 128-wide k stage.  8 waves: wave w owns output rows
// 16 (w & 3).. and, of every stage's 8 scale groups, groups 4 (w >> 2) ..
// + 3, for all the tile's token blocks (the two waves of a row block add
// their halves through LDS at the end), so each weight operand is built
// once; the stage loop is instantiated per token-block count.  Each k step is
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
    return pf_down_hoff(F, qtype) + 2 * kDnPieceB + 8 * kPfRows * 4 + kPfRows * 4;   // + the rows' pair indices
}

// Q6_K: at most 128 registers, so two workgroups (76 KB of LDS each) share a
// compute unit; the Q4_K form's scale decode needs more registers than that.
template <bool Q6>
__global__ __launch_bounds__(kDnThreads) __attribute__((amdgpu_waves_per_eu(Q6 ? 4 : 2))) void pf_down_kernel(
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
    const int kg = wave >> 2;                                 // this wave's half of each stage's 8 groups
    const int ntb = (nrows + 15) >> 4;                        // token blocks holding pairs (1..4), uniform
    f32x4_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the tile rows' pair indices, staged in LDS now (read at the stores,
    // each would put a memory round trip before its store)
    int32_t* opair = reinterpret_cast<int32_t*>(smem + soff + 8 * kPfRows * 4);
    if (tid < kPfRows) opair[tid] = pairs[row0 + (tid < nrows ? tid : 0)];

    // The matrix work of stage st for the tile's first NTB token blocks: this
    // wave's four scale groups (4 kg .. 4 kg + 3 of the stage's eight; the
    // other wave of the row block takes the rest), each weight operand built
    // once and used by every token block.  NTB is fixed per instantiation.
    auto compute = [&](auto ntb_c, int st) __attribute__((always_inline)) {
        constexpr int NTB = decltype(ntb_c)::value;
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
        for (int G4 = 0; G4 < 4; ++G4) {                      // one 16-wide group per k step
            const int G = 4 * kg + G4;                        // group within the stage
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
                pf_q4k_scale_min(hdr.y, hdr.z, hdr.w, J, scj, mj);
                sc = dq * (float)scj;
            }
            const s16x4_t bw = pf_bf16x4(q);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int xo = hoff + (16 * tb + col) * kDnRowB + (16 * G + 4 * g) * 2;
                f32x4_t t = pf_mfma(*reinterpret_cast<const s16x4_t*>(smem + xo), bw, f32x4_t{0.f, 0.f, 0.f, 0.f});
                t = pf_mfma(*reinterpret_cast<const s16x4_t*>(smem + kDnPieceB + xo), bw, t);
                acc[tb][0] += sc * t[0];
                acc[tb][1] += sc * t[1];
                acc[tb][2] += sc * t[2];
                acc[tb][3] += sc * t[3];
            }
        }
        // the offset (and the Q4_K min) of this wave's 4 groups: acc -= S . off,
        // one f32 rank-4 matrix step per token block (k = group = lane / 16)
        const int gi = 8 * half + 4 * kg + g;                 // this lane's group (its k slot)
        float off;
        if (q6) {
            off = 160.f * dq * (float)(int8_t)blk[192 + gi];  // (128 + q) - 160 = q - 32
        } else {
            int scj, mj;
            pf_q4k_scale_min(hdr.y, hdr.z, hdr.w, gi >> 1, scj, mj);
            off = 128.f * dq * (float)scj + dm * (float)mj;
        }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const float sa = reinterpret_cast<const float*>(smem + soff)[(4 * kg + g) * kPfRows + 16 * tb + col];
            acc[tb] = pf_mfma_f32(sa, -off, acc[tb]);
        }
    };
    auto run = [&](auto ntb_c) __attribute__((always_inline)) {
        for (int st = 0; st < nst; ++st) {
            __syncthreads();
            store_stage();
            __syncthreads();
            if (st + 1 < nst) load_stage(st + 1);
            compute(ntb_c, st);
        }
    };

    load_stage(0);
#pragma unroll
    for (int u = 0; u < kDnMaxW16; ++u) {
        const int q = u * kDnThreads + tid;
        if (q < n16) *reinterpret_cast<u32x4v_t*>(smem + 16 * q) = rwt[u];
    }
    if (ntb == 1) run(std::integral_constant<int, 1>{});
    else if (ntb == 2) run(std::integral_constant<int, 2>{});
    else if (ntb == 3) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 4>{});

    // waves 4-7 hand their half of each row's sums to waves 0-3 through LDS
    // (the h staging area, free after the last stage), which add and store
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem + hoff);      // [row block][tb][r][lane]
    if (kg == 1) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (tb < ntb) red[(((wave & 3) * 4 + tb) * 4 + r) * kWave + lane] = acc[tb][r];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * g + r;
                if (t < nrows)
                    Y[(int64_t)opair[t] * H + h0 + orow] =
                        acc[tb][r] + red[(((wave & 3) * 4 + tb) * 4 + r) * kWave + lane];
            }
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
    size_t counts, offsets, tile_off, pairs, xhi, xlo, xs32, tinv, hhi, hlo, hs16, y, total;
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
    L.xlo = o;      o += pf_align((size_t)T * H * 2);
    L.xs32 = o;     o += pf_align((size_t)T * (H / 32) * 4);
    L.tinv = o;     o += pf_align((size_t)T * 4);
    L.hhi = o;      o += pf_align(n * F * 2);
    L.hlo = o;      o += pf_align(n * F * 2);
    L.hs16 = o;     o += pf_align(n * (F / 16) * 4);
    L.y = o;        o += pf_align(n * H * 4);
    L.total = o;
    return L;
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

    hipLaunchKernelGGL(pf_xpieces_kernel, dim3((unsigned)T), dim3(kPfXThreads), 0, stream, hidden, H,
                       reinterpret_cast<uint32_t*>(base + L.xhi), reinterpret_cast<uint32_t*>(base + L.xlo),
                       reinterpret_cast<float*>(base + L.xs32), reinterpret_cast<float*>(base + L.tinv));
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const unsigned slots = (unsigned)(((n + kPfRows - 1) / kPfRows + E + 7) / 8 * 8);
    static LdsLimit gu_lds;
    if ((err = ensure_lds(reinterpret_cast<const void*>(pf_gateup_kernel), gu_lds, kGuLds)) != hipSuccess)
        return err;
    hipLaunchKernelGGL(pf_gateup_kernel, dim3((unsigned)(F / kGuFeat) * slots), dim3(kGuThreads), kGuLds,
                       stream, reinterpret_cast<const uint16_t*>(base + L.xhi),
                       reinterpret_cast<const uint16_t*>(base + L.xlo),
                       reinterpret_cast<const float*>(base + L.xs32),
                       reinterpret_cast<const float*>(base + L.tinv), H, offsets, tile_off, pairs, E, k,
                       gate.base, gate.stride, up.base, up.stride, F, reinterpret_cast<uint16_t*>(base + L.hhi),
                       reinterpret_cast<uint16_t*>(base + L.hlo), reinterpret_cast<float*>(base + L.hs16));
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
