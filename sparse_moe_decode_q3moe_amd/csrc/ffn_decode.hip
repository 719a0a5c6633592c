// Expert FFN for decode-sized batches (aprender issue #3714: "File facts"
// fixes the expert layout, gap G3 the steps, G8 the device-side gather and
// weighted accumulate).
//
// ffn_fused8_kernel (H = 2048, T <= 4, k <= 8): the whole expert FFN in one
// persistent launch, optionally with the routing inside (the MoE block of
// q3moe_moe_ffn); workgroups hand the router partial sums and h to each
// other as tagged words.  Gate/up take the activations as three int8
// pieces (exact int32 dot products); down takes each 16-weight group as
// a * sum(q h) + c * sum(h) in f32.  Described in detail at the kernel.
//
// Other shapes, two kernels per call:
//   gu_decode_kernel   one wave per task = (token-slot pair, R rows of the
//                      selected expert's gate AND up matrices): direct
//                      HBM->LDS loads of both R-row tiles, dequantise in
//                      registers, h = silu(g) * u written as activation
//                      pieces for the down kernel.
//   down_decode_kernel one workgroup per (token, 8 output rows): every wave
//                      loads the 8-row tiles of two slots' down matrices and
//                      those slots' h pieces, dequantises, multiplies by the
//                      routing weight, and the workgroup sums the slots in
//                      slot order (deterministic, no atomics).
//   Weights as exact small integers (bf16 128 + q); the gate/up input as
//   three bf16 pieces (hi + mid + lo) and h as two (hi + lo);
//   v_dot2_f32_bf16 with f32 accumulation; the per-block scales, the Q4_K
//   min term and the integer offsets are applied per 16/32 group in f32.
//
// Weights are never repacked: tiles are read in place at base + e*stride.
#include <atomic>

#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace q3moe {

namespace {

constexpr int kGuWaves = 4;
constexpr int kDnWaves = 4;
constexpr int kDnRows = 8;          // output rows per down workgroup
constexpr int kDnSlotsPerWave = 2;  // lanes 0-31 one slot, lanes 32-63 the next
constexpr uint32_t kBf16Bias = 0x43004300u;   // bf16 128.0 in both halves

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// 16 bytes of data read once (expert weights), loaded non-temporally so the
// stream does not evict reused lines (code, routing, counters) from L2.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Bytes q0..q3 of v (each < 128) as bf16 pairs (128 + q0, 128 + q2) and
// (128 + q1, 128 + q3): the byte goes into the mantissa under exponent byte
// 0x43, in the value order of an activation piece slot.
constexpr uint32_t kBias8 = 0x43434343u;
__device__ __forceinline__ uint32_t bf16_pair_even(uint32_t v) {
    return __builtin_amdgcn_perm(kBias8, v, 0x04020400u);
}
__device__ __forceinline__ uint32_t bf16_pair_odd(uint32_t v) {
    return __builtin_amdgcn_perm(kBias8, v, 0x04030401u);
}

__device__ __forceinline__ void store_h_piece(uint8_t* __restrict__ hp, int64_t value_index,
                                              float h) {
    // value i lives in slot i/4 at half-word (i%4 == 0: 0, 1: 2, 2: 1, 3: 3) of
    // the hi pair dwords, and the same half-word of the lo pair dwords (+8 B)
    const uint32_t hb = bf16_rne_bits(h);
    const uint32_t lb = bf16_rne_bits(h - bf16_bits_to_float(hb));
    const int pos = (int)(value_index & 3);
    const int hw = ((pos & 1) << 1) | (pos >> 1);
    uint16_t* slot = reinterpret_cast<uint16_t*>(hp + (value_index >> 2) * kSlotBytes);
    // device-scope stores write through the per-XCD L2, so a down wave on
    // any XCD that later reads them with coherent loads sees them
    __hip_atomic_store(slot + hw, (uint16_t)hb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(slot + 4 + hw, (uint16_t)lb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A whole slot (values i..i+3, i a multiple of 4) with device-scope stores.
__device__ __forceinline__ void store_h_slot(uint8_t* __restrict__ hp, int64_t value_index,
                                             uint4 slot) {
    uint32_t* d = reinterpret_cast<uint32_t*>(hp + (value_index >> 2) * kSlotBytes);
    __hip_atomic_store(d + 0, slot.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d + 1, slot.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d + 2, slot.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(d + 3, slot.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Q4_K scale and min of sub-block j (compile-time j) from the three dwords
// holding the 12 packed bytes.
template <int J>
__device__ __forceinline__ void q4k_sm_const(uint32_t s0, uint32_t s1, uint32_t s2, int& sc, int& mn) {
    if constexpr (J < 4) {
        sc = (s0 >> (8 * J)) & 63;
        mn = (s1 >> (8 * J)) & 63;
    } else {
        constexpr int jj = J - 4;
        sc = ((s2 >> (8 * jj)) & 15) | (((s0 >> (8 * jj + 6)) & 3) << 4);
        mn = ((s2 >> (8 * jj + 4)) & 15) | (((s1 >> (8 * jj + 6)) & 3) << 4);
    }
}

// The same with a run-time sub-block index.
__device__ __forceinline__ void q4k_sm_var(uint32_t s0, uint32_t s1, uint32_t s2, int j, int& sc, int& mn) {
    if (j < 4) {
        sc = (s0 >> (8 * j)) & 63;
        mn = (s1 >> (8 * j)) & 63;
    } else {
        const int jj = j - 4;
        sc = ((s2 >> (8 * jj)) & 15) | (((s0 >> (8 * jj + 6)) & 3) << 4);
        mn = ((s2 >> (8 * jj + 4)) & 15) | (((s1 >> (8 * jj + 6)) & 3) << 4);
    }
}

// Eight quant dwords (32 bytes, chunk c of a Q4_K block) against the pieces of
// the matching activations: returns the two raw dot products
// A = sum (128 + 8 q_lo) x~ over sub-block 2c's 32 weights, B likewise for
// 2c+1.  The nibble sits in the top of the bf16 mantissa (exact), so the 128
// offset is 16x the largest weight rather than 128x: the sums stay close to
// the useful part and lose less to f32 rounding when the offset is removed.
// xlo (the third pieces, or nullptr for two-piece activations) in the
// piece_lo_off layout of the same block.
__device__ __forceinline__ void q4k_chunk_dots(const uint32_t* qw, const uint8_t* xblk,
                                               const uint8_t* xlo, int c, float& A, float& B) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint4 xa = *reinterpret_cast<const uint4*>(xblk + (16 * c + q) * kSlotBytes);
        const uint4 xb = *reinterpret_cast<const uint4*>(xblk + (16 * c + 8 + q) * kSlotBytes);
        const uint32_t lo = (qw[q] << 3) & 0x78787878u, hi = (qw[q] >> 1) & 0x78787878u;
        const uint32_t p0 = bf16_pair_even(lo), p1 = bf16_pair_odd(lo);
        const uint32_t p2 = bf16_pair_even(hi), p3 = bf16_pair_odd(hi);
        a = dot2_bf16(p0, xa.x, a);
        a = dot2_bf16(p1, xa.y, a);
        a = dot2_bf16(p0, xa.z, a);
        a = dot2_bf16(p1, xa.w, a);
        b = dot2_bf16(p2, xb.x, b);
        b = dot2_bf16(p3, xb.y, b);
        b = dot2_bf16(p2, xb.z, b);
        b = dot2_bf16(p3, xb.w, b);
        if (xlo) {
            const uint2 la = *reinterpret_cast<const uint2*>(xlo + (16 * c + q) * 8);
            const uint2 lb = *reinterpret_cast<const uint2*>(xlo + (16 * c + 8 + q) * 8);
            a = dot2_bf16(p0, la.x, a);
            a = dot2_bf16(p1, la.y, a);
            b = dot2_bf16(p2, lb.x, b);
            b = dot2_bf16(p3, lb.y, b);
        }
    }
    A = a;
    B = b;
}

// Whole Q4_K block (256 weights) in LDS against its 256 activations' pieces
// (xblk) and group sums (gsum, 16 values).
__device__ __forceinline__ float q4k_block_dot(const uint8_t* blk, const uint8_t* xblk,
                                               const uint8_t* xlo, const float* gsum) {
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    const float d8 = 0.125f * half_bits_to_float(hdr.x & 0xffffu);   // weights enter as 128 + 8q
    const float dmin = half_bits_to_float(hdr.x >> 16);
    float row = 0.f;
#define Q3MOE_Q4K_CHUNK(C)                                                                  \
    {                                                                                       \
        const uint4 qa = *reinterpret_cast<const uint4*>(blk + 16 + 32 * (C));              \
        const uint4 qb = *reinterpret_cast<const uint4*>(blk + 32 + 32 * (C));              \
        const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};            \
        float A, B;                                                                         \
        q4k_chunk_dots(qw, xblk, xlo, (C), A, B);                                           \
        int sc0, mn0, sc1, mn1;                                                             \
        q4k_sm_const<2 * (C)>(hdr.y, hdr.z, hdr.w, sc0, mn0);                               \
        q4k_sm_const<2 * (C) + 1>(hdr.y, hdr.z, hdr.w, sc1, mn1);                           \
        const float sx0 = gsum[4 * (C)] + gsum[4 * (C) + 1];                                \
        const float sx1 = gsum[4 * (C) + 2] + gsum[4 * (C) + 3];                            \
        row += d8 * ((float)sc0 * (A - 128.f * sx0) + (float)sc1 * (B - 128.f * sx1)) -     \
               dmin * ((float)mn0 * sx0 + (float)mn1 * sx1);                                \
    }
    Q3MOE_Q4K_CHUNK(0)
    Q3MOE_Q4K_CHUNK(1)
    Q3MOE_Q4K_CHUNK(2)
    Q3MOE_Q4K_CHUNK(3)
#undef Q3MOE_Q4K_CHUNK
    return row;
}

// Convert one token's H activations (global f32) into pieces + group sums
// in LDS, using all threads of the workgroup.  H/4 is a multiple of 64 so
// every wave that enters the loop is full.
__device__ __forceinline__ void activations_to_pieces(const float* __restrict__ x, int H,
                                                      uint8_t* xp, uint8_t* xlo, float* gs, int tid,
                                                      int nthr) {
    for (int s = tid; s < H / 4; s += nthr) {
        const Pieces4x3 pc = make_pieces4x3(reinterpret_cast<const float4*>(x)[s]);
        *reinterpret_cast<uint4*>(xp + piece_slot_off(s)) = pc.slot;
        *reinterpret_cast<uint2*>(xlo + piece_lo_off(s)) = pc.lo;
        float g = pc.sum + __shfl_xor(pc.sum, 1, kWave);
        g += __shfl_xor(g, 2, kWave);
        if ((s & 3) == 0) gs[s >> 2] = g;
    }
}

// Gate/up task geometry for NB = H/256 dividing 32: R = 32/NB rows of one
// expert's gate and up matrices, 2 x 32 super-blocks = 9,216 bytes.
template <int NB>
struct GuTask {
    static constexpr int H = NB * kQK;
    static constexpr int R = 32 / NB;
    static constexpr int ROWB = NB * kQ4KBytes;
    static constexpr int TASKB = R * ROWB;                  // bytes per matrix
};

template <int NB>
__device__ __forceinline__ void gu_issue(const uint8_t* __restrict__ gbase, int64_t gstride,
                                         const uint8_t* __restrict__ ubase, int64_t ustride, int e,
                                         int64_t r0, uint8_t* wg, int lane) {
    using G = GuTask<NB>;
    wave_copy_to_lds(wg, gbase + (int64_t)e * gstride + r0 * G::ROWB, G::TASKB, lane);
    wave_copy_to_lds(wg + G::TASKB, ubase + (int64_t)e * ustride + r0 * G::ROWB, G::TASKB, lane);
}

// Lane = m*32 + rho*NB + b: matrix m (0 gate, 1 up), row rho of the task,
// super-block b of the row.  Writes h = silu(g)*u of the R rows as pieces.
template <int NB>
__device__ __forceinline__ void gu_compute(const uint8_t* wg, const uint8_t* xp, const uint8_t* xlo,
                                           const float* gs, bool valid, int lane,
                                           uint8_t* __restrict__ hpieces, int64_t value_base) {
    using G = GuTask<NB>;
    const int m = lane >> 5, rho = (lane & 31) / NB, b = lane % NB;
    float row = valid ? q4k_block_dot(wg + m * G::TASKB + rho * G::ROWB + b * kQ4KBytes,
                                      xp + b * kBlockPieceStride, xlo + b * kBlockLoStride, gs + b * 16)
                      : 0.f;
#pragma unroll
    for (int o = 1; o < NB; o <<= 1) row += __shfl_xor(row, o, kWave);
    const float up = __shfl_xor(row, 32, kWave);
    const float h = silu_f(row) * up;                  // meaningful where m == 0 && b == 0
    if constexpr (G::R >= 4) {
        // gather rows 4q..4q+3 into the lane of row 4q and store the whole slot
        const float h1 = __shfl(h, (lane + NB) & 63, kWave);
        const float h2 = __shfl(h, (lane + 2 * NB) & 63, kWave);
        const float h3 = __shfl(h, (lane + 3 * NB) & 63, kWave);
        if (m == 0 && b == 0 && (rho & 3) == 0)
            store_h_slot(hpieces, value_base + rho, make_pieces4(make_float4(h, h1, h2, h3)).slot);
    } else {
        if (m == 0 && b == 0) store_h_piece(hpieces, value_base + rho, h);
    }
}

// Gate/up for H = 2048 (8 super-blocks per row, 4 rows of gate and 4 of up
// per task) with each lane owning a column chunk: lane = b*8 + c*2 + hp owns
// quant bytes 32c + 16hp .. +15 of super-block b, i.e. 16 weights of
// sub-block 2c (low nibbles) and 16 of sub-block 2c+1 (high nibbles).  The
// lane loads its weights straight into registers (16 quant bytes and one
// dword of the 16-byte block header per row, the four lanes of a quad
// fetching the four dwords and DPP broadcasts rebuilding the header: a
// quarter of the address work of a 16-byte header load in every lane), so
// nothing goes through LDS and each row is consumed as soon as its loads
// land.  The 8 row partials are folded across
// the wave with a transposed butterfly: after it, lanes 8q..8q+7 hold row q
// (q < 4 gate row q, else up row q-4).
//
// Activations enter as three int8 pieces per value: for each 32-value group
// (one Q4_K sub-block) a power of two s with max|x| / s < 127.5 and
//   x = s * (p1 + p2 / 2^7 + p3 / 2^14) + r,   |r| <= s * 2^-15,
// p1 in [-127, 127], p2 and p3 in [-64, 64] (each a rounded residual, all
// steps exact in f32).  The nibbles are int8 values 0..15, so v_dot4_i32_i8
// gives each piece's dot product over 4 weights exactly in int32, and
// 2^14 S1 + 2^7 S2 + S3 (< 2^30 for 16 weights) is the whole sub-block dot
// in units of s * 2^-14, exact until its one conversion to f32.  The min
// term uses the exact f32 sums of the activations.
//
// Per token in LDS (kI8TokenBytes): piece P at P * kI8PieceBytes as
// [half][lane][16 bytes] (half 0: the lane's low-nibble values, 1: its
// high-nibble values), then the 64 group scales s * 2^-14 (f32, group
// b*8 + j), then the 16-value sums as [half][lane] (f32).
constexpr int kI8PieceBytes = 2 * kWave * 16;
constexpr int kI8ScaleOff = 3 * kI8PieceBytes;
constexpr int kI8SumOff = kI8ScaleOff + 64 * 4;
constexpr int kI8TokenBytes = kI8SumOff + 2 * kWave * 4;

struct XCols {
    uint4 p[3][2];           // [piece][half]: 16 int8 pieces each
    float sa, sb;            // group scales (times 2^-14) of the two halves
    float slo, shi;          // sums of the lane's 16 low-nibble / high-nibble values
    uint32_t sel;            // byte selector of the lane's two sub-blocks' scale bytes
    uint32_t shh;            // 4 (sub-blocks 0-3) or 6 (4-7): where their top scale bits sit
    bool hiform;             // sub-blocks 4-7: low scale bits in the third scale dword
};

template <int NP>
__device__ __forceinline__ XCols load_xcols(const uint8_t* xt, int lane) {
    const int b = lane >> 3, c = (lane >> 1) & 3;
    XCols x;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            x.p[q][h] = *reinterpret_cast<const uint4*>(xt + q * kI8PieceBytes + h * (kWave * 16) + lane * 16);
    const float* sc = reinterpret_cast<const float*>(xt + kI8ScaleOff);
    const float* sm = reinterpret_cast<const float*>(xt + kI8SumOff);
    x.sa = sc[b * 8 + 2 * c];
    x.sb = sc[b * 8 + 2 * c + 1];
    x.slo = sm[lane];
    x.shi = sm[kWave + lane];
    const uint32_t jx = (2 * c) & 3, jy = jx + 1;
    x.sel = jx | ((jx + 4) << 8) | (jy << 16) | ((jy + 4) << 24);
    x.hiform = c >= 2;
    x.shh = x.hiform ? 6 : 4;
    return x;
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// The first step of a dot-product chain: the three-operand form with an
// inline zero accumulator (the builtin picks the two-operand form, whose
// accumulator is also its result, and first moves a zero into it).
__device__ __forceinline__ int sdot4_first(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// One row's contribution of this lane: hdr = the block header (d, dmin, 12
// scale bytes), qv = the lane's 16 quant bytes.  NP = 3: the three pieces
// of the exact form, A and B in units of s * 2^-14; NP = 1: the single int8
// piece of the int8-activation mode, in units of its group scale.
template <int NP>
__device__ __forceinline__ float q4k_cols_row(uint4 hdr, uint4 qv, const XCols& x) {
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    int a1, a2 = 0, a3 = 0, b1, b2 = 0, b3 = 0;
    {
        const uint32_t lo = qw[0] & 0x0f0f0f0fu;               // 4 weights of sub-block 2c
        const uint32_t hi = (qw[0] >> 4) & 0x0f0f0f0fu;        // 4 weights of sub-block 2c+1
        a1 = sdot4_first(lo, x.p[0][0].x);
        b1 = sdot4_first(hi, x.p[0][1].x);
        if constexpr (NP == 3) {
            a2 = sdot4_first(lo, x.p[1][0].x);
            a3 = sdot4_first(lo, x.p[2][0].x);
            b2 = sdot4_first(hi, x.p[1][1].x);
            b3 = sdot4_first(hi, x.p[2][1].x);
        }
    }
#pragma unroll
    for (int q = 1; q < 4; ++q) {
        const uint32_t lo = qw[q] & 0x0f0f0f0fu;
        const uint32_t hi = (qw[q] >> 4) & 0x0f0f0f0fu;
        a1 = sdot4(lo, (&x.p[0][0].x)[q], a1);
        b1 = sdot4(hi, (&x.p[0][1].x)[q], b1);
        if constexpr (NP == 3) {
            a2 = sdot4(lo, (&x.p[1][0].x)[q], a2);
            a3 = sdot4(lo, (&x.p[2][0].x)[q], a3);
            b2 = sdot4(hi, (&x.p[1][1].x)[q], b2);
            b3 = sdot4(hi, (&x.p[2][1].x)[q], b3);
        }
    }
    const int A = NP == 3 ? a1 * 16384 + a2 * 128 + a3 : a1;
    const int B = NP == 3 ? b1 * 16384 + b2 * 128 + b3 : b1;
    // [sc(2c), mn(2c), sc(2c+1), mn(2c+1)] as bytes, branch-free: the low four
    // bits come from the first two scale dwords (sub-blocks 0-3) or from the
    // third one's nibbles (4-7), the top two from bits 4-5 or 6-7 of the first two
    const uint32_t q = __builtin_amdgcn_perm(hdr.z, hdr.y, x.sel);
    const uint32_t r = __builtin_amdgcn_perm(hdr.w >> 4, hdr.w, x.sel);
    const uint32_t low4 = (x.hiform ? r : q) & 0x0f0f0f0fu;
    const uint32_t sm = low4 | (((q >> x.shh) & 0x03030303u) << 4);
    const float d = half_bits_to_float(hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    const float sc0 = (float)(sm & 0xffu), mn0 = (float)((sm >> 8) & 0xffu);
    const float sc1 = (float)((sm >> 16) & 0xffu), mn1 = (float)(sm >> 24);
    return d * (sc0 * ((float)A * x.sa) + sc1 * ((float)B * x.sb)) - dmin * (mn0 * x.slo + mn1 * x.shi);
}

// A float moved across lanes by a DPP pattern within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRor8 = 0x128;         // row_ror:8, i.e. lane i <-> i ^ 8 within a row

// Sum v[0..7] over the 64 lanes; returns row (lane >> 3)'s total.  A
// transposed butterfly: each exchange halves the values a lane carries
// (xor 32 and 16 across rows through the LDS crossbar, xor 8 by DPP), then
// the 8 lanes of a row group add their values with three DPP steps.
__device__ __forceinline__ float fold8_rows(const float v[8], int lane) {
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
    float a[4], c[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = b5 ? v[i] : v[i + 4];
        const float keep = b5 ? v[i + 4] : v[i];
        a[i] = keep + __shfl_xor(send, 32, kWave);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b4 ? a[i] : a[i + 2];
        const float keep = b4 ? a[i + 2] : a[i];
        c[i] = keep + __shfl_xor(send, 16, kWave);
    }
    const float send = b3 ? c[0] : c[1];
    float r = (b3 ? c[1] : c[0]) + dpp_f32<kDppRor8>(send);
    r += dpp_f32<kDppXor1>(r);
    r += dpp_f32<kDppXor2>(r);
    r += dpp_f32<kDppHalfMirror>(r);
    return r;
}

// grid: T*k*(F/R)/kGuWaves workgroups of kGuWaves waves, one task per wave.
template <int NB>
__global__ __launch_bounds__(kGuWaves * kWave) void gu_decode_kernel(
    const float* __restrict__ hidden, int64_t F, int32_t E, int32_t k,
    const int32_t* __restrict__ idx, const uint8_t* __restrict__ gbase, int64_t gstride,
    const uint8_t* __restrict__ ubase, int64_t ustride, uint8_t* __restrict__ hpieces) {
    using G = GuTask<NB>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t* wg = smem + wave * 2 * G::TASKB;
    uint8_t* xp = smem + kGuWaves * 2 * G::TASKB;
    float* gs = reinterpret_cast<float*>(xp + NB * kBlockPieceStride);
    uint8_t* xlo = reinterpret_cast<uint8_t*>(gs + NB * 16);

    const int tiles = (int)(F / G::R);                    // tasks per pair, a multiple of kGuWaves
    const int64_t task = (int64_t)blockIdx.x * kGuWaves + wave;
    const int64_t p = task / tiles;                       // same for the whole workgroup
    const int64_t t = p / k;
    const int64_t r0 = (task % tiles) * G::R;
    const int e = idx[p];
    const bool valid = e >= 0 && e < E;
    if (valid) gu_issue<NB>(gbase, gstride, ubase, ustride, e, r0, wg, lane);
    activations_to_pieces(hidden + t * G::H, G::H, xp, xlo, gs, tid, kGuWaves * kWave);
    wait_all_loads();
    __syncthreads();
    gu_compute<NB>(wg, xp, xlo, gs, valid, lane, hpieces, p * F + r0);
}

// ----------------------------------------------------------------- down --

// Q6_K: lane handles (n, lh) of its row's block: l = 16lh..16lh+15 for all
// four r, i.e. 64 weights in four 16-weight scale groups.
__device__ __forceinline__ float q6k_lane_dot(const uint8_t* lds, int boff, int n, int lh,
                                              const uint8_t* xblk, const float* gsum) {
    const uint4 La = lds_read16_a2(lds, boff + 64 * n + 16 * lh);        // r = 0 (lo), 2 (hi)
    const uint4 Lb = lds_read16_a2(lds, boff + 64 * n + 32 + 16 * lh);   // r = 1 (lo), 3 (hi)
    const uint4 Hd = lds_read16_a2(lds, boff + 128 + 32 * n + 16 * lh);
    const uint32_t la[4] = {La.x, La.y, La.z, La.w};
    const uint32_t lb[4] = {Lb.x, Lb.y, Lb.z, Lb.w};
    const uint32_t hd[4] = {Hd.x, Hd.y, Hd.z, Hd.w};
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int lq = 0; lq < 4; ++lq) {
        uint32_t q[4];
        q[0] = (la[lq] & 0x0f0f0f0fu) | ((hd[lq] << 4) & 0x30303030u);
        q[1] = (lb[lq] & 0x0f0f0f0fu) | ((hd[lq] << 2) & 0x30303030u);
        q[2] = ((la[lq] >> 4) & 0x0f0f0f0fu) | (hd[lq] & 0x30303030u);
        q[3] = ((lb[lq] >> 4) & 0x0f0f0f0fu) | ((hd[lq] >> 2) & 0x30303030u);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint4 x = *reinterpret_cast<const uint4*>(
                xblk + (32 * n + 8 * r + 4 * lh + lq) * kSlotBytes);
            const uint32_t p0 = (q[r] & 0x00ff00ffu) | kBf16Bias;
            const uint32_t p1 = ((q[r] >> 8) & 0x00ff00ffu) | kBf16Bias;
            float a = acc[r];
            a = dot2_bf16(p0, x.x, a);
            a = dot2_bf16(p1, x.y, a);
            a = dot2_bf16(p0, x.z, a);
            a = dot2_bf16(p1, x.w, a);
            acc[r] = a;
        }
    }
    const float d = half_bits_to_float(lds[boff + 208] | (lds[boff + 209] << 8));
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int g = 8 * n + 2 * r + lh;
        const float sc = (float)(int8_t)lds[boff + 192 + g];
        sum += sc * (acc[r] - 160.f * gsum[g]);
    }
    return d * sum;
}

// Q4_K down rows: lane handles chunk c (sub-blocks 2c, 2c+1, 64 weights).
__device__ __forceinline__ float q4k_lane_dot(const uint8_t* blk, int c, const uint8_t* xblk,
                                              const float* gsum) {
    const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
    const uint4 qa = *reinterpret_cast<const uint4*>(blk + 16 + 32 * c);
    const uint4 qb = *reinterpret_cast<const uint4*>(blk + 32 + 32 * c);
    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float A, B;
    q4k_chunk_dots(qw, xblk, nullptr, c, A, B);
    int sc0, mn0, sc1, mn1;
    q4k_sm_var(hdr.y, hdr.z, hdr.w, 2 * c, sc0, mn0);
    q4k_sm_var(hdr.y, hdr.z, hdr.w, 2 * c + 1, sc1, mn1);
    const float d = half_bits_to_float(hdr.x & 0xffffu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    const float sx0 = gsum[4 * c] + gsum[4 * c + 1];
    const float sx1 = gsum[4 * c + 2] + gsum[4 * c + 3];
    return 0.125f * d * ((float)sc0 * (A - 128.f * sx0) + (float)sc1 * (B - 128.f * sx1)) -
           dmin * ((float)mn0 * sx0 + (float)mn1 * sx1);
}

// Geometry of a down slot region in LDS: the 8-row tile of one expert's down
// matrix, 16 bytes of padding (the unaligned Q6_K reads look up to 4 bytes
// ahead), that slot's h pieces (padded blocks) and their group sums.
struct DnGeom {
    int nb, bb, rowb, tile, tile_pad, pieces, sums, per_slot;
    bool q6;
    __host__ __device__ DnGeom(int64_t F, int32_t qtype) {
        nb = (int)(F / kQK);
        q6 = qtype == 2;
        bb = q6 ? kQ6KBytes : kQ4KBytes;
        rowb = nb * bb;
        tile = kDnRows * rowb;                            // multiple of 16
        tile_pad = tile + 16;
        pieces = nb * kBlockPieceStride;
        sums = nb * 16 * 4;
        per_slot = tile_pad + pieces + sums;
    }
};

__device__ __forceinline__ void dn_issue_weights(uint8_t* reg, const DnGeom& g,
                                                 const uint8_t* __restrict__ dbase, int64_t dstride,
                                                 int e, int64_t r0, int lane) {
    wave_stream_to_lds(reg, dbase + (int64_t)e * dstride + r0 * g.rowb, g.tile, lane);
}

__device__ __forceinline__ void dn_issue_h(uint8_t* reg, const DnGeom& g, const uint8_t* hsrc,
                                           int lane) {
    for (int b = 0; b < g.nb; ++b)
        wave_copy_to_lds_coherent(reg + g.tile_pad + b * kBlockPieceStride, hsrc + b * 1024, 1024,
                                  lane);
}

// Group sums (16 values = 4 slots per group) of a slot region's h pieces.
__device__ __forceinline__ void dn_group_sums(uint8_t* reg, const DnGeom& g, int lane) {
    const uint8_t* xs = reg + g.tile_pad;
    float* gs = reinterpret_cast<float*>(reg + g.tile_pad + g.pieces);
    for (int gi = lane; gi < g.nb * 16; gi += kWave) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v += slot_sum(*reinterpret_cast<const uint4*>(xs + piece_slot_off(4 * gi + i)));
        gs[gi] = v;
    }
}

// This lane's share (quarter u of every super-block) of output row rho.
__device__ __forceinline__ float dn_lane_row(const uint8_t* reg, const DnGeom& g, int rho, int u) {
    const uint8_t* xs = reg + g.tile_pad;
    const float* gs = reinterpret_cast<const float*>(xs + g.pieces);
    float y = 0.f;
    for (int b = 0; b < g.nb; ++b) {
        const int boff = rho * g.rowb + b * g.bb;
        y += g.q6 ? q6k_lane_dot(reg, boff, u >> 1, u & 1, xs + b * kBlockPieceStride, gs + b * 16)
                  : q4k_lane_dot(reg + boff, u, xs + b * kBlockPieceStride, gs + b * 16);
    }
    return y;
}

// grid: (T, H/8).  Dynamic LDS: 4 waves x 2 slot regions + the slot-result
// table.  Lane = sh*32 + rho*4 + u: slot sh of the wave's pair, output row
// rho, quarter u of each super-block.
__global__ __launch_bounds__(kDnWaves * kWave) void down_decode_kernel(
    int64_t H, int64_t F, int32_t E, int32_t k, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const uint8_t* __restrict__ dbase, int32_t qtype,
    int64_t dstride, const uint8_t* __restrict__ hpieces, float* __restrict__ out,
    int accumulate) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const DnGeom g(F, qtype);
    uint8_t* wbase = smem + wave * kDnSlotsPerWave * g.per_slot;
    float* ys = reinterpret_cast<float*>(smem + kDnWaves * kDnSlotsPerWave * g.per_slot);

    const int64_t t = blockIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kDnRows;
    const int sh = lane >> 5, rho = (lane >> 2) & 7, u = lane & 3;
    const int group = kDnWaves * kDnSlotsPerWave;

    for (int s0 = 0; s0 < k; s0 += group) {
        int ev[kDnSlotsPerWave];
#pragma unroll
        for (int j = 0; j < kDnSlotsPerWave; ++j) {
            const int s = s0 + wave * kDnSlotsPerWave + j;
            ev[j] = s < k ? idx[t * k + s] : -1;
            if (ev[j] >= 0 && ev[j] < E) {
                uint8_t* reg = wbase + j * g.per_slot;
                dn_issue_weights(reg, g, dbase, dstride, ev[j], r0, lane);
                dn_issue_h(reg, g, hpieces + (t * k + s) * F * 4, lane);
            }
        }
        wait_all_loads();
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kDnSlotsPerWave; ++j) dn_group_sums(wbase + j * g.per_slot, g, lane);
        __syncthreads();
        const int s = s0 + wave * kDnSlotsPerWave + sh;
        const int e = ev[sh];
        const bool valid = s < k && e >= 0 && e < E;
        float y = valid ? dn_lane_row(wbase + sh * g.per_slot, g, rho, u) : 0.f;
        y += __shfl_xor(y, 1, kWave);
        y += __shfl_xor(y, 2, kWave);
        if (u == 0 && s < k) ys[s * kDnRows + rho] = valid ? w[t * k + s] * y : 0.f;
        __syncthreads();
    }
    if (tid < kDnRows) {
        float acc = 0.f;
        for (int s = 0; s < k; ++s) acc += ys[s * kDnRows + tid];
        float* o = out + t * H + r0 + tid;
        *o = accumulate ? *o + acc : acc;
    }
}

// The 8 rows of one gate/up task as this lane's registers: the block header
// and the lane's 16 quant bytes of gate rows r0..r0+3, then of up rows.
// hw[i]: dword lane % 4 of row i's 16-byte block header (the quad's four
// lanes hold the whole header; DPP broadcasts rebuild it in every lane).
struct GuRows {
    uint32_t hw[8];
    uint4 qv[8];
};

__device__ __forceinline__ uint32_t load_stream4(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Lane k of each quad, in every lane of the quad.
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, K * 0x55, 0xf, 0xf, false);
}

// Loads are unconditional (an out-of-range expert reads expert 0's rows and
// its result is dropped), so they form one straight-line group that the
// scheduler keeps ahead of the arithmetic that waits on older loads.
__device__ __forceinline__ void gu_rows_load(GuRows& g, int e, int32_t E,
                                             const uint8_t* __restrict__ gbase, int64_t gstride,
                                             const uint8_t* __restrict__ ubase, int64_t ustride,
                                             int64_t r0, int lane) {
    using G = GuTask<8>;
    const int b = lane >> 3, c = (lane >> 1) & 3, hp = lane & 1;
    const int qoff = 16 + 32 * c + 16 * hp;
    const int64_t es = e >= 0 && e < E ? e : 0;
    const uint8_t* g0 = gbase + es * gstride + r0 * G::ROWB + b * kQ4KBytes;
    const uint8_t* u0 = ubase + es * ustride + r0 * G::ROWB + b * kQ4KBytes;
    const int hoff = 4 * (lane & 3);          // the quad shares one block: 4 B each
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint8_t* row = (i < 4 ? g0 : u0) + (i & 3) * G::ROWB;
        g.hw[i] = load_stream4(row + hoff);
        g.qv[i] = load_stream16(row + qoff);
    }
}

// h = silu(gate) * up of the task's 4 rows, published as tagged words: the
// f32 value in the low half and this call's tag in the high half of one
// 64-bit device-scope store, so a reader that sees the tag sees the value.
template <int NP>
__device__ __forceinline__ void gu_rows_finish(const GuRows& g, const XCols& x, int lane,
                                               uint64_t* __restrict__ hbuf, int64_t value_base,
                                               uint32_t tag) {
    // rows in load order, each fenced off so that it waits only for its own
    // loads (they complete in order).  A pair whose expert is out of range
    // computes on expert 0's rows; its h is never read (the down stage skips
    // that slot).
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 hdr = make_uint4(quad_bcast<0>(g.hw[i]), quad_bcast<1>(g.hw[i]),
                                     quad_bcast<2>(g.hw[i]), quad_bcast<3>(g.hw[i]));
        v[i] = q4k_cols_row<NP>(hdr, g.qv[i], x);
        __builtin_amdgcn_sched_barrier(0);
    }
    const float r = fold8_rows(v, lane);               // lanes 8q..: row q
    const float up = __shfl_xor(r, 32, kWave);          // lane 8q (q < 4) gets up row q
    const float h = silu_f(r) * up;
    if (lane < 32 && (lane & 7) == 0)
        __hip_atomic_store(hbuf + value_base + (lane >> 3),
                           ((uint64_t)tag << 32) | __float_as_uint(h), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ fused path --
//
// One persistent kernel for the whole expert FFN of a few tokens at H = 2048.
// Each workgroup (one per CU) has 8 waves: 6 compute gate/up tasks from
// registers, 2 request the workgroup's down tiles (8 output rows of every
// selected expert) into LDS, so the down weights stream while gate/up
// computes; all 8 then share the down projection of those rows.
//
// Hand-off of h between workgroups without counters: every h value is
// published as one 64-bit word, its f32 bits beside a tag that identifies
// this call (derived from an epoch counter in the workspace).  A down thread
// keeps re-reading the 16 words it needs, with device-scope loads, until all
// carry this call's tag, so the data itself is the signal and no write has
// to be acknowledged before another can be issued.  Before they read h, the
// down threads have already pulled their share of the down tiles out of LDS
// as quant bytes and per-row group factors (a, c) in registers; after h
// arrives each row takes 16 byte conversions, 16 FMAs and one a, c step,
// then the cross-lane sum.  The epoch: each workgroup reads it first and then
// stores a presence word with the tag; workgroup 0 advances it once every
// presence word carries the tag (the next call is a later launch, so nothing
// of this call reads it again), and nothing is counted at exit.  Every wait
// is bounded: one that runs out sets the status word instead of hanging.
constexpr int kFzGu = 6;
constexpr int kFzDn = 2;
constexpr int kFzWaves = kFzGu + kFzDn;
constexpr int kFzNB = 8;                               // H = 2048
constexpr int kSpinLimit = 1 << 22;
constexpr int kStripes = 16;
constexpr int kLineInts = 32;                          // 128-byte spacing of counters
// int32 offsets inside the workspace's synchronisation header
constexpr int kSyncStatus = 0;
constexpr int kSyncEpoch = 32;                         // calls completed on this workspace
constexpr int kSyncExit = 64;                          // + kLineInts * stripe
constexpr int kSyncExitTop = kSyncExit + kStripes * kLineInts;
static_assert((kSyncExitTop + 1) * 4 <= (int)kFfnRouteSyncOffset, "sync header too small");
// The one-layer kernel's presence words: workgroup w stores a tagged word at
// kSyncPresence + w once it has read the epoch (64-bit words, in the
// header's second half past the route counter).
constexpr int kSyncPresence = 6144 / 8;
constexpr int kMaxPresence = 256;
static_assert((kSyncPresence + kMaxPresence) * 8 <= (int)kFfnSyncBytes, "presence words outside the header");
static_assert(kFfnRouteSyncOffset + kRouteCounterBytes <= (size_t)kSyncPresence * 8,
              "the route kernel's counters overlap the presence words");

__device__ __forceinline__ int stripe_members(int stripe, int grid) {
    return grid / kStripes + (stripe < grid % kStripes ? 1 : 0);
}

// The tag of the call that runs with epoch counter value `epoch`: odd, so it
// never equals the zero high half of a cleared workspace, and different for
// consecutive calls; the constant keeps it unlike small integers left in
// memory by other uses.
__device__ __forceinline__ uint32_t h_tag(uint32_t epoch) {
    return (2u * epoch + 1u) ^ 0x6a09e666u;
}

constexpr int kFzMaxSlots = 8;                        // the fused path serves k <= 8
constexpr int kFzMaxTokens = 4;                        // and T <= 4 (T*k routing entries <= 32)
constexpr int kDnGroup = 16;                           // columns per down thread unit
constexpr int kFzMaxUnits = 256;                       // router units (expert x column part) in the kernel
constexpr int kFzRouteNper = 4;                        // experts per lane in the in-kernel top-k: E <= 256
static_assert(kFzWaves * kWave * 4 == kFzNB * kQK, "one float4 of activations per thread and token");

struct FusedLds {
    int xp_bytes, dn_off, h_off, res_off, flag_off, rp_off, lg_off, key_off,
        key32_off, sel_off, scnt_off, total;
};

__host__ __device__ inline FusedLds fused_lds(int64_t T, int64_t F, int32_t qtype) {
    const DnGeom d(F, qtype);
    FusedLds L;
    L.xp_bytes = kI8TokenBytes;                                     // int8 pieces, scales, sums per token
    L.dn_off = (int)T * L.xp_bytes;                                 // down tiles, one per slot
    L.h_off = L.dn_off + kFzMaxSlots * d.tile_pad;                  // h of the unit's token, f32 [slot][F]
    L.res_off = L.h_off + kFzMaxSlots * (int)F * 4;                 // [wave][row] partial sums
    L.flag_off = L.res_off + kFzWaves * kDnRows * 4;                // down waves whose tiles landed
    // routing in the kernel: per-wave router sums [wave][token], then the
    // logits, their keys and the selection
    L.rp_off = L.flag_off + 16;
    L.lg_off = L.rp_off + kFzWaves * kFzMaxTokens * 8;                 // [token][expert] logits
    L.key_off = L.lg_off + kFzMaxTokens * kFzRouteNper * kWave * 8;    // their order keys
    L.key32_off = L.key_off + kFzMaxTokens * kFzRouteNper * kWave * 8; // and 32-bit screen keys
    L.sel_off = L.key32_off + kFzMaxTokens * kFzRouteNper * kWave * 4; // top-k: idx, value
    L.scnt_off = L.sel_off + kFzMaxTokens * kFzMaxSlots * 12;         // top-k slot counters
    L.total = L.scnt_off + kFzMaxTokens * kFzMaxSlots * 4;
    return L;
}

// Down-stage unit of a thread: 16 consecutive columns (one Q6_K scale group,
// half a Q4_K sub-block) of one slot's tile, for all 8 rows.  Each weight is
// a * q + c with the row's group factors (Q6_K: a = d * scale, c = -32 a;
// Q4_K: a = d * sc, c = -dmin * m): the 16 quants q (0..63) come out of the
// raw tile in LDS as bytes, four per word in column order (q[row][i / 4]
// byte i % 4), and a, c as f32.  The row's dot product with h is then
// a * sum(q h) + c * sum(h).
__device__ __forceinline__ void dn_unit_quants(const uint8_t* tile, const DnGeom& g, int grp,
                                               uint32_t (&q)[kDnRows][4], float (&a)[kDnRows],
                                               float (&c)[kDnRows]) {
    const int b = grp / (kQK / kDnGroup), j = grp % (kQK / kDnGroup);
#pragma unroll
    for (int rho = 0; rho < kDnRows; ++rho) {
        const int boff = rho * g.rowb + b * g.bb;
        if (g.q6) {
            // group j: weights 16j..16j+15 with scale j; low four bits in nibble
            // r/2 of ql bytes 64n + 32(r%2) + 16lh + i, top two bits at 2r of
            // qh byte 32n + 16lh + i (n = j/8, r = (j/2)%4, lh = j%2)
            const int n = j >> 3, r = (j >> 1) & 3, lh = j & 1;
            const uint4 ql = lds_read16_a2(tile, boff + 64 * n + 32 * (r & 1) + 16 * lh);
            const uint4 qh = lds_read16_a2(tile, boff + 128 + 32 * n + 16 * lh);
            const uint32_t l4[4] = {ql.x, ql.y, ql.z, ql.w}, h4[4] = {qh.x, qh.y, qh.z, qh.w};
            const int ls = 4 * (r >> 1), hs = 2 * r;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                q[rho][i] = ((l4[i] >> ls) & 0x0f0f0f0fu) | (((h4[i] >> hs) & 0x03030303u) << 4);
            const float d = half_bits_to_float(tile[boff + 208] | (tile[boff + 209] << 8));
            a[rho] = d * (float)(int8_t)tile[boff + 192 + j];
            c[rho] = -32.f * a[rho];
        } else {
            // half j%2 of sub-block j/2: nibble (j/2)%2 of qs bytes 32(j/4) + 16(j%2) + i
            const int sb = j >> 1;
            const uint4 hdr = *reinterpret_cast<const uint4*>(tile + boff);
            const uint4 qs = *reinterpret_cast<const uint4*>(tile + boff + 16 + 32 * (sb >> 1) + 16 * (j & 1));
            const uint32_t q4[4] = {qs.x, qs.y, qs.z, qs.w};
            const int sh = 4 * (sb & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) q[rho][i] = (q4[i] >> sh) & 0x0f0f0f0fu;
            int sc, mn;
            q4k_sm_var(hdr.y, hdr.z, hdr.w, sb, sc, mn);
            a[rho] = half_bits_to_float(hdr.x & 0xffffu) * (float)sc;
            c[rho] = -half_bits_to_float(hdr.x >> 16) * (float)mn;
        }
    }
}

// n tagged words from src into LDS (their 32-bit payloads, dst[i] for word
// i), once each carries `tag`.  n is even and src 16-byte aligned: thread tid
// reads word pairs tid + i * kThr with 16-byte device-scope loads (sc1, the
// coherence of the compiler's device-scope atomic loads; a 16-byte load moves
// a CU's share in fewer, wider requests than 8-byte atomics), so each load
// instruction of a wave covers 1 KiB of consecutive words; a wave re-reads
// its words until all of them carry the tag.  A wait that runs out ORs
// `bit` into the status word.
constexpr int kPollPairs = 6;                          // word pairs per thread and round

// One chunk of that wait: the word pairs c0 + tid + i * kThr (i <
// kPollPairs, those below np) into v, re-read until this wave's all carry
// the tag (or the spin limit runs out: `bit` into the status word).
template <int kThr>
__device__ __forceinline__ void poll_pairs(const uint64_t* src, int np, int c0, uint32_t tag,
                                           int tid, u32x4_t (&v)[kPollPairs], int32_t* status,
                                           int bit) {
    const uint64_t* p[kPollPairs];
#pragma unroll
    for (int i = 0; i < kPollPairs; ++i) {
        const int pi = c0 + tid + i * kThr;
        p[i] = src + 2 * (pi < np ? pi : np - 1);
    }
    int spins = 0;
    while (true) {
        // the six loads and the wait for them in one asm block, so no
        // register of a load in flight is reused before it lands
        asm volatile(
            "global_load_dwordx4 %0, %6, off sc1\n\t"
            "global_load_dwordx4 %1, %7, off sc1\n\t"
            "global_load_dwordx4 %2, %8, off sc1\n\t"
            "global_load_dwordx4 %3, %9, off sc1\n\t"
            "global_load_dwordx4 %4, %10, off sc1\n\t"
            "global_load_dwordx4 %5, %11, off sc1\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5])
            : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5])
            : "memory");
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kPollPairs; ++i)
            ok = ok && (c0 + tid + i * kThr >= np || (v[i].y == tag && v[i].w == tag));
        if (__all(ok)) break;
        if (++spins > kSpinLimit) {
            if (!ok) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int kThr>
__device__ __forceinline__ void wait_tagged(const uint64_t* src, int n, uint32_t tag,
                                            uint32_t* dst, int tid, int32_t* status, int bit) {
    const int np = n >> 1;
    for (int c0 = 0; c0 < np; c0 += kThr * kPollPairs) {
        u32x4_t v[kPollPairs];
        poll_pairs<kThr>(src, np, c0, tag, tid, v, status, bit);
#pragma unroll
        for (int i = 0; i < kPollPairs; ++i) {
            const int pi = c0 + tid + i * kThr;
            if (pi < np) *reinterpret_cast<uint2*>(dst + 2 * pi) = make_uint2(v[i].x, v[i].z);
        }
    }
}

// The router logits of the in-kernel routing from the tagged partial sums:
// pair t * U + u (U = E * P units, u = e * P + part) holds part `part` of
// expert e's logit for token t as a double in two tagged words.  The pairs
// are polled as by wait_tagged (np = T * U <= kThr * kPollPairs, one chunk);
// the P parts of an expert then sit in P consecutive lanes of one wave (P a
// power of two <= 8), and the lane holding part 0 sums them in part order,
// starting from 0.0 as a loop over the parts would, and stores the logit with
// its order keys.  No LDS round trip of the partials.
template <int kThr>
__device__ __forceinline__ void router_logits_from_partials(const uint64_t* src, int np, int P,
                                                            int E, int U, uint32_t tag, int tid,
                                                            int lane, int32_t* status, double* lgt,
                                                            uint64_t* keys, uint32_t* keys32) {
    u32x4_t v[kPollPairs];
    poll_pairs<kThr>(src, np, 0, tag, tid, v, status, 4);
#pragma unroll
    for (int i = 0; i < kPollPairs; ++i) {
        if (i * kThr >= np) break;                      // uniform
        const int pi = tid + i * kThr;
        const double d = __builtin_bit_cast(double, ((uint64_t)v[i].z << 32) | v[i].x);
        double sum = 0.0;
        for (int q = 0; q < P; ++q) sum += __shfl(d, (lane + q) & (kWave - 1), kWave);
        if (pi < np && (pi & (P - 1)) == 0) {
            const int t = pi / U, e = (pi - t * U) / P;
            lgt[t * E + e] = sum;
            keys[t * E + e] = order_key(sum);
            keys32[t * E + e] = order_key32(sum);
        }
    }
}
static_assert(kPollPairs == 6, "the wait above names each of its registers");

// The activations of the T tokens as int8 pieces in LDS (layout at
// kI8PieceBytes): thread tid converts values 4*tid .. 4*tid+3 of every token;
// 8 consecutive threads hold one 32-value group, 4 one 16-value half.  A
// group whose maximum is not finite gets a NaN scale, so it poisons the rows
// that read it as the plain products would.
__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d) {
    return ((uint32_t)(int)a & 0xffu) | (((uint32_t)(int)b & 0xffu) << 8) |
           (((uint32_t)(int)c & 0xffu) << 16) | ((uint32_t)(int)d << 24);
}

// NP = 1 (the int8-activation mode) stores one piece per value instead: for
// each 32-value group d = max|x| / 127 and p = rint(x / d) (both quotients
// correctly rounded f32 divisions, ties to even; d = 0 and p = 0 for an
// all-zero group), the group scale d and the 16-value sums d * sum(p).
template <int MT, int NP>
__device__ __forceinline__ void build_x_pieces(const float4 (&xv)[MT], int64_t T, uint8_t* smem,
                                               int tid) {
    const int v0 = 4 * tid, bl = v0 >> 8, w = v0 & 255, j = w >> 5;
    const int lane = bl * 8 + (j >> 1) * 2 + ((w >> 4) & 1), half = j & 1;
    const int off = half * (kWave * 16) + lane * 16 + (w & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < T) {                                           // whole workgroup in or out
            uint8_t* xt = smem + t * kI8TokenBytes;
            const float4 v = xv[t];
            float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
            // 1 where a value is NaN or infinite (fmaxf would drop a NaN)
            float bad = (fabsf(v.x) <= 3.4028235e38f && fabsf(v.y) <= 3.4028235e38f &&
                         fabsf(v.z) <= 3.4028235e38f && fabsf(v.w) <= 3.4028235e38f) ? 0.f : 1.f;
#pragma unroll
            for (int sh = 1; sh < 8; sh <<= 1) {
                m = fmaxf(m, __shfl_xor(m, sh, kWave));
                bad = fmaxf(bad, __shfl_xor(bad, sh, kWave));
            }
            const bool finite = bad == 0.f;
            if constexpr (NP == 1) {
                const float d = finite ? __fdiv_rn(m, 127.f) : __builtin_nanf("");
                const bool q = finite && m > 0.f;
                const float p0 = q ? rintf(__fdiv_rn(v.x, d)) : 0.f, p1 = q ? rintf(__fdiv_rn(v.y, d)) : 0.f;
                const float p2 = q ? rintf(__fdiv_rn(v.z, d)) : 0.f, p3 = q ? rintf(__fdiv_rn(v.w, d)) : 0.f;
                *reinterpret_cast<uint32_t*>(xt + off) = pack_i8x4(p0, p1, p2, p3);
                int is = (int)p0 + (int)p1 + (int)p2 + (int)p3;
                is += __shfl_xor(is, 1, kWave);
                is += __shfl_xor(is, 2, kWave);
                if ((tid & 3) == 0)
                    reinterpret_cast<float*>(xt + kI8SumOff)[half * kWave + lane] = (float)is * d;
                if ((tid & 7) == 0) reinterpret_cast<float*>(xt + kI8ScaleOff)[bl * 8 + j] = d;
                continue;
            }
            // s = 2^e with m / s in [63.75, 127.5): e from the exponent of m
            int e = finite && m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 7 : 0;
            if (ldexpf(m, -e) >= 127.5f) ++e;
            const float vv[4] = {v.x, v.y, v.z, v.w};
            float p1[4], p2[4], p3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float q = ldexpf(vv[i], -e);
                p1[i] = finite ? rintf(q) : 0.f;
                const float r1 = (q - p1[i]) * 128.f;
                p2[i] = finite ? rintf(r1) : 0.f;
                const float r2 = (r1 - p2[i]) * 128.f;
                p3[i] = finite ? rintf(r2) : 0.f;
            }
            *reinterpret_cast<uint32_t*>(xt + off) = pack_i8x4(p1[0], p1[1], p1[2], p1[3]);
            *reinterpret_cast<uint32_t*>(xt + kI8PieceBytes + off) = pack_i8x4(p2[0], p2[1], p2[2], p2[3]);
            *reinterpret_cast<uint32_t*>(xt + 2 * kI8PieceBytes + off) = pack_i8x4(p3[0], p3[1], p3[2], p3[3]);
            float g = (v.x + v.y) + (v.z + v.w);
            g += __shfl_xor(g, 1, kWave);
            g += __shfl_xor(g, 2, kWave);
            if ((tid & 3) == 0)
                reinterpret_cast<float*>(xt + kI8SumOff)[half * kWave + lane] = g;
            if ((tid & 7) == 0)
                reinterpret_cast<float*>(xt + kI8ScaleOff)[bl * 8 + j] =
                    finite ? ldexpf(1.f, e - 14) : __builtin_nanf("");
        } else {
            // consume the (clamped) load anyway, so that every path has
            // waited for it and its registers can be reused without a
            // conservative wait for all later loads
            asm volatile("" ::"v"(xv[t].x), "v"(xv[t].y), "v"(xv[t].z), "v"(xv[t].w));
        }
    }
}

// Value of lane `src` (wave-uniform) of v.
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// grid: at most one workgroup per CU, kFzWaves waves each.  sync is the
// workspace's synchronisation header: its counters are zero when the kernel
// starts and zero again when it ends.  The routing entries (T*k <= 32) live
// in one register per lane of every wave and are read with readlane.
// With the routing inside, norm_gain (if not null) applies the input
// RMSNorm first: the FFN input is gain * x / sqrt(mean(x^2) + eps) of the
// token's hidden row x.  hidden and out may then be the same buffer (the
// residual update x += MoE(RMSNorm(x))): every workgroup has read all of
// hidden before it publishes its router partials, and no workgroup writes
// out before it has seen all of them.  Hence neither pointer is restrict.
template <bool kRoute, int NP>
__global__ __launch_bounds__(kFzWaves * kWave) void ffn_fused8_kernel(
    const float* hidden, int64_t T, int64_t F, int32_t E, int32_t k,
    const int32_t* __restrict__ idx, const float* __restrict__ w,
    const uint8_t* __restrict__ gbase, int64_t gstride, const uint8_t* __restrict__ ubase,
    int64_t ustride, const uint8_t* __restrict__ dbase, int32_t dqtype, int64_t dstride,
    float* out, int accumulate, uint64_t* __restrict__ hbuf,
    int32_t* __restrict__ sync, const float* __restrict__ router, int32_t P,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint64_t* __restrict__ rbuf,
    const float* __restrict__ norm_gain, float eps) {
    using G = GuTask<kFzNB>;
    constexpr int kThr = kFzWaves * kWave;
    extern __shared__ __align__(16) uint8_t smem[];
    // the wave index as a scalar, so that the gate/up and down branches are
    // uniform and each keeps exact counts of its own outstanding loads
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grid = (int)gridDim.x, wg = (int)blockIdx.x;
    const FusedLds L = fused_lds(T, F, dqtype);
    const DnGeom dg(F, dqtype);
    int32_t* status = sync + kSyncStatus;
    float* res = reinterpret_cast<float*>(smem + L.res_off);

    const int tiles = (int)(F / G::R);                      // T*k*tiles < 2^31 (T <= 4, k <= 8)
    const int n_gu = (int)T * k * tiles;
    const int64_t row_units = G::H / kDnRows;
    const int64_t n_dn = T * row_units;
    const int gu_step = grid * kFzGu;
    const bool is_gu = wave < kFzGu;

    // ---- (1) this call's epoch (every workgroup reads it here and then
    // stores its presence word; workgroup 0 advances the epoch once it has
    // seen every presence word), routing, activation pieces.
    const int nr = (int)(T * k);
    const uint32_t epoch = (uint32_t)__hip_atomic_load(sync + kSyncEpoch, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
    // the tag as a scalar now, while only this small load is in flight
    const uint32_t tag = __builtin_amdgcn_readfirstlane(h_tag(epoch));
    uint64_t* presence = reinterpret_cast<uint64_t*>(sync) + kSyncPresence;
    if (tid == 0)
        __hip_atomic_store(presence + wg, ((uint64_t)tag << 32) | (uint32_t)wg, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    // LDS counters: gate/up waves whose activation pieces are written, down
    // waves whose tiles have landed
    int32_t* x_ready = reinterpret_cast<int32_t*>(smem + L.flag_off);
    int32_t* dn_ready = x_ready + 1;
    if (tid == 0) {
        *x_ready = 0;
        *dn_ready = 0;
    }
    __syncthreads();                          // the counters are zero before anyone counts

    int64_t unit = wg;
    int tau = wg * kFzGu + wave;
    int p = (tau < n_gu ? tau : 0) / tiles, r0 = ((tau < n_gu ? tau : 0) % tiles) * G::R;
    GuRows rows;

    // The T tokens' activations as pieces in LDS, built by the six gate/up
    // waves (waves 0 and 1 also take the last quarter of the vector).  The
    // activation loads are unconditional (clamped), so the build waits only
    // for them and not for weight requests issued after them.
    auto build_pieces = [&](bool issue_weights, int e0) {
        constexpr int kXThr = kFzGu * kWave;              // 384 threads, one float4 each
        constexpr int kXRest = kFzNB * kQK / 4 - kXThr;   // 128 float4 left for waves 0 and 1
        const bool second = tid < kXRest;
        float4 xv[kFzMaxTokens], xw[kFzMaxTokens];
#pragma unroll
        for (int j = 0; j < kFzMaxTokens; ++j) {
            const float4* hx = reinterpret_cast<const float4*>(hidden + (j < T ? j : T - 1) * G::H);
            xv[j] = hx[tid];
            xw[j] = hx[kXThr + (second ? tid : 0)];
        }
        if (issue_weights)
            gu_rows_load(rows, e0, E, gbase, gstride, ubase, ustride, r0, lane);
        __builtin_amdgcn_sched_barrier(0);
        build_x_pieces<kFzMaxTokens, NP>(xv, T, smem, tid);
        if (second) build_x_pieces<kFzMaxTokens, NP>(xw, T, smem, kXThr + tid);
        else asm volatile("" ::"v"(xw[0].x), "v"(xw[1].x), "v"(xw[2].x), "v"(xw[3].x));
        __builtin_amdgcn_sched_barrier(0);
    };

    int my_idx;
    float my_w;
    if constexpr (kRoute) {
        // Routing in the kernel (the route entry point's result, computed
        // redundantly by every workgroup from shared partial logits).
        double* rp = reinterpret_cast<double*>(smem + L.rp_off);      // [wave][token]
        const int U = E * P, HP = (int)(G::H / P);
        // (a0) thread tid holds values 4*tid .. 4*tid+3 of every token's
        // input (H = 2048 = 4 x 512 threads); with the norm they become
        // gain * x * inv, inv = 1 / sqrt(mean(x^2) + eps), the squares summed
        // in double and each value formed in double and rounded once.
        float4 xv[kFzMaxTokens];
#pragma unroll
        for (int t = 0; t < kFzMaxTokens; ++t)
            xv[t] = reinterpret_cast<const float4*>(hidden + (t < T ? t : T - 1) * G::H)[tid];
        if (norm_gain) {
            const float4 g4 = reinterpret_cast<const float4*>(norm_gain)[tid];
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    const float4 v = xv[t];
                    double ss = (double)v.x * v.x;
                    ss = fma((double)v.y, (double)v.y, ss);
                    ss = fma((double)v.z, (double)v.z, ss);
                    ss = fma((double)v.w, (double)v.w, ss);
                    const double sw = wave_sum_dpp_f64(ss);
                    if (lane == 0) rp[wave * kFzMaxTokens + t] = sw;
                }
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    double tot = 0.0;
#pragma unroll
                    for (int wv = 0; wv < kFzWaves; ++wv) tot += rp[wv * kFzMaxTokens + t];
                    const double inv = 1.0 / sqrt(tot / (double)G::H + (double)eps);
                    const float4 v = xv[t];
                    xv[t] = make_float4((float)((double)g4.x * v.x * inv), (float)((double)g4.y * v.y * inv),
                                        (float)((double)g4.z * v.z * inv), (float)((double)g4.w * v.w * inv));
                }
            }
            __syncthreads();                  // rp is reused by the router sums
        }
        // (a) this workgroup's router unit(s): expert u / P, column part u % P
        // (the threads holding that part's columns); f64 sums of the exact
        // f32 products, published as two tagged words
        for (int u = wg; u < U; u += grid) {
            const int e = u / P, part = u % P;
            double acc[kFzMaxTokens];
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) acc[t] = 0.0;
            if ((4 * tid) / HP == part) {
                const float4 r = reinterpret_cast<const float4*>(router + (int64_t)e * G::H)[tid];
#pragma unroll
                for (int t = 0; t < kFzMaxTokens; ++t) {
                    if (t < T) {
                        const float4 x4 = xv[t];
                        double a = fma((double)r.x, (double)x4.x, 0.0);
                        a = fma((double)r.y, (double)x4.y, a);
                        a = fma((double)r.z, (double)x4.z, a);
                        acc[t] = fma((double)r.w, (double)x4.w, a);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    const double sw = wave_sum_dpp_f64(acc[t]);
                    if (lane == 0) rp[wave * kFzMaxTokens + t] = sw;
                }
            }
            __syncthreads();
            if (tid < T) {
                double sum = 0.0;
#pragma unroll
                for (int wv = 0; wv < kFzWaves; ++wv) sum += rp[wv * kFzMaxTokens + tid];
                const uint64_t bits = __builtin_bit_cast(uint64_t, sum);
                uint64_t* dst = rbuf + ((int64_t)tid * U + u) * 2;
                __hip_atomic_store(dst, ((uint64_t)tag << 32) | (uint32_t)bits, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, ((uint64_t)tag << 32) | (uint32_t)(bits >> 32),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }
        // the activation pieces, by every wave, while the partial logits
        // travel (thread tid converts the values it holds)
        build_x_pieces<kFzMaxTokens, NP>(xv, T, smem, tid);
        // (b) every partial logit of every token, then (c) the top-k of token
        // t on wave t; logit = the sum of the expert's parts in part order
        // logits of every token (the sum of an expert's parts in part order)
        // straight from the polled registers, then the top-k by rank
        // counting over the whole workgroup
        double* lgt = reinterpret_cast<double*>(smem + L.lg_off);     // [token][expert]
        uint64_t* keys = reinterpret_cast<uint64_t*>(smem + L.key_off);
        uint32_t* keys32 = reinterpret_cast<uint32_t*>(smem + L.key32_off);
        int32_t* sel_idx = reinterpret_cast<int32_t*>(smem + L.sel_off);
        double* sel_val = reinterpret_cast<double*>(sel_idx + kFzMaxTokens * kFzMaxSlots);
        int32_t* slot_cnt = reinterpret_cast<int32_t*>(smem + L.scnt_off);
        if (tid < nr) slot_cnt[tid] = 0;
        router_logits_from_partials<kThr>(rbuf, (int)T * U, P, E, U, tag, tid, lane, status, lgt,
                                          keys, keys32);
        __syncthreads();
        // the top-k on the screen keys; if equal screen keys reach the chosen
        // (a slot counter other than 1, the same verdict in every wave) the
        // exact selection replaces it
        topk_rank_screen<kThr>(lgt, keys32, (int)T, E, k, tid, sel_idx, sel_val, slot_cnt);
        __syncthreads();
        if (!__all(lane >= nr || slot_cnt[lane] == 1)) {
            topk_rank_select<kThr>(lgt, keys, keys32, (int)T, E, k, tid, sel_idx, sel_val);
            __syncthreads();
        }
        // the chosen experts first: the gate/up weight requests need only
        // them, so they go out before the routing weights are formed
        my_idx = lane < nr ? sel_idx[lane] : -1;
        if (is_gu)
            gu_rows_load(rows, lane_value(my_idx, p), E, gbase, gstride, ubase, ustride, r0, lane);
        // every wave forms all T*k routing weights itself (lane l < T*k:
        // token l / k, rank l % k) while those loads are in flight: the
        // softmax over the token's chosen logits in double, its rank-0 logit
        // subtracted, normalised by their sum in rank order and rounded to
        // f32, as topk_wave does
        {
            const int tl = lane < nr ? lane / k : 0;
            const double top = sel_val[tl * k];
            const double ex = lane < nr ? exp(sel_val[lane] - top) : 0.0;
            double den = 0.0;
            for (int tt = 0; tt < T; ++tt) {
                double d = 0.0;
                for (int r = 0; r < k; ++r) d += readlane_f64(ex, tt * k + r);
                if (tt == tl) den = d;
            }
            my_w = lane < nr ? (float)(ex / den) : 0.f;
        }
        if (wg == 0 && tid < nr) {
            topk_idx[tid] = my_idx;
            topk_w[tid] = my_w;
        }
    } else {
        const int ri = lane < nr ? lane : nr - 1;         // loads without a branch
        my_idx = lane < nr ? idx[ri] : -1;
        my_w = lane < nr ? w[ri] : 0.f;
        if (is_gu) {
            build_pieces(true, lane_value(my_idx, p));
            // the six gate/up waves meet on an LDS counter (the down waves,
            // busy with their tiles, are not part of this)
            if (lane == 0) __hip_atomic_fetch_add(x_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            int spins = 0;
            while (__hip_atomic_load(x_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kFzGu &&
                   ++spins <= kSpinLimit)
                __builtin_amdgcn_s_sleep(1);
        }
    }

    if (is_gu) {
        // gate/up tasks: the first task's weights are on their way; read the
        // token's pieces and compute it, then load and compute the rest.
        // Raised issue priority: the gate/up waves are the critical path, and
        // two SIMDs also run a down wave's quant extraction beside them.
        __builtin_amdgcn_s_setprio(2);
        if (tau < n_gu) {
            int xc = p / k;                   // token whose pieces x holds
            XCols x = load_xcols<NP>(smem + xc * kI8TokenBytes, lane);
            gu_rows_finish<NP>(rows, x, lane, hbuf, (int64_t)p * F + r0, tag);
            for (tau += gu_step; tau < n_gu; tau += gu_step) {
                p = tau / tiles;
                r0 = (tau % tiles) * G::R;
                gu_rows_load(rows, lane_value(my_idx, p), E, gbase, gstride, ubase, ustride, r0, lane);
                const int t = p / k;
                if (t != xc) {
                    x = load_xcols<NP>(smem + t * kI8TokenBytes, lane);
                    xc = t;
                }
                gu_rows_finish<NP>(rows, x, lane, hbuf, (int64_t)p * F + r0, tag);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    // The down waves request the first unit's tiles and count themselves
    // ready once they have landed.  A separate branch after the gate/up one,
    // on a condition the compiler cannot relate to is_gu: merged with it, the
    // direct-to-LDS loads would appear pending on the gate/up path and turn
    // its waits for single loads into waits for all of them.
    int dn_wave = __builtin_amdgcn_readfirstlane(is_gu ? 0 : 1);
    asm volatile("" : "+s"(dn_wave));
    if (dn_wave) {
        if (unit < n_dn) {
            const int dw = wave - kFzGu;
            const int64_t t = unit / row_units, r0d = (unit % row_units) * kDnRows;
            for (int s = dw; s < k; s += kFzDn) {
                const int e = lane_value(my_idx, (int)(t * k + s));
                if (e >= 0 && e < E)
                    dn_issue_weights(smem + L.dn_off + s * dg.tile_pad, dg, dbase, dstride, e, r0d, lane);
            }
        }
        wait_all_loads();
        if (lane == 0)
            __hip_atomic_fetch_add(dn_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (wg == 0 && wave == kFzWaves - 1) {
            // Every workgroup has read this call's epoch once its presence
            // word carries the tag; the epoch then advances for the next call
            // (a later launch on the stream), with no count at exit.  The
            // wait is bounded: running out sets bit 16 of the status word.
            bool all = false;
            for (int spins = 0; !all && spins <= kSpinLimit; ++spins) {
                bool mine = true;
                for (int i = lane; i < grid; i += kWave) {
                    const uint64_t v = __hip_atomic_load(presence + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    mine = mine && (uint32_t)(v >> 32) == tag;
                }
                all = __all(mine);
                if (!all) __builtin_amdgcn_s_sleep(1);
            }
            if (lane == 0) {
                if (!all) __hip_atomic_fetch_or(status, 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sync + kSyncEpoch, (int32_t)(epoch + 1u), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // ---- (2) down projection and combine.  The down units are shared by
    // waves 0-3 (gate/up done first) and the two down waves, 64 per wave:
    // unit u = (slot u / G, 16-column group u % G) for the 8 rows of the
    // workgroup's output unit.  Waves 4 and 5, still on gate/up, only help
    // read h.
    const int groups = (int)(F / kDnGroup);
    const int n_units = k * groups;
    constexpr int kUnitThr = (kFzWaves - 2) * kWave;
    const int uw = wave < 4 ? wave : (wave >= kFzGu ? wave - 2 : -1);
    const int iters = (n_units + kUnitThr - 1) / kUnitThr;   // the same for every wave
    float* hl = reinterpret_cast<float*>(smem + L.h_off);
    for (int j = 0; unit < n_dn; unit += grid, ++j) {
        const int64_t t = unit / row_units, r0 = (unit % row_units) * kDnRows;
        if (j > 0) {
            for (int s = wave; s < k; s += kFzWaves) {
                const int e = lane_value(my_idx, (int)(t * k + s));
                if (e >= 0 && e < E)
                    dn_issue_weights(smem + L.dn_off + s * dg.tile_pad, dg, dbase, dstride, e, r0, lane);
            }
            wait_all_loads();
            __syncthreads();                  // this unit's tiles are in LDS
        } else if (uw >= 0) {
            // the first unit's tiles: wait until both down waves report them
            int spins = 0;
            while (__hip_atomic_load(dn_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kFzDn &&
                   ++spins <= kSpinLimit)
                __builtin_amdgcn_s_sleep(1);
        }
        float acc[kDnRows];
#pragma unroll
        for (int rho = 0; rho < kDnRows; ++rho) acc[rho] = 0.f;
        for (int it = 0; it < iters; ++it) {
            const int u = uw * kWave + lane + it * kUnitThr;
            const bool active = uw >= 0 && u < n_units;
            const int uc = active ? u : 0;
            const int s = uc / groups, grp = uc % groups;
            const int e = __shfl(my_idx, (int)(t * k) + s, kWave);
            const float ws = __shfl(my_w, (int)(t * k) + s, kWave);
            const bool valid = active && e >= 0 && e < E;
            uint32_t qb[kDnRows][4];
            float fa[kDnRows], fc[kDnRows];
            if (uw >= 0) dn_unit_quants(smem + L.dn_off + s * dg.tile_pad, dg, grp, qb, fa, fc);
            if (it == 0) {
                // the token's h: every slot's F values, published by gate/up
                // waves anywhere on the device
                wait_tagged<kThr>(hbuf + t * k * F, k * (int)F, tag, reinterpret_cast<uint32_t*>(hl), tid, status, 2);
                __syncthreads();
            }
            if (uw >= 0) {
                float hv[kDnGroup];
#pragma unroll
                for (int i = 0; i < kDnGroup; i += 4) {
                    const float4 h4 = *reinterpret_cast<const float4*>(hl + s * F + grp * kDnGroup + i);
                    hv[i] = h4.x; hv[i + 1] = h4.y; hv[i + 2] = h4.z; hv[i + 3] = h4.w;
                }
                float hsum = 0.f;
#pragma unroll
                for (int i = 0; i < kDnGroup; ++i) hsum += hv[i];
#pragma unroll
                for (int rho = 0; rho < kDnRows; ++rho) {
                    float sq = 0.f;
#pragma unroll
                    for (int i = 0; i < kDnGroup; ++i)
                        sq = fmaf((float)((qb[rho][i >> 2] >> (8 * (i & 3))) & 0xffu), hv[i], sq);
                    const float y = fmaf(fa[rho], sq, fc[rho] * hsum);
                    acc[rho] += valid ? ws * y : 0.f;
                }
            }
        }
        const float r = fold8_rows(acc, lane);            // lanes 8q..: row q of this wave
        if ((lane & 7) == 0) res[wave * kDnRows + (lane >> 3)] = r;
        __syncthreads();
        if (wave == 0 && lane < kDnRows) {                // fixed order over the waves
            float o = 0.f;
#pragma unroll
            for (int wv = 0; wv < kFzWaves; ++wv) o += res[wv * kDnRows + lane];
            float* dst = out + t * G::H + r0 + lane;
            *dst = accumulate ? *dst + o : o;
        }
    }

}

// --------------------------------------------------------- layer stack --
//
// The MoE blocks of several stacked layers in ONE persistent launch: for
// layer l = 0..nl-1, x <- x + MoE_l(RMSNorm_l(x)), each layer with its own
// router, norm gain and expert tensors (its own down type).  Each layer runs
// the phases of ffn_fused8_kernel<true, 3> with the input RMSNorm; between
// layers the residual stream travels as tagged words too: the workgroup that
// owns output rows r0..r0+7 of a token publishes x_{l+1} for them, and every
// workgroup polls all of x_{l+1} before layer l+1's norm and router.  So the
// launch ramp and drain are paid once per stack instead of once per layer.
// Buffers are reused from layer to layer without counters.  The grid is
// chosen so that every workgroup owns at least one router unit and one down
// unit; then each rewrite waits, through a chain of tagged words, for every
// read of the old contents:
//   x_{l+1} row  <- every h word of its token in layer l <- (the h writer
//                   read) every router word of layer l <- every workgroup
//                   has read all of x_l (it publishes only after that);
//   router words of layer l+1 <- all of x_{l+1}, i.e. every workgroup is
//                   past its down units of layer l, and so past its reads of
//                   layer l's router words and h words;
//   h words of layer l+1 <- every router word of layer l+1 (as above).
// The last layer writes x itself, after every workgroup has read it in
// layer 0 by the first chain.  The tags (one per call and layer, with the
// top bit set so they never equal the one-layer kernel's) tell old words
// from new.  The layer table travels in the kernel arguments (48 layers of
// 56 bytes); longer stacks run as several launches.
constexpr int kMaxStackLayers = 48;

struct StackLayer {
    const float* router;
    const float* gain;
    const uint8_t* gate;
    const uint8_t* up;
    const uint8_t* down;
    int32_t gstride, ustride, dstride;              // expert strides in bytes (< 2^31)
    int32_t dqtype;
};

struct StackJob {
    StackLayer layer[kMaxStackLayers];
};

__device__ __forceinline__ uint32_t stack_tag(uint32_t epoch, int l) {
    return 0x80000000u | ((2u * (epoch * (uint32_t)(kMaxStackLayers + 1) + (uint32_t)l) + 1u) & 0x7fffffffu);
}

// 4 consecutive f32 values published as tagged words, once all carry `tag`
// (the wave waits together; a wait that runs out ORs `bit` into the status).
// The four words are read as two 16-byte device-coherent loads, issued and
// waited for in one asm block (src 16-byte aligned).
__device__ __forceinline__ float4 poll_x4(const uint64_t* src, uint32_t tag, int32_t* status, int bit) {
    u32x4_t a, b;
    int spins = 0;
    while (true) {
        asm volatile(
            "global_load_dwordx4 %0, %2, off sc1\n\t"
            "global_load_dwordx4 %1, %2, off offset:16 sc1\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(a), "=&v"(b)
            : "v"(src)
            : "memory");
        const bool ok = a.y == tag && a.w == tag && b.y == tag && b.w == tag;
        if (__all(ok)) break;
        if (++spins > kSpinLimit) {
            if (!ok) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return make_float4(__uint_as_float(a.x), __uint_as_float(a.z), __uint_as_float(b.x), __uint_as_float(b.z));
}

// grid: at most one workgroup per CU (all resident at once), kFzWaves waves
// each.  x [T][2048] f32 holds the input and receives the output (in place);
// topk_idx / topk_w [nl][T][k] receive every layer's routing; xbuf holds the
// tagged residual stream [T][2048] between layers.  The LDS layout is the
// one-layer kernel's for a Q6_K down tile (the larger one), so every layer
// fits it.
__global__ __launch_bounds__(kFzWaves * kWave) void ffn_stack_kernel(
    float* x, int64_t T_, int64_t F_, int32_t E_, int32_t k_, int32_t nl, float eps, int32_t P_,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint64_t* __restrict__ hbuf,
    int32_t* __restrict__ sync, uint64_t* __restrict__ rbuf, uint64_t* __restrict__ xbuf,
    const StackJob job) {
    using G = GuTask<kFzNB>;
    constexpr int kThr = kFzWaves * kWave;
    extern __shared__ __align__(16) uint8_t smem[];
    int32_t* status = sync + kSyncStatus;
    const uint32_t epoch = (uint32_t)__hip_atomic_load(sync + kSyncEpoch, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
    int32_t exit_ticket = -1;

    for (int l = 0; l < nl; ++l) {
        // the thread index, opaque to the compiler in each layer: otherwise
        // every address derived from it is hoisted out of the layer loop and
        // held in registers through the whole body; likewise the sizes and
        // everything derived from them
        int tid_ = (int)threadIdx.x;
        int64_t T = T_, F = F_;
        int32_t E = E_, k = k_, P = P_;
        asm volatile("" : "+v"(tid_), "+s"(T), "+s"(F), "+s"(E), "+s"(k), "+s"(P));
        const int tid = tid_, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool is_gu = wave < kFzGu;
        const int grid = (int)gridDim.x, wg = (int)blockIdx.x;
        const FusedLds L = fused_lds(T, F, 2);
        float* res = reinterpret_cast<float*>(smem + L.res_off);
        const int tiles = (int)(F / G::R);
        const int n_gu = (int)T * k * tiles;
        const int64_t row_units = G::H / kDnRows;
        const int64_t n_dn = T * row_units;
        const int gu_step = grid * kFzGu;
        const int nr = (int)(T * k);
        int32_t* x_ready = reinterpret_cast<int32_t*>(smem + L.flag_off);
        int32_t* dn_ready = x_ready + 1;
        double* rp = reinterpret_cast<double*>(smem + L.rp_off);      // [wave][token]
        const int U = E * P, HP = (int)(G::H / P);
        const StackLayer& Ly = job.layer[l];
        const uint32_t tag = __builtin_amdgcn_readfirstlane(stack_tag(epoch, l));
        const uint32_t xtag = __builtin_amdgcn_readfirstlane(stack_tag(epoch, l + 1));
        const bool last = l == nl - 1;
        const DnGeom dg(F, Ly.dqtype);
        __syncthreads();                      // the previous layer is done with every LDS region
        if (tid == 0) {
            *x_ready = 0;
            *dn_ready = 0;
        }
        __syncthreads();

        int64_t unit = wg;
        int tau = wg * kFzGu + wave;
        int p = (tau < n_gu ? tau : 0) / tiles, r0 = ((tau < n_gu ? tau : 0) % tiles) * G::R;
        GuRows rows;

        // the layer's loads that do not depend on x_l, issued before its wait:
        // the norm gain and the first router unit's row values (every thread
        // reads its float4 of the row; only the unit's column part is used)
        const float4 g4 = reinterpret_cast<const float4*>(Ly.gain)[tid];
        const int e_first = (wg < U ? wg : 0) / P;
        const float4 r_first = reinterpret_cast<const float4*>(Ly.router + (int64_t)e_first * G::H)[tid];

        // (a0) values 4*tid .. 4*tid+3 of every token's x_l: the input for
        // layer 0, the tagged stream after it; then the layer's RMSNorm
        float4 xv[kFzMaxTokens];
#pragma unroll
        for (int t = 0; t < kFzMaxTokens; ++t) {
            const int tc = t < T ? t : (int)T - 1;
            xv[t] = l == 0 ? reinterpret_cast<const float4*>(x + (int64_t)tc * G::H)[tid]
                           : poll_x4(xbuf + (int64_t)tc * G::H + 4 * tid, tag, status, 8);
        }
        {
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    const float4 v = xv[t];
                    double ss = (double)v.x * v.x;
                    ss = fma((double)v.y, (double)v.y, ss);
                    ss = fma((double)v.z, (double)v.z, ss);
                    ss = fma((double)v.w, (double)v.w, ss);
                    const double sw = wave_sum_dpp_f64(ss);
                    if (lane == 0) rp[wave * kFzMaxTokens + t] = sw;
                }
            }
            __syncthreads();
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    double tot = 0.0;
#pragma unroll
                    for (int wv = 0; wv < kFzWaves; ++wv) tot += rp[wv * kFzMaxTokens + t];
                    const double inv = 1.0 / sqrt(tot / (double)G::H + (double)eps);
                    const float4 v = xv[t];
                    xv[t] = make_float4((float)((double)g4.x * v.x * inv), (float)((double)g4.y * v.y * inv),
                                        (float)((double)g4.z * v.z * inv), (float)((double)g4.w * v.w * inv));
                }
            }
            __syncthreads();                  // rp is reused by the router sums
        }
        // (a) this workgroup's router unit(s), published as tagged words
        for (int u = wg; u < U; u += grid) {
            const int e = u / P, part = u % P;
            double acc[kFzMaxTokens];
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) acc[t] = 0.0;
            if ((4 * tid) / HP == part) {
                const float4 r = u == wg ? r_first : reinterpret_cast<const float4*>(Ly.router + (int64_t)e * G::H)[tid];
#pragma unroll
                for (int t = 0; t < kFzMaxTokens; ++t) {
                    if (t < T) {
                        const float4 x4 = xv[t];
                        double a = fma((double)r.x, (double)x4.x, 0.0);
                        a = fma((double)r.y, (double)x4.y, a);
                        a = fma((double)r.z, (double)x4.z, a);
                        acc[t] = fma((double)r.w, (double)x4.w, a);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < kFzMaxTokens; ++t) {
                if (t < T) {
                    const double sw = wave_sum_dpp_f64(acc[t]);
                    if (lane == 0) rp[wave * kFzMaxTokens + t] = sw;
                }
            }
            __syncthreads();
            if (tid < T) {
                double sum = 0.0;
#pragma unroll
                for (int wv = 0; wv < kFzWaves; ++wv) sum += rp[wv * kFzMaxTokens + tid];
                const uint64_t bits = __builtin_bit_cast(uint64_t, sum);
                uint64_t* dst = rbuf + ((int64_t)tid * U + u) * 2;
                __hip_atomic_store(dst, ((uint64_t)tag << 32) | (uint32_t)bits, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 1, ((uint64_t)tag << 32) | (uint32_t)(bits >> 32),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
        }
        build_x_pieces<kFzMaxTokens, 3>(xv, T, smem, tid);
        // (b) logits from every workgroup's partial sums, the top-k
        double* lgt = reinterpret_cast<double*>(smem + L.lg_off);
        uint64_t* keys = reinterpret_cast<uint64_t*>(smem + L.key_off);
        uint32_t* keys32 = reinterpret_cast<uint32_t*>(smem + L.key32_off);
        int32_t* sel_idx = reinterpret_cast<int32_t*>(smem + L.sel_off);
        double* sel_val = reinterpret_cast<double*>(sel_idx + kFzMaxTokens * kFzMaxSlots);
        int32_t* slot_cnt = reinterpret_cast<int32_t*>(smem + L.scnt_off);
        if (tid < nr) slot_cnt[tid] = 0;
        router_logits_from_partials<kThr>(rbuf, (int)T * U, P, E, U, tag, tid, lane, status, lgt,
                                          keys, keys32);
        __syncthreads();
        topk_rank_screen<kThr>(lgt, keys32, (int)T, E, k, tid, sel_idx, sel_val, slot_cnt);
        __syncthreads();
        if (!__all(lane >= nr || slot_cnt[lane] == 1)) {
            topk_rank_select<kThr>(lgt, keys, keys32, (int)T, E, k, tid, sel_idx, sel_val);
            __syncthreads();
        }
        const int my_idx = lane < nr ? sel_idx[lane] : -1;
        if (is_gu)
            gu_rows_load(rows, lane_value(my_idx, p), E, Ly.gate, Ly.gstride, Ly.up, Ly.ustride, r0, lane);
        float my_w;
        {
            const int tl = lane < nr ? lane / k : 0;
            const double top = sel_val[tl * k];
            const double ex = lane < nr ? exp(sel_val[lane] - top) : 0.0;
            double den = 0.0;
            for (int tt = 0; tt < T; ++tt) {
                double d = 0.0;
                for (int r = 0; r < k; ++r) d += readlane_f64(ex, tt * k + r);
                if (tt == tl) den = d;
            }
            my_w = lane < nr ? (float)(ex / den) : 0.f;
        }
        if (wg == 0 && tid < nr) {
            topk_idx[(int64_t)l * nr + tid] = my_idx;
            topk_w[(int64_t)l * nr + tid] = my_w;
        }

        if (is_gu) {
            __builtin_amdgcn_s_setprio(2);
            if (tau < n_gu) {
                int xc = p / k;
                XCols xcol = load_xcols<3>(smem + xc * kI8TokenBytes, lane);
                gu_rows_finish<3>(rows, xcol, lane, hbuf, (int64_t)p * F + r0, tag);
                for (tau += gu_step; tau < n_gu; tau += gu_step) {
                    p = tau / tiles;
                    r0 = (tau % tiles) * G::R;
                    gu_rows_load(rows, lane_value(my_idx, p), E, Ly.gate, Ly.gstride, Ly.up, Ly.ustride, r0,
                                 lane);
                    const int t = p / k;
                    if (t != xc) {
                        xcol = load_xcols<3>(smem + t * kI8TokenBytes, lane);
                        xc = t;
                    }
                    gu_rows_finish<3>(rows, xcol, lane, hbuf, (int64_t)p * F + r0, tag);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        int dn_wave = __builtin_amdgcn_readfirstlane(is_gu ? 0 : 1);
        asm volatile("" : "+s"(dn_wave));
        if (dn_wave) {
            if (unit < n_dn) {
                const int dw = wave - kFzGu;
                const int64_t t = unit / row_units, r0d = (unit % row_units) * kDnRows;
                for (int s = dw; s < k; s += kFzDn) {
                    const int e = lane_value(my_idx, (int)(t * k + s));
                    if (e >= 0 && e < E)
                        dn_issue_weights(smem + L.dn_off + s * dg.tile_pad, dg, Ly.down, Ly.dstride, e, r0d, lane);
                }
            }
            wait_all_loads();
            if (lane == 0)
                __hip_atomic_fetch_add(dn_ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }

        // (c) down projection and combine; the residual stream goes on as
        // tagged words (the last layer writes x)
        const int groups = (int)(F / kDnGroup);
        const int n_units = k * groups;
        constexpr int kUnitThr = (kFzWaves - 2) * kWave;
        const int uw = wave < 4 ? wave : (wave >= kFzGu ? wave - 2 : -1);
        const int iters = (n_units + kUnitThr - 1) / kUnitThr;
        float* hl = reinterpret_cast<float*>(smem + L.h_off);
        for (int j = 0; unit < n_dn; unit += grid, ++j) {
            const int64_t t = unit / row_units, r0u = (unit % row_units) * kDnRows;
            if (j > 0) {
                for (int s = wave; s < k; s += kFzWaves) {
                    const int e = lane_value(my_idx, (int)(t * k + s));
                    if (e >= 0 && e < E)
                        dn_issue_weights(smem + L.dn_off + s * dg.tile_pad, dg, Ly.down, Ly.dstride, e, r0u, lane);
                }
                wait_all_loads();
                __syncthreads();
            } else if (uw >= 0) {
                int spins = 0;
                while (__hip_atomic_load(dn_ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kFzDn &&
                       ++spins <= kSpinLimit)
                    __builtin_amdgcn_s_sleep(1);
            }
            float acc[kDnRows];
#pragma unroll
            for (int rho = 0; rho < kDnRows; ++rho) acc[rho] = 0.f;
            for (int it = 0; it < iters; ++it) {
                const int u = uw * kWave + lane + it * kUnitThr;
                const bool active = uw >= 0 && u < n_units;
                const int uc = active ? u : 0;
                const int s = uc / groups, grp = uc % groups;
                const int e = __shfl(my_idx, (int)(t * k) + s, kWave);
                const float ws = __shfl(my_w, (int)(t * k) + s, kWave);
                const bool valid = active && e >= 0 && e < E;
                uint32_t qb[kDnRows][4];
                float fa[kDnRows], fc[kDnRows];
                if (uw >= 0) dn_unit_quants(smem + L.dn_off + s * dg.tile_pad, dg, grp, qb, fa, fc);
                if (it == 0) {
                    wait_tagged<kThr>(hbuf + t * k * F, k * (int)F, tag, reinterpret_cast<uint32_t*>(hl), tid, status, 2);
                    if (last && tid == 0 && unit + grid >= n_dn) {
                        int lane0 = 0;
                        asm volatile("" : "+v"(lane0));
                        exit_ticket = __hip_atomic_fetch_add(sync + kSyncExit + (wg % kStripes) * kLineInts + lane0, 1,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    __syncthreads();
                }
                if (uw >= 0) {
                    float hv[kDnGroup];
#pragma unroll
                    for (int i = 0; i < kDnGroup; i += 4) {
                        const float4 h4 = *reinterpret_cast<const float4*>(hl + s * F + grp * kDnGroup + i);
                        hv[i] = h4.x; hv[i + 1] = h4.y; hv[i + 2] = h4.z; hv[i + 3] = h4.w;
                    }
                    float hsum = 0.f;
#pragma unroll
                    for (int i = 0; i < kDnGroup; ++i) hsum += hv[i];
#pragma unroll
                    for (int rho = 0; rho < kDnRows; ++rho) {
                        float sq = 0.f;
#pragma unroll
                        for (int i = 0; i < kDnGroup; ++i)
                            sq = fmaf((float)((qb[rho][i >> 2] >> (8 * (i & 3))) & 0xffu), hv[i], sq);
                        const float y = fmaf(fa[rho], sq, fc[rho] * hsum);
                        acc[rho] += valid ? ws * y : 0.f;
                    }
                }
            }
            const float r = fold8_rows(acc, lane);
            if ((lane & 7) == 0) res[wave * kDnRows + (lane >> 3)] = r;
            __syncthreads();
            if (wave == 0 && lane < kDnRows) {                // fixed order over the waves
                float o = 0.f;
#pragma unroll
                for (int wv = 0; wv < kFzWaves; ++wv) o += res[wv * kDnRows + lane];
                const int64_t row = t * G::H + r0u + lane;
                // x_l of the row: the input (layer 0) or this workgroup's own
                // word of the stream (it owns the row in every layer)
                const float xo = l == 0 ? x[row]
                                        : __uint_as_float((uint32_t)__hip_atomic_load(
                                              xbuf + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                const float xn = xo + o;
                if (last) x[row] = xn;
                else __hip_atomic_store(xbuf + row, ((uint64_t)xtag << 32) | __float_as_uint(xn),
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // exit: the last workgroup advances the epoch and zeroes the counters
    if (threadIdx.x == 0) {
        const int grid = (int)gridDim.x, wg = (int)blockIdx.x;
        const int st = wg % kStripes;
        const int32_t done = exit_ticket >= 0
                                 ? exit_ticket
                                 : __hip_atomic_fetch_add(sync + kSyncExit + st * kLineInts, 1,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == stripe_members(st, grid) - 1) {
            const int used = grid < kStripes ? grid : kStripes;
            const int32_t top = __hip_atomic_fetch_add(sync + kSyncExitTop, 1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            if (top == used - 1) {
                for (int i = 0; i < kStripes; ++i)
                    __hip_atomic_store(sync + kSyncExit + i * kLineInts, 0, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sync + kSyncExitTop, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(sync + kSyncEpoch, (int32_t)(epoch + 1u), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

constexpr size_t kMaxLdsPerWorkgroup = 160 * 1024;

// Compute-unit count of the current device, cached per device (an immutable
// device fact; the cache only saves the query on later calls).
int cu_count() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        return 0;
    if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

size_t gu_lds_bytes(int nb) {
    const int R = 32 / nb;
    const size_t taskb = (size_t)R * nb * kQ4KBytes;
    return kGuWaves * 2 * taskb + (size_t)nb * kBlockPieceStride + (size_t)nb * 16 * 4 +
           (size_t)nb * kBlockLoStride;
}

size_t down_lds_bytes(int64_t F, int32_t qtype) {
    const DnGeom g(F, qtype);
    return (size_t)kDnWaves * kDnSlotsPerWave * g.per_slot + (size_t)kMaxTopK * kDnRows * 4;
}

template <int NB>
hipError_t launch_gu(const float* hidden, int64_t T, int64_t F, int32_t E, int32_t k,
                     const int32_t* idx, const ExpertTensor& gate, const ExpertTensor& up,
                     uint8_t* hp, hipStream_t stream) {
    constexpr int R = 32 / NB;
    const int64_t tasks = T * k * (F / R);
    const size_t lds = gu_lds_bytes(NB);
    static LdsLimit lds_set;
    hipError_t err = ensure_lds(reinterpret_cast<const void*>(gu_decode_kernel<NB>), lds_set, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gu_decode_kernel<NB>, dim3((unsigned)(tasks / kGuWaves)), dim3(kGuWaves * kWave),
                       lds, stream, hidden, F, E, k, idx, gate.base, gate.stride, up.base, up.stride, hp);
    return hipGetLastError();
}

hipError_t launch_down(const float* w, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k,
                       const int32_t* idx, const ExpertTensor& down, const uint8_t* hp, float* out,
                       int accumulate, hipStream_t stream) {
    const size_t lds = down_lds_bytes(F, down.qtype);
    static LdsLimit lds_set;
    hipError_t err = ensure_lds(reinterpret_cast<const void*>(down_decode_kernel), lds_set, (int)lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(down_decode_kernel, dim3((unsigned)T, (unsigned)(H / kDnRows)),
                       dim3(kDnWaves * kWave), lds, stream, H, F, E, k, idx, w, down.base, down.qtype,
                       down.stride, hp, out, accumulate);
    return hipGetLastError();
}

template <bool kRoute, int NP>
hipError_t launch_fused8(const float* hidden, int64_t T, int64_t F, int32_t E, int32_t k,
                         const int32_t* idx, const float* w, const ExpertTensor& gate,
                         const ExpertTensor& up, const ExpertTensor& down, float* out,
                         int accumulate, uint8_t* hp, int32_t* sync, int grid,
                         const float* router, int P, int32_t* topk_idx, float* topk_w,
                         uint64_t* rbuf, const float* norm_gain, float eps, hipStream_t stream) {
    const FusedLds L = fused_lds(T, F, down.qtype);
    static LdsLimit lds_set;
    hipError_t err = ensure_lds(reinterpret_cast<const void*>(ffn_fused8_kernel<kRoute, NP>), lds_set, L.total);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((ffn_fused8_kernel<kRoute, NP>), dim3((unsigned)grid), dim3(kFzWaves * kWave),
                       (size_t)L.total, stream, hidden, T, F, E, k, idx, w, gate.base, gate.stride,
                       up.base, up.stride, down.base, down.qtype, down.stride, out, accumulate,
                       reinterpret_cast<uint64_t*>(hp), sync, router, (int32_t)P, topk_idx, topk_w,
                       rbuf, norm_gain, eps);
    return hipGetLastError();
}

// Workgroups of ffn_fused8_kernel<kRoute> that one compute unit of the
// current device holds at once with `lds` bytes of dynamic LDS (the
// occupancy calculator's answer for this kernel's registers, waves and LDS),
// cached per (device, LDS size); 0 when the device cannot run it.
template <bool kRoute, int NP>
int fused_blocks_per_cu(int lds) {
    static std::atomic<int64_t> cache[kMaxDevices];   // (lds << 16) | (blocks + 1)
    static LdsLimit lds_set;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c != 0 && (c >> 16) == lds) return (int)(c & 0xffff) - 1;
    }
    const void* fn = reinterpret_cast<const void*>(ffn_fused8_kernel<kRoute, NP>);
    if (ensure_lds(fn, lds_set, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kFzWaves * kWave, (size_t)lds) != hipSuccess ||
        n < 0)
        n = 0;
    if (dev < kMaxDevices) cache[dev].store(((int64_t)lds << 16) | (int64_t)(n + 1), std::memory_order_relaxed);
    return n;
}

// Workgroups of the fused kernel for this shape (one per compute unit at
// most), or 0 when the shape is outside it.  The kernel's workgroups wait on
// each other, so all of them must be resident at once: the grid never
// exceeds the compute units times the workgroups one unit holds (the
// occupancy calculator's figure), and a device that holds none at this LDS
// size takes the two-kernel path.
int fused_grid(int64_t T, int64_t H, int64_t F, int32_t k, int32_t dqtype, bool route, int np = 3) {
    if (H != (int64_t)kFzNB * kQK || k > kFzMaxSlots || T > kFzMaxTokens || T < 1) return 0;
    const int lds = fused_lds(T, F, dqtype).total;
    if ((size_t)lds > kMaxLdsPerWorkgroup) return 0;
    const int cus = cu_count();
    if (cus <= 0) return 0;
    const int per_cu = !route ? fused_blocks_per_cu<false, 3>(lds)
                       : np == 1 ? fused_blocks_per_cu<true, 1>(lds) : fused_blocks_per_cu<true, 3>(lds);
    if (per_cu < 1) return 0;
    const int64_t tiles = F / GuTask<kFzNB>::R;
    const int64_t need = (T * k * tiles + kFzGu - 1) / kFzGu;
    const int64_t units = T * (H / kDnRows);
    const int64_t want = need > units ? need : units;
    const int64_t cap = cus < kMaxPresence ? cus : kMaxPresence;   // one presence word per workgroup
    return (int)(want < cap ? want : cap);
}

// Column parts per router row in the fused kernel: the largest power of two
// up to 8 that keeps E * P within the workgroup count (one router unit per
// workgroup) and the unit table.
int route_parts(int32_t E, int grid) {
    int P = 1;
    while (P < 8 && (int64_t)E * P * 2 <= grid && (int64_t)E * P * 2 <= kFzMaxUnits) P *= 2;
    return P;
}

template <int NB>
hipError_t launch_decode_nb(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                            int32_t k, const int32_t* idx, const float* w, const ExpertTensor& gate,
                            const ExpertTensor& up, const ExpertTensor& down, float* out,
                            int accumulate, uint8_t* hp, int32_t* sync, hipStream_t stream) {
    if constexpr (NB == kFzNB) {
        const int grid = fused_grid(T, H, F, k, down.qtype, false);
        if (grid > 0)
            return launch_fused8<false, 3>(hidden, T, F, E, k, idx, w, gate, up, down, out, accumulate,
                                        hp, sync, grid, nullptr, 1, nullptr, nullptr, nullptr, nullptr,
                                        0.f, stream);
    }
    hipError_t err = launch_gu<NB>(hidden, T, F, E, k, idx, gate, up, hp, stream);
    if (err != hipSuccess) return err;
    return launch_down(w, T, H, F, E, k, idx, down, hp, out, accumulate, stream);
}

}  // namespace

bool decode_ffn_supported(int64_t H, int64_t F, int32_t k) {
    const int64_t nb = H / kQK;
    return (nb == 1 || nb == 2 || nb == 4 || nb == 8 || nb == 16) && F % kQK == 0 && k >= 1;
}


hipError_t launch_decode_ffn(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const int32_t* idx, const float* w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ws,
                             hipStream_t stream) {
    int32_t* sync = static_cast<int32_t*>(ws);
    uint8_t* hp = static_cast<uint8_t*>(ws) + kFfnSyncBytes;
    switch (H / kQK) {
        case 1: return launch_decode_nb<1>(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, hp, sync, stream);
        case 2: return launch_decode_nb<2>(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, hp, sync, stream);
        case 4: return launch_decode_nb<4>(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, hp, sync, stream);
        case 8: return launch_decode_nb<8>(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, hp, sync, stream);
        case 16: return launch_decode_nb<16>(hidden, T, H, F, E, k, idx, w, gate, up, down, out, accumulate, hp, sync, stream);
        default: return hipErrorInvalidValue;
    }
}

bool expert_ffn_fused(int64_t T, int64_t H, int64_t F, int32_t k, int32_t dqtype) {
    return T < kPrefillMinTokens && decode_ffn_supported(H, F, k) && H / kQK == kFzNB &&
           fused_grid(T, H, F, k, dqtype, false) > 0;
}

bool moe_decode_fused(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, int32_t dqtype,
                      int act_pieces) {
    return E <= kFzRouteNper * kWave && fused_grid(T, H, F, k, dqtype, true, act_pieces) > 0;
}

size_t moe_route_words_bytes(int64_t T, int32_t E) {
    return (size_t)(T > 0 ? T : 0) * (size_t)E * 8 * 2 * sizeof(uint64_t);   // up to 8 parts
}

hipError_t launch_moe_decode(const float* hidden, int64_t T, int64_t H, int64_t F, int32_t E,
                             int32_t k, const float* router, int32_t* topk_idx, float* topk_w,
                             const ExpertTensor& gate, const ExpertTensor& up,
                             const ExpertTensor& down, float* out, int accumulate, void* ffn_ws,
                             void* route_words, const float* norm_gain, float eps, hipStream_t stream,
                             int act_pieces) {
    if (act_pieces != 1 && act_pieces != 3) return hipErrorInvalidValue;
    int grid = fused_grid(T, H, F, k, down.qtype, true, act_pieces);
    if (grid <= 0 || E > kFzRouteNper * kWave) return hipErrorInvalidValue;
    int32_t* sync = static_cast<int32_t*>(ffn_ws);
    uint8_t* hp = static_cast<uint8_t*>(ffn_ws) + kFfnSyncBytes;
    auto* rw = static_cast<uint64_t*>(route_words);
    const int P = route_parts(E, grid);
    // In place (out == hidden), a workgroup may overwrite rows of hidden only
    // once every workgroup has read them.  It writes after seeing every router
    // word, and a workgroup publishes its router words only after it has read
    // all of hidden: so every workgroup must own a router unit (route_parts
    // gives the same P for the smaller grid).
    if (static_cast<const void*>(hidden) == static_cast<const void*>(out) && E * P < grid) grid = E * P;
    if (act_pieces == 1)
        return launch_fused8<true, 1>(hidden, T, F, E, k, nullptr, nullptr, gate, up, down, out,
                                      accumulate, hp, sync, grid, router, P, topk_idx, topk_w, rw,
                                      norm_gain, eps, stream);
    return launch_fused8<true, 3>(hidden, T, F, E, k, nullptr, nullptr, gate, up, down, out, accumulate,
                                  hp, sync, grid, router, P, topk_idx, topk_w, rw, norm_gain, eps,
                                  stream);
}

namespace {

// Workgroups of ffn_stack_kernel one compute unit holds at once with `lds`
// bytes of dynamic LDS (the occupancy calculator's answer), cached per
// (device, LDS size); 0 when the device cannot run it.
int stack_blocks_per_cu(int lds) {
    static std::atomic<int64_t> cache[kMaxDevices];
    static LdsLimit lds_set;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c != 0 && (c >> 16) == lds) return (int)(c & 0xffff) - 1;
    }
    const void* fn = reinterpret_cast<const void*>(ffn_stack_kernel);
    if (ensure_lds(fn, lds_set, lds) != hipSuccess) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kFzWaves * kWave, (size_t)lds) != hipSuccess ||
        n < 0)
        n = 0;
    if (dev < kMaxDevices) cache[dev].store(((int64_t)lds << 16) | (int64_t)(n + 1), std::memory_order_relaxed);
    return n;
}

// Grid of the stack kernel (0: shape outside it), and its router parts.
// At most one workgroup per compute unit (all resident), and no more
// workgroups than down units (T * H / 8) or router units (E * P): every
// workgroup owns one of each, which the kernel's buffer reuse relies on.
int stack_grid(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, int* P) {
    if (H != (int64_t)kFzNB * kQK || k > kFzMaxSlots || T > kFzMaxTokens || T < 1 ||
        E > kFzRouteNper * kWave || F % kQK != 0)
        return 0;
    const int lds = fused_lds(T, F, 2).total;       // the Q6_K tile layout serves both down types
    if ((size_t)lds > kMaxLdsPerWorkgroup) return 0;
    const int cus = cu_count();
    if (cus <= 0 || stack_blocks_per_cu(lds) < 1) return 0;
    const int64_t units = T * (H / kDnRows);
    int grid = (int)(units < cus ? units : cus);
    *P = route_parts(E, grid);
    if ((int64_t)E * *P < grid) grid = E * *P;
    return grid;
}

}  // namespace

bool moe_stack_fused(int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, const MoeLayerTensors* layers,
                     int32_t n_layers) {
    for (int32_t l = 0; l < n_layers; ++l)
        if (layers[l].gate.stride > INT32_MAX || layers[l].up.stride > INT32_MAX ||
            layers[l].down.stride > INT32_MAX)
            return false;
    int P = 1;
    return stack_grid(T, H, F, E, k, &P) > 0;
}

size_t moe_stack_xbuf_bytes(int64_t T, int64_t H) {
    return (size_t)(T > 0 ? T : 0) * (size_t)(H > 0 ? H : 0) * sizeof(uint64_t);
}

hipError_t launch_moe_stack(float* x, int64_t T, int64_t H, int64_t F, int32_t E, int32_t k, float eps,
                            const MoeLayerTensors* layers, int32_t n_layers, int32_t* topk_idx,
                            float* topk_w, void* ffn_ws, void* route_words, void* xbuf,
                            hipStream_t stream) {
    int P = 1;
    const int grid = stack_grid(T, H, F, E, k, &P);
    if (grid <= 0) return hipErrorInvalidValue;
    const FusedLds L = fused_lds(T, F, 2);
    static LdsLimit lds_set;
    hipError_t err = ensure_lds(reinterpret_cast<const void*>(ffn_stack_kernel), lds_set, L.total);
    if (err != hipSuccess) return err;
    int32_t* sync = static_cast<int32_t*>(ffn_ws);
    auto* hb = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ffn_ws) + kFfnSyncBytes);
    const int64_t nr = T * k;
    for (int32_t l0 = 0; l0 < n_layers; l0 += kMaxStackLayers) {
        const int32_t nl = n_layers - l0 < kMaxStackLayers ? n_layers - l0 : kMaxStackLayers;
        StackJob job{};
        for (int32_t i = 0; i < nl; ++i) {
            const MoeLayerTensors& s = layers[l0 + i];
            if (s.gate.stride > INT32_MAX || s.up.stride > INT32_MAX || s.down.stride > INT32_MAX)
                return hipErrorInvalidValue;
            job.layer[i] = StackLayer{s.router, s.gain, s.gate.base, s.up.base, s.down.base,
                                      (int32_t)s.gate.stride, (int32_t)s.up.stride, (int32_t)s.down.stride,
                                      s.down.qtype};
        }
        hipLaunchKernelGGL(ffn_stack_kernel, dim3((unsigned)grid), dim3(kFzWaves * kWave), (size_t)L.total,
                           stream, x, T, F, E, k, nl, eps, (int32_t)P, topk_idx + l0 * nr,
                           topk_w + l0 * nr, hb, sync, static_cast<uint64_t*>(route_words),
                           static_cast<uint64_t*>(xbuf), job);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace q3moe
