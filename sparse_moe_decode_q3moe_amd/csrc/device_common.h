// Device helpers shared by the q3moe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3moe {

constexpr int kWave = 64;
constexpr int kQK = 256;          // weights per k-quant super-block
constexpr int kQ4KBytes = 144;
constexpr int kQ6KBytes = 210;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// 16 bytes from LDS at a 2-byte-aligned offset: five aligned dword reads
// realigned with v_alignbyte.  Reads up to 4 bytes past the 16 requested,
// so LDS tiles read this way carry 16 bytes of tail padding.
__device__ __forceinline__ uint4 lds_read16_a2(const uint8_t* lds, int off) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (off & ~3));
    const uint32_t sh = (uint32_t)(off & 3);
    uint32_t a0 = p[0], a1 = p[1], a2 = p[2], a3 = p[3], a4 = p[4];
    uint4 r;
    r.x = __builtin_amdgcn_alignbyte(a1, a0, sh);
    r.y = __builtin_amdgcn_alignbyte(a2, a1, sh);
    r.z = __builtin_amdgcn_alignbyte(a3, a2, sh);
    r.w = __builtin_amdgcn_alignbyte(a4, a3, sh);
    return r;
}

// Q4_K 6-bit scale / min of sub-block j (0..7) from the 12 packed bytes S.
__device__ __forceinline__ void q4k_scale_min(const uint8_t* S, int j, int& sc, int& mn) {
    if (j < 4) {
        sc = S[j] & 63;
        mn = S[j + 4] & 63;
    } else {
        sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
        mn = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
}

// Partial dot product of one 16-byte quant chunk m (0..7) of a Q4_K block
// held in LDS with the block's 256 inputs x (LDS or registers via pointer).
// Chunk m covers quant bytes 32c + 16h' .. +15 (c = m/2, h' = m%2); their
// low nibbles are weights 64c + 16h' + i (sub-block 2c) and their high
// nibbles weights 64c + 32 + 16h' + i (sub-block 2c+1).  The min term uses
// sum(x) over the same positions: sum((d*sc*q - dmin*mn) x)
//   = d*sc*sum(q x) - dmin*mn*sum(x).
__device__ __forceinline__ float q4k_chunk_dot(const uint8_t* blk, int m, const float* x) {
    const uint32_t hdr = *reinterpret_cast<const uint32_t*>(blk);
    const float d = half_bits_to_float(hdr & 0xffffu);
    const float dmin = half_bits_to_float(hdr >> 16);
    const int c = m >> 1, hp = m & 1;
    int sc0, mn0, sc1, mn1;
    q4k_scale_min(blk + 4, 2 * c, sc0, mn0);
    q4k_scale_min(blk + 4, 2 * c + 1, sc1, mn1);
    const uint4 qv = *reinterpret_cast<const uint4*>(blk + 16 + 32 * c + 16 * hp);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const float* xl = x + 64 * c + 16 * hp;
    const float* xh = xl + 32;
    float sl = 0.f, sh = 0.f, xsl = 0.f, xsh = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(xl + 4 * i);
        const float4 b = *reinterpret_cast<const float4*>(xh + 4 * i);
        const uint32_t w = qw[i];
        sl += (float)(w & 15) * a.x + (float)((w >> 8) & 15) * a.y +
              (float)((w >> 16) & 15) * a.z + (float)((w >> 24) & 15) * a.w;
        sh += (float)((w >> 4) & 15) * b.x + (float)((w >> 12) & 15) * b.y +
              (float)((w >> 20) & 15) * b.z + (float)((w >> 28) & 15) * b.w;
        xsl += (a.x + a.y) + (a.z + a.w);
        xsh += (b.x + b.y) + (b.z + b.w);
    }
    return d * ((float)sc0 * sl + (float)sc1 * sh) - dmin * ((float)mn0 * xsl + (float)mn1 * xsh);
}

// Partial dot product of one 16-weight unit v (0..15) of a Q6_K block held
// in LDS at a 2-byte-aligned offset `boff` with the block's inputs x.
// Unit v = (n, r, lh) with n = v/8, r = (v%8)/2, lh = v%2 covers weights
// 128n + 32r + 16lh + i (i < 16): low 4 bits from byte 64n + 32(r&1) +
// 16lh + i (low nibble for r < 2, high for r >= 2), high 2 bits from byte
// 128 + 32n + 16lh + i at bit 2r, scale 192 + 8n + 2r + lh, fp16 d at 208.
__device__ __forceinline__ float q6k_unit_dot(const uint8_t* lds, int boff, int v, const float* x) {
    const int n = v >> 3, r = (v & 7) >> 1, lh = v & 1;
    const uint4 lo = lds_read16_a2(lds, boff + 64 * n + 32 * (r & 1) + 16 * lh);
    const uint4 hi = lds_read16_a2(lds, boff + 128 + 32 * n + 16 * lh);
    const int sc = (int)(int8_t)lds[boff + 192 + 8 * n + 2 * r + lh];
    const float d = half_bits_to_float(lds[boff + 208] | (lds[boff + 209] << 8));
    const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t hw[4] = {hi.x, hi.y, hi.z, hi.w};
    const int lshift = (r >= 2) ? 4 : 0;
    const int hshift = 2 * r;
    const float* xs = x + 128 * n + 32 * r + 16 * lh;
    float sq = 0.f, sx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(xs + 4 * i);
        const uint32_t l4 = (lw[i] >> lshift) & 0x0f0f0f0fu;
        const uint32_t h2 = (hw[i] >> hshift) & 0x03030303u;
        const uint32_t q = l4 | (h2 << 4);
        sq += (float)(q & 63) * a.x + (float)((q >> 8) & 63) * a.y +
              (float)((q >> 16) & 63) * a.z + (float)((q >> 24) & 63) * a.w;
        sx += (a.x + a.y) + (a.z + a.w);
    }
    return d * (float)sc * (sq - 32.f * sx);
}

// ---------------------------------------------------------------------------
// Activation pieces.  The decode kernels multiply k-quant weights, which are
// small integers once the per-block scales are factored out, by activations
// split into two bf16 pieces, x = hi + lo (hi = bf16(x), lo = bf16(x - hi),
// both round-to-nearest-even; |x - hi - lo| <= 2^-18 |x|).  A weight q is
// exact as the bf16 value 128 + q (q < 128), so v_dot2_f32_bf16 forms
// sum (128 + q)(hi + lo) with exact products; the 128 offset is removed with
// the per-16 group sums of hi + lo.
//
// Layout of a vector of K values (K a multiple of 256): slot s holds values
// 4s..4s+3 in 16 bytes:
//   dword 0 = hi(4s)   | hi(4s+2) << 16     dword 2 = lo(4s)   | lo(4s+2) << 16
//   dword 1 = hi(4s+1) | hi(4s+3) << 16     dword 3 = lo(4s+1) | lo(4s+3) << 16
// which matches the weight pairs (w & 0x000F000F) / (w >> 8 & 0x000F000F)
// taken from a dword of four consecutive quant bytes.  In global memory the
// slots are contiguous (K*4 bytes); in LDS every 64 slots (one 256-value
// super-block) are followed by 16 bytes of padding so that lanes reading
// the same slot of different blocks hit different banks.
constexpr int kSlotBytes = 16;
constexpr int kBlockPieceStride = 64 * kSlotBytes + 16;   // 1040 bytes per 256 values in LDS

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// f32 -> bf16 bits, round to nearest even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    return (uint16_t)bf16_rne_bits(f);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

struct Pieces4 {
    uint4 slot;     // the 16-byte slot
    float sum;      // (hi + lo) summed over the 4 values
};

__device__ __forceinline__ Pieces4 make_pieces4(float4 v) {
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t hb[4], lb[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hb[i] = bf16_rne_bits(x[i]);
        const float r = x[i] - bf16_bits_to_float(hb[i]);
        lb[i] = bf16_rne_bits(r);
        s += bf16_bits_to_float(hb[i]) + bf16_bits_to_float(lb[i]);
    }
    Pieces4 p;
    p.slot = make_uint4(hb[0] | (hb[2] << 16), hb[1] | (hb[3] << 16), lb[0] | (lb[2] << 16),
                        lb[1] | (lb[3] << 16));
    p.sum = s;
    return p;
}

// Three pieces of 4 values: x = hi + mid + lo, each bf16 round-to-nearest-
// even of what the previous ones leave, so |x - hi - mid - lo| <= 2^-27 |x|.
// The slot holds (hi, mid) in the two-piece layout above; `lo` holds the third
// piece as dword 0 = lo(4s) | lo(4s+2) << 16, dword 1 = lo(4s+1) | lo(4s+3) << 16.
// Used for the gate/up input, whose rounding the outputs amplify most.
struct Pieces4x3 {
    uint4 slot;
    uint2 lo;
    float sum;      // (hi + mid + lo) summed over the 4 values
};

__device__ __forceinline__ Pieces4x3 make_pieces4x3(float4 v) {
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t hb[4], mb[4], lb[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hb[i] = bf16_rne_bits(x[i]);
        const float r1 = x[i] - bf16_bits_to_float(hb[i]);
        mb[i] = bf16_rne_bits(r1);
        const float r2 = r1 - bf16_bits_to_float(mb[i]);
        lb[i] = bf16_rne_bits(r2);
        s += (bf16_bits_to_float(hb[i]) + bf16_bits_to_float(mb[i])) + bf16_bits_to_float(lb[i]);
    }
    Pieces4x3 p;
    p.slot = make_uint4(hb[0] | (hb[2] << 16), hb[1] | (hb[3] << 16), mb[0] | (mb[2] << 16),
                        mb[1] | (mb[3] << 16));
    p.lo = make_uint2(lb[0] | (lb[2] << 16), lb[1] | (lb[3] << 16));
    p.sum = s;
    return p;
}

// LDS layout of the third pieces: 8 bytes per slot, 64 slots per 256 values
// followed by 16 bytes of padding.
constexpr int kBlockLoStride = 64 * 8 + 16;
__device__ __forceinline__ int piece_lo_off(int s) { return (s >> 6) * kBlockLoStride + (s & 63) * 8; }

__device__ __forceinline__ float slot_sum(uint4 s) {
    auto f = [](uint32_t w) { return bf16_bits_to_float(w & 0xffffu) + bf16_bits_to_float(w >> 16); };
    return (f(s.x) + f(s.y)) + (f(s.z) + f(s.w));
}

// LDS byte offset of slot s in the padded layout.
__device__ __forceinline__ int piece_slot_off(int s) { return (s >> 6) * kBlockPieceStride + (s & 63) * kSlotBytes; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copy by one wave (gfx950 global_load_lds_dwordx4): lane i
// of each 1 KiB step moves bytes [16i, 16i+16) of that step; nbytes must be a
// multiple of 16 and both addresses 16-byte aligned.  The loads are only
// issued here; the caller waits (s_waitcnt vmcnt) before reading the LDS.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void wave_copy_to_lds(uint8_t* lds, const uint8_t* __restrict__ g,
                                                 int nbytes, int lane) {
    const int n16 = nbytes >> 4;
    for (int base = 0; base < n16; base += kWave) {
        if (base + lane < n16)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g + (base + lane) * 16),
                                             (lds_ptr_t)(lds + base * 16), 16, 0, 0);
    }
}

// The same for data read once (expert weights): non-temporal loads, so the
// stream does not evict reused lines (code, routing, counters) from L2.
constexpr int kCachePolicyNt = 2;
__device__ __forceinline__ void wave_stream_to_lds(uint8_t* lds, const uint8_t* __restrict__ g,
                                                   int nbytes, int lane) {
    const int n16 = nbytes >> 4;
    for (int base = 0; base < n16; base += kWave) {
        if (base + lane < n16)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g + (base + lane) * 16),
                                             (lds_ptr_t)(lds + base * 16), 16, 0, kCachePolicyNt);
    }
}

// The same with device-scope coherent loads (sc1): they bypass the per-XCD
// L2, so they see data that another XCD wrote with device-scope stores
// without an L2 invalidate.
constexpr int kCachePolicySc1 = 16;

__device__ __forceinline__ void wave_copy_to_lds_coherent(uint8_t* lds, const uint8_t* g,
                                                          int nbytes, int lane) {
    const int n16 = nbytes >> 4;
    for (int base = 0; base < n16; base += kWave) {
        if (base + lane < n16)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g + (base + lane) * 16),
                                             (lds_ptr_t)(lds + base * 16), 16, 0, kCachePolicySc1);
    }
}

__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace q3moe
