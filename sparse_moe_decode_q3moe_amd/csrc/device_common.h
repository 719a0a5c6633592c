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

}  // namespace q3moe
