// The two ends of the model around the 48 decoder layers of a decode step:
// the token embedding gather and the Q6_K output head (aprender issue #3714,
// "File facts": hidden 2048, the output matrix stored as Q6_K; the embedding
// and head rows are k-quant rows of H inputs, read in place).
//
// embed_kernel: one workgroup per token; every thread dequantises weights
//   of the token's row straight from HBM (one row is 1,152 or 1,680 bytes,
//   so the gather is a handful of dependent loads; nothing to stage).
//
// head_q6k_kernel: the logits GEMV over the vocabulary, a single 255 MB
//   stream at the 30B-A3B shape.  Each wave takes groups of 8 consecutive
//   rows (8 x 1,680 = 13,440 contiguous bytes): coalesced 16-byte loads of
//   the next group go out into registers while the current group, stored
//   to the wave's LDS slot, is consumed.  Lane u owns one 32-weight unit of
//   every row (block u / 8, unit (n, r) = ((u / 4) % 2, u % 4): weights
//   128n + 32r + l of the block), so its 32 activations are fixed for the
//   whole kernel: they are split once into three int8 pieces with a
//   power-of-two group scale, x = s (p1 + p2 / 2^7 + p3 / 2^14) + r with
//   |r| <= s 2^-15, and held in registers.  Per row the lane forms the 6-bit
//   quants of its unit (4 bits from the low-nibble plane, 2 from the high
//   plane), and v_dot4_i32_i8 gives each piece's dot product over 4 weights
//   exactly; sum((q - 32) p) = sum(q p) - 32 sum(p) stays an exact int32 per
//   16-weight scale group until its one conversion to f32, then the group's
//   scale d * s_j and the activation scale apply.  The 8 row partials fold
//   across the wave with a transposed butterfly.
#include "device_common.h"
#include "internal.h"

namespace q3moe {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- embedding --

// Weight i (0..255) of a Q4_K block: i = 64c + 32h + l, quant (Q[32c + l] >>
// 4h) & 15, sub-block j = 2c + h; d * sc * q - dmin * m rounded once (d * sc
// and dmin * m are exact in f32).
__device__ __forceinline__ float q4k_weight(const uint8_t* blk, int i) {
    const int c = i >> 6, h = (i >> 5) & 1, l = i & 31;
    const int q = (blk[16 + 32 * c + l] >> (4 * h)) & 15;
    int sc, mn;
    q4k_scale_min(blk + 4, 2 * c + h, sc, mn);
    const float d = half_bits_to_float(blk[0] | (blk[1] << 8));
    const float dmin = half_bits_to_float(blk[2] | (blk[3] << 8));
    return fmaf(d * (float)sc, (float)q, -(dmin * (float)mn));
}

// Weight i of a Q6_K block: i = 128n + 32r + l, low four bits from byte
// 64n + 32(r & 1) + l (low nibble for r < 2), top two from byte 128 + 32n + l
// at bit 2r, int8 scale 192 + 8n + 2r + l / 16, fp16 d at 208; d * s exact in
// f32, times (q - 32) rounded once.
__device__ __forceinline__ float q6k_weight(const uint8_t* blk, int i) {
    const int n = i >> 7, r = (i >> 5) & 3, l = i & 31;
    const int lo = blk[64 * n + 32 * (r & 1) + l] >> (4 * (r >> 1)) & 15;
    const int hi = (blk[128 + 32 * n + l] >> (2 * r)) & 3;
    const int s = (int8_t)blk[192 + 8 * n + 2 * r + (l >> 4)];
    const float d = half_bits_to_float(blk[208] | (blk[209] << 8));
    return (d * (float)s) * (float)((lo | (hi << 4)) - 32);
}

constexpr int kEmbThreads = 256;

// grid: T workgroups.
__global__ __launch_bounds__(kEmbThreads) void embed_kernel(const int32_t* __restrict__ tokens,
                                                             const uint8_t* __restrict__ table,
                                                             int32_t qtype, int64_t V, int64_t H,
                                                             float* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t v = tokens[t];
    float* o = out + t * H;
    if (v < 0 || v >= V) {
        for (int64_t i = threadIdx.x; i < H; i += kEmbThreads) o[i] = __builtin_nanf("");
        return;
    }
    const int bb = qtype == 2 ? kQ6KBytes : kQ4KBytes;
    const uint8_t* row = table + v * (H / kQK) * bb;
    for (int64_t i = threadIdx.x; i < H; i += kEmbThreads) {
        const uint8_t* blk = row + (i / kQK) * bb;
        const int w = (int)(i % kQK);
        o[i] = qtype == 2 ? q6k_weight(blk, w) : q4k_weight(blk, w);
    }
}

// ----------------------------------------------------------- output head --

constexpr int kHdWaves = 4;
constexpr int kHdRows = 8;                               // rows per wave group
constexpr int kHdNB = 8;                                 // H = 2048: one unit per lane
constexpr int kHdRowB = kHdNB * kQ6KBytes;               // 1,680
constexpr int kHdGrpB = kHdRows * kHdRowB;               // 13,440 = 840 x 16
constexpr int kHdChunks = kHdGrpB / 16;
constexpr int kHdLoads = (kHdChunks + kWave - 1) / kWave;   // 14 per lane
constexpr int kHdSlot = kHdGrpB + 16;                    // + tail for the 2-byte-aligned reads
static_assert(kHdGrpB % 16 == 0, "row groups are whole 16-byte chunks");
static_assert(kHdNB * 8 == kWave, "one 32-weight unit per lane and row");

// The lane's 32 activations as three int8 pieces (8 dwords each, 4 values
// per dword in order), the per-16 piece sums and the scale s * 2^-14.
struct HeadX {
    uint32_t p[3][8];
    int ps[3][2];
    float sx;
};

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
    return ((uint32_t)(int)a & 0xffu) | (((uint32_t)(int)b & 0xffu) << 8) |
           (((uint32_t)(int)c & 0xffu) << 16) | ((uint32_t)(int)d << 24);
}

__device__ __forceinline__ HeadX head_x_unit(const float* __restrict__ x) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 f = reinterpret_cast<const float4*>(x)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    float m = 0.f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        finite = finite && fabsf(v[i]) <= 3.4028235e38f;
        m = fmaxf(m, fabsf(v[i]));
    }
    // s = 2^e with m / s in [63.75, 127.5)
    int e = finite && m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 7 : 0;
    if (ldexpf(m, -e) >= 127.5f) ++e;
    HeadX X;
#pragma unroll
    for (int q = 0; q < 3; ++q) X.ps[q][0] = X.ps[q][1] = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float p1[4], p2[4], p3[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float q = ldexpf(v[4 * k + i], -e);
            p1[i] = finite ? rintf(q) : 0.f;
            const float r1 = (q - p1[i]) * 128.f;
            p2[i] = finite ? rintf(r1) : 0.f;
            const float r2 = (r1 - p2[i]) * 128.f;
            p3[i] = finite ? rintf(r2) : 0.f;
            X.ps[0][k >> 2] += (int)p1[i];
            X.ps[1][k >> 2] += (int)p2[i];
            X.ps[2][k >> 2] += (int)p3[i];
        }
        X.p[0][k] = pack4(p1[0], p1[1], p1[2], p1[3]);
        X.p[1][k] = pack4(p2[0], p2[1], p2[2], p2[3]);
        X.p[2][k] = pack4(p3[0], p3[1], p3[2], p3[3]);
    }
    X.sx = finite ? ldexpf(1.f, e - 14) : __builtin_nanf("");
    return X;
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Sum v[0..7] over the wave; lanes 8q .. 8q+7 receive row q's total.  Each
// exchange halves the values a lane carries (xor 32, 16, 8), then the 8 lanes
// of a row add up.
__device__ __forceinline__ float fold8(const float (&v)[8], int lane) {
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
    float a[4], c[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = (b5 ? v[i + 4] : v[i]) + __shfl_xor(b5 ? v[i] : v[i + 4], 32, kWave);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        c[i] = (b4 ? a[i + 2] : a[i]) + __shfl_xor(b4 ? a[i] : a[i + 2], 16, kWave);
    float r = (b3 ? c[1] : c[0]) + __shfl_xor(b3 ? c[0] : c[1], 8, kWave);
    r += __shfl_xor(r, 4, kWave);
    r += __shfl_xor(r, 2, kWave);
    r += __shfl_xor(r, 1, kWave);
    return r;
}

// grid: persistent, kHdWaves waves per workgroup; TT tokens per pass.
template <int TT>
__global__ __launch_bounds__(kHdWaves * kWave) void head_q6k_kernel(
    const float* __restrict__ x, const uint8_t* __restrict__ W, int64_t V,
    float* __restrict__ logits) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t* buf = smem + wave * kHdSlot;
    constexpr int64_t H = kHdNB * kQK;

    // the lane's unit and its activations (fixed for the whole kernel)
    const int b = lane >> 3, n = (lane >> 2) & 1, r = lane & 3;
    HeadX X[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) X[t] = head_x_unit(x + t * H + 256 * b + 128 * n + 32 * r);
    const int ls = 4 * (r >> 1), hs = 2 * r;
    const int qlo = 64 * n + 32 * (r & 1), qho = 128 + 32 * n, sco = 192 + 8 * n + 2 * r;

    const int64_t ngroups = (V + kHdRows - 1) / kHdRows;
    const int64_t gstride = (int64_t)gridDim.x * kHdWaves;
    int64_t g = (int64_t)blockIdx.x * kHdWaves + wave;
    uint4 pre[kHdLoads];
    auto load = [&](int64_t gg) {
        const int64_t rows = V - gg * kHdRows < kHdRows ? V - gg * kHdRows : kHdRows;
        const int nch = (int)(rows * kHdRowB / 16);
        const uint8_t* src = W + gg * kHdGrpB;
#pragma unroll
        for (int i = 0; i < kHdLoads; ++i) {
            const int c = lane + i * kWave;
            const int cc = c < nch ? c : nch - 1;          // clamped: no branch, no stray address
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + 16 * cc));
            pre[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    if (g < ngroups) load(g);
    for (; g < ngroups; g += gstride) {
#pragma unroll
        for (int i = 0; i < kHdLoads; ++i) {
            const int c = lane + i * kWave;
            if (c < kHdChunks) *reinterpret_cast<uint4*>(buf + 16 * c) = pre[i];
        }
        if (g + gstride < ngroups) load(g + gstride);
        float acc[TT][kHdRows];
#pragma unroll
        for (int rho = 0; rho < kHdRows; ++rho) {
            const int boff = rho * kHdRowB + b * kQ6KBytes;
            const uint4 l0 = lds_read16_a2(buf, boff + qlo), l1 = lds_read16_a2(buf, boff + qlo + 16);
            const uint4 h0 = lds_read16_a2(buf, boff + qho), h1 = lds_read16_a2(buf, boff + qho + 16);
            const uint32_t L[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            const uint32_t Hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            uint32_t q[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                q[k] = ((L[k] >> ls) & 0x0f0f0f0fu) | (((Hh[k] >> hs) & 0x03030303u) << 4);
            const uint32_t scw = *reinterpret_cast<const uint16_t*>(buf + boff + sco);
            const float s0 = (float)(int8_t)(scw & 0xffu), s1 = (float)(int8_t)(scw >> 8);
            const float d = half_bits_to_float(*reinterpret_cast<const uint16_t*>(buf + boff + 208));
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                int a1 = 0, a2 = 0, a3 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a1 = sdot4(q[k], X[t].p[0][k], a1);
                    a2 = sdot4(q[k], X[t].p[1][k], a2);
                    a3 = sdot4(q[k], X[t].p[2][k], a3);
                    c1 = sdot4(q[k + 4], X[t].p[0][k + 4], c1);
                    c2 = sdot4(q[k + 4], X[t].p[1][k + 4], c2);
                    c3 = sdot4(q[k + 4], X[t].p[2][k + 4], c3);
                }
                const int A = (a1 - 32 * X[t].ps[0][0]) * 16384 + (a2 - 32 * X[t].ps[1][0]) * 128 +
                              (a3 - 32 * X[t].ps[2][0]);
                const int C = (c1 - 32 * X[t].ps[0][1]) * 16384 + (c2 - 32 * X[t].ps[1][1]) * 128 +
                              (c3 - 32 * X[t].ps[2][1]);
                acc[t][rho] = d * (s0 * (float)A + s1 * (float)C) * X[t].sx;
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float y = fold8(acc[t], lane);
            const int64_t row = g * kHdRows + (lane >> 3);
            if ((lane & 7) == 0 && row < V) logits[t * V + row] = y;
        }
    }
}

int cu_count_now() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

}  // namespace

hipError_t launch_embed(const int32_t* tokens, int64_t T, const uint8_t* table, int32_t qtype,
                        int64_t V, int64_t H, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)T), dim3(kEmbThreads), 0, stream, tokens, table,
                       qtype, V, H, out);
    return hipGetLastError();
}

bool output_head_supported(int64_t H, int32_t qtype) { return H == kHdNB * kQK && qtype == 2; }

hipError_t launch_output_head(const float* x, int64_t T, const uint8_t* W, int64_t V, float* logits,
                              hipStream_t stream) {
    const int64_t ngroups = (V + kHdRows - 1) / kHdRows;
    const int cus = cu_count_now();
    int64_t grid = (ngroups + kHdWaves - 1) / kHdWaves;
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * 2;
    if (grid > cap) grid = cap;
    const size_t lds = (size_t)kHdWaves * kHdSlot;
    for (int64_t t0 = 0; t0 < T;) {
        const int64_t tt = T - t0 >= 2 ? 2 : 1;
        if (tt == 2)
            hipLaunchKernelGGL(head_q6k_kernel<2>, dim3((unsigned)grid), dim3(kHdWaves * kWave), lds,
                               stream, x + t0 * kHdNB * kQK, W, V, logits + t0 * V);
        else
            hipLaunchKernelGGL(head_q6k_kernel<1>, dim3((unsigned)grid), dim3(kHdWaves * kWave), lds,
                               stream, x + t0 * kHdNB * kQK, W, V, logits + t0 * V);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        t0 += tt;
    }
    return hipSuccess;
}

}  // namespace q3moe
