// Wave-level pieces of the routing step shared by the route kernels and the
// fused route + expert-FFN kernel: double-precision wave reductions over DPP
// and the top-k selection with renormalised softmax weights (aprender issue
// #3714, gap G3: the top-8 over the 128 router logits; equal logits go to the
// lower expert index).
#pragma once

#include "device_common.h"

namespace q3moe {

// Lane `src` (wave-uniform) of a double.
__device__ __forceinline__ double readlane_f64(double v, int src) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// A double moved across lanes by a DPP pattern (both halves; lanes without a
// source keep their own value).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
    const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xf, 0xf, false);
    const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)nhi << 32) | nlo);
}
constexpr int kDppQuadXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// Wave-wide max / sum of a double, uniform in every lane: DPP inside each row
// of 16 lanes, then the four row results combined in a fixed order.  No LDS
// round trips on the dependent chain.
__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<kDppQuadXor1>(v));
    v = fmax(v, dpp_f64<kDppQuadXor2>(v));
    v = fmax(v, dpp_f64<kDppRowRor4>(v));
    v = fmax(v, dpp_f64<kDppRowRor8>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)),
                fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

__device__ __forceinline__ double wave_sum_dpp_f64(double v) {
    v += dpp_f64<kDppQuadXor1>(v);
    v += dpp_f64<kDppQuadXor2>(v);
    v += dpp_f64<kDppRowRor4>(v);
    v += dpp_f64<kDppRowRor8>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// An unsigned key with the selection order below on doubles: larger values
// give larger keys, -0 and +0 the same key, NaN the smallest key (0) below
// every number.  With ties broken by the lower index this is a strict total
// order.
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v == 0.0 ? 0.0 : v);
    const uint64_t k = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return v != v ? 0ull : k;
}

// Wave-wide max of a float, uniform in every lane (DPP within rows of 16,
// then the four row results).
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadXor1, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadXor2, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor4, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor8, 0xf, 0xf, false)));
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// One wave: top-k and weights of one token whose logits lane e % 64 holds in
// v[e / 64] (experts beyond E are never chosen).  Order: the larger logit
// first, every number before NaN, equal logits (and NaNs) by the lower
// expert index.  Each of the k rounds screens with the logits rounded to f32
// (a wave maximum over DPP), which keeps every lane whose f32 value equals
// the maximum as a candidate: rounding is monotonic, so the true winner is
// among them.  A single candidate wins outright; several are compared on
// their exact order keys, lowest index first.  Weights: the softmax over the
// selected logits in double, the first selected logit subtracted, normalised
// by their sum in rank order, rounded to f32.  Writes idx[0..k), w[0..k).
template <int NPER>
__device__ __forceinline__ void topk_wave(const double v_in[NPER], int32_t E, int32_t k,
                                          int lane, int32_t* __restrict__ idx,
                                          float* __restrict__ w) {
    float f[NPER];
    uint64_t key[NPER];
    bool live[NPER];
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
        live[j] = lane + kWave * j < E;
        f[j] = v_in[j] != v_in[j] ? -__builtin_inff() : (float)v_in[j];   // NaN screens as -inf
        key[j] = order_key(v_in[j]);
    }
    double my_v = 0.0, top = 0.0;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
        float lm = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < NPER; ++j)
            if (live[j]) lm = fmaxf(lm, f[j]);
        const float m = wave_max_f32(lm);
        uint64_t cand[NPER];
        int ncand = 0, win = -1;
#pragma unroll
        for (int j = 0; j < NPER; ++j) {
            cand[j] = __ballot(live[j] && f[j] == m);
            ncand += __builtin_popcountll(cand[j]);
            if (win < 0 && cand[j]) win = kWave * j + __builtin_ctzll(cand[j]);
        }
        if (ncand > 1) {
            // exact: the largest key among the candidates, lowest index first
            uint64_t best = 0;
            win = -1;
#pragma unroll
            for (int j = 0; j < NPER; ++j) {
                for (uint64_t c = cand[j]; c; c &= c - 1) {
                    const int l = __builtin_ctzll(c);
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[j], l);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key[j] >> 32), l);
                    const uint64_t kk = ((uint64_t)hi << 32) | lo;
                    if (win < 0 || kk > best) {
                        best = kk;
                        win = kWave * j + l;
                    }
                }
            }
        }
        double val = 0.0;
#pragma unroll
        for (int j = 0; j < NPER; ++j)
            if (win >> 6 == j) val = readlane_f64(v_in[j], win & 63);
        if (r == 0) top = val;
        if (lane == r) {
            my_v = val;
            my_i = win;
        }
#pragma unroll
        for (int j = 0; j < NPER; ++j)
            if (lane + kWave * j == win) live[j] = false;
    }
    // lane r < k holds rank r; normaliser summed in rank order
    const double ex = lane < k ? exp(my_v - top) : 0.0;
    double den = 0.0;
    for (int r = 0; r < k; ++r)
        den += readlane_f64(ex, r);
    if (lane < k) {
        idx[lane] = my_i;
        w[lane] = (float)(ex / den);
    }
}

// order_key's screen in 32 bits: the same order on the logits rounded to f32
// (monotonic, so a strictly larger screen key means a strictly larger logit).
__device__ __forceinline__ uint32_t order_key32(double v) {
    const float f = (float)v;
    const uint32_t b = __float_as_uint(f == 0.f ? 0.f : f);
    const uint32_t k = (b >> 31) ? ~b : (b | 0x80000000u);
    return v != v ? 0u : k;
}

// The top-k of T tokens' logits by rank counting, with every thread of the
// workgroup: lg[t*E + e] holds the logits, key[] their order_key and key32[]
// their order_key32 (all in LDS).  4 consecutive threads count, over every
// fourth expert each, how many experts rank above expert e of
// token t: every larger screen key counts, equal screen keys are decided on
// the exact keys and indices.  The expert whose count c is below k is the
// token's rank-c choice (sel_idx/sel_val[t*k + c] in LDS).  The same
// choices as topk_wave, with the work spread over the workgroup.
template <int kThr>
__device__ __forceinline__ void topk_rank_select(const double* lg, const uint64_t* key,
                                                 const uint32_t* key32, int T, int E, int k,
                                                 int tid, int32_t* sel_idx, double* sel_val) {
    const int units = T * E * 4;
    for (int u0 = 0; u0 < units; u0 += kThr) {
        const int u = u0 + tid;
        const bool act = u < units;
        const int item = act ? (u >> 2) : 0, qtr = u & 3;
        const int t = item / E, e = item % E;
        const uint32_t* row = key32 + t * E;
        const uint32_t me = row[e];
        // quarter q takes the keys j = q + 4i (four banks per read step)
        const int nj = (E - qtr + 3) >> 2;
        const uint32_t* rq = row + qtr;
        int gt = 0, ge = 0;
        int i = 0;
        for (; i + 8 <= nj; i += 8) {                   // 8 reads in flight, no branches
            uint32_t kj[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) kj[m] = rq[4 * (i + m)];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                gt += (int)(kj[m] > me);
                ge += (int)(kj[m] >= me);
            }
        }
        for (; i < nj; ++i) {
            const uint32_t kj = rq[4 * i];
            gt += (int)(kj > me);
            ge += (int)(kj >= me);
        }
        // equal screen keys other than e itself: decide those exactly
        const bool self_here = (e & 3) == qtr;
        if (__any(ge - gt > (self_here ? 1 : 0))) {
            const uint64_t* krow = key + t * E;
            const uint64_t mk = krow[e];
            int tie = 0;
            for (int jj = qtr; jj < E; jj += 4) {
                const uint64_t kj = krow[jj];
                tie += (row[jj] == me && jj != e && (kj > mk || (kj == mk && jj < e))) ? 1 : 0;
            }
            gt += tie;
        }
        int cnt = gt;
        cnt += __shfl_xor(cnt, 1, kWave);
        cnt += __shfl_xor(cnt, 2, kWave);
        if (act && qtr == 0 && cnt < k) {
            sel_idx[t * k + cnt] = e;
            sel_val[t * k + cnt] = lg[t * E + e];
        }
    }
}

// The same selection when no two of the chosen screen keys are equal, at
// half the comparisons: 4 consecutive threads count, over every fourth
// expert each, only the experts whose screen key is strictly larger than
// expert e's.  Distinct screen keys order the logits exactly (rounding is
// monotonic), so an expert whose count c is below k is the token's rank-c
// choice; it also adds one to slot c's counter (slot_cnt, zero on entry).
// Equal screen keys at or above the k-th place give two experts the same
// count, so some slot counter ends other than 1; the caller then runs
// topk_rank_select, which decides equal screen keys exactly.
template <int kThr>
__device__ __forceinline__ void topk_rank_screen(const double* lg, const uint32_t* key32, int T,
                                                 int E, int k, int tid, int32_t* sel_idx,
                                                 double* sel_val, int32_t* slot_cnt) {
    const int units = T * E * 4;
    for (int u0 = 0; u0 < units; u0 += kThr) {
        const int u = u0 + tid;
        const bool act = u < units;
        const int item = act ? (u >> 2) : 0, qtr = u & 3;
        const int t = T == 1 ? 0 : item / E, e = item - t * E;
        const uint32_t* row = key32 + t * E;
        const uint32_t me = row[e];
        int gt = 0;
        if ((E & 15) == 0) {
            // quarter q takes the 4-key chunks j = 16i + 4q + c: at every
            // step the four quarters of a wave read four consecutive 16-byte
            // chunks (16 banks, each read broadcast to its 16 lanes)
            const uint4* rq = reinterpret_cast<const uint4*>(row) + qtr;
            const int nb = E >> 4;
            int i = 0;
            for (; i + 8 <= nb; i += 8) {               // 8 reads (32 keys) in flight, no branches
                uint4 kj[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) kj[m] = rq[4 * (i + m)];
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    gt += (int)(kj[m].x > me) + (int)(kj[m].y > me) + (int)(kj[m].z > me) +
                          (int)(kj[m].w > me);
            }
            for (; i < nb; ++i) {
                const uint4 kv = rq[4 * i];
                gt += (int)(kv.x > me) + (int)(kv.y > me) + (int)(kv.z > me) + (int)(kv.w > me);
            }
        } else {
            // quarter q takes the keys j = q + 4i (four consecutive words,
            // four banks, at every step of a wave); quarters of 32
            // consecutive keys would all fall in one bank
            const int nj = (E - qtr + 3) >> 2;
            const uint32_t* rq = row + qtr;
            int i = 0;
            for (; i + 8 <= nj; i += 8) {               // 8 reads in flight, no branches
                uint32_t kj[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) kj[m] = rq[4 * (i + m)];
#pragma unroll
                for (int m = 0; m < 8; ++m) gt += (int)(kj[m] > me);
            }
            for (; i < nj; ++i) gt += (int)(rq[4 * i] > me);
        }
        // the 4 quarter counts of an expert sit in one quad of lanes
        int cnt = gt + __builtin_amdgcn_update_dpp(0, gt, kDppQuadXor1, 0xf, 0xf, false);
        cnt += __builtin_amdgcn_update_dpp(0, cnt, kDppQuadXor2, 0xf, 0xf, false);
        if (act && qtr == 0 && cnt < k) {
            sel_idx[t * k + cnt] = e;
            sel_val[t * k + cnt] = lg[t * E + e];
            __hip_atomic_fetch_add(slot_cnt + t * k + cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

}  // namespace q3moe
