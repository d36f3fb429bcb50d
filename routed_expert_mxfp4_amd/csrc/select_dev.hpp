// select_dev.hpp -- wave-level top-k selection and softmax (device code).
//
// One wave selects the k largest of E <= 64*PL logits of one token: larger
// logit first, lower expert index first among equal logits (the layer's tie
// rule), then a softmax over the k selected logits in fp64 (no extra
// scaling).  Lane l holds experts l, l+64, ...
//
// Each round takes the wave maximum of an order-preserving 32-bit key of the
// lane-local best logit, then the minimum expert index among the lanes that
// hold that key.  Both reductions rotate within rows of 16 lanes with DPP
// (cheap VALU moves) and combine the four rows through scalar registers.
#pragma once

#include "moe_internal.hpp"

namespace moe {

// DPP row_ror:n (rotate right by n within each row of 16 lanes).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_ror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x120 + N, 0xF, 0xF, false);
}

// Wave max / min: rotate within rows of 16 (all lanes of a row end with the
// row's result), then combine the four rows from lanes 0, 16, 32, 48 with
// readlane; the result is wave-uniform (scalar registers).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_row_ror<8>(v));
    v = max(v, dpp_row_ror<4>(v));
    v = max(v, dpp_row_ror<2>(v));
    v = max(v, dpp_row_ror<1>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp_row_ror<8>(v));
    v = min(v, dpp_row_ror<4>(v));
    v = min(v, dpp_row_ror<2>(v));
    v = min(v, dpp_row_ror<1>(v));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return min(min(a, b), min(c, d));
}

// Order-preserving key of a logit: a > b (as floats) <=> key(a) > key(b).
// -0 is folded into +0 (equal as floats) and NaN ranks with -inf.  Keys of
// real logits are >= key(-inf) = 0x007FFFFF, so 0 marks "taken".
__device__ __forceinline__ uint32_t logit_key(float v) {
    if (v != v) v = -INFINITY;
    if (v == 0.0f) v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// LDS scratch of one wave for wave_topk_softmax (uint32 words, 16-byte
// aligned): candidate keys at 64.., their experts at 128.., spare write
// targets at 192 and 193.
constexpr int kTopkScratch = 196;

// Sum of a double over lanes 0..31 (lanes past them are ignored): rotations
// within rows of 16 lanes, then rows 0 and 1 through scalar registers.
__device__ __forceinline__ double sum_lanes32_f64(double v) {
#pragma unroll
    for (int r = 8; r >= 1; r >>= 1) {
        const unsigned long long u = __double_as_longlong(v);
        int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
        if (r == 8) {
            lo = __builtin_amdgcn_update_dpp(lo, lo, 0x128, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(hi, hi, 0x128, 0xF, 0xF, false);
        } else if (r == 4) {
            lo = __builtin_amdgcn_update_dpp(lo, lo, 0x124, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(hi, hi, 0x124, 0xF, 0xF, false);
        } else if (r == 2) {
            lo = __builtin_amdgcn_update_dpp(lo, lo, 0x122, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(hi, hi, 0x122, 0xF, 0xF, false);
        } else {
            lo = __builtin_amdgcn_update_dpp(lo, lo, 0x121, 0xF, 0xF, false);
            hi = __builtin_amdgcn_update_dpp(hi, hi, 0x121, 0xF, 0xF, false);
        }
        v += __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) |
                                               (uint32_t)lo));
    }
    const unsigned long long u = __double_as_longlong(v);
    const uint32_t lo0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 0);
    const uint32_t hi0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 0);
    const uint32_t lo1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 16);
    const uint32_t hi1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 16);
    return __longlong_as_double((long long)(((unsigned long long)hi0 << 32) | lo0)) +
           __longlong_as_double((long long)(((unsigned long long)hi1 << 32) | lo1));
}

// C <= 64 candidates, one per lane (lane < C: key ka, expert ea; other
// lanes key 0, expert ~0): each one's rank in (key descending, expert
// ascending) order is counted against the others, whose keys come by
// readlane, and the lane of rank r < k receives its expert and logit with
// one ds_permute.
__device__ __forceinline__ void wave_rank_select(uint32_t ka, uint32_t ea, int C, int k,
                                                 int *my_e, float *my_v) {
    const int lane = threadIdx.x & 63;
    int rank = 0;
    for (int j0 = 0; j0 < C; j0 += 4) {               // four independent compares a pass
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = min(j0 + q, C - 1);
            const uint32_t kb = (uint32_t)__builtin_amdgcn_readlane((int)ka, j);
            const uint32_t eb = (uint32_t)__builtin_amdgcn_readlane((int)ea, j);
            rank += (j0 + q < C && (kb > ka || (kb == ka && eb < ea))) ? 1 : 0;
        }
    }
    // a permutation: candidates go to their rank (< C), the others stay
    const int tgt = lane < C ? rank : lane;
    const uint32_t se = (uint32_t)__builtin_amdgcn_ds_permute(tgt << 2, (int)ea);
    const uint32_t sk = (uint32_t)__builtin_amdgcn_ds_permute(tgt << 2, (int)ka);
    if (lane < k) {
        *my_e = (int)se;
        *my_v = key_logit(sk);
    }
}

// Softmax over the k selected logits (lane j < k holds the j-th, descending):
// exp(v - v_0) in fp64, summed over lanes 0..31 in a fixed order, one
// division and one rounding per weight.
__device__ __forceinline__ void wave_softmax_tail(int my_e, float my_v, int k, int *sel_e,
                                                  float *sel_w) {
    const int lane = threadIdx.x & 63;
    const double vmax = (double)__shfl(my_v, 0, 64);
    const double ex = lane < k ? exp((double)my_v - vmax) : 0.0;
    const double sum = sum_lanes32_f64(ex);
    *sel_e = my_e;
    *sel_w = (float)(ex / sum);
}

// Selects the top-k (k <= 32) of one token's logits row.  On return lane
// j < k holds the j-th selected expert in *sel_e and its weight in *sel_w.
// sc: this wave's kTopkScratch words of LDS.
//
// tau is a lower bound of the k-th largest of the 64 lane maxima: the
// largest t with #{lanes : lmax >= t} >= k among the keys whose low 16 bits
// are zero (bisection on the top 16 bits, one ballot per bit).  The k-th
// largest lane maximum is at most the k-th largest key (those k lane maxima
// are k distinct keys), so every selected expert has key >= tau.  The keys
// >= tau (k and a few more on real logits) are gathered -- each lane's
// count, a prefix sum over the wave from one ballot per count bit, then
// branch-free LDS writes -- and each one's rank in (key descending, expert
// ascending) order is counted against the others, whose keys come by
// readlane.  The lane of rank r hands its candidate to lane r with one
// ds_permute.  If more than 64 keys lie at or above tau (massive ties), k
// rounds of wave-wide max/min select instead.
template <int PL>
__device__ __forceinline__ void wave_topk_softmax(const float *__restrict__ row, int E, int k,
                                                  uint32_t *sc, int *sel_e, float *sel_w) {
    const int lane = threadIdx.x & 63;
    uint32_t key[PL];
    float v[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) v[i] = row[min(lane + 64 * i, E - 1)];   // all loads first
#pragma unroll
    for (int i = 0; i < PL; ++i) key[i] = lane + 64 * i < E ? logit_key(v[i]) : 0u;
    float my_v = 0.f;
    int my_e = 0;
    uint32_t lmax = 0u;
#pragma unroll
    for (int i = 0; i < PL; ++i) lmax = max(lmax, key[i]);
    uint32_t tau = 0u;
#pragma unroll 1
    for (int bit = 31; bit >= 16; --bit) {
        const uint32_t t = tau | (1u << bit);
        if ((int)__popcll(__ballot(lmax >= t)) >= k) tau = t;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) cnt += (key[i] != 0u && key[i] >= tau) ? 1 : 0;
    int base = 0, C = 0;                            // exclusive prefix of cnt, total
#pragma unroll
    for (int b = 0; (1 << b) <= PL; ++b) {
        const unsigned long long m = __ballot((cnt >> b) & 1);
        base += (int)__popcll(m & below) << b;
        C += (int)__popcll(m) << b;
    }
    if (C <= 64) {
        int p = base;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const bool c = key[i] != 0u && key[i] >= tau;
            sc[c ? 64 + p : 192] = key[i];
            sc[c ? 128 + p : 193] = (uint32_t)(lane + 64 * i);
            p += c ? 1 : 0;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the writes have landed
        __builtin_amdgcn_wave_barrier();
        const uint32_t ka = lane < C ? sc[64 + lane] : 0u;
        const uint32_t ea = lane < C ? sc[128 + lane] : 0xFFFFFFFFu;
        wave_rank_select(ka, ea, C, k, &my_e, &my_v);
    } else {
        for (int j = 0; j < k; ++j) {
            uint32_t bk = 0u;
            int bi = 0;
#pragma unroll
            for (int i = 0; i < PL; ++i)          // ascending e: ties keep the lower e
                if (key[i] > bk) {
                    bk = key[i];
                    bi = i;
                }
            const uint32_t gk = wave_max_u32(bk);
            const uint32_t cand = (bk == gk) ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu;
            const uint32_t ge = wave_min_u32(cand);
            if ((int)(ge & 63u) == lane) {
                const int gi = (int)(ge >> 6);
#pragma unroll
                for (int i = 0; i < PL; ++i)
                    if (i == gi) key[i] = 0u;
            }
            if (lane == j) {
                my_e = (int)ge;
                my_v = key_logit(gk);
            }
        }
    }
    wave_softmax_tail(my_e, my_v, k, sel_e, sel_w);
}

}  // namespace moe
