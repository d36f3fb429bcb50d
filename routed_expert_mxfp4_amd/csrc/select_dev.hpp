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
// aligned).
constexpr int kTopkScratch = 192;

// Selects the top-k (k <= 32) of one token's logits row.  On return lane
// j < k holds the j-th selected expert in *sel_e and its weight in *sel_w.
// sc: this wave's kTopkScratch words of LDS.
//
// tau, the k-th largest of the 64 lane maxima (found by bisection on the
// key), is at most the k-th largest key: those k lane maxima are k distinct
// keys >= tau.  So every selected expert has key >= tau.  The keys >= tau
// (about k + a few on real logits) are gathered and each one's rank in (key
// descending, expert ascending) order is counted against the others.  If
// more than 64 keys lie at or above tau (massive ties), k rounds of
// wave-wide max/min select instead.
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
    // tau = the largest t with #{lanes : lmax >= t} >= k, by bisection on
    // the key (each step one compare whose result is the ballot)
    uint32_t tau = 0u;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = tau | (1u << bit);
        if ((int)__popcll(__ballot(lmax >= t)) >= k) tau = t;
    }
    int C = 0;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const bool c = key[i] != 0u && key[i] >= tau;
        const unsigned long long m = __ballot(c);
        const int pos = C + (int)__popcll(m & below);
        if (c && pos < 64) {
            sc[64 + pos] = key[i];
            sc[128 + pos] = (uint32_t)(lane + 64 * i);
        }
        C += (int)__popcll(m);
    }
    if (C <= 64) {
        int rank = 64;
        uint32_t ka = 0u, ea = 0u;
        const uint4 *sc4 = reinterpret_cast<const uint4 *>(sc);
        if (lane < C) {
            ka = sc[64 + lane];
            ea = sc[128 + lane];
            rank = 0;
        }
        // candidates past C are ignored (keys there may be stale)
#pragma unroll
        for (int j4 = 0; j4 < 16; ++j4) {
            if (4 * j4 < C) {
                const uint4 kb4 = sc4[16 + j4], eb4 = sc4[32 + j4];
                const uint32_t kb[4] = {kb4.x, kb4.y, kb4.z, kb4.w};
                const uint32_t eb[4] = {eb4.x, eb4.y, eb4.z, eb4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    rank += (4 * j4 + q < C && (kb[q] > ka || (kb[q] == ka && eb[q] < ea))) ? 1 : 0;
            }
        }
        if (lane >= C) rank = 64;
        if (rank < k) {
            sc[rank] = ea;
            sc[32 + rank] = ka;
        }
        if (lane < k) {
            my_e = (int)sc[lane];
            my_v = key_logit(sc[32 + lane]);
        }
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
    const double vmax = (double)__shfl(my_v, 0, 64);
    const double ex = lane < k ? exp((double)my_v - vmax) : 0.0;
    double sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    *sel_e = my_e;
    *sel_w = (float)(ex / sum);
}

}  // namespace moe
