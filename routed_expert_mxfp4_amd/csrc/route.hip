// route.hip -- router logits (canonical fp64 order), wave-level top-k and
// softmax over the selected logits, for gfx950.
//
// Canonical logit (the pages name the router, not its arithmetic): the d
// inputs are split into 64 equal chunks; lane c of a wave sums chunk c in
// fp64 in ascending order (each bf16*bf16 product is exact in fp64, so an
// fma equals the separate multiply and add); the 64 chunk sums are combined
// by xor-butterfly levels of width 1, 2, ..., 32, which adds exactly the
// pairs (0,1),(2,3),... then ((0,1),(2,3)),... of a fixed pairwise tree;
// the bias is added in fp64 and the result rounded once to fp32.
//
// Top-k: descending logit, lower expert index first on equal logits; the
// routing weights are a softmax over the k selected logits, no extra scale.
#include "moe_internal.hpp"

namespace moe {
namespace {

template <int VEC>
struct VecLoad;
template <>
struct VecLoad<8> {
    __device__ static void load(const uint16_t *p, uint32_t (&v)[4]) {
        uint4 q = *reinterpret_cast<const uint4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <>
struct VecLoad<4> {
    __device__ static void load(const uint16_t *p, uint32_t (&v)[4]) {
        uint2 q = *reinterpret_cast<const uint2 *>(p);
        v[0] = q.x; v[1] = q.y;
    }
};
template <>
struct VecLoad<2> {
    __device__ static void load(const uint16_t *p, uint32_t (&v)[4]) {
        v[0] = *reinterpret_cast<const uint32_t *>(p);
    }
};
template <>
struct VecLoad<1> {
    __device__ static void load(const uint16_t *p, uint32_t (&v)[4]) { v[0] = p[0]; }
};

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xFFFF0000u); }

// One wave (64 lanes) computes TT tokens x TE experts.  Lane c owns chunk c
// (P = d/64 consecutive inputs) of every token and expert row in the tile.
template <int TT, int TE, int VEC>
__global__ __launch_bounds__(64) void router_logits_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int d, int E) {
    const int lane = threadIdx.x;
    const int e0 = blockIdx.x * TE;
    const int t0 = blockIdx.y * TT;
    const int P = d >> 6;
    const uint16_t *xr[TT];
    const uint16_t *wrow[TE];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
        int t = min(t0 + i, T - 1);                  // padding rows: discarded
        xr[i] = x + (size_t)t * d + (size_t)lane * P;
    }
#pragma unroll
    for (int j = 0; j < TE; ++j) {
        int e = min(e0 + j, E - 1);
        wrow[j] = wr + (size_t)e * d + (size_t)lane * P;
    }
    double acc[TT][TE];
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) acc[i][j] = 0.0;

    for (int p = 0; p < P; p += VEC) {
        uint32_t xv[TT][4], wv[TE][4];
#pragma unroll
        for (int i = 0; i < TT; ++i) VecLoad<VEC>::load(xr[i] + p, xv[i]);
#pragma unroll
        for (int j = 0; j < TE; ++j) VecLoad<VEC>::load(wrow[j] + p, wv[j]);
#pragma unroll
        for (int q = 0; q < VEC; ++q) {              // ascending element order
#pragma unroll
            for (int i = 0; i < TT; ++i) {
                double xe = (q & 1) ? bf16_hi(xv[i][q >> 1]) : bf16_lo(xv[i][q >> 1]);
#pragma unroll
                for (int j = 0; j < TE; ++j) {
                    double we = (q & 1) ? bf16_hi(wv[j][q >> 1]) : bf16_lo(wv[j][q >> 1]);
                    acc[i][j] = fma(xe, we, acc[i][j]);
                }
            }
        }
    }
    // fixed pairwise tree over the 64 chunk sums
#pragma unroll
    for (int w = 1; w < 64; w <<= 1)
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int j = 0; j < TE; ++j) acc[i][j] += __shfl_xor(acc[i][j], w, 64);

#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int t = t0 + i, e = e0 + j;
            if (lane == i * TE + j && t < T && e < E) {
                double l = acc[i][j] + (bias ? (double)bias[e] : 0.0);
                logits[(size_t)t * E + e] = (float)l;       // one RNE rounding
            }
        }
}

template <int TT, int TE>
hipError_t launch_logits_tile(const uint16_t *x, const uint16_t *wr, const float *bias,
                              float *logits, int T, int d, int E, hipStream_t s) {
    dim3 grid((E + TE - 1) / TE, (T + TT - 1) / TT);
    const int P = d / 64;
    if (P % 8 == 0)
        router_logits_kernel<TT, TE, 8><<<grid, 64, 0, s>>>(x, wr, bias, logits, T, d, E);
    else if (P % 4 == 0)
        router_logits_kernel<TT, TE, 4><<<grid, 64, 0, s>>>(x, wr, bias, logits, T, d, E);
    else if (P % 2 == 0)
        router_logits_kernel<TT, TE, 2><<<grid, 64, 0, s>>>(x, wr, bias, logits, T, d, E);
    else
        router_logits_kernel<TT, TE, 1><<<grid, 64, 0, s>>>(x, wr, bias, logits, T, d, E);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// top-k + softmax: one wave per token; lane l holds experts l, l+64, ...
// ---------------------------------------------------------------------------
struct Cand {
    float v;
    int e;
};

__device__ __forceinline__ bool better(float va, int ea, float vb, int eb) {
    return va > vb || (va == vb && ea < eb);
}

template <int PL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ logits,
                                                           int32_t *__restrict__ ids,
                                                           float *__restrict__ w, int T,
                                                           int E, int k) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[PL];
    const float *row = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        int e = lane + 64 * i;
        float a = e < E ? row[e] : -INFINITY;
        v[i] = (a != a) ? -INFINITY : a;             // NaN ranks lowest
    }
    uint32_t taken = 0;
    float my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off, 64);
            int oe = __shfl_xor(be, off, 64);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }
    // softmax over the selected logits (fp64), max = the first selected
    double vmax = (double)__shfl(my_v, 0, 64);
    double ex = lane < k ? exp((double)my_v - vmax) : 0.0;
    double sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = (float)(ex / sum);
    }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias,
                                float *logits, int T, int d, int E, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (T < 4) return launch_logits_tile<1, 4>(x, wr, bias, logits, T, d, E, s);
    return launch_logits_tile<4, 8>(x, wr, bias, logits, T, d, E, s);
}

hipError_t launch_topk_softmax(const float *logits, int32_t *ids, float *w, int T, int E,
                               int k, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    const int pl = (E + 63) / 64;
    if (pl <= 4)
        topk_softmax_kernel<4><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
    else if (pl <= 8)
        topk_softmax_kernel<8><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
    else
        topk_softmax_kernel<16><<<grid, 256, 0, s>>>(logits, ids, w, T, E, k);
    return hipGetLastError();
}

}  // namespace moe
