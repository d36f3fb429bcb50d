// tail.hip -- the MoE tail around the routed layer on gfx950: the RMSNorm
// that feeds the router and the experts, and the shared expert for few
// tokens (for many tokens its GEMMs are in shared_gemm.hip).
//
// The pages' model-shape MoE tail is the weighted reduction, RMSNorm, the
// routed-up activation quantisation and the residual adds (Moonshine README,
// "Run layer-major prefill"); shared experts and norms are in the bf16/Q8
// static tier beside the routers, not in the MXFP4 expert store (Moonshine
// README, "How the engine works", tier diagram).
//
// Block: xn = RMSNorm(x) * gamma (bf16); out = x + routed(xn) + shared(xn),
// shared(xn) = W_dn (silu(W_gate xn) * (W_up xn)) with bf16 weights.
#include "moe_internal.hpp"

namespace moe {
namespace {

// fp64 -> bf16 bits, round to nearest even, straight from fp64 (no fp32
// step, which could round twice).  Normal range: drop the 45 low fraction
// bits with a nearest-even carry (the carry may ripple into the exponent);
// the result has 8 significant bits and converts to fp32 exactly (or is
// >= 2^128: infinity).  Below 2^-126 the bf16 grid is the multiples of
// 2^-133: scale by 2^133 (exact), round to an integer (nearest even), scale
// back.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return (uint16_t)(sign | 0x7FC0u);    // NaN
    if (a >= 0x3810000000000000ull) {                                     // |v| >= 2^-126
        uint64_t r = a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1ull);
        r &= ~0x00001FFFFFFFFFFFull;
        if (r >= 0x47F0000000000000ull) return (uint16_t)(sign | 0x7F80u); // >= 2^128
        const float fv = (float)__longlong_as_double((long long)r);
        return (uint16_t)(sign | (__float_as_uint(fv) >> 16));
    }
    const double q = rint(__longlong_as_double((long long)a) * 0x1p133);
    const float fv = (float)(q * 0x1p-133);
    return (uint16_t)(sign | (__float_as_uint(fv) >> 16));
}

__device__ __forceinline__ double bf16_to_f64(uint32_t b) {
    return (double)__uint_as_float(b << 16);
}

// Sum of squares of one lane's chunk (P consecutive bf16 at c), in fp64 in
// ascending order (v * v is exact in fp64).  P % 8 == 0: 16-byte loads,
// four in flight; else element by element.
__device__ __forceinline__ double chunk_sumsq(const uint16_t *c, int P) {
    double s = 0.0;
    if ((P & 7) == 0) {
        const uint4 *q = reinterpret_cast<const uint4 *>(c);
        const int n = P >> 3;
        int j = 0;
        for (; j + 4 <= n; j += 4) {
            const uint4 w4[4] = {q[j], q[j + 1], q[j + 2], q[j + 3]};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t w[4] = {w4[r].x, w4[r].y, w4[r].z, w4[r].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const double lo = bf16_to_f64(w[i] & 0xFFFFu), hi = bf16_to_f64(w[i] >> 16);
                    s = s + lo * lo;
                    s = s + hi * hi;
                }
            }
        }
        for (; j < n; ++j) {
            const uint4 w4 = q[j];
            const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const double lo = bf16_to_f64(w[i] & 0xFFFFu), hi = bf16_to_f64(w[i] >> 16);
                s = s + lo * lo;
                s = s + hi * hi;
            }
        }
    } else {
        for (int i = 0; i < P; ++i) {
            const double v = bf16_to_f64(c[i]);
            s = s + v * v;
        }
    }
    return s;
}

// Grid (T, S), one wave per block: block (t, s) normalises the s-th of S
// equal spans of row t (S > 1 spreads a few tokens over many CUs).  Every
// block first finds the row's sum of squares in the canonical order: lane c
// sums chunk c (d / 64 consecutive elements) in fp64, ascending, and
// xor-butterfly levels 1, 2, .., 32 add exactly the pairs of the fixed
// pairwise tree over the 64 chunk sums (addition is commutative, so both
// partners hold the same bits).  Then, in fp64: ms = ss / d,
// den = sqrt(ms + eps), xn_i = bf16((x_i / den) * gamma_i).  IEEE division
// and square root are correctly rounded, so the result does not depend on
// how the work is spread.
__global__ __launch_bounds__(64) void rmsnorm_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ gamma,
                                                     float eps, uint16_t *__restrict__ xn,
                                                     int d) {
    const int t = blockIdx.x, lane = threadIdx.x;
    const uint16_t *xrow = x + (size_t)t * d;
    const int P = d >> 6;
    double s = chunk_sumsq(xrow + (size_t)lane * P, P);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m, 64);
    const double ms = s / (double)d;
    const double den = sqrt(ms + (double)eps);
    const int nv = d >> 3, S = (int)gridDim.y;
    const int v0 = (int)(((long long)nv * blockIdx.y) / S);
    const int v1 = (int)(((long long)nv * (blockIdx.y + 1)) / S);
    const uint4 *xr = reinterpret_cast<const uint4 *>(xrow);
    const uint4 *gr = reinterpret_cast<const uint4 *>(gamma);
    uint4 *orow = reinterpret_cast<uint4 *>(xn + (size_t)t * d);
    for (int v = v0 + lane; v < v1; v += 64) {
        const uint4 xv = xr[v];
        const uint4 gv = gr[v];
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double lo = (bf16_to_f64(xw[i] & 0xFFFFu) / den) * bf16_to_f64(gw[i] & 0xFFFFu);
            const double hi = (bf16_to_f64(xw[i] >> 16) / den) * bf16_to_f64(gw[i] >> 16);
            ow[i] = (uint32_t)f64_to_bf16_rne(lo) | ((uint32_t)f64_to_bf16_rne(hi) << 16);
        }
        orow[v] = uint4{ow[0], ow[1], ow[2], ow[3]};
    }
}

__device__ __forceinline__ float dot8_bf16(uint4 w, uint4 xv, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                          __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                          __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                          __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                          __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    return acc;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Shared expert gate/up for NT <= 8 tokens: one wave per pair (gate row n,
// up row fs + n), both rows streamed once with 16-byte loads (a wave reads
// 1 KB of each row per turn) and used for every token; xn comes from L2.
// h[t][n] = silu(g) * u in fp32.
template <int NT>
__global__ __launch_bounds__(256) void shared_gate_up_kernel(const uint16_t *__restrict__ xn,
                                                             const uint16_t *__restrict__ sgu,
                                                             float *__restrict__ h, int d,
                                                             int fs) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= fs) return;
    const uint4 *g = reinterpret_cast<const uint4 *>(sgu + (size_t)n * d);
    const uint4 *u = reinterpret_cast<const uint4 *>(sgu + (size_t)(fs + n) * d);
    const int nv = d >> 3;
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
    int v = lane;
    for (; v + 64 < nv; v += 128) {
        const uint4 g0 = g[v], u0 = u[v], g1 = g[v + 64], u1 = u[v + 64];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint4 *xr = reinterpret_cast<const uint4 *>(xn + (size_t)t * d);
            const uint4 x0 = xr[v], x1 = xr[v + 64];
            ag[t] = dot8_bf16(g1, x1, dot8_bf16(g0, x0, ag[t]));
            au[t] = dot8_bf16(u1, x1, dot8_bf16(u0, x0, au[t]));
        }
    }
    if (v < nv) {
        const uint4 g0 = g[v], u0 = u[v];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint4 x0 = reinterpret_cast<const uint4 *>(xn + (size_t)t * d)[v];
            ag[t] = dot8_bf16(g0, x0, ag[t]);
            au[t] = dot8_bf16(u0, x0, au[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float gs = wave_sum_f32(ag[t]), us = wave_sum_f32(au[t]);
        if (lane == t) h[(size_t)t * fs + n] = silu_mul(gs, us);
    }
}

// Shared expert down for NT <= 8 tokens, with the block's residual add in
// the epilogue: one wave per output column m streams row m of W_dn [d][fs]
// once; out[t][m] = bf16(x[t][m] + y[t][m] + sum_n h[t][n] W_dn[m][n]),
// x the block input and y the routed layer's output (both bf16).
template <int NT>
__global__ __launch_bounds__(256) void shared_down_add_kernel(
    const float *__restrict__ h, const uint16_t *__restrict__ sdn,
    const uint16_t *__restrict__ xres, const uint16_t *__restrict__ yr,
    uint16_t *__restrict__ out, int d, int fs) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= d) return;
    const uint4 *w = reinterpret_cast<const uint4 *>(sdn + (size_t)m * fs);
    const int nv = fs >> 3;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
    for (int v = lane; v < nv; v += 64) {
        const uint4 wv = w[v];
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 *hr = reinterpret_cast<const float4 *>(h + (size_t)t * fs) + 2 * v;
            const float4 a = hr[0], b = hr[1];
            const float hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[t] = fmaf(bf16_bits_to_f32(ww[i] & 0xFFFFu), hv[2 * i], acc[t]);
                acc[t] = fmaf(bf16_bits_to_f32(ww[i] >> 16), hv[2 * i + 1], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float s = wave_sum_f32(acc[t]);
        if (lane == t) {
            const size_t i = (size_t)t * d + m;
            out[i] = f32_to_bf16_rne((bf16_bits_to_f32(xres[i]) + bf16_bits_to_f32(yr[i])) + s);
        }
    }
}

template <int NT>
hipError_t shared_gemv_nt(const uint16_t *xn, const uint16_t *sgu, const uint16_t *sdn,
                          const uint16_t *xres, const uint16_t *yr, float *h, uint16_t *out,
                          int d, int fs, hipStream_t s) {
    // fs == 0 (no shared expert): the down pass adds x and y alone
    if (fs > 0) {
        const hipError_t e = timed_launch("shared_gate_up", shared_gate_up_kernel<NT>,
                                          dim3((fs + 3) / 4), dim3(256), 0, s, xn, sgu, h, d, fs);
        if (e != hipSuccess) return e;
    }
    return timed_launch("shared_down_add", shared_down_add_kernel<NT>, dim3((d + 3) / 4),
                        dim3(256), 0, s, h, sdn, xres, yr, out, d, fs);
}

}  // namespace

// A few tokens are spread over up to 32 blocks each (each block recomputes
// the row's 14 KB sum of squares from L2); from 512 tokens on, one block
// per token.
hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *gamma, float eps, uint16_t *xn,
                          int T, int d, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int split = T >= 512 ? 1 : min(32, max(1, min(512 / T, (d >> 3) / 64)));
    return timed_launch("rmsnorm", rmsnorm_kernel, dim3(T, split), dim3(64), 0, s, x, gamma,
                        eps, xn, d);
}

hipError_t launch_shared_gemv(const uint16_t *xn, const uint16_t *sgu, const uint16_t *sdn,
                              const uint16_t *xres, const uint16_t *yr, float *h, uint16_t *out,
                              int T, int d, int fs, hipStream_t s) {
    switch (T) {
    case 1: return shared_gemv_nt<1>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 2: return shared_gemv_nt<2>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 3: return shared_gemv_nt<3>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 4: return shared_gemv_nt<4>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 5: return shared_gemv_nt<5>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 6: return shared_gemv_nt<6>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 7: return shared_gemv_nt<7>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    case 8: return shared_gemv_nt<8>(xn, sgu, sdn, xres, yr, h, out, d, fs, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
