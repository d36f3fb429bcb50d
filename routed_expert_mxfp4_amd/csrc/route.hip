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
#include <atomic>

#include "moe_internal.hpp"
#include "select_dev.hpp"

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
        (void)timed_launch("router_logits", router_logits_kernel<TT, TE, 8>, dim3(grid), dim3(64), 0, s, x, wr, bias, logits, T, d, E);
    else if (P % 4 == 0)
        (void)timed_launch("router_logits", router_logits_kernel<TT, TE, 4>, dim3(grid), dim3(64), 0, s, x, wr, bias, logits, T, d, E);
    else if (P % 2 == 0)
        (void)timed_launch("router_logits", router_logits_kernel<TT, TE, 2>, dim3(grid), dim3(64), 0, s, x, wr, bias, logits, T, d, E);
    else
        (void)timed_launch("router_logits", router_logits_kernel<TT, TE, 1>, dim3(grid), dim3(64), 0, s, x, wr, bias, logits, T, d, E);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One token with d % 512 == 0: router rows staged through LDS.
// ---------------------------------------------------------------------------
// Lane c of a wave sums chunk c (P consecutive inputs) of one router row.  A
// direct load would have the 64 lanes of a wave read 64 rows 2P bytes apart,
// so every 16-byte load touches 64 cache lines; instead the block copies its
// router rows into LDS with coalesced 16-byte loads, laid out chunk by
// chunk with 16 bytes of padding (a chunk stride of 2P+16 bytes keeps the
// 16 lanes of a b128 read on distinct banks), and each lane then reads its
// own chunk from LDS.  The lane's chunk of x goes straight to registers.
constexpr int kStagePieces = 16;                    // d <= 8192
constexpr int kRouterRowsPerBlock = 4;              // one token: router rows (waves) per block

// RPB router rows per block (one wave each); a block stages its rows with
// RPB * 64 threads, each loading d / 512 sixteen-byte pieces.
template <int RPB>
__global__ __launch_bounds__(64 * RPB) void router_small_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int d, int E) {
    constexpr int kThreads = 64 * RPB;
    constexpr int kPer = kStagePieces;              // pieces per thread: d / 512 <= 16
    extern __shared__ uint4 wrs[];                  // [RPB][64][(2P+16)/16] + 1 spare
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int P = d >> 6;
    const int q_per_chunk = P >> 3;                 // 16-byte pieces per chunk
    const int cstride = q_per_chunk + 1;            // in uint4, with padding
    const int e0 = blockIdx.x * RPB;
    const int pieces = 64 * q_per_chunk;            // 16-byte pieces per row
    const int total = RPB * pieces;                 // <= kThreads * kPer
    // n / pieces and n / q_per_chunk by multiply-high with ceil(2^32 / D):
    // exact for n, D < 2^16 (n D < 2^32), which holds here (n < 4096,
    // D <= 1024); the wave-uniform magic numbers cost one scalar division
    // each instead of a vector division per piece
    const uint64_t mg_p = ((1ull << 32) + (uint64_t)pieces - 1) / (uint64_t)pieces;
    const uint64_t mg_q = ((1ull << 32) + (uint64_t)q_per_chunk - 1) / (uint64_t)q_per_chunk;
    auto div_p = [mg_p](int n) { return (int)(((uint64_t)(uint32_t)n * mg_p) >> 32); };
    auto div_q = [mg_q](int n) { return (int)(((uint64_t)(uint32_t)n * mg_q) >> 32); };
    // every load first, then every LDS store: one memory round trip
    uint4 buf[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = min((int)threadIdx.x + kThreads * j, total - 1);
        const int r = div_p(i), q = i - r * pieces;
        buf[j] = reinterpret_cast<const uint4 *>(wr + (size_t)min(e0 + r, E - 1) * d)[q];
    }
    // every load completes here, then unconditional stores (pieces past the
    // end go to a spare slot)
    loads_done(buf);
    const int spare = RPB * 64 * cstride;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = (int)threadIdx.x + kThreads * j;
        const int r = div_p(i), q = i - r * pieces;
        const int c = div_q(q), w = q - c * q_per_chunk;
        wrs[i < total ? (r * 64 + c) * cstride + w : spare] = buf[j];
    }
    __syncthreads();
    const int e = e0 + wid;
    const uint4 *wc = wrs + (wid * 64 + lane) * cstride;
    double acc = 0.0;
    // the lane's chunk of x (one token) is loaded into registers up front
    const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)lane * P);
    uint4 xv[kStagePieces];
#pragma unroll
    for (int w = 0; w < kStagePieces; ++w) xv[w] = xr[min(w, q_per_chunk - 1)];
#pragma unroll
    for (int w = 0; w < kStagePieces; ++w) {
        if (w < q_per_chunk) {
            const uint4 wv = wc[w];
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
            const uint32_t xx[4] = {xv[w].x, xv[w].y, xv[w].z, xv[w].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {                  // ascending element order
                acc = fma(bf16_lo(xx[q]), bf16_lo(ww[q]), acc);
                acc = fma(bf16_hi(xx[q]), bf16_hi(ww[q]), acc);
            }
        }
    }
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) acc += __shfl_xor(acc, w, 64);
    if (e < E && lane == 0) logits[e] = (float)(acc + (bias ? (double)bias[e] : 0.0));
}

// ---------------------------------------------------------------------------
// Few tokens (8 <= T < 256, d % 512 == 0): TE router rows staged through LDS
// for TT tokens.  The block copies its router rows into LDS with coalesced
// 16-byte loads, chunk by chunk with 16 bytes of padding (as above); wave w
// then takes tokens t0 + (TT / 4) w .., lane c summing chunk c of every
// token and row of the tile in ascending element order, the x chunk pieces
// loaded straight from memory a few slices ahead.  The same arithmetic and
// order as router_logits_kernel, so the logits are identical; the router
// rows are read once per TT tokens with whole cache lines.
constexpr int kLtTE = 8;                            // router rows per block
constexpr int kLtTT = 16;                           // tokens per block (4 per wave)
constexpr int kLtAhead = 2;                         // x slices in flight ahead

__global__ __launch_bounds__(256) void router_lds_tile_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int d, int E) {
    constexpr int TPW = kLtTT / 4;                  // tokens per wave
    extern __shared__ uint4 wrs[];                  // [kLtTE][64][cstride]
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int P = d >> 6;
    const int q_per_chunk = P >> 3;                 // 16-byte pieces per chunk
    const int cstride = q_per_chunk + 1;
    const int e0 = blockIdx.x * kLtTE;
    const int t0 = blockIdx.y * kLtTT + wid * TPW;
    const int pieces = 64 * q_per_chunk;            // 16-byte pieces per row
    const int total = kLtTE * pieces;
    // staging, 16 pieces a thread per round: every load of a round first,
    // then its LDS stores
    for (int base = 0; base < total; base += 256 * 16) {
        uint4 buf[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = min(base + (int)threadIdx.x + 256 * j, total - 1);
            const int r = i / pieces, q = i - r * pieces;
            buf[j] = reinterpret_cast<const uint4 *>(wr + (size_t)min(e0 + r, E - 1) * d)[q];
        }
        loads_done(buf);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int i = base + (int)threadIdx.x + 256 * j;
            if (i < total) {
                const int r = i / pieces, q = i - r * pieces;
                const int c = q / q_per_chunk, w = q - c * q_per_chunk;
                wrs[(r * 64 + c) * cstride + w] = buf[j];
            }
        }
    }
    __syncthreads();
    const uint4 *xr[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
        xr[i] = reinterpret_cast<const uint4 *>(x + (size_t)min(t0 + i, T - 1) * d + (size_t)lane * P);
    double acc[TPW][kLtTE];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < kLtTE; ++j) acc[i][j] = 0.0;
    uint4 xq[kLtAhead + 1][TPW];
#pragma unroll
    for (int a = 0; a < kLtAhead; ++a)
#pragma unroll
        for (int i = 0; i < TPW; ++i) xq[a][i] = xr[i][min(a, q_per_chunk - 1)];
    const uint4 *wc = wrs + lane * cstride;
    for (int w = 0; w < q_per_chunk; ++w) {
        // slice w + kLtAhead's x pieces, then slice w's products
        const int wn = min(w + kLtAhead, q_per_chunk - 1);
        uint4 xn[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) xn[i] = xr[i][wn];
        uint32_t wv[kLtTE][4];
#pragma unroll
        for (int j = 0; j < kLtTE; ++j) {
            const uint4 v = wc[j * 64 * cstride + w];
            wv[j][0] = v.x; wv[j][1] = v.y; wv[j][2] = v.z; wv[j][3] = v.w;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {               // ascending element order
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const uint4 xv = xq[0][i];
                const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
                const double xe = (q & 1) ? bf16_hi(xw[q >> 1]) : bf16_lo(xw[q >> 1]);
#pragma unroll
                for (int j = 0; j < kLtTE; ++j) {
                    const double we = (q & 1) ? bf16_hi(wv[j][q >> 1]) : bf16_lo(wv[j][q >> 1]);
                    acc[i][j] = fma(xe, we, acc[i][j]);
                }
            }
        }
#pragma unroll
        for (int a = 0; a < kLtAhead; ++a)
#pragma unroll
            for (int i = 0; i < TPW; ++i) xq[a][i] = a + 1 < kLtAhead ? xq[a + 1][i] : xn[i];
    }
    // fixed pairwise tree over the 64 chunk sums
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int j = 0; j < kLtTE; ++j) acc[i][j] += __shfl_xor(acc[i][j], m, 64);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int j = 0; j < kLtTE; ++j) {
            const int t = t0 + i, e = e0 + j;
            if (lane == i * kLtTE + j && t < T && e < E) {
                const double l = acc[i][j] + (bias ? (double)bias[e] : 0.0);
                logits[(size_t)t * E + e] = (float)l;   // one RNE rounding
            }
        }
}

// ---------------------------------------------------------------------------
// top-k + softmax: one wave per token.
// ---------------------------------------------------------------------------
template <int PL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ logits,
                                                           int32_t *__restrict__ ids,
                                                           float *__restrict__ w, int T,
                                                           int E, int k) {
    __shared__ __align__(16) uint32_t tsc[4][kTopkScratch];
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int e;
    float wt;
    wave_topk_softmax<PL>(logits + (size_t)t * E, E, k, tsc[threadIdx.x >> 6], &e, &wt);
    if (lane < k) {
        ids[(size_t)t * k + lane] = e;
        w[(size_t)t * k + lane] = wt;
    }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias,
                                float *logits, int T, int d, int E, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int P = d / 64;
    if (T == 1 && P % 8 == 0 && d <= 8192) {
        // 4 router rows per block, or 1 when that leaves CUs idle (E < 768)
        const int rpb = E >= 4 * 192 ? kRouterRowsPerBlock : 1;
        const size_t lds = (size_t)rpb * 64 * ((P / 8) + 1) * 16 + 16;   // + spare slot
        if (rpb == 1)
            (void)timed_launch("router_logits", router_small_kernel<1>, dim3(E), dim3(64), lds, s,
                               x, wr, bias, logits, T, d, E);
        else
            (void)timed_launch("router_logits", router_small_kernel<kRouterRowsPerBlock>,
                               dim3((E + kRouterRowsPerBlock - 1) / kRouterRowsPerBlock),
                               dim3(64 * kRouterRowsPerBlock), lds, s, x, wr, bias, logits, T, d, E);
        return hipGetLastError();
    }
    // larger token tiles re-read the router rows fewer times (8 x 8 at
    // T = 64: 67.6 us against 86.0 us for 4 x 8)
    if (T < 4) return launch_logits_tile<1, 4>(x, wr, bias, logits, T, d, E, s);
    if (T < 8) return launch_logits_tile<4, 8>(x, wr, bias, logits, T, d, E, s);
    if (P % 8 == 0 && d <= 8192) {
        // router rows staged through LDS, 16 tokens per block (up to 136 KB
        // of LDS: the launch limit is raised once per process)
        static std::atomic<bool> attr{false};
        const size_t lds = (size_t)kLtTE * 64 * ((P / 8) + 1) * 16;
        if (!attr.load(std::memory_order_acquire)) {
            const hipError_t e = hipFuncSetAttribute((const void *)router_lds_tile_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)(kLtTE * 64 * 17 * 16));
            if (e != hipSuccess) return e;
            attr.store(true, std::memory_order_release);
        }
        dim3 grid((E + kLtTE - 1) / kLtTE, (T + kLtTT - 1) / kLtTT);
        (void)timed_launch("router_logits", router_lds_tile_kernel, dim3(grid), dim3(256), lds, s,
                           x, wr, bias, logits, T, d, E);
        return hipGetLastError();
    }
    return launch_logits_tile<8, 8>(x, wr, bias, logits, T, d, E, s);
}

hipError_t launch_topk_softmax(const float *logits, int32_t *ids, float *w, int T, int E,
                               int k, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + 3) / 4);
    const int pl = (E + 63) / 64;
    if (pl <= 4)
        (void)timed_launch("topk_softmax", topk_softmax_kernel<4>, dim3(grid), dim3(256), 0, s, logits, ids, w, T, E, k);
    else if (pl <= 8)
        (void)timed_launch("topk_softmax", topk_softmax_kernel<8>, dim3(grid), dim3(256), 0, s, logits, ids, w, T, E, k);
    else
        (void)timed_launch("topk_softmax", topk_softmax_kernel<16>, dim3(grid), dim3(256), 0, s, logits, ids, w, T, E, k);
    return hipGetLastError();
}

}  // namespace moe
