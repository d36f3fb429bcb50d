// route_filter.hip -- routing for many tokens: approximate logits on the
// bf16 matrix cores, then the canonical logit only where it can matter.
//
// The canonical logit of (t, e) is the router dot product summed in the
// fixed fp64 order of route.hip, plus the bias, rounded once to fp32.  For
// prefill-sized T computing all T x E of them in fp64 dominates the layer,
// yet only the k largest per token are ever used.  So:
//   1. zt[t][e] = x[t] . wr[e] on v_mfma_f32_16x16x32_bf16 (bf16 products
//      are exact in fp32; the fp32 additions are the only error), and the
//      row norms |x_t|, |w_e| (computed in fp64, rounded up).
//   2. Per token, a certified interval for every canonical logit:
//        |z_te - (zt_te + b_e)| <= B_te
//        B_te = gamma |x_t| |w_e| (1 + 2^-20) + 2^-23 (|zt_te + b_e| + gamma |x_t| |w_e|)
//               + 1e-30
//      with gamma = 2 (d/64 + 128) 2^-23 / (1 - 2 (d/64 + 128) 2^-23).  The
//      GEMM sums each 64-wide K stage on its own (two chained MFMAs, the
//      first from zero: 64 products in any internal order, at most 63
//      roundings) and adds the d/64 stage sums in fp32, so the error is at
//      most (63 + d/64) u sum |x_i w_i| to first order, whatever order and
//      rounding the MFMA uses inside (u = 2^-23 also covers truncating
//      adders); gamma doubles that with room to spare, Cauchy-Schwarz gives
//      sum |x_i w_i| <= |x_t| |w_e|, and 2^-23 |z| covers the final rounding
//      of the canonical value.  Rows holding a subnormal, infinite or NaN
//      bf16 get an infinite norm (no finite interval), which forces the
//      exact path below.
//   3. tau = the k-th largest lower end.  An expert whose upper end is
//      below tau is below k others for certain, so it is not selected; the
//      canonical logits of the others (the candidates, usually ~17) are
//      computed exactly, and top-k + softmax run over them alone.  A token with any non-finite interval, or
//      more than kCandMax candidates (e.g. massively tied logits), takes
//      the canonical logits of all E experts instead.
// The selected experts and weights are therefore exactly those of the
// canonical logits; only the amount of fp64 work depends on the data.
#include "moe_internal.hpp"
#include "select_dev.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCandMax = kRouteCandMax;

// ---------------------------------------------------------------------------
// Row norms in fp64, rounded up to fp32; +inf if the row holds a subnormal,
// infinite or NaN bf16.  One wave per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void row_norm_kernel(const uint16_t *__restrict__ m, int R,
                                                       int d, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    const uint16_t *row = m + (size_t)r * d;
    double ss = 0.0;
    bool odd = false;
    for (int i = lane * 8; i < d; i += 64 * 8) {
        const uint4 q = *reinterpret_cast<const uint4 *>(row + i);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t b = (w[j] >> (16 * h)) & 0xFFFFu;
                const uint32_t ex = (b >> 7) & 0xFFu, mant = b & 0x7Fu;
                odd |= ex == 0xFFu || (ex == 0u && mant != 0u);
                const double v = (double)__uint_as_float(b << 16);
                ss = fma(v, v, ss);
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const bool any_odd = __ballot(odd) != 0ull;
    if (lane == 0) {
        // sqrt in fp64 (relative error ~1e-16) then a margin far above it
        const float n = (float)(sqrt(ss) * (1.0 + 1.0 / 1048576.0));
        out[r] = any_odd || !(n < INFINITY) ? INFINITY : n;
    }
}

// ---------------------------------------------------------------------------
// zt = x . wr^T on bf16 MFMA.  Block: 128 tokens x 128 experts, four waves
// in 2 x 2 (64 x 64 each, 4 x 4 tiles of 16 x 16), K in stages of 64
// staged through LDS (double buffer, next stage held in registers while the
// current one computes).  Rows past T or E are clamped loads, discarded.
// ---------------------------------------------------------------------------
constexpr int kFT = 128, kFE = 128, kFK = 64;
constexpr int kFStride = 2 * kFK + 16;                 // bytes per LDS row (conflict-free b128)
constexpr int kFOperand = kFT * kFStride;              // 18432
constexpr int kFLds = 2 * 2 * kFOperand;               // 73728

__global__ __launch_bounds__(256) void filter_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ wr,
                                                          float *__restrict__ zt, int T, int d,
                                                          int E) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    const int t0 = blockIdx.y * kFT, e0 = blockIdx.x * kFE;
    const int r16 = lane & 15, g = lane >> 4;
    // this thread's 4 + 4 sixteen-byte pieces of each stage
    const uint16_t *pa[4], *pb[4];
    int so[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i, row = idx >> 3, pc = idx & 7;
        pa[i] = x + (size_t)min(t0 + row, T - 1) * d + pc * 8;
        pb[i] = wr + (size_t)min(e0 + row, E - 1) * d + pc * 8;
        so[i] = row * kFStride + pc * 16;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nst = d / kFK;
    uint4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4 *>(pa[i]);
        rb[i] = *reinterpret_cast<const uint4 *>(pb[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4 *>(lds + so[i]) = ra[i];
        *reinterpret_cast<uint4 *>(lds + kFOperand + so[i]) = rb[i];
    }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        uint8_t *cur = lds + (s & 1) * 2 * kFOperand;
        uint8_t *nxt = lds + ((s + 1) & 1) * 2 * kFOperand;
        // the next stage (the last one again on the final pass: a harmless
        // rewrite of the idle buffer keeps the loop free of branches)
        const size_t koff = (size_t)min(s + 1, nst - 1) * kFK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *reinterpret_cast<const uint4 *>(pa[i] + koff);
            rb[i] = *reinterpret_cast<const uint4 *>(pb[i] + koff);
        }
        // this stage's products summed on their own (the first MFMA starts
        // from zero), then added to the running sum in fp32: the summation
        // chains stay short, which keeps the certified bound tight
        f32x4_t part[4][4];
#pragma unroll
        for (int ks = 0; ks < kFK / 32; ++ks) {
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *reinterpret_cast<const bf16x8_t *>(
                    cur + (wm * 64 + mt * 16 + r16) * kFStride + ks * 64 + 16 * g);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                bfr[nt] = *reinterpret_cast<const bf16x8_t *>(
                    cur + kFOperand + (wn * 64 + nt * 16 + r16) * kFStride + ks * 64 + 16 * g);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    part[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[mt], bfr[nt], ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : part[mt][nt],
                        0, 0, 0);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][nt][i] += part[mt][nt][i];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4 *>(nxt + so[i]) = ra[i];
            *reinterpret_cast<uint4 *>(nxt + kFOperand + so[i]) = rb[i];
        }
        __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + wm * 64 + mt * 16 + 4 * g + i;
            if (t < T) {
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const int e = e0 + wn * 64 + nt * 16 + r16;
                    if (e < E) zt[(size_t)t * E + e] = acc[mt][nt][i];
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Certified selection (one wave per token), then canonical refinement and
// top-k/softmax (one block per token).
// ---------------------------------------------------------------------------
// fp32 bounds that contain a finite double: round toward -inf / +inf (one
// step of the fp32 grid when the nearest rounding went the wrong way).
__device__ __forceinline__ float f32_step_down(float f) {
    const uint32_t u = __float_as_uint(f);
    if (f == 0.f) return -__uint_as_float(1u);             // largest negative subnormal
    return __uint_as_float(f > 0.f ? u - 1u : u + 1u);
}
__device__ __forceinline__ float f32_down(double v) {
    const float f = (float)v;
    return (double)f > v ? f32_step_down(f) : f;
}
__device__ __forceinline__ float f32_up(double v) {
    const float f = (float)v;
    return (double)f < v ? -f32_step_down(-f) : f;
}

// The canonical logit of (token row xr, expert row wrow): lane c sums its
// P = d / 64 inputs in ascending order in fp64, the 64 sums meet in the
// fixed xor-butterfly tree, the bias is added in fp64, one rounding.  Same
// arithmetic, in the same order, as the router kernels of route.hip.
__device__ __forceinline__ float canonical_logit(const uint16_t *xr, const uint16_t *wrow, int P,
                                                 int lane, double bias) {
    const uint16_t *xc = xr + (size_t)lane * P, *wc = wrow + (size_t)lane * P;
    double acc = 0.0;
    int p = 0;
    if ((P & 7) == 0) {
        for (; p < P; p += 8) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xc + p);
            const uint4 wv = *reinterpret_cast<const uint4 *>(wc + p);
            const uint32_t xx[4] = {xv.x, xv.y, xv.z, xv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fma((double)__uint_as_float(xx[q] << 16), (double)__uint_as_float(ww[q] << 16), acc);
                acc = fma((double)__uint_as_float(xx[q] & 0xFFFF0000u),
                          (double)__uint_as_float(ww[q] & 0xFFFF0000u), acc);
            }
        }
    } else {
        for (; p < P; ++p)
            acc = fma((double)__uint_as_float((uint32_t)xc[p] << 16),
                      (double)__uint_as_float((uint32_t)wc[p] << 16), acc);
    }
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) acc += __shfl_xor(acc, w, 64);
    return (float)(acc + bias);
}

// canonical_logit with the lane's chunks (8 NQ inputs) already in registers.
template <int NQ>
__device__ __forceinline__ float canonical_from_regs(const uint4 (&xq)[NQ], const uint4 (&wq)[NQ],
                                                     int lane, double bias) {
    double acc = 0.0;
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
        const uint32_t xx[4] = {xq[p].x, xq[p].y, xq[p].z, xq[p].w};
        const uint32_t ww[4] = {wq[p].x, wq[p].y, wq[p].z, wq[p].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = fma((double)__uint_as_float(xx[q] << 16), (double)__uint_as_float(ww[q] << 16), acc);
            acc = fma((double)__uint_as_float(xx[q] & 0xFFFF0000u),
                      (double)__uint_as_float(ww[q] & 0xFFFF0000u), acc);
        }
    }
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) acc += __shfl_xor(acc, w, 64);
    return (float)(acc + bias);
}

// Per token (one wave): the certified intervals, tau and the candidate
// list, written to cand[t][..] in ascending expert order with their number
// in ncand_out[t] (-1: the token takes all E canonical logits).
template <int PL>
__global__ __launch_bounds__(256) void select_cand_kernel(
    const float *__restrict__ zt, const float *__restrict__ nx, const float *__restrict__ nw,
    const float *__restrict__ bias, int32_t *__restrict__ cand, int32_t *__restrict__ ncand_out,
    int T, int E, int k, double gamma) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wid;
    if (t >= T) return;                                    // no block-level sync below
    int32_t *mycand = cand + (size_t)t * kCandMax;
    const double gx = gamma * (double)nx[t];
    uint32_t lok[PL], upk[PL];
    bool bad = !(gx < INFINITY);
    float zl[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) zl[i] = zt[(size_t)t * E + min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        lok[i] = 0u;
        upk[i] = 0u;
        if (e < E) {
            const double zf = (double)zl[i] + (bias ? (double)bias[e] : 0.0);
            const double sb = gx * (double)nw[e];
            const double B = sb * (1.0 + 1.0 / 1048576.0) + (fabs(zf) + sb) * (1.0 / 8388608.0) + 1e-30;
            const double lo = zf - B, up = zf + B;
            if (!(fabs(lo) < INFINITY) || !(fabs(up) < INFINITY)) bad = true;
            lok[i] = logit_key(f32_down(lo));
            upk[i] = logit_key(f32_up(up));
        }
    }
    bad = __ballot(bad) != 0ull;
    int ncand = 0;
    if (!bad) {
        // tau: the k-th largest lower end (with multiplicity)
        uint32_t kk[PL];
#pragma unroll
        for (int i = 0; i < PL; ++i) kk[i] = lok[i];
        uint32_t tau = 0u;
        for (int j = 0; j < k; ++j) {
            uint32_t bk = 0u;
#pragma unroll
            for (int i = 0; i < PL; ++i) bk = max(bk, kk[i]);
            const uint32_t gk = wave_max_u32(bk);
            const unsigned long long m = __ballot(bk == gk);
            // the lowest lane holding the maximum drops one copy of it;
            // selects, not branches, keep the kk[] in place
            bool take = lane == (int)__builtin_ctzll(m);
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                const bool hit = take && kk[i] == gk;
                kk[i] = hit ? 0u : kk[i];
                take = take && !hit;
            }
            tau = gk;
        }
        int base = 0;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const bool c = lane + 64 * i < E && upk[i] >= tau;
            const unsigned long long m = __ballot(c);
            const int pos = base + (int)__popcll(m & ((1ull << lane) - 1ull));
            if (c && pos < kCandMax) mycand[pos] = lane + 64 * i;
            base += (int)__popcll(m);
        }
        ncand = base;
        bad = ncand > kCandMax;
    }
    if (lane == 0) ncand_out[t] = bad ? -1 : ncand;       // -1: all E experts
}

// The canonical logits of the candidates, then the token's top-k + softmax:
// block = one token.  Its four waves take candidates wid, wid + 4, .. and
// park the logits in LDS.  With P = 8 NQ the lane's chunk of x stays in
// registers and each candidate's chunk of its router row is loaded in one go
// (every load before any use); else both chunks stream from memory.  Wave 0
// then ranks the candidates (at most 64, one per lane), or, for a token that
// takes all E experts, runs the full-row selection over them.  Either way
// the k selected and their order are those of the full row of canonical
// logits, since the candidates hold its top k, and the weights come from the
// same softmax tail as the unfiltered path.
template <int NQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void refine_topk_kernel(
    const float *__restrict__ bias, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ wr, const int32_t *__restrict__ cand,
    const int32_t *__restrict__ ncand_in, int32_t *__restrict__ ids, float *__restrict__ tw,
    int T, int d, int E, int k) {
    __shared__ __align__(16) float zc[kMaxExperts];
    __shared__ __align__(16) uint32_t tsc[kTopkScratch];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = blockIdx.x;
    if (t >= T) return;                                    // whole block: before any barrier
    const int nc = ncand_in[t];
    const bool all = nc < 0;
    const int n = all ? E : min(nc, kCandMax);
    const int P = d >> 6;
    const uint16_t *xr = x + (size_t)t * d;
    const int32_t *mycand = cand + (size_t)t * kCandMax;
    if constexpr (NQ > 0) {
        uint4 xq[NQ];
        const uint4 *xc = reinterpret_cast<const uint4 *>(xr + (size_t)lane * P);
#pragma unroll
        for (int q = 0; q < NQ; ++q) xq[q] = xc[q];
        for (int c = wid; c < n; c += 4) {
            const int e = all ? c : mycand[c];
            if ((unsigned)e >= (unsigned)E) continue;
            const uint4 *wc = reinterpret_cast<const uint4 *>(wr + (size_t)e * d + (size_t)lane * P);
            uint4 wq[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) wq[q] = wc[q];
            // an empty asm that "changes" the x chunk each pass keeps the
            // compiler from hoisting its 8 NQ fp64 conversions out of the
            // loop (2 VGPRs each), which would cap the kernel at one wave
            // per SIMD
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                asm volatile("" : "+v"(xq[q].x), "+v"(xq[q].y), "+v"(xq[q].z), "+v"(xq[q].w));
            const float z = canonical_from_regs<NQ>(xq, wq, lane, bias ? (double)bias[e] : 0.0);
            if (lane == 0) zc[c] = z;
        }
    } else {
        for (int c = wid; c < n; c += 4) {
            const int e = all ? c : mycand[c];
            if ((unsigned)e >= (unsigned)E) continue;
            const float z = canonical_logit(xr, wr + (size_t)e * d, P, lane,
                                            bias ? (double)bias[e] : 0.0);
            if (lane == 0) zc[c] = z;
        }
    }
    __syncthreads();
    if (wid != 0) return;
    // a fresh copy of the lane index: the 64-bit offsets built from it are
    // then formed here, not kept in registers across the loop above
    int li = lane;
    asm volatile("" : "+v"(li));
    int se = 0;
    float sw = 0.f;
    if (all) {
        wave_topk_softmax<kMaxExperts / 64>(zc, E, k, tsc, &se, &sw);
    } else {
        const int e = li < n ? mycand[li] : -1;
        const bool ok = (unsigned)e < (unsigned)E;
        const uint32_t ka = ok ? logit_key(zc[li]) : 0u;
        const uint32_t ea = ok ? (uint32_t)e : 0xFFFFFFFFu;
        int my_e = 0;
        float my_v = 0.f;
        wave_rank_select(ka, ea, n, k, &my_e, &my_v);
        wave_softmax_tail(my_e, my_v, k, &se, &sw);
    }
    if (li < k) {
        ids[(size_t)t * k + li] = se;
        tw[(size_t)t * k + li] = sw;
    }
}

bool g_filter_attr = false;

}  // namespace

bool route_filter_ok(int T, int d, int E) {
    return T >= kRouteFilterMinT && d % 64 == 0 && E <= kMaxExperts;
}

hipError_t launch_route_filtered(const uint16_t *x, const uint16_t *wr, const float *bias,
                                 float *zt, float *nx, float *nw, int32_t *cand, int32_t *ncand,
                                 int32_t *ids, float *tw, int T, int d, int E, int k,
                                 hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipError_t e;
    if (!g_filter_attr) {
        e = hipFuncSetAttribute((const void *)filter_gemm_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kFLds);
        if (e != hipSuccess) return e;
        g_filter_attr = true;
    }
    {
        DiagScope ds("router_norms", s);
        row_norm_kernel<<<(T + 3) / 4, 256, 0, s>>>(x, T, d, nx);
        row_norm_kernel<<<(E + 3) / 4, 256, 0, s>>>(wr, E, d, nw);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        dim3 grid((E + kFE - 1) / kFE, (T + kFT - 1) / kFT);
        (void)timed_launch("router_filter_gemm", filter_gemm_kernel, dim3(grid), dim3(256), kFLds, s, x, wr, zt, T, d, E);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const double c = 2.0 * (double)(d / 64 + 128) / 8388608.0;
    const double gamma = c / (1.0 - c);
    const int pl = (E + 63) / 64;
    {
        const unsigned grid = (unsigned)((T + 3) / 4);
        if (pl <= 4)
            (void)timed_launch("router_select", select_cand_kernel<4>, dim3(grid), dim3(256), 0, s, zt, nx, nw, bias, cand, ncand, T, E, k, gamma);
        else if (pl <= 8)
            (void)timed_launch("router_select", select_cand_kernel<8>, dim3(grid), dim3(256), 0, s, zt, nx, nw, bias, cand, ncand, T, E, k, gamma);
        else
            (void)timed_launch("router_select", select_cand_kernel<16>, dim3(grid), dim3(256), 0, s, zt, nx, nw, bias, cand, ncand, T, E, k, gamma);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        // the register-resident chunk covers d = 512 * NQ; other d take the
        // loop that reads both chunks from memory
        const int P = d / 64;
        if (P == 112)
            (void)timed_launch("router_refine", refine_topk_kernel<14>, dim3(T), dim3(256), 0, s, bias, x, wr, cand, ncand, ids, tw, T, d, E, k);
        else if (P == 64)
            (void)timed_launch("router_refine", refine_topk_kernel<8>, dim3(T), dim3(256), 0, s, bias, x, wr, cand, ncand, ids, tw, T, d, E, k);
        else
            (void)timed_launch("router_refine", refine_topk_kernel<0>, dim3(T), dim3(256), 0, s, bias, x, wr, cand, ncand, ids, tw, T, d, E, k);
    }
    return hipGetLastError();
}

}  // namespace moe
