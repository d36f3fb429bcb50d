// ffn_fp8.hip -- routed expert FFN with FP8 experts on gfx950: E4M3FN codes
// (one byte per weight, K contiguous) with one fp32 scale per 128 x 128
// block of each matrix.
//
// The pages' FP8 lane pairs an exhaustive OCP E4M3FN oracle with a fused
// GEMV and a bounded BF16-dequant prefill floor (Moonshine README, "GLM 5.3
// Flash status").  Here a grouped dequant-GEMV serves fewer than 128
// tokens (ffn_fp8_mfma.hip takes over from there): each wave
// streams whole weight rows with 16-byte loads (16 codes per lane), gfx950
// converts code pairs exactly to bf16 (against bf16 x) or fp32 (against fp32
// h) -- the bf16 copy of a weight lives only in registers -- and each
// 16-element partial sum is multiplied by its block's fp32 scale.  Every
// decoded weight is reused for all token rows of the expert staged in LDS
// (up to kRows8 per pass).
//
// Gate/up: h[p][n] = silu(x_t . Wg[n]) * (x_t . Wu[n]) (fp32), p over the
// expert's rows (t = sorted_rows[p] / k); gate rows [0, f), up [f, 2f).
// Down: rows_out[p][m] = h[p] . Wd[m] (bf16), expert-major.
#include "moe_internal.hpp"
#include "select_dev.hpp"

namespace moe {
namespace {

constexpr int kPairs8 = 16;      // gate/up output pairs per block
constexpr int kRows8 = 4;        // token rows of one expert per LDS pass
constexpr int kDnRows8 = 64;     // down output rows per block

__device__ __forceinline__ float silu_mul8(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// The expert group of blockIdx.y from device data, bounds-checked.
__device__ __forceinline__ bool group8(const int32_t *plan, const int32_t *offsets, int a,
                                       int E, int nrows, int &e, int &row0, int &ne) {
    if (a >= plan[0]) return false;
    e = plan[1 + a];
    if ((unsigned)e >= (unsigned)E) return false;
    row0 = offsets[e];
    ne = offsets[e + 1] - row0;
    return row0 >= 0 && ne > 0 && row0 + ne <= nrows;
}

// 16 E4M3FN codes (byte i = element i) dotted with 16 bf16 values (x0:
// elements 0..7, x1: 8..15), fp32 accumulate.  The scaled convert (scale
// 1.0) gives the codes' exact bf16 values, low byte first.
__device__ __forceinline__ float dot16_fp8_bf16(uint4 c, uint4 x0, uint4 x1, float acc) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[i], 1.0f, false);
        const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[i], 1.0f, true);
        acc = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2_t, xw[2 * i]), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2_t, xw[2 * i + 1]),
                                              acc, false);
    }
    return acc;
}

// 16 E4M3FN codes dotted with 16 fp32 values h[0..15].
__device__ __forceinline__ float dot16_fp8_f32(uint4 c, const float4 (&hv)[4], float acc) {
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[i], 1.0f, false);
        const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(cw[i], 1.0f, true);
        acc = fmaf(lo.x, hv[i].x, acc);
        acc = fmaf(lo.y, hv[i].y, acc);
        acc = fmaf(hi.x, hv[i].z, acc);
        acc = fmaf(hi.y, hv[i].w, acc);
    }
    return acc;
}

// Block (kPairs8 output pairs, expert a = blockIdx.y); wave w takes pairs
// w, w + 4, ..; lane l takes the 16-code chunks c = l + 64 i of a row, two
// chunks per turn so that four 16-byte loads are in flight.
__global__ __launch_bounds__(256) void fp8_gate_up_kernel(
    const uint16_t *__restrict__ x, Fp8Args W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_rows, const int32_t *__restrict__ plan,
    float *__restrict__ h, int T, int d, int E, int k, int f, int rpp) {
    const int nrows = T * k;
    int e, row0, ne;
    if (!group8(plan, offsets, blockIdx.y, E, nrows, e, row0, ne)) return;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t *codes = W.gu_codes + (size_t)e * 2 * f * d;
    const int sbk = d >> 7;                               // scale blocks along K
    const float *scales = W.gu_scales + (size_t)e * (2 * f >> 7) * sbk;
    extern __shared__ uint4 xs4[];                        // [rpp][d / 8]
    const int nvec = d >> 3, nch = d >> 4;
    const int n_base = blockIdx.x * kPairs8;

    for (int r0 = 0; r0 < ne; r0 += rpp) {
        const int R = min(rpp, ne - r0);
        __syncthreads();
        for (int i = threadIdx.x; i < R * nvec; i += 256) {
            const int r = i / nvec, v = i - r * nvec;
            const int row = sorted_rows[row0 + r0 + r];
            const int tok = (unsigned)row < (unsigned)nrows ? row / k : 0;
            xs4[r * nvec + v] = reinterpret_cast<const uint4 *>(x + (size_t)tok * d)[v];
        }
        __syncthreads();
        for (int p = wid; p < kPairs8; p += 4) {
            const int n = n_base + p;
            const uint4 *grow = reinterpret_cast<const uint4 *>(codes + (size_t)n * d);
            const uint4 *urow = reinterpret_cast<const uint4 *>(codes + (size_t)(f + n) * d);
            const float *gsc = scales + (size_t)(n >> 7) * sbk;
            const float *usc = scales + (size_t)((f + n) >> 7) * sbk;
            float g[kRows8], u[kRows8];
#pragma unroll
            for (int r = 0; r < kRows8; ++r) g[r] = u[r] = 0.f;
            for (int c = lane; c < nch; c += 128) {
                const bool two = c + 64 < nch;
                const uint4 cg0 = grow[c], cu0 = urow[c];
                const uint4 cg1 = two ? grow[c + 64] : uint4{0, 0, 0, 0};
                const uint4 cu1 = two ? urow[c + 64] : uint4{0, 0, 0, 0};
                const float sg0 = gsc[c >> 3], su0 = usc[c >> 3];
                const float sg1 = two ? gsc[(c + 64) >> 3] : 0.f;
                const float su1 = two ? usc[(c + 64) >> 3] : 0.f;
#pragma unroll
                for (int r = 0; r < kRows8; ++r) {
                    if (r < R) {
                        const uint4 *xv = xs4 + r * nvec;
                        g[r] += sg0 * dot16_fp8_bf16(cg0, xv[2 * c], xv[2 * c + 1], 0.f);
                        u[r] += su0 * dot16_fp8_bf16(cu0, xv[2 * c], xv[2 * c + 1], 0.f);
                        if (two) {
                            const int c1 = c + 64;
                            g[r] += sg1 * dot16_fp8_bf16(cg1, xv[2 * c1], xv[2 * c1 + 1], 0.f);
                            u[r] += su1 * dot16_fp8_bf16(cu1, xv[2 * c1], xv[2 * c1 + 1], 0.f);
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < kRows8; ++r) {
                if (r < R) {
                    const float gs = wave_sum_f32(g[r]), us = wave_sum_f32(u[r]);
                    if (lane == 0) h[(size_t)(row0 + r0 + r) * f + n] = silu_mul8(gs, us);
                }
            }
        }
    }
}

// Block (kDnRows8 output rows, expert a); wave w owns rows 16 w .. 16 w + 15
// as four groups of 16 lanes with 4 rows each; lane gl of a group takes the
// 16-code chunks gl + 16 i of those rows.
__global__ __launch_bounds__(256) void fp8_down_kernel(
    const float *__restrict__ h, Fp8Args W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ plan, uint16_t *__restrict__ rows_out, int T, int d, int E,
    int k, int f, int rpp) {
    const int nrows = T * k;
    int e, row0, ne;
    if (!group8(plan, offsets, blockIdx.y, E, nrows, e, row0, ne)) return;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4, gl = lane & 15;
    const uint8_t *codes = W.dn_codes + (size_t)e * d * f;
    const int sbk = f >> 7;
    const float *scales = W.dn_scales + (size_t)e * (d >> 7) * sbk;
    extern __shared__ float4 hs4[];                       // [rpp][f / 4]
    const int nv = f >> 2, nch = f >> 4;
    const int m_base = blockIdx.x * kDnRows8 + wid * 16 + grp * 4;

    for (int r0 = 0; r0 < ne; r0 += rpp) {
        const int R = min(rpp, ne - r0);
        __syncthreads();
        for (int i = threadIdx.x; i < R * nv; i += 256) {
            const int r = i / nv, v = i - r * nv;
            hs4[r * nv + v] = reinterpret_cast<const float4 *>(h + (size_t)(row0 + r0 + r) * f)[v];
        }
        __syncthreads();
        float acc[4][kRows8];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRows8; ++r) acc[q][r] = 0.f;
        for (int c = gl; c < nch; c += 16) {
            uint4 cq[4];
            float sq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m_base + q;
                cq[q] = reinterpret_cast<const uint4 *>(codes + (size_t)m * f)[c];
                sq[q] = scales[(size_t)(m >> 7) * sbk + (c >> 3)];
            }
#pragma unroll
            for (int r = 0; r < kRows8; ++r) {
                if (r < R) {
                    const float4 *hr = hs4 + r * nv + 4 * c;
                    const float4 hv[4] = {hr[0], hr[1], hr[2], hr[3]};
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q][r] += sq[q] * dot16_fp8_f32(cq[q], hv, 0.f);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRows8; ++r) {
                if (r < R) {
                    const float v = group16_sum_f32(acc[q][r]);
                    if (gl == 0)
                        rows_out[(size_t)(row0 + r0 + r) * d + m_base + q] = f32_to_bf16_rne(v);
                }
            }
    }
}

// Decode-sized T (<= 8 rows per expert): the gate and up rows of a wave's
// pairs are streamed one row at a time, double-buffered -- the next row's
// loads (d bytes of codes and its block scales) are in flight while the
// current row is reduced -- against the token row staged once in LDS.  Lane
// l owns the 16-code chunks l + 64 i (i < NCL) of every row.
constexpr int kRxPairs8 = 32;       // pairs per block (8 per wave)
constexpr int kStageX8 = 4;         // x staging: d <= 4 * 256 * 8 = 8192

template <int NCL>
struct Row8 {
    uint4 c[NCL];
    float s[NCL];
};

template <int NCL>
__device__ __forceinline__ void load_row8(const uint8_t *codes, const float *scales, int row,
                                          int d, int sbk, int nch, int lane, Row8<NCL> &rb) {
    const uint4 *r = reinterpret_cast<const uint4 *>(codes + (size_t)row * d);
    const float *sr = scales + (size_t)(row >> 7) * sbk;
#pragma unroll
    for (int i = 0; i < NCL; ++i) {
        const int c = min(lane + 64 * i, nch - 1);
        rb.c[i] = r[c];
        rb.s[i] = sr[c >> 3];
    }
}

template <int NCL>
__device__ __forceinline__ float row_dot8(const Row8<NCL> &rb, const uint4 *__restrict__ xs,
                                          int lane, int nch) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NCL; ++i) {
        const int c = lane + 64 * i;
        const int cc = min(c, nch - 1);
        const float p = dot16_fp8_bf16(rb.c[i], xs[2 * cc], xs[2 * cc + 1], 0.f);
        acc += c < nch ? p * rb.s[i] : 0.f;
        __builtin_amdgcn_sched_barrier(0);
    }
    return wave_sum_f32(acc);
}

template <int NCL>
__global__ __launch_bounds__(256) void fp8_gate_up_rx_kernel(
    const uint16_t *__restrict__ x, Fp8Args W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_rows, const int32_t *__restrict__ plan,
    float *__restrict__ h, int T, int d, int E, int k, int f) {
    const int nrows = T * k;
    int e, row0, ne;
    if (!group8(plan, offsets, blockIdx.y, E, nrows, e, row0, ne)) return;
    extern __shared__ uint4 xs[];                         // d / 8 x 16 B, + 1 spare
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = d >> 4, nvec = d >> 3, sbk = d >> 7;
    const uint8_t *codes = W.gu_codes + (size_t)e * 2 * f * d;
    const float *scales = W.gu_scales + (size_t)e * (2 * f >> 7) * sbk;
    constexpr int kPerWave = kRxPairs8 / 4;               // pairs n_base + 4 q
    const int n_base = blockIdx.x * kRxPairs8 + wid;
    for (int r = 0; r < ne; ++r) {
        const int row = sorted_rows[row0 + r];
        const int tok = (unsigned)row < (unsigned)nrows ? row / k : 0;
        Row8<NCL> A, B;
        load_row8<NCL>(codes, scales, n_base, d, sbk, nch, lane, A);   // before the x sync
        __syncthreads();
        {
            const uint4 *xrow = reinterpret_cast<const uint4 *>(x + (size_t)tok * d);
            uint4 tmp[kStageX8];
#pragma unroll
            for (int j = 0; j < kStageX8; ++j)
                tmp[j] = xrow[min((int)threadIdx.x + 256 * j, nvec - 1)];
            loads_done(tmp);
#pragma unroll
            for (int j = 0; j < kStageX8; ++j) {
                const int i = (int)threadIdx.x + 256 * j;
                xs[i < nvec ? i : nvec] = tmp[j];
            }
        }
        __syncthreads();
        float *hrow = h + (size_t)(row0 + r) * f;
#pragma unroll 1
        for (int q = 0; q < kPerWave; ++q) {
            const int n = n_base + 4 * q;
            load_row8<NCL>(codes, scales, f + n, d, sbk, nch, lane, B);          // up row
            __builtin_amdgcn_sched_barrier(0);
            const float g = row_dot8<NCL>(A, xs, lane, nch);
            __builtin_amdgcn_sched_barrier(0);
            if (q + 1 < kPerWave)
                load_row8<NCL>(codes, scales, n + 4, d, sbk, nch, lane, A);     // next gate row
            __builtin_amdgcn_sched_barrier(0);
            const float u = row_dot8<NCL>(B, xs, lane, nch);
            if (lane == 0) hrow[n] = silu_mul8(g, u);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One token (T = 1): the top-k and the grouping happen inside the gate/up
// pass, as in the MXFP4 one-token kernel.  Every block selects the token's
// experts from the logits row (one wave) after staging x; in ascending
// expert order the a-th selected expert is the one whose h row is a
// (blockIdx.y = a), routed from top-k slot sorted_rows[a].  Block (0, 0)
// writes the grouping (ids, weights, counts, offsets, sorted_rows, row_pos,
// plan) for the later kernels.  The gate/up rows are streamed as in
// fp8_gate_up_rx_kernel.
template <int NCL>
__global__ __launch_bounds__(256) void fp8_gate_up_token_kernel(
    const float *__restrict__ logits, const uint16_t *__restrict__ x, Fp8Args W,
    int32_t *__restrict__ ids, float *__restrict__ tw, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
    int32_t *__restrict__ row_pos, int32_t *__restrict__ plan, float *__restrict__ h, int d,
    int E, int k, int f) {
    extern __shared__ uint4 xs[];                         // d / 8 x 16 B, + 1 spare
    __shared__ __align__(16) uint32_t tsc[kTopkScratch];
    __shared__ int sel[kMaxTopK];                         // selected experts, ascending
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = d >> 4, nvec = d >> 3, sbk = d >> 7;
    const bool first = blockIdx.x == 0 && blockIdx.y == 0;
    {
        const uint4 *xrow = reinterpret_cast<const uint4 *>(x);
        uint4 tmp[kStageX8];
#pragma unroll
        for (int j = 0; j < kStageX8; ++j)
            tmp[j] = xrow[min((int)threadIdx.x + 256 * j, nvec - 1)];
        loads_done(tmp);
#pragma unroll
        for (int j = 0; j < kStageX8; ++j) {
            const int i = (int)threadIdx.x + 256 * j;
            xs[i < nvec ? i : nvec] = tmp[j];
        }
    }
    if (wid == 0) {
        int e;
        float wt;
        wave_topk_softmax<16>(logits, E, k, tsc, &e, &wt);
        int rank = 0;                                     // place among the selected
        for (int i = 0; i < k; ++i) rank += __shfl(e, i) < e ? 1 : 0;
        if (lane < k) {
            sel[rank] = e;
            if (first) {
                ids[lane] = e;
                tw[lane] = wt;
                sorted_rows[rank] = lane;
                row_pos[lane] = rank;
                plan[1 + rank] = e;
            }
        }
        if (first && lane == 0) plan[0] = k;
    }
    __syncthreads();
    if (first) {
        for (int c = threadIdx.x; c <= E; c += 256) {
            int below = 0, hit = 0;
            for (int i = 0; i < k; ++i) {
                below += sel[i] < c ? 1 : 0;
                hit += sel[i] == c ? 1 : 0;
            }
            offsets[c] = below;
            if (c < E) counts[c] = hit;
        }
    }
    const int a = blockIdx.y;
    const int e = sel[a];
    if ((unsigned)e >= (unsigned)E) return;
    const uint8_t *codes = W.gu_codes + (size_t)e * 2 * f * d;
    const float *scales = W.gu_scales + (size_t)e * (2 * f >> 7) * sbk;
    constexpr int kPerWave = kRxPairs8 / 4;               // pairs n_base + 4 q
    const int n_base = blockIdx.x * kRxPairs8 + wid;
    float *hrow = h + (size_t)a * f;
    Row8<NCL> A, B;
    load_row8<NCL>(codes, scales, n_base, d, sbk, nch, lane, A);
#pragma unroll 1
    for (int q = 0; q < kPerWave; ++q) {
        const int n = n_base + 4 * q;
        load_row8<NCL>(codes, scales, f + n, d, sbk, nch, lane, B);              // up row
        __builtin_amdgcn_sched_barrier(0);
        const float g = row_dot8<NCL>(A, xs, lane, nch);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 1 < kPerWave)
            load_row8<NCL>(codes, scales, n + 4, d, sbk, nch, lane, A);         // next gate row
        __builtin_amdgcn_sched_barrier(0);
        const float u = row_dot8<NCL>(B, xs, lane, nch);
        if (lane == 0) hrow[n] = silu_mul8(g, u);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Down + combine for small T: block (ROWS output rows, token t); wave j
// computes slot j's expert output for the block's rows (j = wid, wid + 16,
// ...) from h row row_pos[t k + j], lane l owning the 16-code chunks l + 64 i
// (i < NCL) of f, whose h values it holds in registers; rows go in batches
// of B in a ring of R batch buffers (R - 1 batches' loads in flight during
// each batch's math).  Each row's partial sums are reduced across the wave
// and parked in LDS; then y = sum_j w_j o_j in fp32, slot order, one writer
// per output.
template <int NCL, int ROWS, int B, int R>
__global__ __launch_bounds__(1024) void fp8_down_combine_kernel(
    const float *__restrict__ h, Fp8Args W, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const int32_t *__restrict__ row_pos,
    uint16_t *__restrict__ y, int T, int d, int E, int k, int f) {
    static_assert(ROWS % B == 0, "whole batches");
    static_assert(R >= 2, "a ring");
    __shared__ float part[kMaxTopK][ROWS];
    const int t = blockIdx.y;
    const int m0 = blockIdx.x * ROWS;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = f >> 4, sbk = f >> 7;
    const int nrows = T * k;
    for (int j = wid; j < k; j += 16) {
        const int e = __builtin_amdgcn_readfirstlane(ids[(size_t)t * k + j]);
        const int p = __builtin_amdgcn_readfirstlane(row_pos[(size_t)t * k + j]);
        if ((unsigned)e < (unsigned)E && (unsigned)p < (unsigned)nrows) {
            const uint8_t *codes = W.dn_codes + (size_t)e * d * f;
            const float *scales = W.dn_scales + (size_t)e * (d >> 7) * sbk;
            const float4 *hrow = reinterpret_cast<const float4 *>(h + (size_t)p * f);
            float4 hv[NCL][4];
#pragma unroll
            for (int i = 0; i < NCL; ++i) {
                const int c = min(lane + 64 * i, nch - 1);
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[i][q] = hrow[4 * c + q];
            }
            constexpr int NB = ROWS / B;
            Row8<NCL> ring[R][B];
#pragma unroll
            for (int b0 = 0; b0 < R - 1 && b0 < NB; ++b0)
#pragma unroll
                for (int rr = 0; rr < B; ++rr)
                    load_row8<NCL>(codes, scales, m0 + b0 * B + rr, f, sbk, nch, lane, ring[b0][rr]);
#pragma unroll
            for (int bi = 0; bi < NB; ++bi) {
                if (bi + R - 1 < NB) {
#pragma unroll
                    for (int rr = 0; rr < B; ++rr)
                        load_row8<NCL>(codes, scales, m0 + (bi + R - 1) * B + rr, f, sbk, nch,
                                       lane, ring[(bi + R - 1) % R][rr]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rr = 0; rr < B; ++rr) {
                    const Row8<NCL> &rb = ring[bi % R][rr];
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < NCL; ++i) {
                        const int c = lane + 64 * i;
                        const float pi = dot16_fp8_f32(rb.c[i], hv[i], 0.f);
                        acc += c < nch ? pi * rb.s[i] : 0.f;
                    }
                    const float o = wave_sum_f32(acc);
                    if (lane == 0) part[j][bi * B + rr] = o;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if (lane < ROWS) {
            part[j][lane] = 0.f;
        }
    }
    __syncthreads();
    if (threadIdx.x < ROWS) {
        float yv = 0.f;
        for (int j = 0; j < k; ++j) yv += topk_w[(size_t)t * k + j] * part[j][threadIdx.x];
        y[(size_t)t * d + m0 + threadIdx.x] = f32_to_bf16_rne(yv);
    }
}

template <int NCL>
hipError_t launch_fp8_rx(const uint16_t *x, Fp8Args w, const int32_t *offsets,
                         const int32_t *sorted_rows, const int32_t *plan, float *h, int T, int d,
                         int E, int k, int f, int amax, hipStream_t s) {
    return timed_launch("fp8_gate_up", fp8_gate_up_rx_kernel<NCL>, dim3(f / kRxPairs8, amax),
                        dim3(256), (size_t)d * 2 + 16, s, x, w, offsets, sorted_rows, plan, h, T,
                        d, E, k, f);
}

}  // namespace

hipError_t launch_fp8_gate_up(const uint16_t *x, Fp8Args w, const int32_t *offsets,
                              const int32_t *sorted_rows, const int32_t *plan, float *h, int T,
                              int d, int E, int k, int f, hipStream_t s) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    if (T <= 8 && d <= 8192 && f % kRxPairs8 == 0) {
        switch ((d + 1023) / 1024) {                      // 16-code chunks per lane
        case 1: return launch_fp8_rx<1>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 2: return launch_fp8_rx<2>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 3: return launch_fp8_rx<3>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 4: return launch_fp8_rx<4>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 5: return launch_fp8_rx<5>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 6: return launch_fp8_rx<6>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        case 7: return launch_fp8_rx<7>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        default: return launch_fp8_rx<8>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s);
        }
    }
    const int rpp = max(1, min(kRows8, 32768 / d));      // <= 64 KB of LDS
    return timed_launch("fp8_gate_up", fp8_gate_up_kernel, dim3(f / kPairs8, amax), dim3(256),
                        (size_t)rpp * d * 2, s, x, w, offsets, sorted_rows, plan, h, T, d, E, k,
                        f, rpp);
}

hipError_t launch_fp8_down(const float *h, Fp8Args w, const int32_t *offsets,
                           const int32_t *plan, uint16_t *rows_out, int T, int d, int E, int k,
                           int f, hipStream_t s) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    const int rpp = max(1, min(kRows8, 16384 / f));      // <= 64 KB of LDS
    return timed_launch("fp8_down", fp8_down_kernel, dim3(d / kDnRows8, amax), dim3(256),
                        (size_t)rpp * f * 4, s, h, w, offsets, plan, rows_out, T, d, E, k, f,
                        rpp);
}

bool fp8_gate_up_token_fusable(int T, int d, int E, int k, int f) {
    return T == 1 && k <= kMaxTopK && k <= E && E <= 1024 && d <= 8192 && d % 128 == 0 &&
           f % kRxPairs8 == 0;
}

hipError_t launch_fp8_gate_up_token(const float *logits, const uint16_t *x, Fp8Args w,
                                    int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                    int32_t *sorted_rows, int32_t *row_pos, int32_t *plan,
                                    float *h, int d, int E, int k, int f, hipStream_t s) {
    const dim3 grid(f / kRxPairs8, k);
    const size_t lds = (size_t)d * 2 + 16;
#define MOE_FP8_TOK(N)                                                                       \
    case N:                                                                                  \
        return timed_launch("fp8_gate_up", fp8_gate_up_token_kernel<N>, grid, dim3(256), lds, s, \
                            logits, x, w, ids, tw, counts, offsets, sorted_rows, row_pos,    \
                            plan, h, d, E, k, f);
    switch ((d + 1023) / 1024) {                          // 16-code chunks per lane
        MOE_FP8_TOK(1) MOE_FP8_TOK(2) MOE_FP8_TOK(3) MOE_FP8_TOK(4)
        MOE_FP8_TOK(5) MOE_FP8_TOK(6) MOE_FP8_TOK(7) MOE_FP8_TOK(8)
    default:
        return hipErrorInvalidValue;
    }
#undef MOE_FP8_TOK
}

bool fp8_down_combine_ok(int T, int d, int k, int f) {
    return T >= 1 && T <= 4 && k <= kMaxTopK && f <= 2048 && f % 128 == 0 && d % 32 == 0;
}

hipError_t launch_fp8_down_combine(const float *h, Fp8Args w, const int32_t *ids,
                                   const float *topk_w, const int32_t *row_pos, uint16_t *y,
                                   int T, int d, int E, int k, int f, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (!fp8_down_combine_ok(T, d, k, f)) return hipErrorInvalidValue;
    // 28 output rows per block where d allows (7168 / 28 = 256 blocks), else 32
    const int ncl = (f / 16 + 63) / 64;
    if (d % 28 == 0) {
        const dim3 grid(d / 28, T);
        if (ncl == 1)
            return timed_launch("fp8_down", fp8_down_combine_kernel<1, 28, 2, 2>, grid, dim3(1024), 0,
                                s, h, w, ids, topk_w, row_pos, y, T, d, E, k, f);
        return timed_launch("fp8_down", fp8_down_combine_kernel<2, 28, 2, 2>, grid, dim3(1024), 0, s,
                            h, w, ids, topk_w, row_pos, y, T, d, E, k, f);
    }
    const dim3 grid(d / 32, T);
    if (ncl == 1)
        return timed_launch("fp8_down", fp8_down_combine_kernel<1, 32, 2, 2>, grid, dim3(1024), 0, s,
                            h, w, ids, topk_w, row_pos, y, T, d, E, k, f);
    return timed_launch("fp8_down", fp8_down_combine_kernel<2, 32, 2, 2>, grid, dim3(1024), 0, s, h,
                        w, ids, topk_w, row_pos, y, T, d, E, k, f);
}

}  // namespace moe
