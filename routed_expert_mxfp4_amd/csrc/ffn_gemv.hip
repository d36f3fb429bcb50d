// ffn_gemv.hip -- routed expert FFN for decode-sized row groups (gfx950).
//
// Decode reads each selected expert once and does little arithmetic per
// byte, so this path is bound by HBM bandwidth: each wave streams whole
// MXFP4 rows with 16-byte loads (one 32-element MX block per lane), decodes
// E2M1 pairs to bf16 with the gfx950 scaled convert (scale 1), takes bf16
// dot products against the activations held in LDS, and applies the block's
// E8M0 scale to the fp32 partial sum with an exact ldexp.  Every decoded
// weight is reused for all rows (tokens) of the expert held in LDS.
//
// Gate/up: for expert e with rows p in [offsets[e], offsets[e+1]),
//   g = x_t . Wg[n], u = x_t . Wu[n], h[p][n] = silu(g) * u   (fp32)
// with t = sorted_rows[p] / k, gate rows [0,f), up rows [f,2f).
// Down: o[p][m] = h[p] . Wd[m] -> bf16 rows_out (expert-major), or fused
// with the weighted combine per token for small T.
#include "moe_internal.hpp"
#include "mx_split.hpp"
#include "select_dev.hpp"

namespace moe {
namespace {

constexpr int kRowsMax = 4;          // token rows of one expert per LDS pass
constexpr int kGuPairs = 16;         // gate/up output pairs per block
constexpr int kDnRows = 64;          // down output rows per block

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + expf(-g)) * u;
}

// Expert-group bounds from device data, checked so that malformed plans can
// never index outside the arrays.
__device__ __forceinline__ bool expert_group(const int32_t *plan, const int32_t *offsets,
                                             int a, int E, int nrows, int &e, int &row0,
                                             int &ne) {
    if (a >= plan[0]) return false;
    e = plan[1 + a];
    if ((unsigned)e >= (unsigned)E) return false;
    row0 = offsets[e];
    ne = offsets[e + 1] - row0;
    return row0 >= 0 && ne > 0 && row0 + ne <= nrows;
}

__global__ __launch_bounds__(256) void gemv_gate_up_kernel(
    const uint16_t *__restrict__ x, ExpertArgs W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_rows, const int32_t *__restrict__ plan,
    float *__restrict__ h, int T, int d, int E, int k, int f, int rows_per_pass) {
    const int nrows = T * k;
    int e, row0, ne;
    if (!expert_group(plan, offsets, blockIdx.y, E, nrows, e, row0, ne)) return;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nblk = d >> 5;
    const size_t code_row = (size_t)d >> 1;
    const uint8_t *codes = W.gu_codes + (size_t)e * 2 * f * code_row;
    const uint8_t *scales = W.gu_scales + (size_t)e * 2 * f * nblk;
    extern __shared__ uint4 xs4[];                // [rows_per_pass][d/8]
    const int nvec = d >> 3;
    const int n_base = blockIdx.x * kGuPairs;

    for (int r0 = 0; r0 < ne; r0 += rows_per_pass) {
        const int R = min(rows_per_pass, ne - r0);
        __syncthreads();
        for (int i = threadIdx.x; i < R * nvec; i += 256) {
            const int r = i / nvec, v = i - r * nvec;
            const int row = sorted_rows[row0 + r0 + r];
            const int tok = (unsigned)row < (unsigned)nrows ? row / k : 0;
            xs4[r * nvec + v] = reinterpret_cast<const uint4 *>(x + (size_t)tok * d)[v];
        }
        __syncthreads();
        for (int p = wid; p < kGuPairs; p += 4) {
            const int n = n_base + p;
            const uint8_t *grow = codes + (size_t)n * code_row;
            const uint8_t *urow = codes + (size_t)(f + n) * code_row;
            const uint8_t *gsc = scales + (size_t)n * nblk;
            const uint8_t *usc = scales + (size_t)(f + n) * nblk;
            float g[kRowsMax], u[kRowsMax];
#pragma unroll
            for (int r = 0; r < kRowsMax; ++r) g[r] = u[r] = 0.f;
            for (int b = lane; b < nblk; b += 64) {
                const uint4 cg = *reinterpret_cast<const uint4 *>(grow + 16 * (size_t)b);
                const uint4 cu = *reinterpret_cast<const uint4 *>(urow + 16 * (size_t)b);
                const uint32_t sg = gsc[b], su = usc[b];
#pragma unroll
                for (int r = 0; r < kRowsMax; ++r) {
                    if (r < R) {
                        const uint4 *xv = xs4 + r * nvec + 4 * b;
                        float pg = 0.f, pu = 0.f;
                        pg = dot8_fp4_bf16(cg.x, xv[0], pg);
                        pu = dot8_fp4_bf16(cu.x, xv[0], pu);
                        pg = dot8_fp4_bf16(cg.y, xv[1], pg);
                        pu = dot8_fp4_bf16(cu.y, xv[1], pu);
                        pg = dot8_fp4_bf16(cg.z, xv[2], pg);
                        pu = dot8_fp4_bf16(cu.z, xv[2], pu);
                        pg = dot8_fp4_bf16(cg.w, xv[3], pg);
                        pu = dot8_fp4_bf16(cu.w, xv[3], pu);
                        g[r] += apply_e8m0(pg, sg);
                        u[r] += apply_e8m0(pu, su);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < kRowsMax; ++r) {
                if (r < R) {
                    const float gs = wave_sum_f32(g[r]);
                    const float us = wave_sum_f32(u[r]);
                    if (lane == 0) h[(size_t)(row0 + r0 + r) * f + n] = silu_mul(gs, us);
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void gemv_down_kernel(
    const float *__restrict__ h, ExpertArgs W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ plan, uint16_t *__restrict__ rows_out, int T, int d, int E,
    int k, int f, int rows_per_pass) {
    const int nrows = T * k;
    int e, row0, ne;
    if (!expert_group(plan, offsets, blockIdx.y, E, nrows, e, row0, ne)) return;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int grp = lane >> 4, gl = lane & 15;
    const int nblk = f >> 5;
    const size_t code_row = (size_t)f >> 1;
    const uint8_t *codes = W.dn_codes + (size_t)e * d * code_row;
    const uint8_t *scales = W.dn_scales + (size_t)e * d * nblk;
    extern __shared__ float4 hs4[];               // [rows_per_pass][f/4]
    const int nv = f >> 2;
    const int m_base = blockIdx.x * kDnRows + wid * 16 + grp * 4;

    for (int r0 = 0; r0 < ne; r0 += rows_per_pass) {
        const int R = min(rows_per_pass, ne - r0);
        __syncthreads();
        for (int i = threadIdx.x; i < R * nv; i += 256) {
            const int r = i / nv, v = i - r * nv;
            hs4[r * nv + v] = reinterpret_cast<const float4 *>(h + (size_t)(row0 + r0 + r) * f)[v];
        }
        __syncthreads();
        float acc[4][kRowsMax];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRowsMax; ++r) acc[q][r] = 0.f;
        for (int b = gl; b < nblk; b += 16) {
            uint4 c[4];
            uint32_t sc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = *reinterpret_cast<const uint4 *>(codes + (size_t)(m_base + q) * code_row +
                                                        16 * (size_t)b);
                sc[q] = scales[(size_t)(m_base + q) * nblk + b];
            }
#pragma unroll
            for (int r = 0; r < kRowsMax; ++r) {
                if (r < R) {
                    const float4 *hv = hs4 + r * nv + 8 * b;
                    float4 hv0 = hv[0], hv1 = hv[1], hv2 = hv[2], hv3 = hv[3];
                    float4 hv4 = hv[4], hv5 = hv[5], hv6 = hv[6], hv7 = hv[7];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float s = 0.f;
                        s = dot8_fp4_f32(c[q].x, hv0, hv1, s);
                        s = dot8_fp4_f32(c[q].y, hv2, hv3, s);
                        s = dot8_fp4_f32(c[q].z, hv4, hv5, s);
                        s = dot8_fp4_f32(c[q].w, hv6, hv7, s);
                        acc[q][r] += apply_e8m0(s, sc[q]);
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < kRowsMax; ++r) {
                if (r < R) {
                    const float v = group16_sum_f32(acc[q][r]);
                    if (gl == 0)
                        rows_out[(size_t)(row0 + r0 + r) * d + m_base + q] = f32_to_bf16_rne(v);
                }
            }
    }
}

// Small T: y[t][m] = sum_j w[t][j] * (h[row_pos[t*k+j]] . Wd_{e_j}[m]) in
// fp32, slot order j = 0..k-1, one wave per (token, 16 output rows).
__global__ __launch_bounds__(64) void down_combine_kernel(
    const float *__restrict__ h, ExpertArgs W, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const int32_t *__restrict__ row_pos,
    uint16_t *__restrict__ y, int T, int d, int E, int k, int f) {
    const int t = blockIdx.y;
    const int lane = threadIdx.x, grp = lane >> 4, gl = lane & 15;
    const int m_base = blockIdx.x * 16 + grp * 4;
    const int nblk = f >> 5;
    const size_t code_row = (size_t)f >> 1;
    const int nrows = T * k;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int p = row_pos[(size_t)t * k + j];
        if ((unsigned)e >= (unsigned)E || (unsigned)p >= (unsigned)nrows) continue;
        const float wj = topk_w[(size_t)t * k + j];
        const uint8_t *codes = W.dn_codes + (size_t)e * d * code_row;
        const uint8_t *scales = W.dn_scales + (size_t)e * d * nblk;
        const float4 *hrow = reinterpret_cast<const float4 *>(h + (size_t)p * f);
        float part[4] = {0.f, 0.f, 0.f, 0.f};
        for (int b = gl; b < nblk; b += 16) {
            uint4 c[4];
            uint32_t sc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = *reinterpret_cast<const uint4 *>(codes + (size_t)(m_base + q) * code_row +
                                                        16 * (size_t)b);
                sc[q] = scales[(size_t)(m_base + q) * nblk + b];
            }
            const float4 *hv = hrow + 8 * b;
            float4 hv0 = hv[0], hv1 = hv[1], hv2 = hv[2], hv3 = hv[3];
            float4 hv4 = hv[4], hv5 = hv[5], hv6 = hv[6], hv7 = hv[7];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = 0.f;
                s = dot8_fp4_f32(c[q].x, hv0, hv1, s);
                s = dot8_fp4_f32(c[q].y, hv2, hv3, s);
                s = dot8_fp4_f32(c[q].z, hv4, hv5, s);
                s = dot8_fp4_f32(c[q].w, hv6, hv7, s);
                part[q] += apply_e8m0(s, sc[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += wj * group16_sum_f32(part[q]);
    }
    if (gl == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) y[(size_t)t * d + m_base + q] = f32_to_bf16_rne(acc[q]);
    }
}

// ---------------------------------------------------------------------------
// Decode-shaped kernels: activations and h in registers, every weight load of
// a row issued before any of it is used, DPP lane reductions.
// ---------------------------------------------------------------------------
constexpr int kRxPairs = 32;         // gate/up pairs per block (8 per wave)
constexpr int kRxRows = 4;           // token rows per weight pass (x split: 4 x d x 2 B of LDS)
// the one-token kernel: 96, 48 or 32 pairs per block (launch_gate_up_token_t)

// Gate/up for decode-sized groups, software-pipelined: lane l owns the MX
// blocks b = l + 64 i (i < NBL) of d; the token row is split once into LDS
// (shared by the block's four waves) and each wave streams its output pairs
// with the next pair's code loads issued before the current pair's dots (on
// the matrix cores, below), so HBM reads and arithmetic overlap instead of
// alternating.
// h elements: fp32, or bf16 (the one-token and few-token paths of the bf16
// mode, whose down pass then dots bf16 pairs, as the gate/up pass does).
__device__ __forceinline__ void put_h(float *p, float v) { *p = v; }
__device__ __forceinline__ void put_h(uint16_t *p, float v) { *p = f32_to_bf16_rne(v); }

template <int NBL>
struct PairBuf {
    uint4 c[2][NBL];       // gate, up
    uint32_t s[2][NBL];
};

template <int NBL>
__device__ __forceinline__ void load_pair(rsrc_t codes, rsrc_t scales, int n, int f, int lane,
                                          int nblk, uint32_t code_row, PairBuf<NBL> &pb) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const uint32_t row = (uint32_t)(n + v * f);                 // wave-uniform
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
            const uint32_t b = (uint32_t)min(lane + 64 * i, nblk - 1);
            pb.c[v][i] = buf_load16(codes, 16u * b, row * code_row);
            pb.s[v][i] = buf_load8(scales, b, row * (uint32_t)nblk);
        }
    }
}

// ---------------------------------------------------------------------------
// Dots on the matrix cores, with the GEMV's load pattern.  A wave
// streams one weight row at a time as the vector-ALU kernel does (lane l
// holds the MX blocks l + 64 i of the row), and one scaled MFMA
// (16x16x128, FP6 x FP4) per i takes those 64 blocks as its B operand -- B
// row l % 16, K group l / 16 is lane l's block, with the block's own E8M0
// scale -- against the same blocks of x as A (each lane's x block split in
// two MX E2M3 terms, two MFMAs).  C[j][j] is then the dot over the four
// blocks of lanes j + 16 g, so the trace of C is the row's dot product; the
// off-diagonal products are not used.  The weights need no conversion on
// the vector ALU; x is split once per token row into LDS.
// ---------------------------------------------------------------------------
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One lane's A operand: its x block as two E2M3 terms and their scales
// (byte 0 hi, byte 1 lo).  Lanes past the end of d hold zero codes.
struct XSplit {
    i32x8_t hi, lo;
    uint32_t sc;
};

// The trace of a 16 x 16 product: lane l holds C[4 (l / 16) + r][l % 16] in
// acc[r], so the diagonal sits in lanes 16 g + c with r = c - 4 g in 0..3.
__device__ __forceinline__ float mfma_trace16(f32x4_t acc, int lane) {
    const int r = (lane & 15) - 4 * (lane >> 4);
    float v = 0.f;
    v = r == 0 ? acc[0] : v;
    v = r == 1 ? acc[1] : v;
    v = r == 2 ? acc[2] : v;
    v = r == 3 ? acc[3] : v;
    return wave_sum_f32(v);
}

template <int NBL>
__device__ __forceinline__ float pair_h_mfma(const PairBuf<NBL> &pb, const XSplit (&xa)[NBL],
                                             int lane, int nblk) {
    f32x4_t cg = {0.f, 0.f, 0.f, 0.f}, cu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        const bool ok = lane + 64 * i < nblk;
        const uint4 wg = pb.c[0][i], wu = pb.c[1][i];
        const i32x8_t bg = {(int)wg.x, (int)wg.y, (int)wg.z, (int)wg.w, 0, 0, 0, 0};
        const i32x8_t bu = {(int)wu.x, (int)wu.y, (int)wu.z, (int)wu.w, 0, 0, 0, 0};
        // lanes past the end carry a duplicate block: scale 2^0 against zero x
        const int sg = ok ? (int)pb.s[0][i] : 127, su = ok ? (int)pb.s[1][i] : 127;
        cg = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[i].hi, bg, cg, 2, 4, 0, (int)xa[i].sc, 0, sg);
        cu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[i].hi, bu, cu, 2, 4, 0, (int)xa[i].sc, 0, su);
        cg = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[i].lo, bg, cg, 2, 4, 1, (int)xa[i].sc, 0, sg);
        cu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa[i].lo, bu, cu, 2, 4, 1, (int)xa[i].sc, 0, su);
    }
    return silu_mul(mfma_trace16(cg, lane), mfma_trace16(cu, lane));
}

// A row (bf16 x or fp32 h) split into records of 64 bytes per MX block in
// LDS: hi codes [0, 24), lo codes [24, 48), scales at 48 (hi) and 49 (lo);
// threads t0, t0 + stride, .. take a block each.
__device__ __forceinline__ void block_values(const uint16_t *__restrict__ row, int b, float (&v)[32]) {
    const uint4 *xb = reinterpret_cast<const uint4 *>(row) + 4 * b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 w = xb[q];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v[8 * q + 2 * t] = __uint_as_float(ww[t] << 16);
            v[8 * q + 2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u);
        }
    }
}
__device__ __forceinline__ void block_values(const float *__restrict__ row, int b, float (&v)[32]) {
    const float4 *hb = reinterpret_cast<const float4 *>(row) + 8 * b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 w = hb[q];
        v[4 * q] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
    }
}
template <typename RT>
__device__ __forceinline__ void split_x_to_lds(const RT *__restrict__ xrow, int nblk, int t0,
                                               int stride, uint4 *xsr) {
    for (int b = t0; b < nblk; b += stride) {
        float v[32];
        block_values(xrow, b, v);
        const SplitBlock sb = split_block32(v);
        xsr[4 * b + 0] = uint4{sb.hi[0], sb.hi[1], sb.hi[2], sb.hi[3]};
        xsr[4 * b + 1] = uint4{sb.hi[4], sb.hi[5], sb.lo[0], sb.lo[1]};
        xsr[4 * b + 2] = uint4{sb.lo[2], sb.lo[3], sb.lo[4], sb.lo[5]};
        xsr[4 * b + 3] = uint4{sb.scales, 0u, 0u, 0u};
    }
}

// The lane's A operands (blocks lane + 64 i) from the split records.
template <int NBL>
__device__ __forceinline__ void load_xsplit(const uint4 *xsr, int lane, int nblk,
                                            XSplit (&xa)[NBL]) {
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
        const int b = lane + 64 * i;
        if (b < nblk) {
            const uint4 q0 = xsr[4 * b], q1 = xsr[4 * b + 1], q2 = xsr[4 * b + 2], q3 = xsr[4 * b + 3];
            xa[i].hi = i32x8_t{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, 0, 0};
            xa[i].lo = i32x8_t{(int)q1.z, (int)q1.w, (int)q2.x, (int)q2.y, (int)q2.z, (int)q2.w, 0, 0};
            xa[i].sc = q3.x;
        } else {
            xa[i].hi = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
            xa[i].lo = xa[i].hi;
            xa[i].sc = 0x7F7Fu;
        }
    }
}

// Experts a = blockIdx.y, blockIdx.y + gridDim.y, ... of the plan.  h row of
// (expert a, its r-th row): row0 + r, or a * hstride + r when hstride > 0
// (the compact rows of the mixed path's small experts).
template <int NBL, typename HT>
__global__ __launch_bounds__(256) void gate_up_regx_kernel(
    const uint16_t *__restrict__ x, ExpertArgs W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_rows, const int32_t *__restrict__ plan,
    HT *__restrict__ h, int T, int d, int E, int k, int f, int hstride) {
    const int nrows = T * k;
    for (int a = blockIdx.y; a < plan[0]; a += gridDim.y) {
    int e, row0, ne;
    if (!expert_group(plan, offsets, a, E, nrows, e, row0, ne)) continue;
    if (hstride > 0 && ne > hstride) continue;
    extern __shared__ uint4 xsr[];                // kRxRows token rows split, d/32 records of 64 B each
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nblk = d >> 5;
    const uint32_t code_row = (uint32_t)d >> 1;
    const rsrc_t codes = make_rsrc(W.gu_codes + (size_t)e * 2 * f * code_row, 2u * f * code_row);
    const rsrc_t scales = make_rsrc(W.gu_scales + (size_t)e * 2 * f * nblk, 2u * f * nblk);
    constexpr int kPerWave = kRxPairs / 4;        // pairs n_base + wid + 4 q
    const int n_base = blockIdx.x * kRxPairs + wid;
    // the expert's rows in chunks of up to kRxRows: each chunk's x rows are
    // split into LDS once and every weight pair, loaded once, is dotted with
    // all of them (weights are not re-streamed per row within a chunk)
    for (int r0 = 0; r0 < ne; r0 += kRxRows) {
        const int nr = min(kRxRows, ne - r0);   // block-uniform
        PairBuf<NBL> A, B;
        load_pair<NBL>(codes, scales, n_base, f, lane, nblk, code_row, A);   // before the x sync
        __syncthreads();                            // the previous chunk's records are read
        for (int r = 0; r < nr; ++r) {
            const int row = sorted_rows[row0 + r0 + r];
            const int tok = (unsigned)row < (unsigned)nrows ? row / k : 0;
            split_x_to_lds(x + (size_t)tok * d, nblk, (int)threadIdx.x, 256, xsr + 4 * nblk * r);
        }
        __syncthreads();
        HT *hrow = h + (size_t)(hstride > 0 ? a * hstride + r0 : row0 + r0) * f;
        if (nr == 1) {
            // one row: its split x stays in registers for the whole pass
            XSplit xa[NBL];
            load_xsplit<NBL>(xsr, lane, nblk, xa);
            // sched_barrier keeps each stage in place: a later pair's loads
            // may not be hoisted above an earlier pair's math (that would
            // only grow the register footprint, not the bytes in flight)
#pragma unroll 1
            for (int q = 0; q < kPerWave; q += 2) {
                load_pair<NBL>(codes, scales, n_base + 4 * (q + 1), f, lane, nblk, code_row, B);
                __builtin_amdgcn_sched_barrier(0);
                const float va = pair_h_mfma<NBL>(A, xa, lane, nblk);
                if (lane == 0) put_h(hrow + n_base + 4 * q, va);
                __builtin_amdgcn_sched_barrier(0);
                if (q + 2 < kPerWave)
                    load_pair<NBL>(codes, scales, n_base + 4 * (q + 2), f, lane, nblk, code_row, A);
                __builtin_amdgcn_sched_barrier(0);
                const float vb = pair_h_mfma<NBL>(B, xa, lane, nblk);
                if (lane == 0) put_h(hrow + n_base + 4 * (q + 1), vb);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // several rows: each row's split x is read from LDS per pair
#pragma unroll 1
            for (int q = 0; q < kPerWave; q += 2) {
                load_pair<NBL>(codes, scales, n_base + 4 * (q + 1), f, lane, nblk, code_row, B);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
                for (int r = 0; r < nr; ++r) {
                    XSplit xa[NBL];
                    load_xsplit<NBL>(xsr + 4 * nblk * r, lane, nblk, xa);
                    const float va = pair_h_mfma<NBL>(A, xa, lane, nblk);
                    if (lane == 0) put_h(hrow + (size_t)r * f + n_base + 4 * q, va);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (q + 2 < kPerWave)
                    load_pair<NBL>(codes, scales, n_base + 4 * (q + 2), f, lane, nblk, code_row, A);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
                for (int r = 0; r < nr; ++r) {
                    XSplit xa[NBL];
                    load_xsplit<NBL>(xsr + 4 * nblk * r, lane, nblk, xa);
                    const float vb = pair_h_mfma<NBL>(B, xa, lane, nblk);
                    if (lane == 0) put_h(hrow + (size_t)r * f + n_base + 4 * (q + 1), vb);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    }
}

// One token (T = 1): the top-k and the grouping happen inside the gate/up
// pass.  Every block selects the token's experts itself from the logits row
// (E floats, read by wave 0) while waves 1..3 split x; the k selected
// experts are distinct, so in ascending expert order the a-th of them is
// the one whose h row is a, routed from top-k slot sorted_rows[a] -- exactly
// the grouping of the permute step.  Block (0, 0) writes that grouping (ids,
// weights, counts, offsets, sorted_rows, row_pos, plan) for the later
// kernels.  Each wave streams its output pairs as gate_up_regx_kernel does,
// the next pair's loads issued before the current pair's products.
template <int NBL, int PAIRS, typename HT, int NWV>
__global__ __launch_bounds__(64 * NWV) void gate_up_mfma_token_kernel(
    const float *__restrict__ logits, const uint16_t *__restrict__ x, ExpertArgs W,
    int32_t *__restrict__ ids, float *__restrict__ tw, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_rows,
    int32_t *__restrict__ row_pos, int32_t *__restrict__ plan, HT *__restrict__ h, int d,
    int E, int k, int f) {
    extern __shared__ uint4 xsr[];                // [d / 32] split records of 64 bytes
    __shared__ __align__(16) uint32_t tsc[kTopkScratch];
    __shared__ int sel[32];                       // selected experts, ascending
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nblk = d >> 5;
    const bool first = blockIdx.x == 0 && blockIdx.y == 0;
    if (wid == 0) {
        int e;
        float wt;
        wave_topk_softmax<16>(logits, E, k, tsc, &e, &wt);
        int rank = 0;                               // place among the selected
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
    } else {
        split_x_to_lds(x, nblk, (int)threadIdx.x - 64, 64 * (NWV - 1), xsr);   // waves 1..
    }
    __syncthreads();
    if (first) {
        for (int c = threadIdx.x; c <= E; c += 64 * NWV) {
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
    XSplit xa[NBL];
    load_xsplit<NBL>(xsr, lane, nblk, xa);
    const uint32_t code_row = (uint32_t)d >> 1;
    const rsrc_t codes = make_rsrc(W.gu_codes + (size_t)e * 2 * f * code_row, 2u * f * code_row);
    const rsrc_t scales = make_rsrc(W.gu_scales + (size_t)e * 2 * f * nblk, 2u * f * nblk);
    constexpr int kPerWave = PAIRS / NWV;         // pairs n_base + wid + NWV q
    static_assert(kPerWave % 2 == 0, "pairs go two at a time");
    const int n_base = blockIdx.x * PAIRS + wid;
    HT *hrow = h + (size_t)a * f;
    PairBuf<NBL> A, B;
    load_pair<NBL>(codes, scales, n_base, f, lane, nblk, code_row, A);
#pragma unroll 1
    for (int q = 0; q < kPerWave; q += 2) {
        load_pair<NBL>(codes, scales, n_base + NWV * (q + 1), f, lane, nblk, code_row, B);
        __builtin_amdgcn_sched_barrier(0);
        const float va = pair_h_mfma<NBL>(A, xa, lane, nblk);
        if (lane == 0) put_h(hrow + n_base + NWV * q, va);
        __builtin_amdgcn_sched_barrier(0);
        if (q + 2 < kPerWave)
            load_pair<NBL>(codes, scales, n_base + NWV * (q + 2), f, lane, nblk, code_row, A);
        __builtin_amdgcn_sched_barrier(0);
        const float vb = pair_h_mfma<NBL>(B, xa, lane, nblk);
        if (lane == 0) put_h(hrow + n_base + NWV * (q + 1), vb);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Down rows for one h row: lane l owns the MX blocks b = l + 64 i (i < NBLD)
// of f, so its slice of h (32 values per block: eight float4, or four uint4
// of bf16 pairs) is loaded once into registers and reused for every output
// row; rows go in batches whose code loads are all in flight together, and
// each row's partial sums are reduced across the wave.  Lanes past the end
// of f load a duplicate of the last block; split_h_slice turns it into zero
// codes, so the loads need no select and can stay in flight.
constexpr int kDnBatch = 4;

template <int NBLD>
__device__ __forceinline__ void load_h_slice(rsrc_t hbuf, uint32_t hrow_off, int lane, int nblk,
                                             float4 (&hv)[NBLD][8]) {
#pragma unroll
    for (int i = 0; i < NBLD; ++i) {
        const uint32_t b = (uint32_t)min(lane + 64 * i, nblk - 1);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            hv[i][q] = __builtin_bit_cast(float4, buf_load16(hbuf, 128u * b + 16u * q, hrow_off));
    }
}

template <int NBLD>
__device__ __forceinline__ void load_h_slice(rsrc_t hbuf, uint32_t hrow_off, int lane, int nblk,
                                             uint4 (&hv)[NBLD][4]) {
#pragma unroll
    for (int i = 0; i < NBLD; ++i) {
        const uint32_t b = (uint32_t)min(lane + 64 * i, nblk - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) hv[i][q] = buf_load16(hbuf, 64u * b + 16u * q, hrow_off);
    }
}

// The lane's h slice of NBLD blocks: eight float4 per block for fp32 h,
// four uint4 (bf16 pairs) for bf16 h.
template <typename HT> struct HPart { typedef float4 type[8]; };
template <> struct HPart<uint16_t> { typedef uint4 type[4]; };

// Down rows in batches of kDnBatch: load_batch issues every code and scale
// load of a batch, dot_batch_mfma does its math (out[rr] = h . Wd[m + rr], every
// lane gets the sums).  Callers issue the next batch's loads before the
// current batch's math.
__device__ __forceinline__ void store_bf16x4(uint16_t *dst, const float (&v)[kDnBatch]) {
    uint2 o;
    o.x = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
    o.y = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<uint2 *>(dst) = o;
}

template <int NBLD, int B = kDnBatch>
struct RowBuf {
    uint4 c[B][NBLD];
    uint32_t s[B][NBLD];
};

template <int NBLD, int B = kDnBatch>
__device__ __forceinline__ void load_batch(rsrc_t codes, rsrc_t scales, int m, int lane,
                                           int nblk, uint32_t code_row, RowBuf<NBLD, B> &rb) {
#pragma unroll
    for (int rr = 0; rr < B; ++rr)
#pragma unroll
        for (int i = 0; i < NBLD; ++i) {
            const uint32_t b = (uint32_t)min(lane + 64 * i, nblk - 1);
            const uint32_t row = (uint32_t)(m + rr);                  // wave-uniform
            rb.c[rr][i] = buf_load16(codes, 16u * b, row * code_row);
            rb.s[rr][i] = buf_load8(scales, b, row * (uint32_t)nblk);
        }
}

// The lane's h slice as the matrix cores' A operand: each MX block of it
// split in two E2M3 terms (lanes past the end of f: zero codes).
__device__ __forceinline__ void h_block_values(const float4 (&hv)[8], float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        v[4 * q] = hv[q].x;
        v[4 * q + 1] = hv[q].y;
        v[4 * q + 2] = hv[q].z;
        v[4 * q + 3] = hv[q].w;
    }
}
__device__ __forceinline__ void h_block_values(const uint4 (&hv)[4], float (&v)[32]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t ww[4] = {hv[q].x, hv[q].y, hv[q].z, hv[q].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v[8 * q + 2 * t] = __uint_as_float(ww[t] << 16);
            v[8 * q + 2 * t + 1] = __uint_as_float(ww[t] & 0xFFFF0000u);
        }
    }
}

template <int NBLD, typename HV>
__device__ __forceinline__ void split_h_slice(const HV (&hv)[NBLD], int lane, int nblk,
                                              XSplit (&ha)[NBLD]) {
#pragma unroll
    for (int i = 0; i < NBLD; ++i) {
        float v[32];
        h_block_values(hv[i], v);
        const SplitBlock sb = split_block32(v);
        const bool ok = lane + 64 * i < nblk;
        ha[i].hi = ok ? i32x8_t{(int)sb.hi[0], (int)sb.hi[1], (int)sb.hi[2], (int)sb.hi[3],
                                (int)sb.hi[4], (int)sb.hi[5], 0, 0}
                      : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        ha[i].lo = ok ? i32x8_t{(int)sb.lo[0], (int)sb.lo[1], (int)sb.lo[2], (int)sb.lo[3],
                                (int)sb.lo[4], (int)sb.lo[5], 0, 0}
                      : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        ha[i].sc = ok ? sb.scales : 0x7F7Fu;
    }
}

// out[rr] = h . Wd[m + rr] for a batch: per row and MX block of the lanes,
// two scaled MFMAs (the h terms against the row's blocks, as in
// pair_h_mfma), the row's dot the trace of the product.
template <int NBLD, int B>
__device__ __forceinline__ void dot_batch_mfma(const RowBuf<NBLD, B> &rb, const XSplit (&ha)[NBLD],
                                               int lane, int nblk, float (&out)[B]) {
    f32x4_t c[B];
#pragma unroll
    for (int rr = 0; rr < B; ++rr) c[rr] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NBLD; ++i) {
        const bool ok = lane + 64 * i < nblk;
#pragma unroll
        for (int rr = 0; rr < B; ++rr) {
            const uint4 w = rb.c[rr][i];
            const i32x8_t bw = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
            const int sw = ok ? (int)rb.s[rr][i] : 127;
            c[rr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ha[i].hi, bw, c[rr], 2, 4, 0, (int)ha[i].sc, 0, sw);
            c[rr] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ha[i].lo, bw, c[rr], 2, 4, 1, (int)ha[i].sc, 0, sw);
        }
    }
#pragma unroll
    for (int rr = 0; rr < B; ++rr) out[rr] = mfma_trace16(c[rr], lane);
}

// Fused down + combine for small T: block (ROWS output rows, token t) of NW
// waves; wave j computes slot j's expert output for the block's rows (j =
// wid, wid + NW, ...) in batches of B rows held in a ring of R batch buffers,
// so R - 1 batches' loads are in flight during each batch's math, and parks
// it in LDS; then y = sum_j w_j o_j in fp32, slot order, one writer per
// output.  ROWS is a multiple of B.
template <int NBLD, int ROWS, int B, int R, int NW, typename HT>
__global__ __launch_bounds__(64 * NW) void down_combine_split_kernel(
    const HT *__restrict__ h, ExpertArgs W, const int32_t *__restrict__ ids,
    const float *__restrict__ topk_w, const int32_t *__restrict__ row_pos,
    uint16_t *__restrict__ y, int T, int d, int E, int k, int f) {
    static_assert(ROWS % B == 0, "whole batches");
    static_assert(R >= 2, "a ring");
    __shared__ float part[kMaxTopK][ROWS];
    const int t = blockIdx.y;
    const int m0 = blockIdx.x * ROWS;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nblk = f >> 5;
    const uint32_t code_row = (uint32_t)f >> 1;
    const int nrows = T * k;
    const rsrc_t hbuf = make_rsrc(h, (uint32_t)min((size_t)nrows * f * sizeof(HT), (size_t)0xFFFFFFF0u));
    for (int j = wid; j < k; j += NW) {
        const int e = __builtin_amdgcn_readfirstlane(ids[(size_t)t * k + j]);
        const int p = __builtin_amdgcn_readfirstlane(row_pos[(size_t)t * k + j]);
        const bool ok = (unsigned)e < (unsigned)E && (unsigned)p < (unsigned)nrows;
        if (ok) {
            const rsrc_t codes = make_rsrc(W.dn_codes + (size_t)e * d * code_row, (uint32_t)d * code_row);
            const rsrc_t scales = make_rsrc(W.dn_scales + (size_t)e * d * nblk, (uint32_t)d * nblk);
            // h first, then the ring's first weight loads, then the split:
            // the split waits for h alone while the weights are in flight
            typename HPart<HT>::type hv[NBLD];
            load_h_slice<NBLD>(hbuf, (uint32_t)p * f * (uint32_t)sizeof(HT), lane, nblk, hv);
            constexpr int NB = ROWS / B;
            RowBuf<NBLD, B> ring[R];
#pragma unroll
            for (int i = 0; i < R - 1 && i < NB; ++i)
                load_batch<NBLD, B>(codes, scales, m0 + i * B, lane, nblk, code_row, ring[i]);
            XSplit ha[NBLD];
            split_h_slice<NBLD>(hv, lane, nblk, ha);
#pragma unroll
            for (int bi = 0; bi < NB; ++bi) {
                if (bi + R - 1 < NB)
                    load_batch<NBLD, B>(codes, scales, m0 + (bi + R - 1) * B, lane, nblk, code_row,
                                        ring[(bi + R - 1) % R]);
                __builtin_amdgcn_sched_barrier(0);
                float out[B];
                dot_batch_mfma<NBLD, B>(ring[bi % R], ha, lane, nblk, out);
                if (lane == 0) {
#pragma unroll
                    for (int rr = 0; rr < B; ++rr) part[j][bi * B + rr] = out[rr];
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

// Expert-major down for decode-sized groups: block (64 output rows, expert
// a), 16 rows per wave.  An expert's token rows go one at a time, the
// lane's split h slice in registers -- or, with kMulti and several rows,
// kDnTokRows at a time through LDS, each weight batch loaded once for all
// of them.  kMulti is off where every expert has one row (the small experts
// of a scaled-MFMA call at a crossover of one row): that path keeps the
// lighter code.
constexpr int kDnTokRows = 4;
template <int NBLD, bool kMulti>
__global__ __launch_bounds__(256) void down_rows_kernel(
    const float *__restrict__ h, ExpertArgs W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ plan, uint16_t *__restrict__ rows_out, int T, int d, int E,
    int k, int f, int hstride) {
    extern __shared__ uint4 hsr[];                // kDnTokRows h rows split, f/32 records of 64 B each
    const int nrows = T * k;
    for (int a = blockIdx.y; a < plan[0]; a += gridDim.y) {
    int e, row0, ne;
    if (!expert_group(plan, offsets, a, E, nrows, e, row0, ne)) continue;
    if (hstride > 0 && ne > hstride) continue;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int nblk = f >> 5;
    const uint32_t code_row = (uint32_t)f >> 1;
    const int m = blockIdx.x * 64 + wid * 16;
    const rsrc_t codes = make_rsrc(W.dn_codes + (size_t)e * d * code_row, (uint32_t)d * code_row);
    const rsrc_t scales = make_rsrc(W.dn_scales + (size_t)e * d * nblk, (uint32_t)d * nblk);
    const rsrc_t hbuf = make_rsrc(h + (size_t)(hstride > 0 ? a * hstride : row0) * f,
                                  (uint32_t)ne * f * 4u);
    auto one_row = [&](int r) {
        // the lane's split h slice stays in registers (issuing batch A's
        // loads before the split costs this kernel a quarter of its waves:
        // more registers live across the split)
        XSplit ha[NBLD];
        {
            float4 hv[NBLD][8];
            load_h_slice<NBLD>(hbuf, (uint32_t)r * f * 4u, lane, nblk, hv);
            split_h_slice<NBLD>(hv, lane, nblk, ha);
        }
        uint16_t *orow = rows_out + (size_t)(row0 + r) * d + m;
        RowBuf<NBLD> A, B;
        load_batch<NBLD>(codes, scales, m, lane, nblk, code_row, A);
#pragma unroll 1
        for (int b0 = 0; b0 < 16; b0 += 2 * kDnBatch) {
            load_batch<NBLD>(codes, scales, m + b0 + kDnBatch, lane, nblk, code_row, B);
            __builtin_amdgcn_sched_barrier(0);
            float out[kDnBatch];
            dot_batch_mfma<NBLD, kDnBatch>(A, ha, lane, nblk, out);
            if (lane == 0) store_bf16x4(orow + b0, out);
            __builtin_amdgcn_sched_barrier(0);
            if (b0 + 2 * kDnBatch < 16)
                load_batch<NBLD>(codes, scales, m + b0 + 2 * kDnBatch, lane, nblk, code_row, A);
            __builtin_amdgcn_sched_barrier(0);
            dot_batch_mfma<NBLD, kDnBatch>(B, ha, lane, nblk, out);
            if (lane == 0) store_bf16x4(orow + b0 + kDnBatch, out);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (!kMulti) {
        for (int r = 0; r < ne; ++r) one_row(r);
        continue;
    }
    if (ne == 1) {
        one_row(0);
        continue;
    }
    // several rows: up to kDnTokRows of them split into LDS by the whole block,
    // then every weight batch, loaded once, is dotted with each of them
    const float *hrows = h + (size_t)(hstride > 0 ? a * hstride : row0) * f;
    for (int r0 = 0; r0 < ne; r0 += kDnTokRows) {
        const int nr = min(kDnTokRows, ne - r0);       // block-uniform
        __syncthreads();                            // the previous chunk's records are read
        for (int r = 0; r < nr; ++r)
            split_x_to_lds(hrows + (size_t)(r0 + r) * f, nblk, (int)threadIdx.x, 256,
                           hsr + 4 * nblk * r);
        __syncthreads();
        RowBuf<NBLD> A, B;
        load_batch<NBLD>(codes, scales, m, lane, nblk, code_row, A);
        uint16_t *orow = rows_out + (size_t)(row0 + r0) * d + m;
#pragma unroll 1
        for (int b0 = 0; b0 < 16; b0 += 2 * kDnBatch) {
            load_batch<NBLD>(codes, scales, m + b0 + kDnBatch, lane, nblk, code_row, B);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
            for (int r = 0; r < nr; ++r) {
                XSplit ha[NBLD];
                load_xsplit<NBLD>(hsr + 4 * nblk * r, lane, nblk, ha);
                float out[kDnBatch];
                dot_batch_mfma<NBLD, kDnBatch>(A, ha, lane, nblk, out);
                if (lane == 0) store_bf16x4(orow + (size_t)r * d + b0, out);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (b0 + 2 * kDnBatch < 16)
                load_batch<NBLD>(codes, scales, m + b0 + 2 * kDnBatch, lane, nblk, code_row, A);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
            for (int r = 0; r < nr; ++r) {
                XSplit ha[NBLD];
                load_xsplit<NBLD>(hsr + 4 * nblk * r, lane, nblk, ha);
                float out[kDnBatch];
                dot_batch_mfma<NBLD, kDnBatch>(B, ha, lane, nblk, out);
                if (lane == 0) store_bf16x4(orow + (size_t)r * d + b0 + kDnBatch, out);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    }
}

}  // namespace

template <int NBL>
hipError_t launch_regx(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                       const int32_t *sorted_rows, const int32_t *plan, float *h, int T, int d,
                       int E, int k, int f, int amax, hipStream_t s, int hstride = 0,
                       bool hb = false) {
    dim3 grid(f / kRxPairs, amax);
    if (hb)
        (void)timed_launch("gemv_gate_up", gate_up_regx_kernel<NBL, uint16_t>, dim3(grid),
                           dim3(256), (size_t)kRxRows * d * 2, s, x, w, offsets, sorted_rows, plan,
                           reinterpret_cast<uint16_t *>(h), T, d, E, k, f, hstride);
    else
        (void)timed_launch("gemv_gate_up", gate_up_regx_kernel<NBL, float>, dim3(grid), dim3(256),
                           (size_t)kRxRows * d * 2, s, x, w, offsets, sorted_rows, plan, h, T, d, E, k,
                           f, hstride);
    return hipGetLastError();
}

bool gemv_bf16_h_ok(int T, int d, int f) {
    return T >= 1 && T <= 4 && d <= 8192 && f <= 4096 && f % kRxPairs == 0;
}

hipError_t launch_gemv_gate_up(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                               const int32_t *sorted_rows, const int32_t *plan, float *h,
                               int T, int d, int E, int k, int f, hipStream_t s, bool hb) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    if (hb && !gemv_bf16_h_ok(T, d, f)) return hipErrorInvalidValue;
    const int nbl = (d / 32 + 63) / 64;               // MX blocks per lane along d
    if (f % kRxPairs == 0 && T <= 64 && nbl <= 4 && d <= 8192) {
        if (nbl == 1) return launch_regx<1>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s, 0, hb);
        if (nbl == 2) return launch_regx<2>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s, 0, hb);
        return launch_regx<4>(x, w, offsets, sorted_rows, plan, h, T, d, E, k, f, amax, s, 0, hb);
    }
    const int rpp = max(1, min(kRowsMax, 32768 / d));   // <= 64 KB of LDS
    dim3 grid(f / kGuPairs, amax);
    (void)timed_launch("gemv_gate_up", gemv_gate_up_kernel, dim3(grid), dim3(256), (size_t)rpp * d * 2, s, x, w, offsets, sorted_rows, plan,
                                                               h, T, d, E, k, f, rpp);
    return hipGetLastError();
}

template <int NBLD>
hipError_t launch_down_rows(const float *h, ExpertArgs w, const int32_t *offsets,
                            const int32_t *plan, uint16_t *rows_out, int T, int d, int E,
                            int k, int f, int amax, hipStream_t s, int hstride = 0) {
    dim3 grid(d / 64, amax);
    // the several-row path only where an expert can have several rows
    if (hstride == 1)
        (void)timed_launch("gemv_down", down_rows_kernel<NBLD, false>, dim3(grid), dim3(256), 0,
                           s, h, w, offsets, plan, rows_out, T, d, E, k, f, hstride);
    else
        (void)timed_launch("gemv_down", down_rows_kernel<NBLD, true>, dim3(grid), dim3(256),
                           (size_t)kDnTokRows * f * 2, s, h, w, offsets, plan, rows_out, T, d, E,
                           k, f, hstride);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const float *h, ExpertArgs w, const int32_t *offsets,
                            const int32_t *plan, uint16_t *rows_out, int T, int d, int E,
                            int k, int f, hipStream_t s) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    const int nbld = (f / 32 + 63) / 64;              // MX blocks per lane along f
    if (T <= 64 && nbld <= 2) {
        if (nbld == 1) return launch_down_rows<1>(h, w, offsets, plan, rows_out, T, d, E, k, f, amax, s);
        return launch_down_rows<2>(h, w, offsets, plan, rows_out, T, d, E, k, f, amax, s);
    }
    const int rpp = max(1, min(kRowsMax, 16384 / f));   // <= 64 KB of LDS
    dim3 grid(d / kDnRows, amax);
    (void)timed_launch("gemv_down", gemv_down_kernel, dim3(grid), dim3(256), (size_t)rpp * f * 4, s, h, w, offsets, plan, rows_out, T, d,
                                                            E, k, f, rpp);
    return hipGetLastError();
}

bool gemv_small_ok(int d, int f) {
    return f % kRxPairs == 0 && d <= 8192 && (f / 32 + 63) / 64 <= 2;
}

// The small-expert passes run in a scaled-MFMA call whose small list may
// be empty (every expert over the crossover): a bounded grid whose blocks
// walk the list (a += gridDim.y) keeps that case to a few microseconds
// instead of one block per possible expert.
constexpr int kSmallGridY = 320;

hipError_t launch_gemv_gate_up_small(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                                     const int32_t *sorted_rows, const int32_t *small,
                                     float *h_small, int T, int d, int E, int k, int f,
                                     int gemv_max, hipStream_t s) {
    const int amax = min(min(E, T * k), kSmallGridY);
    if (amax <= 0) return hipSuccess;
    const int nbl = (d / 32 + 63) / 64;
    if (nbl == 1)
        return launch_regx<1>(x, w, offsets, sorted_rows, small, h_small, T, d, E, k, f, amax, s,
                              gemv_max);
    if (nbl == 2)
        return launch_regx<2>(x, w, offsets, sorted_rows, small, h_small, T, d, E, k, f, amax, s,
                              gemv_max);
    return launch_regx<4>(x, w, offsets, sorted_rows, small, h_small, T, d, E, k, f, amax, s,
                          gemv_max);
}

hipError_t launch_gemv_down_small(const float *h_small, ExpertArgs w, const int32_t *offsets,
                                  const int32_t *small, uint16_t *rows_out, int T, int d, int E,
                                  int k, int f, int gemv_max, hipStream_t s) {
    const int amax = min(min(E, T * k), kSmallGridY);
    if (amax <= 0) return hipSuccess;
    if ((f / 32 + 63) / 64 == 1)
        return launch_down_rows<1>(h_small, w, offsets, small, rows_out, T, d, E, k, f, amax, s,
                                   gemv_max);
    return launch_down_rows<2>(h_small, w, offsets, small, rows_out, T, d, E, k, f, amax, s,
                               gemv_max);
}

bool gate_up_token_fusable(int T, int d, int E, int k, int f) {
    const int nbl = (d / 32 + 63) / 64;
    return T == 1 && k <= 32 && k <= E && E <= 1024 && (f % 48 == 0 || f % 32 == 0) &&
           nbl <= 4 && d <= 8192;
}

template <int NBL, int PAIRS, typename HT, int NWV>
hipError_t launch_token_n(const float *logits, const uint16_t *x, ExpertArgs w, int32_t *ids,
                          float *tw, int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                          int32_t *row_pos, int32_t *plan, HT *h, int d, int E, int k, int f,
                          hipStream_t s) {
    return timed_launch("gemv_gate_up", gate_up_mfma_token_kernel<NBL, PAIRS, HT, NWV>,
                        dim3(f / PAIRS, k), dim3(64 * NWV), (size_t)d * 2 + 16, s, logits, x, w, ids, tw, counts, offsets,
                        sorted_rows, row_pos, plan, h, d, E, k, f);
}

template <int PAIRS, int NWV, typename HT>
hipError_t launch_gate_up_token_p(const float *logits, const uint16_t *x, ExpertArgs w,
                                  int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                  int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, HT *h,
                                  int d, int E, int k, int f, hipStream_t s) {
    const int nbl = (d / 32 + 63) / 64;
    if (nbl == 1)
        return launch_token_n<1, PAIRS, HT, NWV>(logits, x, w, ids, tw, counts, offsets,
                                                 sorted_rows, row_pos, plan, h, d, E, k, f, s);
    if (nbl == 2)
        return launch_token_n<2, PAIRS, HT, NWV>(logits, x, w, ids, tw, counts, offsets,
                                                 sorted_rows, row_pos, plan, h, d, E, k, f, s);
    return launch_token_n<4, PAIRS, HT, NWV>(logits, x, w, ids, tw, counts, offsets, sorted_rows,
                                             row_pos, plan, h, d, E, k, f, s);
}

template <typename HT>
hipError_t launch_gate_up_token_t(const float *logits, const uint16_t *x, ExpertArgs w,
                                  int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                  int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, HT *h,
                                  int d, int E, int k, int f, hipStream_t s) {
#define TOKEN_CFG(P, NW)                                                                   \
    return launch_gate_up_token_p<P, NW>(logits, x, w, ids, tw, counts, offsets, sorted_rows, \
                                         row_pos, plan, h, d, E, k, f, s)
    // wide rows (d > 4096: two pairs in flight are 4 x 3.6 KB a wave at
    // d = 7168): one block per CU streams best when the grid fills the chip
    // (K3 shape: 96 pairs, 256 blocks, 37.4 us against 38.2 us for 48); the
    // narrower rows of d = 4096 want two blocks per CU (64 pairs: 20.0 us
    // against 17.4 us for 32)
    if (d > 4096 && f % 96 == 0 && (f / 96) * k >= 256) TOKEN_CFG(96, 4);
    if (f % 48 == 0) TOKEN_CFG(48, 4);
    TOKEN_CFG(32, 4);
#undef TOKEN_CFG
}

hipError_t launch_gate_up_token(const float *logits, const uint16_t *x, ExpertArgs w,
                                int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, float *h,
                                int d, int E, int k, int f, hipStream_t s, bool hb) {
    if (hb) {
        if (!gemv_bf16_h_ok(1, d, f)) return hipErrorInvalidValue;
        return launch_gate_up_token_t(logits, x, w, ids, tw, counts, offsets, sorted_rows,
                                      row_pos, plan, reinterpret_cast<uint16_t *>(h), d, E, k, f,
                                      s);
    }
    return launch_gate_up_token_t(logits, x, w, ids, tw, counts, offsets, sorted_rows, row_pos,
                                  plan, h, d, E, k, f, s);
}

// rows per batch and batch buffers of the fused down + combine
// (batches of 4 rows; a ring of 3 batch buffers for one MX block of h per
// lane, 2 for two, whose registers allow no more at 8 waves)
constexpr int kDcB = 4;

template <int NBLD, int ROWS, int NW, typename HT>
void launch_dc(const HT *h, ExpertArgs w, const int32_t *ids, const float *topk_w,
               const int32_t *row_pos, uint16_t *y, int T, int d, int E, int k, int f,
               hipStream_t s) {
    constexpr int R = NBLD == 1 ? 3 : 2;
    (void)timed_launch("down_combine", down_combine_split_kernel<NBLD, ROWS, kDcB, R, NW, HT>,
                       dim3(d / ROWS, T), dim3(64 * NW), 0, s, h, w, ids, topk_w, row_pos, y, T, d,
                       E, k, f);
}

template <int NBLD, int NW, typename HT>
void launch_dc_rows(int rows, const HT *h, ExpertArgs w, const int32_t *ids,
                    const float *topk_w, const int32_t *row_pos, uint16_t *y, int T, int d,
                    int E, int k, int f, hipStream_t s) {
    if (rows == 28) launch_dc<NBLD, 28, NW>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
    else if (rows == 16) launch_dc<NBLD, 16, NW>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
    else launch_dc<NBLD, 32, NW>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
}

template <int NBLD, typename HT>
hipError_t launch_dc_split(const HT *h, ExpertArgs w, const int32_t *ids,
                           const float *topk_w, const int32_t *row_pos, uint16_t *y, int T,
                           int d, int E, int k, int f, hipStream_t s) {
    // about one block per CU: 28 output rows per block where d allows
    // (7168 / 28 = 256), else 16 (4096 / 16 = 256) or 32; 8 waves, a wave
    // taking slots wid, wid + 8, .. (at k = 16 two slots a wave with three
    // batches in flight: 18.6 us against 19.4 for 16 waves of one slot and
    // two batches)
    const int rows = d % 28 == 0 ? 28 : (d % 16 == 0 && d / 16 <= 512 ? 16 : 32);
    launch_dc_rows<NBLD, 8>(rows, h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
    return hipGetLastError();
}

hipError_t launch_down_combine(const float *h, ExpertArgs w, const int32_t *ids,
                               const float *topk_w, const int32_t *row_pos, uint16_t *y,
                               int T, int d, int E, int k, int f, hipStream_t s, bool hb) {
    if (T <= 0) return hipSuccess;
    const int nbld = (f / 32 + 63) / 64;
    if (hb) {
        if (!gemv_bf16_h_ok(T, d, f)) return hipErrorInvalidValue;
        const uint16_t *hh = reinterpret_cast<const uint16_t *>(h);
        if (nbld == 1) return launch_dc_split<1>(hh, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
        return launch_dc_split<2>(hh, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
    }
    if (nbld <= 2) {
        if (nbld == 1) return launch_dc_split<1>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
        return launch_dc_split<2>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f, s);
    }
    dim3 grid(d / 16, T);
    (void)timed_launch("down_combine", down_combine_kernel, dim3(grid), dim3(64), 0, s, h, w, ids, topk_w, row_pos, y, T, d, E, k, f);
    return hipGetLastError();
}

}  // namespace moe
