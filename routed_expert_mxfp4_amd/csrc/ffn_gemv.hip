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
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
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
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
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

}  // namespace

hipError_t launch_gemv_gate_up(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                               const int32_t *sorted_rows, const int32_t *plan, float *h,
                               int T, int d, int E, int k, int f, hipStream_t s) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    const int rpp = max(1, min(kRowsMax, 32768 / d));   // <= 64 KB of LDS
    dim3 grid(f / kGuPairs, amax);
    gemv_gate_up_kernel<<<grid, 256, (size_t)rpp * d * 2, s>>>(x, w, offsets, sorted_rows, plan,
                                                               h, T, d, E, k, f, rpp);
    return hipGetLastError();
}

hipError_t launch_gemv_down(const float *h, ExpertArgs w, const int32_t *offsets,
                            const int32_t *plan, uint16_t *rows_out, int T, int d, int E,
                            int k, int f, hipStream_t s) {
    const int amax = min(E, T * k);
    if (amax <= 0) return hipSuccess;
    const int rpp = max(1, min(kRowsMax, 16384 / f));   // <= 64 KB of LDS
    dim3 grid(d / kDnRows, amax);
    gemv_down_kernel<<<grid, 256, (size_t)rpp * f * 4, s>>>(h, w, offsets, plan, rows_out, T, d,
                                                            E, k, f, rpp);
    return hipGetLastError();
}

hipError_t launch_down_combine(const float *h, ExpertArgs w, const int32_t *ids,
                               const float *topk_w, const int32_t *row_pos, uint16_t *y,
                               int T, int d, int E, int k, int f, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid(d / 16, T);
    down_combine_kernel<<<grid, 64, 0, s>>>(h, w, ids, topk_w, row_pos, y, T, d, E, k, f);
    return hipGetLastError();
}

}  // namespace moe
