// combine.hip -- weighted combine of each token's k expert outputs (gfx950).
//
// y[t][m] = sum_j w[t][j] * rows_out[row_pos[t*k+j]][m], accumulated in fp32
// in slot order and rounded once to bf16 (the MoE tail's weighted reduction:
// Moonshine README, "Run layer-major prefill").  Each thread owns 8
// consecutive outputs of one token, so every y element has exactly one
// writer (no atomics) and all loads and stores are 16 bytes wide.
//
// In the pre-norm block the same pass also does the tail's adds: with resid
// (bf16 [T][d], the block input) and extra (fp32 [T][d], the shared expert's
// output; NULL: none) the accumulator starts at resid + extra, so
// out = bf16(x + s + sum_j w_j rows_j) is written once.
#include "moe_internal.hpp"

namespace moe {
namespace {

template <int G>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ rows_out,
                                                      const int32_t *__restrict__ row_pos,
                                                      const float *__restrict__ topk_w,
                                                      const uint16_t *__restrict__ resid,
                                                      const float *__restrict__ extra,
                                                      uint16_t *__restrict__ y, int T, int d,
                                                      int k) {
    const int t = blockIdx.y;
    const int v = blockIdx.x * blockDim.x + threadIdx.x;   // 8-element vector index
    if (v >= (d >> 3)) return;
    const int nrows = T * k;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (resid) {
        const uint4 r = reinterpret_cast<const uint4 *>(resid + (size_t)t * d)[v];
        float4 e0 = {0.f, 0.f, 0.f, 0.f}, e1 = e0;
        if (extra) {
            const float4 *e = reinterpret_cast<const float4 *>(extra + (size_t)t * d) + 2 * v;
            e0 = e[0];
            e1 = e[1];
        }
        const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = bf16_bits_to_f32(rw[i] & 0xFFFFu) + ev[2 * i];
            acc[2 * i + 1] = bf16_bits_to_f32(rw[i] >> 16) + ev[2 * i + 1];
        }
    }
    // slots in groups of G: all loads of a group are issued before use
    for (int j0 = 0; j0 < k; j0 += G) {
        uint4 q[G];
        float wj[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int j = min(j0 + jj, k - 1);
            int p = row_pos[(size_t)t * k + j];
            const bool ok = j0 + jj < k && (unsigned)p < (unsigned)nrows;
            p = ok ? p : 0;
            wj[jj] = ok ? topk_w[(size_t)t * k + j] : 0.f;
            q[jj] = reinterpret_cast<const uint4 *>(rows_out + (size_t)p * d)[v];
        }
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            if (j0 + jj < k) {
                const uint32_t wds[4] = {q[jj].x, q[jj].y, q[jj].z, q[jj].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += wj[jj] * bf16_bits_to_f32(wds[i] & 0xFFFFu);
                    acc[2 * i + 1] += wj[jj] * bf16_bits_to_f32(wds[i] >> 16);
                }
            }
        }
    }
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    reinterpret_cast<uint4 *>(y + (size_t)t * d)[v] = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t *rows_out, const int32_t *row_pos,
                          const float *topk_w, uint16_t *y, int T, int d, int k,
                          hipStream_t s, const uint16_t *resid, const float *extra) {
    if (T <= 0) return hipSuccess;
    // 128-thread blocks when they tile the row exactly (d = 7168: 7 blocks,
    // no idle lanes); every slot's load in flight at once for k <= 16
    const int nv = d >> 3;
    const int bs = nv % 128 == 0 ? 128 : 256;
    dim3 grid((nv + bs - 1) / bs, T);
    if (k > 8)
        (void)timed_launch("combine", combine_kernel<16>, dim3(grid), dim3(bs), 0, s, rows_out,
                           row_pos, topk_w, resid, extra, y, T, d, k);
    else
        (void)timed_launch("combine", combine_kernel<8>, dim3(grid), dim3(bs), 0, s, rows_out,
                           row_pos, topk_w, resid, extra, y, T, d, k);
    return hipGetLastError();
}

}  // namespace moe
