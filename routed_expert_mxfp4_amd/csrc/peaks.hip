// peaks.hip -- what this GPU actually sustains for the two resources the
// layer's kernels are bound by, measured the way those kernels use them:
//
//   * a streaming read of n bytes from HBM in one launch (16-byte loads,
//     eight per thread in flight, grid-stride), the ceiling a bandwidth-bound
//     kernel reading the same n bytes can reach, ramp-up and tail included;
//   * the issue rate of the matrix instructions the expert GEMMs use, from
//     registers with no memory traffic: the scaled v_mfma_scale_f32_16x16x128
//     _f8f6f4 (and its 32x32x64 shape) for a given pair of operand formats,
//     and the bf16 v_mfma_f32_32x32x16 of the shared expert.
//
// Both write one value per block (a checksum / the sum of the accumulators)
// so that no load or product can be dropped.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src,
                                                          size_t n16, uint32_t *__restrict__ out) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] ^= red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

// Sixteen independent accumulation chains per wave, each with its own
// operand registers: the 16x16x128 shape's result latency is long against
// its issue time, and only this much independent work (with up to eight
// waves per SIMD) comes near its issue rate.  Operands differ per lane and
// chain so that nothing folds.  Scale code 127 (2^0) for both operands.
template <int FA, int FB>
__global__ __launch_bounds__(256) void mfma_scaled_rate_kernel(int iters, float *__restrict__ out) {
    constexpr int kCh = 16;
    const int lane = threadIdx.x & 63;
    const int v = 0x22222222 ^ (lane & 7);
    i32x8_t a[kCh], b[kCh];
    f32x4_t c[kCh];
#pragma unroll
    for (int j = 0; j < kCh; ++j) {
        const int vj = v ^ (j << 8);
        a[j] = i32x8_t{vj, vj, vj, vj, vj, vj, vj, vj};
        b[j] = i32x8_t{vj ^ 1, vj ^ 1, vj ^ 1, vj ^ 1, vj ^ 1, vj ^ 1, vj ^ 1, vj ^ 1};
        c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int i = 0; i < iters; i += 4) {
#pragma unroll
        for (int j = 0; j < kCh; ++j)
            c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b[j], c[j], FA, FB, 0, 127, 0, 127);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kCh; ++j) s += c[j][j & 3];
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// The 32x32x64 shape of the same instruction family (16 accumulators).
template <int FA, int FB>
__global__ __launch_bounds__(256) void mfma_scaled32_rate_kernel(int iters, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int v = 0x22222222 ^ (lane & 7);
    const i32x8_t a = {v, v, v, v, v, v, v, v};
    const i32x8_t b = {v ^ 1, v ^ 1, v ^ 1, v ^ 1, v ^ 1, v ^ 1, v ^ 1, v ^ 1};
    f32x16_t c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, FA, FB, 0, 127, 0, 127);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, FA, FB, 0, 127, 0, 127);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, FA, FB, 0, 127, 0, 127);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, FA, FB, 0, 127, 0, 127);
    }
    const float s = (c0[0] + c1[5]) + (c2[10] + c3[15]);
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_rate_kernel(int iters, float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (float)(lane + j));
        b[j] = (__bf16)(0.002f * (float)(lane - j));
    }
    f32x16_t c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    const float s = (c0[0] + c1[5]) + (c2[10] + c3[15]);
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks,
                              hipStream_t s) {
    if (src == nullptr || out == nullptr || blocks <= 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return hipErrorInvalidValue;
    return timed_launch("stream_read", stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                        static_cast<const uint4 *>(src), bytes / 16, out);
}

hipError_t launch_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t s) {
    if (out == nullptr || blocks <= 0 || iters <= 0 || iters % 4 != 0) return hipErrorInvalidValue;
    switch (kind) {
    case 0:   // FP6 E2M3 x FP4 E2M1
        return timed_launch("mfma_rate", mfma_scaled_rate_kernel<2, 4>, dim3(blocks), dim3(256), 0, s, iters, out);
    case 1:   // FP8 E4M3 x FP4 E2M1
        return timed_launch("mfma_rate", mfma_scaled_rate_kernel<0, 4>, dim3(blocks), dim3(256), 0, s, iters, out);
    case 2:   // FP4 E2M1 x FP4 E2M1
        return timed_launch("mfma_rate", mfma_scaled_rate_kernel<4, 4>, dim3(blocks), dim3(256), 0, s, iters, out);
    case 3:   // FP8 E4M3 x FP8 E4M3
        return timed_launch("mfma_rate", mfma_scaled_rate_kernel<0, 0>, dim3(blocks), dim3(256), 0, s, iters, out);
    case 4:   // bf16 x bf16, 32x32x16
        return timed_launch("mfma_rate", mfma_bf16_rate_kernel, dim3(blocks), dim3(256), 0, s, iters, out);
    case 5:   // FP6 E2M3 x FP4 E2M1, 32x32x64
        return timed_launch("mfma_rate", mfma_scaled32_rate_kernel<2, 4>, dim3(blocks), dim3(256), 0, s, iters, out);
    case 6:   // FP4 E2M1 x FP4 E2M1, 32x32x64
        return timed_launch("mfma_rate", mfma_scaled32_rate_kernel<4, 4>, dim3(blocks), dim3(256), 0, s, iters, out);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
