// blas.cpp -- the shared expert's two dense bf16 GEMMs for many tokens, on
// the ROCm library GEMM (rocBLAS).  They are plain library GEMMs (bf16
// operands, fp32 accumulate and output) with no fused epilogue, so the
// library's tuned gfx950 kernels serve them; the SwiGLU between them and the
// residual add after them are this library's own kernels.
//
// One rocBLAS handle per device, created on first use and kept until the
// process ends; the caller's stream is set on it for every call, under a
// lock, so concurrent callers do not race on the handle's stream.  Atomics
// are disabled on the handle: GEMM results are then identical run to run.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <map>
#include <mutex>

#include "moe_internal.hpp"

namespace moe {
namespace {

std::mutex g_blas_mu;
std::map<int, rocblas_handle> g_handles;

rocblas_handle handle_for_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    auto it = g_handles.find(dev);
    if (it != g_handles.end()) return it->second;
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
        rocblas_destroy_handle(h);
        return nullptr;
    }
    g_handles[dev] = h;
    return h;
}

}  // namespace

// Row-major c[M][N] = a[M][K] * b[N][K]^T.  In rocBLAS's column-major terms
// that is C^T (N x M, ld N) = B (stored K x N, ld K, transposed) * A^T
// (stored K x M, ld K).
hipError_t blas_gemm_bf16_nt(const uint16_t *a, const uint16_t *b, float *c, int M, int N,
                             int K, hipStream_t s) {
    if (M <= 0 || N <= 0) return hipSuccess;
    std::lock_guard<std::mutex> lk(g_blas_mu);
    rocblas_handle h = handle_for_current_device();
    if (!h) return hipErrorInvalidHandle;
    if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorInvalidHandle;
    const float alpha = 1.0f, beta = 0.0f;
    const rocblas_status st = rocblas_gemm_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &alpha, b,
        rocblas_datatype_bf16_r, K, a, rocblas_datatype_bf16_r, K, &beta, c, rocblas_datatype_f32_r,
        N, c, rocblas_datatype_f32_r, N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) return hipErrorLaunchFailure;
    return hipGetLastError();
}

}  // namespace moe
