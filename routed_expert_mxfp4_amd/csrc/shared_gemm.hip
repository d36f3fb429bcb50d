// shared_gemm.hip -- the shared expert's two dense bf16 GEMMs for many
// tokens, on gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16), with the
// SwiGLU fused into the gate/up GEMM's epilogue.
//
//   gate/up: h[t][n]  = bf16(silu(g) * u),  g = xn[t] . Wgu[n],
//                                           u = xn[t] . Wgu[fs + n]
//   down:    sx[t][m] = h[t] . Wdn[m]   (fp32, added by the combine pass)
//
// Both are "row times row" products: every operand is K-contiguous, which
// is the matrix core's operand layout (lane l holds row l % 32 and eight
// consecutive K elements of a 32 x 16 slice).  fp32 accumulation.
//
// Block tile 128 x 128, K step 64, four waves (2 x 2) of 64 x 64, i.e.
// 2 x 2 MFMA tiles of 32 x 32 per wave.  Operand tiles go global ->
// registers -> LDS with a 16-byte pad per row (16-byte fragment reads of 32
// consecutive rows then touch distinct banks), double-buffered: the next
// step's global loads are in flight during the current step's MFMAs, one
// barrier per step.
//
// In the gate/up GEMM a block takes 64 gate rows and the matching 64 up
// rows of Wgu (LDS rows 0..63 and 64..127), and each wave one 32-column
// slice of each, so a lane holds g and u of the same (t, n) in the same
// register of its two accumulator tiles: the SwiGLU needs no exchange.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kRow = kBK + 8;                     // bf16 per LDS row (16-byte pad)
constexpr int kTile = 128 * kRow;                 // bf16 per operand tile
constexpr int kLds = 2 * 2 * kTile * 2;           // [buffer][A, B] tiles, bytes: 73728

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Which B row (weight row) LDS row r of the block's B tile holds.
template <bool kSwiGLU>
__device__ __forceinline__ int b_row(int r, int nb, int fs, int N) {
    if (kSwiGLU) {
        const int n = nb * 64 + (r & 63);          // gate column n (clamped: unused)
        return (r < 64 ? 0 : fs) + min(n, fs - 1);
    }
    return min(nb * kBN + r, N - 1);
}

// One thread's four 16-byte pieces of each operand tile: piece p = c * 256 +
// tid is row p / 8, K piece p % 8.  Rows past the end are clamped (their
// results are never stored); K pieces past K are zero.
struct Stage {
    uint4 a[4], b[4];
};

template <bool kSwiGLU>
__device__ __forceinline__ void load_stage(Stage &st, const uint16_t *__restrict__ A,
                                           const uint16_t *__restrict__ B, int m0, int nb,
                                           int k0, int M, int N, int K, int fs, int tid) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int p = c * 256 + tid, r = p >> 3, kp = k0 + 8 * (p & 7);
        const bool in_k = kp < K;
        const size_t ar = (size_t)min(m0 + r, M - 1), br = (size_t)b_row<kSwiGLU>(r, nb, fs, N);
        st.a[c] = in_k ? *reinterpret_cast<const uint4 *>(A + ar * K + kp) : uint4{0, 0, 0, 0};
        st.b[c] = in_k ? *reinterpret_cast<const uint4 *>(B + br * K + kp) : uint4{0, 0, 0, 0};
    }
}

__device__ __forceinline__ void store_stage(const Stage &st, uint16_t *la, uint16_t *lb, int tid) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int p = c * 256 + tid, r = p >> 3, kq = 8 * (p & 7);
        *reinterpret_cast<uint4 *>(la + r * kRow + kq) = st.a[c];
        *reinterpret_cast<uint4 *>(lb + r * kRow + kq) = st.b[c];
    }
}

__device__ __forceinline__ bf16x8_t frag(const uint16_t *tile, int row, int kq) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(tile + row * kRow + kq));
}

// kSwiGLU: A = xn [M][K = d], B = Wgu [2 fs][d], out = h bf16 [M][fs];
// else:    A = h [M][K = fs], B = Wdn [N = d][fs], out = sx fp32 [M][N].
// Blocks are spread over the 8 XCDs so that each XCD takes a contiguous run
// of tiles, N fastest: the N tiles of one row tile share its A rows in L2.
template <bool kSwiGLU>
__global__ __launch_bounds__(256) void shared_gemm_kernel(const uint16_t *__restrict__ A,
                                                          const uint16_t *__restrict__ B,
                                                          void *__restrict__ out, int M, int N,
                                                          int K, int fs, int nbn, int tiles) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int per = (tiles + 7) >> 3;
    const int u = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    if ((int)(blockIdx.x >> 3) >= per || u >= tiles) return;
    const int mt = u / nbn, nb = u - mt * nbn;
    const int m0 = mt * kBM;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int l32 = lane & 31, kh = 8 * (lane >> 5);
    // this wave's A rows and B rows in the tiles
    const int ar0 = wm * 64 + l32;
    const int br0 = kSwiGLU ? wn * 32 + l32 : wn * 64 + l32;
    const int br1 = kSwiGLU ? 64 + wn * 32 + l32 : wn * 64 + 32 + l32;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = (K + kBK - 1) / kBK;
    Stage st;
    load_stage<kSwiGLU>(st, A, B, m0, nb, 0, M, N, K, fs, tid);
    store_stage(st, lds, lds + kTile, tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) load_stage<kSwiGLU>(st, A, B, m0, nb, (kt + 1) * kBK, M, N, K, fs, tid);
        const uint16_t *la = lds + (kt & 1) * 2 * kTile, *lb = la + kTile;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kq = ks * 16 + kh;
            const bf16x8_t a0 = frag(la, ar0, kq), a1 = frag(la, ar0 + 32, kq);
            const bf16x8_t b0 = frag(lb, br0, kq), b1 = frag(lb, br1, kq);
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) {
            uint16_t *na = lds + ((kt + 1) & 1) * 2 * kTile;
            store_stage(st, na, na + kTile, tid);
        }
        __syncthreads();
    }

    // register r of a 32 x 32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4,
    // column lane % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= M) continue;
            if (kSwiGLU) {
                const int n = nb * 64 + wn * 32 + l32;
                if (n < fs)
                    static_cast<uint16_t *>(out)[(size_t)row * fs + n] =
                        f32_to_bf16_rne(silu_mul(acc[i][0][r], acc[i][1][r]));
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = nb * kBN + wn * 64 + 32 * j + l32;
                    if (col < N) static_cast<float *>(out)[(size_t)row * N + col] = acc[i][j][r];
                }
            }
        }
}

bool g_attr_done = false;

hipError_t set_attrs() {
    if (g_attr_done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)shared_gemm_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)shared_gemm_kernel<false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess) g_attr_done = true;
    return e;
}

dim3 xcd_grid(int tiles) { return dim3((unsigned)(8 * ((tiles + 7) / 8))); }

}  // namespace

hipError_t launch_shared_gate_up_gemm(const uint16_t *xn, const uint16_t *sgu, uint16_t *h, int T,
                                      int d, int fs, hipStream_t s) {
    if (T <= 0 || fs <= 0) return hipSuccess;
    hipError_t e = set_attrs();
    if (e != hipSuccess) return e;
    const int nbn = (fs + 63) / 64, tiles = ((T + kBM - 1) / kBM) * nbn;
    return timed_launch("shared_gemm_gate_up", shared_gemm_kernel<true>, xcd_grid(tiles),
                        dim3(256), kLds, s, xn, sgu, (void *)h, T, 2 * fs, d, fs, nbn, tiles);
}

hipError_t launch_shared_down_gemm(const uint16_t *h, const uint16_t *sdn, float *sx, int T,
                                   int d, int fs, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipError_t e = set_attrs();
    if (e != hipSuccess) return e;
    const int nbn = (d + kBN - 1) / kBN, tiles = ((T + kBM - 1) / kBM) * nbn;
    return timed_launch("shared_gemm_down", shared_gemm_kernel<false>, xcd_grid(tiles), dim3(256),
                        kLds, s, h, sdn, (void *)sx, T, d, fs, fs, nbn, tiles);
}

}  // namespace moe
