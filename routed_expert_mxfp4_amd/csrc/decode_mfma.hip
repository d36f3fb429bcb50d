// decode_mfma.hip -- the down GEMV and weighted combine of one token on the
// gfx950 scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// y[m] = sum over the k selected experts a of W_dn[e_a][m] . h'_a, where
// h'_a = w_a * h_a already carries the routing weight and comes split into
// two MX E2M3 terms per 32 elements (the gate/up kernel's epilogue).  Each
// MFMA multiplies 16 weight rows x 128 K -- the E2M1 codes and E8M0 scales
// as stored are the FP4 A operand and its scale -- by h' as the FP6 B
// operand: column 0 the hi term, column 1 the lo term, columns 2..15 zero.
// C[m][0] + C[m][1] is then row m's share; the experts follow each other
// along K in the same accumulator, so the combine is the accumulation.  No
// dequantisation runs on the vector ALU.
//
// Each wave issues all of an expert's code loads (16 rows x f/2 bytes)
// before multiplying, one expert ahead.  Deterministic: fixed order
// throughout, one writer per output.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRec = 64;              // bytes per h' record (one 32-element block)

// One expert's weight rows of the block: NSTEP 16-byte code pieces and the
// row's scales (NSTEP / 4 pieces of 16 bytes) per lane.
template <int NSTEP>
struct DnBuf {
    uint4 c[NSTEP];
    uint4 sc[NSTEP / 4];
};

template <int NSTEP>
__device__ __forceinline__ void dn_issue(DnBuf<NSTEP> &b, const ExpertArgs &W, int e, int E, int d,
                                         uint32_t row, uint32_t code_row, int nb, int g) {
    const int ev = (unsigned)e < (unsigned)E ? e : 0;
    const rsrc_t codes = make_rsrc(W.dn_codes + (size_t)ev * d * code_row, (uint32_t)d * code_row);
    const rsrc_t scales = make_rsrc(W.dn_scales + (size_t)ev * d * nb, (uint32_t)d * (uint32_t)nb);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
        b.c[s] = buf_load16(codes, row * code_row + 64u * s + 16u * (uint32_t)g, 0);
#pragma unroll
    for (int q = 0; q < NSTEP / 4; ++q) b.sc[q] = buf_load16(scales, row * (uint32_t)nb + 16u * q, 0);
}

// acc += this expert's 16 rows x f against h' (records at rec0 in LDS).
template <int NSTEP>
__device__ __forceinline__ void dn_mfma(f32x4_t &acc, const DnBuf<NSTEP> &b, const uint8_t *lds,
                                        uint32_t rec0, uint32_t zero_rec, int r16, int g) {
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
        // the B operand: this lane's column r16 (0: hi, 1: lo term) and K
        // block g of step s; columns 2..15 read the zero record
        const uint32_t rec = rec0 + (uint32_t)(4 * s + g) * kRec;
        const uint32_t bsrc = r16 < 2 ? rec + 24u * (uint32_t)r16 : zero_rec;
        const uint32_t ssrc = r16 < 2 ? rec + 48u + (uint32_t)r16 : zero_rec + 48u;
        const uint4 b0 = *reinterpret_cast<const uint4 *>(lds + bsrc);
        const uint2 b1 = *reinterpret_cast<const uint2 *>(lds + bsrc + 16);
        const uint32_t bs = lds[ssrc];
        // the A scale: byte g of dword s % 4 of the row's scale piece s / 4
        const uint4 sq = b.sc[s >> 2];
        const uint32_t sw = (s & 3) == 0 ? sq.x : (s & 3) == 1 ? sq.y : (s & 3) == 2 ? sq.z : sq.w;
        const uint32_t as = sw >> (8 * g);
        const i32x8_t A = {(int)b.c[s].x, (int)b.c[s].y, (int)b.c[s].z, (int)b.c[s].w, 0, 0, 0, 0};
        const i32x8_t B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 2, 0, (int)as, 0, (int)bs);
    }
}

// Block b owns output rows [R b, R b + R), R = 28 or 32 (d = 7168 makes 256
// blocks of 28, one per CU), as two 16-row tiles starting at R b and
// R b + 16; the second tile's rows past R b + R are not loaded (their
// buffer loads fall outside the weight range and return zero codes) and
// not written.  Eight waves: wave w takes tile w % 2 and the experts
// a = w / 2, w / 2 + 4, ...; each tile's four partial sums are added in
// wave order.
template <int NSTEP>
__global__ __launch_bounds__(512) void down_token_mfma_kernel(
    const uint8_t *__restrict__ hq, ExpertArgs W, const int32_t *__restrict__ plan,
    uint16_t *__restrict__ y, int d, int E, int k, int f, int R) {
    extern __shared__ __align__(16) uint8_t lds[];   // k * f/32 records of h', then a zero record
    __shared__ float part[8][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tile = wid & 1, a0 = wid >> 1;
    const int r16 = lane & 15, g = lane >> 4;
    const int nb = f >> 5;                           // MX blocks of h' per expert
    const int m_base = blockIdx.x * R;
    const uint32_t code_row = (uint32_t)f >> 1;
    const uint32_t row = 16 * tile + r16 < R ? (uint32_t)(m_base + 16 * tile + r16) : (uint32_t)d;

    // the first expert's weight loads go out before h' is staged
    DnBuf<NSTEP> X, Y;
    if (a0 < k) dn_issue<NSTEP>(X, W, plan[1 + a0], E, d, row, code_row, nb, g);

    // stage h' of every selected expert, and a zero record whose scale bytes
    // are 127 (2^0) for the zero columns 2..15
    const int recs16 = k * nb * (kRec / 16);
    const uint4 *src = reinterpret_cast<const uint4 *>(hq);
    uint4 *dst = reinterpret_cast<uint4 *>(lds);
    for (int i = tid; i < recs16; i += 512) dst[i] = src[i];
    if (tid < kRec / 16) dst[recs16 + tid] = tid == 3 ? uint4{0x7F7Fu, 0u, 0u, 0u} : uint4{0u, 0u, 0u, 0u};
    __syncthreads();

    const uint32_t zero_rec = (uint32_t)(k * nb * kRec);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // experts a = a0, a0 + 4, ...: two buffers, the next expert's loads in
    // flight during the current one's MFMAs
    for (int a = a0; a < k; a += 8) {
        if (a + 4 < k) dn_issue<NSTEP>(Y, W, plan[1 + a + 4], E, d, row, code_row, nb, g);
        if ((unsigned)plan[1 + a] < (unsigned)E)
            dn_mfma<NSTEP>(acc, X, lds, (uint32_t)(a * nb * kRec), zero_rec, r16, g);
        if (a + 8 < k) dn_issue<NSTEP>(X, W, plan[1 + a + 8], E, d, row, code_row, nb, g);
        if (a + 4 < k && (unsigned)plan[1 + a + 4] < (unsigned)E)
            dn_mfma<NSTEP>(acc, Y, lds, (uint32_t)((a + 4) * nb * kRec), zero_rec, r16, g);
    }
    // columns 0 and 1 of rows 4 g + i sit in lanes 16 g and 16 g + 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float v = acc[i] + __shfl_down(acc[i], 1, 64);
        if (r16 == 0) part[wid][4 * g + i] = v;
    }
    __syncthreads();
    if (tid < 32) {
        const int t = tid >> 4, r = tid & 15;
        const int m = m_base + 16 * t + r;
        if (16 * t + r < R) {
            const float v = ((part[t][r] + part[t + 2][r]) + part[t + 4][r]) + part[t + 6][r];
            y[m] = f32_to_bf16_rne(v);
        }
    }
}

}  // namespace

hipError_t launch_down_token_mfma(const uint8_t *hq, ExpertArgs w, const int32_t *plan,
                                  uint16_t *y, int d, int E, int k, int f, hipStream_t s) {
    const size_t lds = (size_t)k * (f / 32) * kRec + kRec;
    const int R = d % 28 == 0 ? 28 : 32;            // d % 16 == 0, so d % 32 == 0 otherwise
    if (d % R != 0) return hipErrorInvalidValue;
    const dim3 grid(d / R);
    switch (f / 128) {
#define MOE_DOWN_CASE(N)                                                                     \
    case N:                                                                                  \
        return timed_launch("down_combine", down_token_mfma_kernel<N>, grid, dim3(512), lds, \
                            s, hq, w, plan, y, d, E, k, f, R);
        MOE_DOWN_CASE(12)
        MOE_DOWN_CASE(24)
#undef MOE_DOWN_CASE
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
