// ffn_fp8_mfma.hip -- the routed expert FFN with FP8 experts on the gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), for many rows per expert.
//
// The FP8 store is E4M3FN codes with one fp32 scale per 128 x 128 block of
// each matrix.  Every E4M3FN value is exactly a bf16 value, so the codes are
// converted exactly (the scaled convert with scale 1.0) when a weight tile
// goes from registers into LDS, the activations stay bf16 as given, and the
// block scale is applied in fp32: the products of each 128-element K chunk
// are accumulated apart (one chunk = two K steps of 64) and then added to
// the result times that chunk's scale.  A block's 128 gate columns, its 128
// up columns and a wave's 64 down columns each lie inside one 128-row scale
// block, so each wave needs one scale per accumulator tile and chunk.
//
//   gate/up: h[p][n] = bf16(silu(x_t . Wg[n]) * (x_t . Wu[n])), t = sorted_rows[p] / k
//   down:    rows_out[p][m] = bf16(h[p] . Wd[m])
//
// Work units are (row tile of <= 128 rows of one expert, column block): a
// block tile of 128 rows x 256 weight rows (gate/up: 128 gate + the matching
// 128 up rows), K step 64, eight waves as 2 (rows) x 4 (columns) of 64 x 64,
// i.e. 2 x 2 MFMA tiles of 32 x 32 each.  Operand tiles go global ->
// registers -> LDS (rows padded by 16 bytes), double-buffered with one
// barrier per step.  Units are ordered column block by column block with an
// expert's row tiles adjacent, so the blocks that share a weight slice run
// together, and the 8 XCDs each take a contiguous run of units.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;                    // rows per tile
constexpr int kTN = 256;                    // weight rows per block
constexpr int kBK = 64;                     // K per step
constexpr int kRow = kBK + 8;               // bf16 per LDS row (16-byte pad)
constexpr int kATile = kTM * kRow;          // bf16
constexpr int kBTile = kTN * kRow;          // bf16
constexpr int kStage = kATile + kBTile;     // bf16 per buffer
constexpr int kLds = 2 * kStage * 2;        // bytes: 110592
constexpr int kThreads = 512;

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// 16 E4M3FN codes -> 16 bf16 (exact), element order kept.
__device__ __forceinline__ void fp8x16_to_bf16(uint4 c, uint4 &lo, uint4 &hi) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    }
    lo = uint4{o[0], o[1], o[2], o[3]};
    hi = uint4{o[4], o[5], o[6], o[7]};
}

__device__ __forceinline__ bf16x8_t frag(const uint16_t *tile, int row, int kq) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(tile + row * kRow + kq));
}

// An expert's rows [r0, r0 + c) from offsets; an inconsistent range counts
// as empty, so that no tile reaches outside the nrows grouped rows.
__device__ __forceinline__ int group_rows(const int32_t *offsets, int e, int nrows, int &r0) {
    r0 = offsets[e];
    const int c = offsets[e + 1] - r0;
    return (r0 >= 0 && c > 0 && r0 <= nrows - c) ? c : 0;
}

// The row tiles of the grouped rows: tiles[0] = their number, then (expert,
// first row, rows) per tile, experts ascending; at most max_tiles.  One
// block.
__global__ __launch_bounds__(1024) void fp8_tile_plan_kernel(const int32_t *__restrict__ offsets,
                                                             int E, int nrows, int max_tiles,
                                                             int32_t *__restrict__ tiles) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    const int per = (E + 1023) / 1024;
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int mine = 0, r0;
    for (int e = e0; e < e1; ++e) mine += (group_rows(offsets, e, nrows, r0) + kTM - 1) / kTM;
    part[tid] = mine;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {            // inclusive scan
        const int v = tid >= s ? part[tid - s] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int base = part[tid] - mine;
    for (int e = e0; e < e1; ++e) {
        const int c = group_rows(offsets, e, nrows, r0);
        for (int i = 0; i * kTM < c && base < max_tiles; ++i, ++base) {
            tiles[1 + 3 * base] = e;
            tiles[2 + 3 * base] = r0 + i * kTM;
            tiles[3 + 3 * base] = min(kTM, c - i * kTM);
        }
    }
    if (tid == 1023) tiles[0] = min(part[1023], max_tiles);
}

// kGU: A = x [T][K = d] gathered by sorted_rows, B = Wgu [E][2f][d], out =
// h bf16 [rows][f]; else A = h [rows][K = f], B = Wdn [E][d][f], out =
// rows_out bf16 [rows][d].  nbn column blocks per tile (gate/up: f / 128,
// down: d / 256 rounded up).
template <bool kGU>
__global__ __launch_bounds__(kThreads) void fp8_mfma_kernel(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ sorted_rows, int k,
    const uint8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ tiles, uint16_t *__restrict__ out, int nrows, int d, int f,
    int nbn) {
    extern __shared__ __align__(16) uint16_t lds[];
    const int n_tiles = tiles[0];
    const int units = n_tiles * nbn;
    const int per = (units + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    if (slot >= per) return;
    const int u = (int)(blockIdx.x & 7) * per + slot;
    if (u >= units) return;
    const int nb = u / n_tiles, t = u - nb * n_tiles;
    const int e = tiles[1 + 3 * t], row0 = tiles[2 + 3 * t], rows = tiles[3 + 3 * t];

    const int K = kGU ? d : f;
    const int brows = kGU ? 2 * f : d;              // weight rows per expert
    const int N = kGU ? f : d;                      // output columns
    const uint8_t *W = codes + (size_t)e * brows * K;
    const float *S = scales + (size_t)e * (brows / 128) * (K / 128);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int T = (int)(nrows / k);
    const int l32 = lane & 31, kh = 8 * (lane >> 5);

    // this thread's two A pieces (row p >> 3, K piece p & 7) and two B
    // pieces (row p >> 2, 16-code piece p & 3), p = c * 512 + tid
    const uint16_t *arow[2];
    const uint8_t *brow[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int pa = c * kThreads + tid, ra = min(pa >> 3, rows - 1);
        const size_t src = kGU ? (size_t)min(max(sorted_rows[row0 + ra] / k, 0), T - 1)
                               : (size_t)(row0 + ra);
        arow[c] = act + src * K + 8 * (pa & 7);
        const int pb = c * kThreads + tid, rb = pb >> 2;
        int wr;
        if (kGU) wr = (rb < 128 ? 0 : f) + nb * 128 + (rb & 127);
        else wr = min(nb * kTN + rb, d - 1);
        brow[c] = W + (size_t)wr * K + 16 * (pb & 3);
    }
    // scales of this wave's two column tiles: gate/up: gate block nb, up
    // block f/128 + nb; down: block (nb * 256 + wn * 64) / 128
    const int srow0 = kGU ? nb : min((nb * kTN + wn * 64) / 128, d / 128 - 1);
    const int srow1 = kGU ? f / 128 + nb : srow0;
    const float *s0 = S + (size_t)srow0 * (K / 128);
    const float *s1 = S + (size_t)srow1 * (K / 128);

    // LDS rows of this wave's fragments
    const int ar0 = wm * 64 + l32;
    const int br0 = kGU ? wn * 32 + l32 : wn * 64 + l32;
    const int br1 = kGU ? 128 + wn * 32 + l32 : wn * 64 + 32 + l32;

    f32x16_t acc[2][2], tmp[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ga0, ga1, gb0, gb1;
#define FP8_LOAD(k0)                                                    \
    do {                                                                \
        ga0 = *reinterpret_cast<const uint4 *>(arow[0] + (k0));         \
        ga1 = *reinterpret_cast<const uint4 *>(arow[1] + (k0));         \
        gb0 = *reinterpret_cast<const uint4 *>(brow[0] + (k0));         \
        gb1 = *reinterpret_cast<const uint4 *>(brow[1] + (k0));         \
    } while (0)
    // LDS places of this thread's pieces
    const int a_off0 = (tid >> 3) * kRow + 8 * (tid & 7);
    const int a_off1 = ((kThreads + tid) >> 3) * kRow + 8 * (tid & 7);
    const int b_off0 = kATile + (tid >> 2) * kRow + 16 * (tid & 3);
    const int b_off1 = kATile + ((kThreads + tid) >> 2) * kRow + 16 * (tid & 3);
#define FP8_STORE(buf)                                                  \
    do {                                                                \
        uint16_t *b_ = (buf);                                           \
        *reinterpret_cast<uint4 *>(b_ + a_off0) = ga0;                  \
        *reinterpret_cast<uint4 *>(b_ + a_off1) = ga1;                  \
        uint4 lo_, hi_;                                                 \
        fp8x16_to_bf16(gb0, lo_, hi_);                                  \
        *reinterpret_cast<uint4 *>(b_ + b_off0) = lo_;                  \
        *reinterpret_cast<uint4 *>(b_ + b_off0 + 8) = hi_;              \
        fp8x16_to_bf16(gb1, lo_, hi_);                                  \
        *reinterpret_cast<uint4 *>(b_ + b_off1) = lo_;                  \
        *reinterpret_cast<uint4 *>(b_ + b_off1 + 8) = hi_;              \
    } while (0)

    const int nk = K / kBK;
    FP8_LOAD(0);
    FP8_STORE(lds);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) FP8_LOAD((kt + 1) * kBK);
        if ((kt & 1) == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) tmp[i][j][r] = 0.f;
        }
        const uint16_t *la = lds + (kt & 1) * kStage, *lb = la + kATile;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kq = ks * 16 + kh;
            const bf16x8_t a0 = frag(la, ar0, kq), a1 = frag(la, ar0 + 32, kq);
            const bf16x8_t b0 = frag(lb, br0, kq), b1 = frag(lb, br1, kq);
            tmp[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, tmp[0][0], 0, 0, 0);
            tmp[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, tmp[0][1], 0, 0, 0);
            tmp[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, tmp[1][0], 0, 0, 0);
            tmp[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, tmp[1][1], 0, 0, 0);
        }
        if (kt & 1) {                                // chunk kt / 2 complete
            const float sa = s0[kt >> 1], sb = s1[kt >> 1];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc[i][0][r] = fmaf(sa, tmp[i][0][r], acc[i][0][r]);
                    acc[i][1][r] = fmaf(sb, tmp[i][1][r], acc[i][1][r]);
                }
        }
        if (more) FP8_STORE(lds + ((kt + 1) & 1) * kStage);
        __syncthreads();
    }

#undef FP8_LOAD
#undef FP8_STORE

    // register r of a 32 x 32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4,
    // column lane % 32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lr = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (lr >= rows) continue;
            uint16_t *orow = out + (size_t)(row0 + lr) * N;
            if (kGU) {
                orow[nb * 128 + wn * 32 + l32] = f32_to_bf16_rne(silu_mul(acc[i][0][r], acc[i][1][r]));
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = nb * kTN + wn * 64 + 32 * j + l32;
                    if (col < d) orow[col] = f32_to_bf16_rne(acc[i][j][r]);
                }
            }
        }
}

bool g_attr_done = false;

hipError_t set_attrs() {
    if (g_attr_done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)fp8_mfma_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)fp8_mfma_kernel<false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess) g_attr_done = true;
    return e;
}

}  // namespace

int fp8_mfma_max_tiles(int T, int E, int k) {
    const long long rows = (long long)T * k;
    return (int)((rows + kTM - 1) / kTM + std::min<long long>(E, rows));
}

size_t fp8_mfma_tiles_bytes(int T, int E, int k) {
    return (size_t)(1 + 3 * (size_t)fp8_mfma_max_tiles(T, E, k)) * 4;
}

bool fp8_mfma_ok(int T, int d, int E, int k, int f) {
    return T >= kMfmaMinT && d % 128 == 0 && f % 128 == 0 && E <= (1 << 20) &&
           (long long)fp8_mfma_max_tiles(T, E, k) * std::max(f / 128, (d + kTN - 1) / kTN) <
               (1LL << 31) - 8;
}

hipError_t launch_fp8_mfma_ffn(const uint16_t *x, Fp8Args w, const int32_t *offsets,
                               const int32_t *sorted_rows, int32_t *tiles, uint16_t *h,
                               uint16_t *rows_out, int T, int d, int E, int k, int f,
                               hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipError_t e = set_attrs();
    if (e != hipSuccess) return e;
    const int max_tiles = fp8_mfma_max_tiles(T, E, k);
    e = timed_launch("fp8_plan", fp8_tile_plan_kernel, dim3(1), dim3(1024), 0, s, offsets, E,
                     T * k, max_tiles, tiles);
    if (e != hipSuccess) return e;
    const int nbn_gu = f / 128, nbn_dn = (d + kTN - 1) / kTN;
    const long long ug = (long long)max_tiles * nbn_gu, ud = (long long)max_tiles * nbn_dn;
    e = timed_launch("fp8_gate_up", fp8_mfma_kernel<true>, dim3((unsigned)(8 * ((ug + 7) / 8))),
                     dim3(kThreads), kLds, s, x, sorted_rows, k, w.gu_codes, w.gu_scales,
                     (const int32_t *)tiles, h, T * k, d, f, nbn_gu);
    if (e != hipSuccess) return e;
    return timed_launch("fp8_down", fp8_mfma_kernel<false>, dim3((unsigned)(8 * ((ud + 7) / 8))),
                        dim3(kThreads), kLds, s, (const uint16_t *)h, sorted_rows, k, w.dn_codes,
                        w.dn_scales, (const int32_t *)tiles, rows_out, T * k, d, f, nbn_dn);
}

}  // namespace moe
