// ffn_fp8_mfma.hip -- the routed expert FFN with FP8 experts on the gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), for many rows per expert.
//
// The FP8 store is E4M3FN codes with one fp32 scale per 128 x 128 block of
// each matrix.  Weight tiles stay FP8 in LDS; when a wave reads its B
// fragment (8 codes per lane) it converts the codes exactly to fp32,
// multiplies them by their block's scale and rounds the products to bf16
// (one rounding per weight: relative error at most 2^-9), so the matrix
// cores see the dequantised weight tile.  Activations are used as given
// (bf16), accumulation is fp32.  A block's gate columns, its up columns and
// a wave's down columns each lie inside one 128-row scale block, so a wave
// needs at most two scales per 128-element K chunk.
//
//   gate/up: h[p][n] = bf16(silu(x_t . Wg[n]) * (x_t . Wu[n])), t = sorted_rows[p] / k
//   down:    rows_out[p][m] = bf16(h[p] . Wd[m])
//
// Work units are (row tile of <= 128 rows of one expert, column block): a
// block tile of up to 128 rows x 512 weight rows (gate/up: 256 gate + the
// matching 256 up rows), K step 64, eight waves.  A row tile runs at the
// smallest height of 32, 64 or 128 rows that holds it (an expert's last
// tile is usually short), so the matrix work follows the rows; at 128 rows
// each wave takes 64 x 128, i.e. 2 x 4 MFMA tiles of 32 x 32 (gate/up: two
// gate tiles and the two up tiles of the same columns, so the SwiGLU is
// local to a lane).
// Operand pieces go global -> registers -> LDS: two steps' loads are in
// flight in registers while a third is multiplied from LDS (two LDS
// buffers, one barrier per step).  LDS layout per buffer: A bf16 rows of 64
// K padded to 144 bytes; B as 8 chunk planes (8 K each) of 512 rows x 8
// bytes, planes 4128 bytes apart, so that a half-wave's fragment reads (32
// rows of one chunk) and its stores (8 rows x 4 pieces) hit distinct banks.
// Units are ordered column block by column block with an expert's row tiles
// adjacent, so the blocks that share a weight slice run together, and the 8
// XCDs each take a contiguous run of units.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;                    // rows per tile
constexpr int kTN = 512;                    // weight rows per block
constexpr int kBK = 64;                     // K per step
constexpr int kRow = kBK + 8;               // bf16 per LDS row of A (16-byte pad)
constexpr int kABytes = kTM * kRow * 2;     // 18432
constexpr int kPlane = kTN * 8 + 32;        // bytes per chunk plane of B: 4128
constexpr int kBBytes = 8 * kPlane;         // 33024
constexpr int kStage = kABytes + kBBytes;   // 51456
constexpr int kLds = 2 * kStage;            // 102912
constexpr int kThreads = 512;

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// A fragment: 8 bf16 of LDS row `row` from K element kq.
__device__ __forceinline__ bf16x8_t afrag(const uint8_t *a, int row, int kq) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(a + row * (kRow * 2) + kq * 2));
}

// B fragment: 8 E4M3FN codes (one lane's K half of a 16-K slice) of LDS
// row `row` from chunk plane `c`, times the block scale, rounded to bf16.
__device__ __forceinline__ bf16x8_t bfrag(const uint8_t *b, int c, int row, float s) {
    const uint2 raw = *reinterpret_cast<const uint2 *>(b + c * kPlane + row * 8);
    const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, 1.0f, false);
    const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, 1.0f, true);
    const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, 1.0f, false);
    const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, 1.0f, true);
    bf16x8_t o;
    o[0] = (__bf16)(v0.x * s);
    o[1] = (__bf16)(v0.y * s);
    o[2] = (__bf16)(v1.x * s);
    o[3] = (__bf16)(v1.y * s);
    o[4] = (__bf16)(v2.x * s);
    o[5] = (__bf16)(v2.y * s);
    o[6] = (__bf16)(v3.x * s);
    o[7] = (__bf16)(v3.y * s);
    return o;
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

// One unit: rows [row0, row0 + rows) of expert e (rows <= MT), column
// block nb.  kGU: A = x [T][K = d] gathered by sorted_rows, B = Wgu
// [E][2f][d], out = h bf16 [rows][f]; else A = h [rows][K = f], B = Wdn
// [E][d][f], out = rows_out bf16 [rows][d].  Columns past the end are
// loaded clamped and not stored.
//
// MT = 128: waves (wm, wn) in 2 x 4 take 64 rows x 128 weight rows (2 x 4
// MFMA tiles); MT = 64: 32 rows x 128 (1 x 4); MT = 32: all 32 rows x 64
// weight rows (1 x 2).  Gate/up: a wave's first half of column tiles are
// gate columns and its second half the up columns of the same f range.
template <bool kGU, int MT>
__device__ __forceinline__ void fp8_tile(const uint16_t *__restrict__ act,
                                         const int32_t *__restrict__ sorted_rows, int k,
                                         const uint8_t *__restrict__ W,
                                         const float *__restrict__ S, uint16_t *__restrict__ out,
                                         int nrows, int d, int f, int nb, int row0, int rows,
                                         uint8_t *lds) {
    constexpr int MTW = MT == 128 ? 2 : 1;          // m-tiles per wave
    constexpr int NTW = MT == 32 ? 2 : 4;           // n-tiles per wave
    constexpr int kAPieces = MT * 8;                // 16-byte A pieces per step
    const int K = kGU ? d : f;
    const int brows = kGU ? 2 * f : d;
    const int N = kGU ? f : d;
    const int T = nrows / k;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int l32 = lane & 31, h = lane >> 5;

    // this thread's A pieces (row p >> 3, 8-element piece p & 7, p = c * 512
    // + tid < MT * 8) and B pieces (row c * 128 + tid / 4, 16-code piece
    // tid % 4), as byte offsets (the step's K offset goes in the scalar
    // offset of the buffer loads)
    const rsrc_t ra = make_rsrc(act, (uint32_t)((size_t)(kGU ? T : nrows) * K * 2));
    const rsrc_t rb = make_rsrc(W, (uint32_t)((size_t)brows * K));
    uint32_t aoff[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int pa = c * kThreads + tid, r = min(pa >> 3, rows - 1);
        const int src = kGU ? min(max(sorted_rows[row0 + r] / k, 0), T - 1) : row0 + r;
        aoff[c] = (uint32_t)src * (uint32_t)K * 2u + 16u * (uint32_t)(pa & 7);
    }
    const bool a_mine0 = tid < kAPieces, a_mine1 = kThreads + tid < kAPieces;
    uint32_t boff[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int r = c * 128 + (tid >> 2);
        int wr;
        if (kGU) wr = (r < 256 ? 0 : f) + min(nb * 256 + (r & 255), f - 1);
        else wr = min(nb * kTN + r, d - 1);
        boff[c] = (uint32_t)wr * (uint32_t)K + 16u * (uint32_t)(tid & 3);
    }
    // this wave's rows and weight rows in the block tile
    const int ar0 = (MT == 128 ? wm * 64 : MT == 64 ? wm * 32 : 0) + l32;
    int br[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        if (MT == 32)
            br[j] = kGU ? (j == 0 ? 0 : 256) + wn * 64 + 32 * wm + l32 : wn * 128 + wm * 64 + 32 * j + l32;
        else
            br[j] = kGU ? (j < 2 ? 0 : 256) + wn * 64 + 32 * (j & 1) + l32 : wn * 128 + 32 * j + l32;
    }
    // scale rows: the wave's gate (or down) columns and, for gate/up, the
    // up columns f / 128 blocks later
    const int srow0 = kGU ? min((nb * 256 + wn * 64) >> 7, f / 128 - 1)
                          : min((nb * kTN + wn * 128) >> 7, d / 128 - 1);
    const float *s0 = S + (size_t)srow0 * (K / 128);
    const float *s1 = S + (size_t)(kGU ? srow0 + f / 128 : srow0) * (K / 128);

    f32x16_t acc[MTW][NTW];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // LDS places of this thread's pieces: A rows tid / 8 and 64 + tid / 8;
    // B rows c * 128 + tid / 4, planes 2 (tid % 4) and 2 (tid % 4) + 1
    const int a_off = (tid >> 3) * (kRow * 2) + 16 * (tid & 7);
    const int b_off = kABytes + 2 * (tid & 3) * kPlane + (tid >> 2) * 8;

    // two register sets of this thread's pieces
    uint4 pa0, pa1, pb0, pb1, pb2, pb3, qa0, qa1, qb0, qb1, qb2, qb3;
#define FP8_LOAD(S, k0)                                                   \
    do {                                                                  \
        const uint32_t ka_ = (uint32_t)(k0) * 2u, kb_ = (uint32_t)(k0);   \
        if (a_mine0) S##a0 = buf_load16(ra, aoff[0], ka_);                \
        if (a_mine1) S##a1 = buf_load16(ra, aoff[1], ka_);                \
        S##b0 = buf_load16(rb, boff[0], kb_);                             \
        S##b1 = buf_load16(rb, boff[1], kb_);                             \
        S##b2 = buf_load16(rb, boff[2], kb_);                             \
        S##b3 = buf_load16(rb, boff[3], kb_);                             \
    } while (0)
#define FP8_STORE_B(v, c, buf)                                                             \
    do {                                                                                   \
        *reinterpret_cast<uint2 *>((buf) + b_off + (c) * 1024) = uint2{v.x, v.y};          \
        *reinterpret_cast<uint2 *>((buf) + b_off + (c) * 1024 + kPlane) = uint2{v.z, v.w}; \
    } while (0)
#define FP8_STORE(S, buf)                                                              \
    do {                                                                               \
        uint8_t *b_ = (buf);                                                           \
        if (a_mine0) *reinterpret_cast<uint4 *>(b_ + a_off) = S##a0;                   \
        if (a_mine1) *reinterpret_cast<uint4 *>(b_ + a_off + 64 * (kRow * 2)) = S##a1; \
        FP8_STORE_B(S##b0, 0, b_);                                                     \
        FP8_STORE_B(S##b1, 1, b_);                                                     \
        FP8_STORE_B(S##b2, 2, b_);                                                     \
        FP8_STORE_B(S##b3, 3, b_);                                                     \
    } while (0)
#define FP8_MULTIPLY(buf, sa, sb)                                                         \
    do {                                                                                  \
        const uint8_t *la_ = (buf), *lb_ = la_ + kABytes;                                 \
        _Pragma("unroll") for (int ks = 0; ks < kBK / 16; ++ks) {                         \
            bf16x8_t a_[MTW];                                                             \
            _Pragma("unroll") for (int i = 0; i < MTW; ++i)                               \
                a_[i] = afrag(la_, ar0 + 32 * i, ks * 16 + 8 * h);                        \
            _Pragma("unroll") for (int j = 0; j < NTW; ++j) {                             \
                const bf16x8_t b = bfrag(lb_, 2 * ks + h, br[j], j < NTW / 2 ? (sa) : (sb)); \
                _Pragma("unroll") for (int i = 0; i < MTW; ++i)                           \
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_[i], b, acc[i][j], 0, 0, 0); \
            }                                                                             \
        }                                                                                 \
    } while (0)

    // K / 64 steps, an even number: each iteration multiplies one 128-K
    // chunk (step kt from LDS buffer 0, kt + 1 from buffer 1)
    const int nk = K / kBK;
    FP8_LOAD(p, 0);
    FP8_STORE(p, lds);
    FP8_LOAD(p, kBK);
    if (nk > 2) FP8_LOAD(q, 2 * kBK);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        const float sa = s0[kt >> 1], sb = kGU ? s1[kt >> 1] : sa;
        FP8_MULTIPLY(lds, sa, sb);
        FP8_STORE(p, lds + kStage);                 // step kt + 1
        if (kt + 3 < nk) FP8_LOAD(p, (kt + 3) * kBK);
        __syncthreads();
        FP8_MULTIPLY(lds + kStage, sa, sb);
        if (kt + 2 < nk) FP8_STORE(q, lds);         // step kt + 2
        if (kt + 4 < nk) FP8_LOAD(q, (kt + 4) * kBK);
        __syncthreads();
    }
#undef FP8_LOAD
#undef FP8_STORE_B
#undef FP8_STORE
#undef FP8_MULTIPLY

    // register r of a 32 x 32 tile holds row 8 (r / 4) + 4 (lane / 32) + r % 4,
    // column lane % 32
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lr = ar0 - l32 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
            if (lr >= rows) continue;
            uint16_t *orow = out + (size_t)(row0 + lr) * N;
            if (kGU) {
#pragma unroll
                for (int j = 0; j < NTW / 2; ++j) {
                    const int col = nb * 256 + (br[j] - l32) + l32;
                    if (col < f)
                        orow[col] = f32_to_bf16_rne(silu_mul(acc[i][j][r], acc[i][j + NTW / 2][r]));
                }
            } else {
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int col = nb * kTN + br[j];
                    if (col < d) orow[col] = f32_to_bf16_rne(acc[i][j][r]);
                }
            }
        }
}

// nbn column blocks per row tile (gate/up: f / 256, down: d / 512, rounded
// up); each row tile runs with the smallest height of 32, 64 or 128 rows
// that holds its rows.
template <bool kGU>
__global__ __launch_bounds__(kThreads) void fp8_mfma_kernel(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ sorted_rows, int k,
    const uint8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ tiles, uint16_t *__restrict__ out, int nrows, int d, int f,
    int nbn) {
    extern __shared__ __align__(16) uint8_t lds[];
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
    const int brows = kGU ? 2 * f : d;
    const uint8_t *W = codes + (size_t)e * brows * K;
    const float *S = scales + (size_t)e * (brows / 128) * (K / 128);
    if (rows > 64)
        fp8_tile<kGU, 128>(act, sorted_rows, k, W, S, out, nrows, d, f, nb, row0, rows, lds);
    else if (rows > 32)
        fp8_tile<kGU, 64>(act, sorted_rows, k, W, S, out, nrows, d, f, nb, row0, rows, lds);
    else
        fp8_tile<kGU, 32>(act, sorted_rows, k, W, S, out, nrows, d, f, nb, row0, rows, lds);
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
    // 32-bit buffer offsets: x, h and one expert's matrix under 4 GiB
    const double lim = 4294967296.0;
    if ((double)T * k * std::max(d, f) * 2.0 >= lim || 2.0 * f * d >= lim) return false;
    return T >= kMfmaMinT && d % 128 == 0 && f % 128 == 0 && E <= (1 << 20) &&
           (long long)fp8_mfma_max_tiles(T, E, k) * std::max((f + 255) / 256, (d + kTN - 1) / kTN) <
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
    const int nbn_gu = (f + 255) / 256, nbn_dn = (d + kTN - 1) / kTN;
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
