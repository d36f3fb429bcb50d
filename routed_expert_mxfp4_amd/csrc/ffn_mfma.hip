// ffn_mfma.hip -- routed expert FFN for prefill-sized row groups on gfx950
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The weights are fed to the matrix cores exactly as stored: E2M1 codes and
// their E8M0 block scales are the B operand and its scale (one lane holds
// one 32-element MX block of one weight row, which is the canonical layout's
// row-major K-contiguous block).  The A operand (activations x for gate/up,
// h for down) is split into two MX E2M3 terms, a = hi + lo with
// hi = MX(a), lo = MX(a - hi), each with its own E8M0 scale per 32 elements
// along K; both terms go through the matrix core (two MFMAs per tile step)
// and accumulate into one fp32 tile.  A single 6-bit term keeps only ~3
// significant bits and misses the output tolerance; two terms keep ~7.
//
// Layouts (per row; a "step" is 128 K elements = 4 MX blocks):
//   q [rows][K/128][2 terms][4 blocks][24 B]   E2M3 codes, 6-bit fields
//                                             packed little-endian
//   s [rows][K/128][2 terms][4 blocks]        E8M0 scale codes
// MFMA operand layout (16x16x128): lane l holds row (l % 16) of a 16-row
// tile and K block (l / 16) of the step; the output tile holds
// C[4 * (l / 16) + i][l % 16] in lane l, register i.
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStepQ = 192;      // bytes of codes per row per step (2 terms x 96)
constexpr int kStepS = 8;        // scale bytes per row per step

// ---------------------------------------------------------------------------
// MX E2M3 conversion (OCP MX v1.0): shared exponent X = floor(log2(amax)) - 2
// clamped to [-127, 127] (E8M0 code X + 127; an all-zero block gets code 0);
// elements v / 2^X rounded to nearest even onto the E2M3 grid (subnormals
// 0, 1/8, .., 7/8; then 1..1.875, 2..3.75, 4..7.5), saturating at 7.5.  The
// code is monotone in the rounded magnitude, so it is computed directly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.f)) return -127;
    int e;
    (void)frexpf(amax, &e);                       // amax = m 2^e, m in [0.5, 1)
    return min(max(e - 1 - 2, -127), 127);
}

__device__ __forceinline__ uint32_t e2m3_encode(float r) {
    const uint32_t sign = (__float_as_uint(r) >> 31) << 5;
    const float a = fabsf(r);
    uint32_t c;
    if (a >= 7.5f) c = 31u;
    else if (a < 2.0f) c = (uint32_t)__builtin_rintf(a * 8.0f);
    else if (a < 4.0f) c = 8u + (uint32_t)__builtin_rintf(a * 4.0f);
    else c = 16u + (uint32_t)__builtin_rintf(a * 2.0f);
    return sign | c;
}

__device__ __forceinline__ float e2m3_decode(uint32_t c) {
    const uint32_t f = (c >> 3) & 3u, m = c & 7u;
    const float mag = f == 0u ? (float)m * 0.125f : ldexpf(1.0f + (float)m * 0.125f, (int)f - 1);
    return (c & 32u) ? -mag : mag;
}

__device__ __forceinline__ float group16_max_f32(float v) {
    v = fmaxf(v, dpp_ror_f32<8>(v));
    v = fmaxf(v, dpp_ror_f32<4>(v));
    v = fmaxf(v, dpp_ror_f32<2>(v));
    v = fmaxf(v, dpp_ror_f32<1>(v));
    return v;
}

template <typename In>
__device__ __forceinline__ float2 load_pair_f32(const In *p);
template <>
__device__ __forceinline__ float2 load_pair_f32<uint16_t>(const uint16_t *p) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
    return make_float2(bf16_bits_to_f32(w & 0xFFFFu), bf16_bits_to_f32(w >> 16));
}
template <>
__device__ __forceinline__ float2 load_pair_f32<float>(const float *p) {
    return *reinterpret_cast<const float2 *>(p);
}

// Packs the 12-bit code pairs of the 16 lanes of a group (lane j: elements
// 2j, 2j+1 of the block) into the block's 24 bytes: lanes j % 4 == 0 write
// 6 bytes (three 16-bit words) covering lanes j .. j+3.
__device__ __forceinline__ void store_block_codes(uint8_t *dst24, uint32_t pair12, int j) {
    const uint32_t p1 = (uint32_t)__shfl_down((int)pair12, 1, 16);
    const uint32_t p2 = (uint32_t)__shfl_down((int)pair12, 2, 16);
    const uint32_t p3 = (uint32_t)__shfl_down((int)pair12, 3, 16);
    if ((j & 3) == 0) {
        const unsigned long long bits = (unsigned long long)pair12 |
                                        ((unsigned long long)p1 << 12) |
                                        ((unsigned long long)p2 << 24) |
                                        ((unsigned long long)p3 << 36);
        uint16_t *w = reinterpret_cast<uint16_t *>(dst24 + 6 * (j >> 2));
        w[0] = (uint16_t)(bits & 0xFFFFu);
        w[1] = (uint16_t)((bits >> 16) & 0xFFFFu);
        w[2] = (uint16_t)((bits >> 32) & 0xFFFFu);
    }
}

// One wave per (row, step): lane l handles elements 2j, 2j+1 (j = l % 16) of
// MX block g = l / 16 of the step.  Rows are `src_row(r)` of the input.
template <typename In>
__global__ __launch_bounds__(256) void mx_split_e2m3_kernel(const In *__restrict__ in, int rows,
                                                            int K, uint8_t *__restrict__ q,
                                                            uint8_t *__restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int nsteps = K >> 7;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long long)rows * nsteps) return;
    const int r = (int)(item / nsteps), st = (int)(item % nsteps);
    const int g = lane >> 4, j = lane & 15;
    const float2 v = load_pair_f32<In>(in + (size_t)r * K + (size_t)st * 128 + g * 32 + 2 * j);
    uint8_t *qrow = q + ((size_t)r * nsteps + st) * kStepQ;
    uint8_t *srow = s + ((size_t)r * nsteps + st) * kStepS;
    // hi term
    const float amax_h = group16_max_f32(fmaxf(fabsf(v.x), fabsf(v.y)));
    const int xh = mx_exponent(amax_h);
    const uint32_t h0 = e2m3_encode(ldexpf(v.x, -xh)), h1 = e2m3_encode(ldexpf(v.y, -xh));
    // lo term: the residual a - hi is exact in fp32
    const float r0 = v.x - ldexpf(e2m3_decode(h0), xh);
    const float r1 = v.y - ldexpf(e2m3_decode(h1), xh);
    const float amax_l = group16_max_f32(fmaxf(fabsf(r0), fabsf(r1)));
    const int xl = mx_exponent(amax_l);
    const uint32_t l0 = e2m3_encode(ldexpf(r0, -xl)), l1 = e2m3_encode(ldexpf(r1, -xl));
    store_block_codes(qrow + g * 24, h0 | (h1 << 6), j);
    store_block_codes(qrow + 96 + g * 24, l0 | (l1 << 6), j);
    if (j == 0) {
        srow[g] = (uint8_t)(xh + 127);
        srow[4 + g] = (uint8_t)(xl + 127);
    }
}

// ---------------------------------------------------------------------------
// Tile plan: per active expert, the number of 128-row tiles and their
// exclusive prefix.  tiles[0] = total, tiles[1 + a] = prefix of expert a.
// ---------------------------------------------------------------------------
constexpr int kBM = 128;

__global__ __launch_bounds__(1024) void mfma_plan_kernel(const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ plan,
                                                         int32_t *__restrict__ tiles, int E) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int nact = plan[0];
    int c = 0;
    if (tid < nact) {
        const int e = plan[1 + tid];
        const int n = ((unsigned)e < (unsigned)E) ? offsets[e + 1] - offsets[e] : 0;
        c = (n + kBM - 1) / kBM;
    }
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64);
        if (lane >= o) inc += u;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wid; ++w) base += wsum[w];
    if (tid < nact) tiles[1 + tid] = base + inc - c;
    if (tid == 1023) tiles[0] = base + inc;
}

// Which (active expert, m-tile) a global m-tile index belongs to: binary
// search over the tile prefix of the plan's active experts.
__device__ __forceinline__ int find_expert(const int32_t *tiles, int nact, int mt) {
    int lo = 0, hi = nact - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tiles[1 + mid] <= mt) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Grouped scaled-MFMA GEMM tile: 128 rows x 128 columns, K in steps of 128,
// 4 waves in a 2 x 2 arrangement (64 x 64 per wave = 4 x 4 MFMA tiles, two A
// terms each).  LDS holds two stages (double buffer); the next step's global
// loads sit in registers while the current step computes.
// ---------------------------------------------------------------------------
constexpr int kAStride = 208;    // LDS bytes per A row (192 + pad: 16-B aligned, conflict-free b64 reads)
constexpr int kBStride = 80;     // LDS bytes per B row (64 + pad: conflict-free b128 reads)

struct alignas(16) Stage {
    uint8_t a[kBM][kAStride];
    uint8_t as[kBM][kStepS];
    uint8_t b[128][kBStride];
    uint8_t bs[128][4];
};

__device__ __forceinline__ i32x8_t load_a_frag(const uint8_t *p) {
    const uint2 w0 = *reinterpret_cast<const uint2 *>(p);
    const uint2 w1 = *reinterpret_cast<const uint2 *>(p + 8);
    const uint2 w2 = *reinterpret_cast<const uint2 *>(p + 16);
    i32x8_t v = {(int)w0.x, (int)w0.y, (int)w1.x, (int)w1.y, (int)w2.x, (int)w2.y, 0, 0};
    return v;
}

__device__ __forceinline__ i32x8_t load_b_frag(const uint8_t *p) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    i32x8_t v = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    return v;
}

// The tile step: 32 MFMAs per wave.  acc[mt][nt] += A(mt) . B(nt) for both
// A terms, scales per lane.
// B rows of the wave's four 16-column tiles: gate/up (kGateUp) takes
// gate rows wn*32 + {0,16} and the matching up rows 64 + wn*32 + {0,16};
// down takes rows wn*64 + {0,16,32,48}.
template <bool kGateUp>
__device__ __forceinline__ int b_tile_row(int wn, int nt) {
    return kGateUp ? (nt >> 1) * 64 + wn * 32 + (nt & 1) * 16 : wn * 64 + nt * 16;
}

template <bool kGateUp>
__device__ __forceinline__ void mfma_step(const Stage &S, int wm, int wn, int lane,
                                          f32x4_t (&acc)[4][4]) {
    const int r16 = lane & 15, g = lane >> 4;
    i32x8_t b[4];
    int bsc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int br = b_tile_row<kGateUp>(wn, nt) + r16;
        b[nt] = load_b_frag(&S.b[br][g * 16]);
        bsc[nt] = S.bs[br][g];
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int ar = wm * 64 + mt * 16 + r16;
        const i32x8_t ahi = load_a_frag(&S.a[ar][g * 24]);
        const i32x8_t alo = load_a_frag(&S.a[ar][96 + g * 24]);
        const int shi = S.as[ar][g], slo = S.as[ar][4 + g];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                ahi, b[nt], acc[mt][nt], 2, 4, 0, shi, 0, bsc[nt]);
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                alo, b[nt], acc[mt][nt], 2, 4, 0, slo, 0, bsc[nt]);
        }
    }
}

// Global -> LDS loads of one step go straight into LDS (gfx950 direct
// loads: lane l of a wave instruction fills LDS bytes base + size * l), so
// no registers hold the next step.  Each LDS region is a run of equal slots
// (A: 13 slots of 16 B per row, the 13th a pad slot that repeats a valid
// piece; B: 5 slots per row; scales in 4-byte slots), and wave w issues the
// instructions covering slots 64 * (4 i + w) .. + 63.
struct StepSrc {
    const uint8_t *aq, *as;
    const int *a_rowidx;
    size_t a_rowq, a_rows;
    const uint8_t *bq, *bsb;
    int b_r0, b_r1;
    size_t b_code_row;
    int b_nblk;
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void direct16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void direct4(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 4, 0, 0);
}

constexpr int kASlots = kBM * (kAStride / 16);     // 1664 = 26 x 64
constexpr int kBSlots = 128 * (kBStride / 16);     // 640  = 10 x 64
static_assert(kASlots % 64 == 0 && kBSlots % 64 == 0, "slot runs must fill waves");

__device__ __forceinline__ void issue_step(Stage &S, const StepSrc &src, int kk, int wid,
                                           int lane) {
    uint8_t *abase = &S.a[0][0];
    for (int i = 0; 64 * (4 * i + wid) < kASlots; ++i) {
        const int s0 = 64 * (4 * i + wid), sl = s0 + lane;
        const int r = sl / (kAStride / 16), pc = min(sl - r * (kAStride / 16), kStepQ / 16 - 1);
        direct16(src.aq + (size_t)src.a_rowidx[r] * src.a_rowq + (size_t)kk * kStepQ + pc * 16,
                 abase + 16 * s0);
    }
    {   // A scales: 256 four-byte slots (2 per row), one instruction per wave
        const int sl = 64 * wid + lane, r = sl >> 1;
        direct4(src.as + (size_t)src.a_rowidx[r] * src.a_rows + (size_t)kk * kStepS + (sl & 1) * 4,
                &S.as[0][0] + 4 * 64 * wid);
    }
    uint8_t *bbase = &S.b[0][0];
    for (int i = 0; 64 * (4 * i + wid) < kBSlots; ++i) {
        const int s0 = 64 * (4 * i + wid), sl = s0 + lane;
        const int n = sl / (kBStride / 16), pc = min(sl - n * (kBStride / 16), 3);
        const int row = n < 64 ? src.b_r0 + n : src.b_r1 + (n - 64);
        direct16(src.bq + (size_t)row * src.b_code_row + (size_t)kk * 64 + pc * 16, bbase + 16 * s0);
    }
    if (wid < 2) {   // B scales: 128 four-byte slots
        const int n = 64 * wid + lane;
        const int row = n < 64 ? src.b_r0 + n : src.b_r1 + (n - 64);
        direct4(src.bsb + (size_t)row * src.b_nblk + (size_t)kk * 4, &S.bs[0][0] + 4 * 64 * wid);
    }
}

// Common GEMM core: computes the 128 x 128 tile into acc (per wave 64 x 64).
template <bool kGateUp>
__device__ __forceinline__ void gemm_tile(Stage *stages, const StepSrc &src, int nsteps, int wm,
                                          int wn, f32x4_t (&acc)[4][4]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    issue_step(stages[0], src, 0, wid, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): this wave's loads landed
    __syncthreads();                                   // ... and every other wave's
    for (int kk = 0; kk < nsteps; ++kk) {
        const int cur = kk & 1;
        if (kk + 1 < nsteps) issue_step(stages[cur ^ 1], src, kk + 1, wid, lane);
        mfma_step<kGateUp>(stages[cur], wm, wn, lane, acc);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// gate/up: tile = 128 rows x (64 gate + 64 up) columns of one expert.
// Epilogue: h = silu(gate) * up in fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_up_mfma_kernel(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xs, ExpertArgs W,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ sorted_rows,
    const int32_t *__restrict__ plan, const int32_t *__restrict__ tiles, float *__restrict__ h,
    int T, int d, int E, int k, int f, int mt_max) {
    extern __shared__ __align__(16) uint8_t smem[];
    Stage *stages = reinterpret_cast<Stage *>(smem);
    __shared__ int a_rowidx[kBM];
    const int nt_blk = blockIdx.x / mt_max;           // 64-column block of f
    const int mt = blockIdx.x - nt_blk * mt_max;      // global m-tile
    const int total = tiles[0];
    if (mt >= total) return;
    const int nact = plan[0];
    const int a = find_expert(tiles, nact, mt);
    const int e = plan[1 + a];
    if ((unsigned)e >= (unsigned)E) return;
    const int nrows = T * k;
    const int row0 = offsets[e], ne = offsets[e + 1] - row0;
    if (row0 < 0 || ne <= 0 || row0 + ne > nrows) return;
    const int m0 = (mt - tiles[1 + a]) * kBM;          // first row of the tile in the expert
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    if (tid < kBM) {
        const int r = min(m0 + tid, ne - 1);
        const int row = sorted_rows[row0 + r];
        a_rowidx[tid] = (unsigned)row < (unsigned)nrows ? row / k : 0;
    }
    __syncthreads();
    const int nsteps = d >> 7, nblk = d >> 5;
    const size_t code_row = (size_t)d >> 1;
    const uint8_t *bq = W.gu_codes + (size_t)e * 2 * f * code_row;
    const uint8_t *bsb = W.gu_scales + (size_t)e * 2 * f * nblk;
    const int n0 = nt_blk * 64;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const StepSrc src{xq, xs, a_rowidx, (size_t)nsteps * kStepQ, (size_t)nsteps * kStepS,
                      bq, bsb, n0, f + n0, code_row, nblk};
    gemm_tile<true>(stages, src, nsteps, wm, wn, acc);
    // epilogue: lane holds rows 4 (l/16) + i, column l % 16 of each tile
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int mtl = 0; mtl < 4; ++mtl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = m0 + wm * 64 + mtl * 16 + 4 * g + i;
            if (r < ne) {
                float *hrow = h + (size_t)(row0 + r) * f + n0 + wn * 32;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float gv = acc[mtl][j][i], uv = acc[mtl][2 + j][i];
                    hrow[j * 16 + c16] = gv / (1.0f + expf(-gv)) * uv;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// down: tile = 128 rows x 128 output columns of one expert -> bf16 rows_out.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void down_mfma_kernel(
    const uint8_t *__restrict__ hq, const uint8_t *__restrict__ hs, ExpertArgs W,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ plan,
    const int32_t *__restrict__ tiles, uint16_t *__restrict__ rows_out, int T, int d, int E,
    int k, int f, int mt_max) {
    extern __shared__ __align__(16) uint8_t smem[];
    Stage *stages = reinterpret_cast<Stage *>(smem);
    __shared__ int a_rowidx[kBM];
    const int nt_blk = blockIdx.x / mt_max;           // 128-column block of d
    const int mt = blockIdx.x - nt_blk * mt_max;
    const int total = tiles[0];
    if (mt >= total) return;
    const int nact = plan[0];
    const int a = find_expert(tiles, nact, mt);
    const int e = plan[1 + a];
    if ((unsigned)e >= (unsigned)E) return;
    const int nrows = T * k;
    const int row0 = offsets[e], ne = offsets[e + 1] - row0;
    if (row0 < 0 || ne <= 0 || row0 + ne > nrows) return;
    const int m0 = (mt - tiles[1 + a]) * kBM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    if (tid < kBM) a_rowidx[tid] = row0 + min(m0 + tid, ne - 1);   // h rows are expert-major
    __syncthreads();
    const int nsteps = f >> 7, nblk = f >> 5;
    const size_t code_row = (size_t)f >> 1;
    const uint8_t *bq = W.dn_codes + (size_t)e * d * code_row;
    const uint8_t *bsb = W.dn_scales + (size_t)e * d * nblk;
    const int n0 = nt_blk * 128;
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const StepSrc src{hq, hs, a_rowidx, (size_t)nsteps * kStepQ, (size_t)nsteps * kStepS,
                      bq, bsb, n0, n0 + 64, code_row, nblk};
    gemm_tile<false>(stages, src, nsteps, wm, wn, acc);
    const int g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int mtl = 0; mtl < 4; ++mtl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = m0 + wm * 64 + mtl * 16 + 4 * g + i;
            if (r < ne) {
                uint16_t *orow = rows_out + (size_t)(row0 + r) * d + n0 + wn * 64;
#pragma unroll
                for (int j = 0; j < 4; ++j) orow[j * 16 + c16] = f32_to_bf16_rne(acc[mtl][j][i]);
            }
        }
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

bool g_attr_done = false;

hipError_t set_lds_attrs() {
    if (g_attr_done) return hipSuccess;
    const int bytes = (int)(2 * sizeof(Stage));
    hipError_t e = hipFuncSetAttribute((const void *)gate_up_mfma_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)down_mfma_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) g_attr_done = true;
    return e;
}

}  // namespace

bool mfma_path_ok(int T, int d, int f) { return d % 128 == 0 && f % 128 == 0 && T >= kMfmaMinT; }

size_t mfma_ws_bytes(int T, int d, int E, int k, int f) {
    const size_t rows = (size_t)T * k;
    return al256((size_t)T * (d / 128) * kStepQ) + al256((size_t)T * (d / 128) * kStepS) +
           al256(rows * (f / 128) * kStepQ) + al256(rows * (f / 128) * kStepS) +
           al256((size_t)(E + 1) * 4);
}

hipError_t launch_mx_split_bf16(const uint16_t *in, int rows, int K, uint8_t *q, uint8_t *s,
                                hipStream_t st) {
    const long long items = (long long)rows * (K / 128);
    if (items <= 0) return hipSuccess;
    mx_split_e2m3_kernel<uint16_t><<<(unsigned)((items + 3) / 4), 256, 0, st>>>(in, rows, K, q, s);
    return hipGetLastError();
}

hipError_t launch_mx_split_f32(const float *in, int rows, int K, uint8_t *q, uint8_t *s,
                               hipStream_t st) {
    const long long items = (long long)rows * (K / 128);
    if (items <= 0) return hipSuccess;
    mx_split_e2m3_kernel<float><<<(unsigned)((items + 3) / 4), 256, 0, st>>>(in, rows, K, q, s);
    return hipGetLastError();
}

hipError_t launch_mfma_ffn(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                           const int32_t *sorted_rows, const int32_t *plan, float *h,
                           uint16_t *rows_out, void *ws, int T, int d, int E, int k, int f,
                           hipStream_t s) {
    hipError_t e = set_lds_attrs();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)T * k;
    char *p = static_cast<char *>(ws);
    uint8_t *xq = reinterpret_cast<uint8_t *>(p);
    p += al256((size_t)T * (d / 128) * kStepQ);
    uint8_t *xs = reinterpret_cast<uint8_t *>(p);
    p += al256((size_t)T * (d / 128) * kStepS);
    uint8_t *hq = reinterpret_cast<uint8_t *>(p);
    p += al256(rows * (f / 128) * kStepQ);
    uint8_t *hs = reinterpret_cast<uint8_t *>(p);
    p += al256(rows * (f / 128) * kStepS);
    int32_t *tiles = reinterpret_cast<int32_t *>(p);

    e = launch_mx_split_bf16(x, T, d, xq, xs, s);
    if (e != hipSuccess) return e;
    mfma_plan_kernel<<<1, 1024, 0, s>>>(offsets, plan, tiles, E);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int mt_max = min(E, (int)rows) + (int)((rows + kBM - 1) / kBM);
    const size_t lds = 2 * sizeof(Stage);
    gate_up_mfma_kernel<<<(unsigned)(mt_max * (f / 64)), 256, lds, s>>>(
        xq, xs, w, offsets, sorted_rows, plan, tiles, h, T, d, E, k, f, mt_max);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_mx_split_f32(h, (int)rows, f, hq, hs, s);
    if (e != hipSuccess) return e;
    down_mfma_kernel<<<(unsigned)(mt_max * (d / 128)), 256, lds, s>>>(
        hq, hs, w, offsets, plan, tiles, rows_out, T, d, E, k, f, mt_max);
    return hipGetLastError();
}

}  // namespace moe
