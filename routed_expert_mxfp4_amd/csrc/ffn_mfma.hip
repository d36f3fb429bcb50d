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
// Split layout: per row, per K step of 128 elements (4 MX blocks), 208 bytes
//   block g (0..3) at 48 g:  [hi codes 0..15][lo codes 0..15]
//                            [hi codes 16..23][lo codes 16..23]
//   192 + 2 g: E8M0 scale of hi, 193 + 2 g: of lo;  200..207: zero
// where "codes" is the block's 24-byte stream of 6-bit E2M3 fields packed
// little-endian (the MFMA operand format).  A lane's fp6 operand (6 dwords)
// is then one 16-byte read plus one 8-byte read per term.
//
// MFMA operand layout (16x16x128): lane l holds row (l % 16) of a 16-row
// tile and K block (l / 16) of the step; the output tile holds
// C[4 * (l / 16) + i][l % 16] in lane l, register i.
#include <algorithm>
#include <utility>

#include "moe_internal.hpp"
#include "mx_split.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStepBytes = 208;  // split bytes per row per K step
constexpr int kSlotsRow = 13;    // 16-byte pieces per row per K step

// The block's 48 code bytes [hi 0..15][lo 0..15][hi 16..23][lo 16..23] as
// three 16-byte words.
__device__ __forceinline__ void split_words(const SplitBlock &b, u32x4_t (&w)[3]) {
    w[0] = u32x4_t{b.hi[0], b.hi[1], b.hi[2], b.hi[3]};
    w[1] = u32x4_t{b.lo[0], b.lo[1], b.lo[2], b.lo[3]};
    w[2] = u32x4_t{b.hi[4], b.hi[5], b.lo[4], b.lo[5]};
}

template <typename In>
__device__ __forceinline__ void load_block32(const In *p, float (&v)[32]);
template <>
__device__ __forceinline__ void load_block32<uint16_t>(const uint16_t *p, float (&v)[32]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t *>(p + 8 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[8 * c + 2 * q] = __uint_as_float(w[q] << 16);
            v[8 * c + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    }
}
template <>
__device__ __forceinline__ void load_block32<float>(const float *p, float (&v)[32]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t *>(p + 4 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[4 * c + q] = w[q];
    }
}

// One lane per 32-element block: item = row * (K / 32) + block.  Block g of
// step st of row r lands at bytes 48 g of the row's step, its scales at
// 192 + 2 g; the lane of block 0 zeroes the step's pad bytes 200..207.
template <typename In>
__global__ __launch_bounds__(256) void mx_split_e2m3_kernel(const In *__restrict__ in,
                                                            uint32_t items, int K,
                                                            uint8_t *__restrict__ q) {
    const uint32_t item = blockIdx.x * 256u + threadIdx.x;
    if (item >= items) return;
    const uint32_t nblk = (uint32_t)K >> 5;
    const uint32_t r = item / nblk, b = item - r * nblk;
    float v[32];
    load_block32<In>(in + (size_t)r * K + 32 * b, v);
    const SplitBlock sb = split_block32(v);
    uint8_t *step = q + ((size_t)r * (nblk >> 2) + (b >> 2)) * kStepBytes;
    u32x4_t w[3];
    split_words(sb, w);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(step + 48 * (b & 3));
    dst[0] = w[0];
    dst[1] = w[1];
    dst[2] = w[2];
    *reinterpret_cast<uint16_t *>(step + 192 + 2 * (b & 3)) = (uint16_t)sb.scales;
    if ((b & 3) == 0) *reinterpret_cast<u32x2_t *>(step + 200) = u32x2_t{0u, 0u};
}

template <typename T>
__device__ __forceinline__ void store_block32(T *p, const f32x32_t &v);
template <>
__device__ __forceinline__ void store_block32<uint16_t>(uint16_t *p, const f32x32_t &v) {
    // one-term MX values carry at most 4 significant bits: exact in bf16
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u32x4_t w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = (__float_as_uint(v[8 * c + 2 * q]) >> 16) |
                   (__float_as_uint(v[8 * c + 2 * q + 1]) & 0xFFFF0000u);
        *reinterpret_cast<u32x4_t *>(p + 8 * c) = w;
    }
}
template <>
__device__ __forceinline__ void store_block32<float>(float *p, const f32x32_t &v) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
        *reinterpret_cast<f32x4_t *>(p + 4 * c) = f32x4_t{v[4 * c], v[4 * c + 1], v[4 * c + 2],
                                                          v[4 * c + 3]};
}

// The activation-MX rounding: each 32-element block of a flat array (rows x
// K with K % 32 == 0, so blocks never cross rows) replaced by its one-term
// MX E2M3 value, decoded exactly -- the hi term of split_block32.  One lane
// per block; out may be in.
template <typename T>
__global__ __launch_bounds__(256) void mx_round_kernel(const T *in, uint32_t items, T *out) {
    const uint32_t item = blockIdx.x * 256u + threadIdx.x;
    if (item >= items) return;
    float v[32];
    load_block32<T>(in + (size_t)item * 32, v);
    const float sc = e8m0_operand(mx_exponent(amax32(v)));
    store_block32<T>(out + (size_t)item * 32, e2m3_unpack32(e2m3_pack32(v, sc), sc));
}

// ---------------------------------------------------------------------------
// Tile plan: per active expert, the number of 128-row tiles and their
// exclusive prefix.  tiles[0] = total, tiles[1 + a] = prefix of expert a.
// Experts with at most gemv_max rows get no tiles: they are listed in
// small[] (small[0] = count, then their ids, ascending) for the GEMV path.
// ---------------------------------------------------------------------------
constexpr int kBM = 128;

__global__ __launch_bounds__(1024) void mfma_plan_kernel(const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ plan,
                                                         int32_t *__restrict__ tiles,
                                                         int32_t *__restrict__ small, int E,
                                                         int gemv_max) {
    __shared__ int wsum[16], ssum[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int nact = plan[0];
    int c = 0, sm = 0, e = -1;
    if (tid < nact) {
        e = plan[1 + tid];
        const int n = ((unsigned)e < (unsigned)E) ? offsets[e + 1] - offsets[e] : 0;
        if (n > gemv_max) c = (n + kBM - 1) / kBM;
        else if (n > 0) sm = 1;
    }
    int inc = c, sinc = sm;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(inc, o, 64), v = __shfl_up(sinc, o, 64);
        if (lane >= o) {
            inc += u;
            sinc += v;
        }
    }
    if (lane == 63) {
        wsum[wid] = inc;
        ssum[wid] = sinc;
    }
    __syncthreads();
    int base = 0, sbase = 0;
    for (int w = 0; w < wid; ++w) {
        base += wsum[w];
        sbase += ssum[w];
    }
    if (tid < nact) tiles[1 + tid] = base + inc - c;
    if (small && sm) small[1 + sbase + sinc - 1] = e;
    if (tid == 1023) {
        tiles[0] = base + inc;
        if (small) small[0] = sbase + sinc;
    }
}

// Which active expert a global m-tile index belongs to: binary search over
// the tile prefix of the plan's active experts.
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
// Grouped GEMM block: one tile of an expert's rows -- MT m-tiles of 16 rows,
// MT = 1, 2, 4 or 8, the smallest that holds them -- times 512 weight rows
// (gate/up: 256 gate rows and the matching 256 up rows; down: 512 output
// columns), K in steps of 128.  Eight waves, two per SIMD, so that while
// one wave waits for a barrier or for its loads to issue, the other keeps
// the matrix core busy.  A tile of 128 rows puts the waves on 2 x 4 parts
// of 64 rows x 128 weight rows (4 x 8 MFMA tiles, 128 accumulators); a
// shorter tile on 1 x 8 parts of all its rows x 64 weight rows.  Two MFMAs
// (hi, lo terms) per tile and step, one in the activation-MX mode.
//
// Data movement: every operand goes global -> LDS with buffer loads that
// write LDS directly (lane l's 16 bytes to m0 + 16 l; bytes past a
// buffer's end read as zero), shared by the eight waves:
//   A  (split activations) MT x 16 rows x 208 B per step;
//   B  (weight codes) 32 operand tiles of 1 KB per step: tile t's lane l
//      holds row 16 t' + l % 16, K block l / 16 of the step, the MFMA's B
//      operand layout, so a fragment read is 16 contiguous bytes per lane;
//   scales of 4 steps at once, 256 B per operand tile (row r's 16 bytes at
//      16 r).
// The weight codes (first touch often from HBM) are loaded two steps ahead
// into three LDS stages, the activations (mostly L2 hits) one step ahead
// into two, and the weight scales once per 4 steps into one buffer that each
// lane copies into registers at the group's first step.  At the top of step
// kk each wave waits until only its loads of step kk + 1's codes remain, a
// barrier publishes every wave's, then the next loads are issued into
// buffers every wave has finished reading, and step kk is multiplied.
// 16-row tiles take a deeper ring instead (four stages of each operand,
// every load three steps ahead; see issue_step_deep).
// ---------------------------------------------------------------------------
constexpr int kWaves = 8;
constexpr int kAStageBytes = kBM * kStepBytes;              // 26624: a 128-row tile's step
constexpr int kBStageBytes = 32 * 1024;                     // 32 operand tiles of 1 KB
constexpr int kSGroupBytes = 32 * 256;                      // scales of 4 steps, 32 tiles
constexpr int kBBase = 2 * kAStageBytes;                    // 2 A stages, 3 B stages, 1 group
constexpr int kSBase = kBBase + 3 * kBStageBytes;
constexpr int kLdsBytes = kSBase + kSGroupBytes;            // 159744 of 160 KB
constexpr int kBLoads = 4;                                  // code loads per wave and step

template <int MT>
struct Tile {
    static constexpr int kMtw = MT == 8 ? 4 : MT;           // m-tiles per wave
    static constexpr int kNtw = MT == 8 ? 8 : 4;            // operand tiles (16 cols) per wave
    static constexpr int kALoads = (MT * 16 * kSlotsRow + 63) / 64;   // 26, 13, 7, 4 wave loads
    static_assert(kALoads <= 4 * kWaves, "four A loads per wave at most");
    static_assert(kALoads * 1024 <= kAStageBytes, "A loads stay in the A stage");
};

typedef __amdgpu_buffer_rsrc_t brsrc_t;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Buffer load of 16 bytes per lane straight into LDS (lane l's bytes at
// lds_addr + 16 l); lds_addr is wave-uniform.  Inline asm: the compiler does
// not see these loads, and waits for them only where this file says
// (vmcnt(0) at the top of a step, or before the epilogue reuses the LDS).
// m0 holds nothing else in these kernels.
__device__ __forceinline__ void lds_load16(brsrc_t r, uint32_t voff, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(r), "s"(lds_addr)
        : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ brsrc_t rsrc_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left free.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int OFF>
__device__ __forceinline__ u32x4_t ds_read128(uint32_t a) {
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read64(uint32_t a) {
    u32x2_t v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t ds_read_u16(uint32_t a) {
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(v) : "v"(a), "i"(OFF));
    return v;
}

struct AFrag {
    i32x8_t hi, lo;
    uint32_t sc;   // byte 0: hi scale, byte 1: lo scale
};

// Issues the five LDS reads of m-tile MT's A fragment (a: this lane's row /
// block address in the stage, s: its scale address).
template <int MT>
__device__ __forceinline__ void read_afrag(AFrag &f, uint32_t a, uint32_t s) {
    constexpr int o = MT * 16 * kStepBytes;
    const u32x4_t h0 = ds_read128<o>(a);
    const u32x4_t l0 = ds_read128<o + 16>(a);
    const u32x2_t h1 = ds_read64<o + 32>(a);
    const u32x2_t l1 = ds_read64<o + 40>(a);
    f.sc = ds_read_u16<o>(s);
    const u32x4_t h1w = __builtin_shufflevector(h1, h1, 0, 1, -1, -1);
    const u32x4_t l1w = __builtin_shufflevector(l1, l1, 0, 1, -1, -1);
    f.hi = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(h0, h1w, 0, 1, 2, 3, 4, 5, -1, -1));
    f.lo = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(l0, l1w, 0, 1, 2, 3, 4, 5, -1, -1));
}

// Waits until at most N LDS reads are outstanding; the fragment's values
// are tied to the wait so that no use is scheduled before it.
template <int N>
__device__ __forceinline__ void afrag_ready(AFrag &f) {
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(f.hi), "+v"(f.lo), "+v"(f.sc) : "n"(N));
}

// N 16-byte reads at base + STRIDE i (i < N), the strides in the
// instructions' offset field: one address register for all of them (the B
// fragments of a wave's operand tiles, 16 bytes per lane each; the rows of
// a scale group).
template <int STRIDE, int... I>
__device__ __forceinline__ void ds_read128_strided(u32x4_t *r, uint32_t base,
                                                   std::integer_sequence<int, I...>) {
    ((r[I] = ds_read128<STRIDE * I>(base)), ...);
}
template <int STRIDE, int N>
__device__ __forceinline__ void ds_read128_rows(u32x4_t (&r)[N], uint32_t base) {
    static_assert(STRIDE * (N - 1) < 65536, "offsets fit the instruction");
    ds_read128_strided<STRIDE>(r, base, std::make_integer_sequence<int, N>());
}

template <int N>
struct BFrags {
    u32x4_t q[N];
    uint32_t sc[N];
};

// Waits until at most PEND LDS reads of the wave are outstanding (those
// issued after the B fragments'); each fragment register is then tied to
// that point (the empty asm statements stay after the wait), so no use is
// scheduled before it.
template <int N, int PEND>
__device__ __forceinline__ void bfrags_ready(BFrags<N> &b) {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(PEND) : "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(b.q[i]), "+v"(b.sc[i]));
}

// The block's tile: which expert, which 128 rows of it, which 512 weight
// rows.  Units (tile, n-block) are numbered expert by expert, and inside an
// expert n-block by n-block, its row tiles next to each other: the blocks
// that read the same weight slice run at the same time.  Blocks are spread
// over the 8 XCDs (consecutive block ids go to consecutive XCDs) so that
// each XCD walks a contiguous range of units: those blocks meet in its L2.
struct TileSel {
    int e, row0, ne, m0, nb;
};

__device__ __forceinline__ bool select_tile(const int32_t *tiles, const int32_t *plan,
                                            const int32_t *offsets, int E, int nrows, int NB,
                                            TileSel &ts) {
    const int total_u = tiles[0] * NB;
    const int per = (total_u + 7) >> 3;
    const int loc = (int)(blockIdx.x >> 3);
    if (loc >= per) return false;
    const int u = (int)(blockIdx.x & 7) * per + loc;
    if (u >= total_u) return false;
    // expert a owns units [tiles[1 + a] * NB, (its tile end) * NB)
    const int nact = plan[0];
    const int a = find_expert(tiles, nact, u / NB);
    const int t0 = tiles[1 + a];
    const int nt = (a + 1 < nact ? tiles[2 + a] : tiles[0]) - t0;
    if (nt <= 0) return false;
    const int v = u - t0 * NB;
    ts.nb = v / nt;
    ts.e = plan[1 + a];
    if ((unsigned)ts.e >= (unsigned)E || ts.nb >= NB) return false;
    ts.row0 = offsets[ts.e];
    ts.ne = offsets[ts.e + 1] - ts.row0;
    if (ts.row0 < 0 || ts.ne <= 0 || ts.row0 + ts.ne > nrows) return false;
    ts.m0 = (v - ts.nb * nt) * kBM;
    if (ts.m0 >= ts.ne) return false;
    return true;
}

// The per-block constants of a tile: where this lane's A pieces, B tiles
// and scale rows come from, and the buffer resources.
struct Plan8 {
    brsrc_t ra, rb, rs;              // split activations, weight codes, weight scales
    uint32_t a_src[4];               // this lane's A piece offsets (step 0)
    uint32_t b_src[4];               // this lane's offsets in its 4 B loads (step 0)
    uint32_t s_src;                  // this lane's scale row offset (group 0)
    uint32_t cstep, sgrp;            // bytes from one step's codes to the next, one group's scales
    int nsteps, n_a;                 // K steps; A loads of this wave
};

// First weight row of operand tile t (16 rows) of the block's 512.
// Gate/up: the tiles a wave multiplies are half gate, half up, the up tile
// j + n/2 matching gate tile j, so that the SwiGLU is local to the wave.
template <bool kGateUp, int MT>
__device__ __forceinline__ int tile_row(int t, int nb, int f) {
    if (!kGateUp) return nb * 512 + 16 * t;
    constexpr int kNtw = Tile<MT>::kNtw, kPer = kNtw / 2;
    const int owner = t / kNtw, j = t - owner * kNtw;
    const int col = nb * 256 + owner * 16 * kPer + 16 * (j < kPer ? j : j - kPer);
    return j < kPer ? col : f + col;
}

template <bool kGateUp, int MT>
__device__ __forceinline__ void plan8(Plan8 &P, const uint8_t *aq, uint32_t a_bytes,
                                      const ExpertArgs &W, int d, int f, int packed,
                                      const TileSel &ts, const int *a_rowidx, int wid,
                                      int lane) {
    const int K = kGateUp ? d : f;
    P.nsteps = K >> 7;
    const uint32_t code_row = (uint32_t)K >> 1, nblk = (uint32_t)K >> 5;
    const uint32_t wrows = kGateUp ? 2u * (uint32_t)f : (uint32_t)d;
    P.ra = rsrc_of(aq, a_bytes);
    P.rb = rsrc_of((kGateUp ? W.gu_codes : W.dn_codes) + (size_t)ts.e * wrows * code_row,
                   wrows * code_row);
    P.rs = rsrc_of((kGateUp ? W.gu_scales : W.dn_scales) + (size_t)ts.e * wrows * nblk,
                   wrows * nblk);
    const uint32_t a_row_bytes = (uint32_t)P.nsteps * kStepBytes;
    constexpr int kRows = MT * 16;
    P.n_a = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = wid + kWaves * j;                       // this wave's j-th A load
        if (i < Tile<MT>::kALoads) P.n_a = j + 1;
        const int p = 64 * min(i, Tile<MT>::kALoads - 1) + lane;
        const int r = p < kRows * kSlotsRow ? p / kSlotsRow : kRows - 1;
        const int pc = p < kRows * kSlotsRow ? p - r * kSlotsRow : kSlotsRow - 1;
        P.a_src[j] = (uint32_t)a_rowidx[r] * a_row_bytes + 16u * (uint32_t)pc;
    }
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = wid + kWaves * j;
        const uint32_t row = (uint32_t)tile_row<kGateUp, MT>(t, ts.nb, f);
        P.b_src[j] = packed ? (row >> 4) * (uint32_t)(K >> 7) * 1024u + 16u * (uint32_t)lane
                            : (row + (uint32_t)r16) * code_row + 16u * (uint32_t)g;
    }
    {
        const int t = 4 * wid + g;                            // this lane's scale row
        const uint32_t row = (uint32_t)tile_row<kGateUp, MT>(t, ts.nb, f);
        P.s_src = packed ? (row >> 4) * (uint32_t)(K >> 9) * 256u + 16u * (uint32_t)r16
                         : (row + (uint32_t)r16) * nblk;
    }
    P.cstep = packed ? 1024u : 64u;
    P.sgrp = packed ? 256u : 16u;
}

// Step kk's activation loads into A stage kk & 1, and at kk % 4 == 0 the
// scale group kk / 4.  P's offsets are those of step kk (scale group kk / 4)
// and move on to the next step (group) in place, so the address of a load
// takes no register beyond the one it lives in.  Wave-uniform branches only.
template <int MT>
__device__ __forceinline__ void issue_a8(Plan8 &P, uint32_t lds, int kk, int wid) {
    const uint32_t st = lds + (uint32_t)((kk & 1) * kAStageBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < P.n_a) {
            lds_load16(P.ra, P.a_src[j],
                       (uint32_t)__builtin_amdgcn_readfirstlane(
                           (int)(st + 1024u * (uint32_t)(wid + kWaves * j))));
            P.a_src[j] += kStepBytes;
        }
    }
    if ((kk & 3) == 0) {
        lds_load16(P.rs, P.s_src,
                   (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(lds + kSBase + 1024u * (uint32_t)wid)));
        P.s_src += P.sgrp;
    }
}

// The next step's weight-code loads (kBLoads per wave) into B stage sb; P's
// code offsets move on one step in place.
__device__ __forceinline__ void issue_b8(Plan8 &P, uint32_t lds, int sb, int wid) {
    const uint32_t st = lds + kBBase + (uint32_t)(sb * kBStageBytes);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
        lds_load16(P.rb, P.b_src[j],
                   (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(st + 1024u * (uint32_t)(wid + kWaves * j))));
        P.b_src[j] += P.cstep;
    }
}

// 16-row tiles (decode-sized experts): an A stage is 4 KB, so four A
// stages, four weight stages and the scale group fit in LDS with every load
// issued three K steps ahead.  Such a tile does little matrix work per step,
// so its weight stream is set by the bytes in flight; twice as many as the
// two-ahead ring keep it going.
constexpr int kDeepAStage = 4096;
constexpr int kDeepBBase = 4 * kDeepAStage;
constexpr int kDeepSBase = kDeepBBase + 4 * kBStageBytes;
static_assert(kDeepSBase + kSGroupBytes <= kLdsBytes, "the deep ring fits the block's LDS");

// All of step kk's loads into stage kk % 4: activations (and, at kk % 4 ==
// 0, the scale group), then the weight codes.
__device__ __forceinline__ void issue_step_deep(const Plan8 &P, uint32_t lds, int kk, int wid) {
    const uint32_t st = (uint32_t)(kk & 3);
    const uint32_t a_st = lds + st * kDeepAStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < P.n_a)
            lds_load16(P.ra, P.a_src[j] + (uint32_t)kk * kStepBytes,
                       (uint32_t)__builtin_amdgcn_readfirstlane(
                           (int)(a_st + 1024u * (uint32_t)(wid + kWaves * j))));
    }
    if ((kk & 3) == 0)
        lds_load16(P.rs, P.s_src + (uint32_t)(kk >> 2) * P.sgrp,
                   (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(lds + kDeepSBase + 1024u * (uint32_t)wid)));
    const uint32_t b_st = lds + kDeepBBase + st * kBStageBytes;
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
        lds_load16(P.rb, P.b_src[j] + (uint32_t)kk * P.cstep,
                   (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(b_st + 1024u * (uint32_t)(wid + kWaves * j))));
}

// 16-row tiles on the canonical store, super-steps of two K steps: a weight
// row's 128 bytes of two steps are one cache line, so each load takes 8 rows
// x 128 bytes (whole lines) instead of 16 rows x 64 bytes (half lines, the
// pattern the operand layout would need).  Lane l of load i (rows 8 i ..
// 8 i + 7 of the block's 512) reads row 8 i + l % 8, bytes 16 (l / 8) of the
// line, and lands at 16 l: piece p of row r sits at 1024 i + 128 p + 16 r,
// so the fragment of step h (0, 1) and K group g of row r is piece 4 h + g.
// Two super-stages of 64 KB (one loading while the other is multiplied),
// four one-step A stages and the scale group.
constexpr int kSupAStage = 4096;
constexpr int kSupBBase = 4 * kSupAStage;
constexpr int kSupBStage = 64 * 1024;
constexpr int kSupSBase = kSupBBase + 2 * kSupBStage;
static_assert(kSupSBase + kSGroupBytes <= kLdsBytes, "the super-step ring fits the block's LDS");

// Super-step S's loads: the activations of steps 2S and 2S + 1 (and, at
// 2S % 4 == 0, the scale group), then the weight lines of both steps into
// super-stage S % 2.
template <bool kGateUp>
__device__ __forceinline__ void issue_super(const Plan8 &P, uint32_t lds, int S, int wid,
                                            const uint32_t (&line_src)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kk = 2 * S + h;
        const uint32_t a_st = lds + (uint32_t)(kk & 3) * kSupAStage;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < P.n_a)
                lds_load16(P.ra, P.a_src[j] + (uint32_t)kk * kStepBytes,
                           (uint32_t)__builtin_amdgcn_readfirstlane(
                               (int)(a_st + 1024u * (uint32_t)(wid + kWaves * j))));
        }
        if ((kk & 3) == 0)
            lds_load16(P.rs, P.s_src + (uint32_t)(kk >> 2) * P.sgrp,
                       (uint32_t)__builtin_amdgcn_readfirstlane(
                           (int)(lds + kSupSBase + 1024u * (uint32_t)wid)));
    }
    const uint32_t b_st = lds + kSupBBase + (uint32_t)(S & 1) * kSupBStage;
#pragma unroll
    for (int j = 0; j < 8; ++j)        // loads 2 t and 2 t + 1 of operand tiles t = wid + 8 (j / 2)
        lds_load16(P.rb, line_src[j] + 128u * (uint32_t)S,
                   (uint32_t)__builtin_amdgcn_readfirstlane(
                       (int)(b_st + 1024u * (uint32_t)(2 * (wid + kWaves * (j >> 1)) + (j & 1)))));
}

// Waits until at most n of the wave's loads are outstanding; n is one of
// the values the deep ring produces (0, or one or two later steps' loads).
__device__ __forceinline__ void deep_wait(int n) {
    switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
}

// The lane's E8M0 codes of one scale group for its operand tiles: byte s of
// sc[nt] is the code of K block 4 s + g of row r16 (step s of the group),
// picked from the row's 16 bytes.
// All N reads are issued before one wait (each row's bytes are then tied to
// that wait, as in bfrags_ready).
template <int N>
__device__ __forceinline__ void read_group_scales(uint32_t (&sc)[N], uint32_t addr,
                                                  uint32_t psel01) {
    u32x4_t r[N];
    ds_read128_rows<256>(r, addr);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < N; ++nt) {
        asm volatile("" : "+v"(r[nt]));
        const uint32_t t01 = __builtin_amdgcn_perm(r[nt].y, r[nt].x, psel01);
        const uint32_t t23 = __builtin_amdgcn_perm(r[nt].w, r[nt].z, psel01);
        sc[nt] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
}

// The A fragments of m-tiles I..kMtw-1, two in flight: m-tile I's is waited
// for, its MFMAs issued against every B fragment, m-tile I + 2's queued, then
// hook(I) (the ring's next global loads, issued between MFMA groups).
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};
template <int I, int MTW, int NTW, bool kSingle, typename H = NoHook>
__device__ __forceinline__ void chain8(f32x4_t (&acc)[MTW][NTW], AFrag (&fa)[2],
                                       const BFrags<NTW> &fb, uint32_t a, uint32_t s,
                                       const H &hook = H()) {
    if constexpr (I < MTW) {
        afrag_ready<(I + 1 < MTW) ? 5 : 0>(fa[I & 1]);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
            const u32x4_t q = fb.q[nt];
            const i32x8_t b = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
            acc[I][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[I & 1].hi, b, acc[I][nt], 2, 4, 0, (int)fa[I & 1].sc, 0, (int)fb.sc[nt]);
            if constexpr (!kSingle)
                acc[I][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fa[I & 1].lo, b, acc[I][nt], 2, 4, 1, (int)fa[I & 1].sc, 0, (int)fb.sc[nt]);
        }
        if constexpr (I + 2 < MTW) read_afrag<I + 2>(fa[I & 1], a, s);
        hook(I);
        chain8<I + 1, MTW, NTW, kSingle>(acc, fa, fb, a, s, hook);
    }
}

// kGateUp: A = split x (token rows), out = hq, the split of h = silu(gate) *
//          up [rows][f] (expert-major rows), the down pass's A;
// else:    A = hq, out = rows_out bf16 [rows][d].
// packed: the weights are in the operand-order layout of prepack_kernel
// (K % 512 == 0): each 1 KB operand tile of a step is contiguous there (16
// rows x 64 B gathered otherwise), each scale group 256 B.
template <bool kGateUp, bool kSingle, int MT>
__device__ __forceinline__ void gemm_tile(const uint8_t *__restrict__ aq, uint32_t a_bytes,
                                          const ExpertArgs &W, uint8_t *__restrict__ hq,
                                          uint16_t *__restrict__ rows_out, int d, int f,
                                          int packed, const TileSel &ts, const int *a_rowidx,
                                          uint8_t *lds) {
    constexpr int kMtw = Tile<MT>::kMtw, kNtw = Tile<MT>::kNtw;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    // this wave's part: m-tiles mbase.., operand tiles nbase..
    const int mbase = MT == 8 ? 4 * (wid & 1) : 0;
    const int nbase = MT == 8 ? 8 * (wid >> 1) : 4 * wid;
    Plan8 P;
    plan8<kGateUp, MT>(P, aq, a_bytes, W, d, f, packed, ts, a_rowidx, wid, lane);
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
    const uint32_t a_lane = (uint32_t)((16 * mbase + r16) * kStepBytes + 48 * g);
    const uint32_t s_lane = (uint32_t)((16 * mbase + r16) * kStepBytes + 192 + 2 * g);

    f32x4_t acc[kMtw][kNtw];
#pragma unroll
    for (int i = 0; i < kMtw; ++i)
#pragma unroll
        for (int j = 0; j < kNtw; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t psel01 = (uint32_t)g | ((4u + (uint32_t)g) << 8);
    uint32_t spk[kNtw];
    // one K step's products from A stage st and B stage sbq
    auto multiply = [&](uint32_t st, uint32_t sbq, int kk, const auto &hook) {
        BFrags<kNtw> fb;
#pragma unroll
        for (int nt = 0; nt < kNtw; ++nt) fb.sc[nt] = spk[nt] >> (8 * (kk & 3));
        ds_read128_rows<1024>(fb.q, sbq + 1024u * (uint32_t)nbase + 16u * (uint32_t)lane);
        AFrag fa[2];
        const uint32_t a = st + a_lane, s = st + s_lane;
        read_afrag<0>(fa[0], a, s);
        if constexpr (kMtw > 1) read_afrag<1>(fa[1], a, s);
        // the B fragments and m-tile 0's A fragment; m-tile 1's may still fly
        bfrags_ready<kNtw, (kMtw > 1 ? 5 : 0)>(fb);
        chain8<0, kMtw, kNtw, kSingle>(acc, fa, fb, a, s, hook);
    };
    if constexpr (MT == 1) {
        if (!packed && (P.nsteps & 1) == 0) {
            // super-steps of two K steps, one ahead (see issue_super)
            uint32_t line_src[8];
            {
                const uint32_t code_row = (uint32_t)(kGateUp ? d : f) >> 1;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = wid + kWaves * (j >> 1);
                    const uint32_t row = (uint32_t)tile_row<kGateUp, MT>(t, ts.nb, f) + 8u * (uint32_t)(j & 1) +
                                         (uint32_t)(lane & 7);
                    line_src[j] = row * code_row + 16u * (uint32_t)(lane >> 3);
                }
            }
            // this lane's fragment offset in a super-stage, step h = 0 (h = 1: + 512)
            const uint32_t frag_lane = 1024u * (uint32_t)(r16 >> 3) + 128u * (uint32_t)g + 16u * (uint32_t)(r16 & 7);
            const uint32_t sgrp_lane = lds_addr + kSupSBase + 256u * (uint32_t)nbase + 16u * (uint32_t)r16;
            const int NS = P.nsteps >> 1;
            issue_super<kGateUp>(P, lds_addr, 0, wid, line_src);
            for (int S = 0; S < NS; ++S) {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));       // super-step S's loads, the only ones out
                __builtin_amdgcn_s_barrier();                   // everyone's; super-step S - 1's stages free
                __builtin_amdgcn_sched_barrier(0);
                if ((S & 1) == 0) read_group_scales<kNtw>(spk, sgrp_lane, psel01);
                __builtin_amdgcn_sched_barrier(0);
                if (S + 1 < NS) issue_super<kGateUp>(P, lds_addr, S + 1, wid, line_src);
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t b_st = lds_addr + kSupBBase + (uint32_t)(S & 1) * kSupBStage;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kk = 2 * S + h;
                    BFrags<kNtw> fb;
#pragma unroll
                    for (int nt = 0; nt < kNtw; ++nt) fb.sc[nt] = spk[nt] >> (8 * (kk & 3));
                    ds_read128_rows<2048>(fb.q, b_st + 2048u * (uint32_t)nbase + frag_lane + 512u * (uint32_t)h);
                    AFrag fa[2];
                    const uint32_t st = lds_addr + (uint32_t)(kk & 3) * kSupAStage;
                    const uint32_t a = st + a_lane, sa = st + s_lane;
                    read_afrag<0>(fa[0], a, sa);
                    bfrags_ready<kNtw, 0>(fb);
                    chain8<0, kMtw, kNtw, kSingle>(acc, fa, fb, a, sa);
                }
            }
        } else {
            // the deep ring: steps 0..2 first, then step kk + 3 at step kk
            const uint32_t sgrp_lane = lds_addr + kDeepSBase + 256u * (uint32_t)nbase + 16u * (uint32_t)r16;
            for (int s0 = 0; s0 < 3 && s0 < P.nsteps; ++s0) issue_step_deep(P, lds_addr, s0, wid);
            for (int kk = 0; kk < P.nsteps; ++kk) {
                // step kk's loads, with those of the (at most two) later steps
                // issued so far still allowed in flight
                const int pend = min(2, P.nsteps - 1 - kk);
                const int scl = (pend >= 1 && ((kk + 1) & 3) == 0) + (pend >= 2 && ((kk + 2) & 3) == 0);
                deep_wait(pend * (P.n_a + kBLoads) + scl);
                __builtin_amdgcn_s_barrier();                   // everyone's; step kk-1's stages free
                __builtin_amdgcn_sched_barrier(0);
                if ((kk & 3) == 0) read_group_scales<kNtw>(spk, sgrp_lane, psel01);
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 3 < P.nsteps) issue_step_deep(P, lds_addr, kk + 3, wid);
                __builtin_amdgcn_sched_barrier(0);
                multiply(lds_addr + (uint32_t)((kk & 3) * kDeepAStage),
                         lds_addr + kDeepBBase + (uint32_t)((kk & 3) * kBStageBytes), kk, NoHook());
            }
        }
    } else {
        // prologue: step 0's activations and scale group, steps 0 and 1's codes
        issue_a8<MT>(P, lds_addr, 0, wid);
        issue_b8(P, lds_addr, 0, wid);
        if (P.nsteps > 1) issue_b8(P, lds_addr, 1, wid);
        const uint32_t sgrp_lane = lds_addr + kSBase + 256u * (uint32_t)nbase + 16u * (uint32_t)r16;
        int sb = 0;                                         // kk % 3
        for (int kk = 0; kk < P.nsteps; ++kk) {
            // step kk's operands: all but step kk + 1's codes, the last loads
            // issued (when there are any)
            if (kk + 1 < P.nsteps)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(kBLoads));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __builtin_amdgcn_s_barrier();                   // everyone's; step kk-1's buffers free
            __builtin_amdgcn_sched_barrier(0);
            if ((kk & 3) == 0) read_group_scales<kNtw>(spk, sgrp_lane, psel01);
            __builtin_amdgcn_sched_barrier(0);
            // the next loads go out between the MFMA groups (step kk + 1's
            // activations after m-tile 0, step kk + 2's codes after the last
            // m-tile), not all at once after the barrier: the eight waves'
            // loads then queue at the texture unit while the matrix cores
            // work
            static_assert(Tile<MT>::kMtw >= 2, "both hooks run");
            const int sbn = sb == 0 ? 2 : sb - 1;
            auto hook = [&](int i) {
                __builtin_amdgcn_sched_barrier(0);
                if (i == 0 && kk + 1 < P.nsteps) issue_a8<MT>(P, lds_addr, kk + 1, wid);
                if (i == Tile<MT>::kMtw - 1 && kk + 2 < P.nsteps) issue_b8(P, lds_addr, sbn, wid);
                __builtin_amdgcn_sched_barrier(0);
            };
            multiply(lds_addr + (uint32_t)((kk & 1) * kAStageBytes),
                     lds_addr + kBBase + (uint32_t)(sb * kBStageBytes), kk, hook);
            sb = sb == 2 ? 0 : sb + 1;
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();                                        // the stages are free for the epilogue

    // epilogue: lane holds rows 4 (l / 16) + i, column l % 16 of each tile
    if (kGateUp) {
        // h = silu(gate) * up, kNtw / 2 * 16 columns of the wave's rows, goes
        // through LDS two m-tiles (32 rows) at a time, then is split one
        // 32-element MX block per lane
        constexpr int kPer = kNtw / 2;                       // gate tiles of the wave
        constexpr int kCols = 16 * kPer;                     // 64 or 32 h columns
        constexpr int kHs = kCols + 4;                       // floats per staged row
        constexpr int kPassMt = kMtw < 2 ? kMtw : 2;
        float *hs = reinterpret_cast<float *>(lds) + wid * 32 * kHs;
        const int hc0 = ts.nb * 256 + (MT == 8 ? (wid >> 1) : wid) * kCols;
        const uint32_t hq_row = (uint32_t)(f >> 7) * kStepBytes;
        uint8_t *hq_step = hq + (size_t)(hc0 >> 7) * kStepBytes;
        const int gb0 = (hc0 & 127) >> 5;
#pragma unroll
        for (int pass = 0; pass < kMtw / kPassMt; ++pass) {
            const int r_first = ts.m0 + 16 * (mbase + kPassMt * pass);
            const int left = ts.ne - r_first;               // rows from this pass on
#pragma unroll
            for (int m = 0; m < kPassMt; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int nt = 0; nt < kPer; ++nt) {
                        const float gv = acc[kPassMt * pass + m][nt][i];
                        const float uv = acc[kPassMt * pass + m][nt + kPer][i];
                        hs[(16 * m + 4 * g + i) * kHs + 16 * nt + r16] = gv / (1.0f + expf(-gv)) * uv;
                    }
            __syncthreads();
            if (left > 0) {
                // buffer stores drop offsets past the pass's live rows
                const uint32_t live = (uint32_t)min(left, 16 * kPassMt) * hq_row;
                const brsrc_t out = rsrc_of(hq_step + (size_t)(ts.row0 + r_first) * hq_row, live);
                const int item = lane, rl = item / (kCols / 32), blk = item % (kCols / 32);
                if (rl < 16 * kPassMt) {
                    float v[32];
                    const float *src = hs + rl * kHs + 32 * blk;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const f32x4_t w = *reinterpret_cast<const f32x4_t *>(src + 4 * c);
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[4 * c + q] = w[q];
                    }
                    const SplitBlock sb = split_block32(v);
                    u32x4_t w[3];
                    split_words(sb, w);
                    const uint32_t o = (uint32_t)rl * hq_row, b = (uint32_t)(gb0 + blk);
#pragma unroll
                    for (int c = 0; c < 3; ++c)
                        __builtin_amdgcn_raw_buffer_store_b128(w[c], out, o + 48u * b + 16u * c, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sb.scales, out, o + 192u + 2u * b,
                                                          0, 0);
                }
            }
            __syncthreads();
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < kMtw; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ts.m0 + 16 * (mbase + mt) + 4 * g + i;
                if (r < ts.ne) {
                    uint16_t *orow = rows_out + (size_t)(ts.row0 + r) * d + ts.nb * 512 + 16 * nbase;
#pragma unroll
                    for (int nt = 0; nt < kNtw; ++nt)
                        orow[16 * nt + r16] = f32_to_bf16_rne(acc[mt][nt][i]);
                }
            }
    }
}

// One block per (m-tile, n-block) unit of the tile plan; the tile's height
// is chosen from its rows (block-uniform, so the branch below and every
// barrier inside gemm_tile are taken by the whole block).
template <bool kGateUp, bool kSingle>
__global__ __launch_bounds__(512, 1) void ffn_mfma_kernel(
    const uint8_t *__restrict__ aq, ExpertArgs W, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_rows, const int32_t *__restrict__ plan,
    const int32_t *__restrict__ tiles, uint8_t *__restrict__ hq, uint16_t *__restrict__ rows_out,
    int T, int d, int E, int k, int f, int packed) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int a_rowidx[kBM];
    const int nrows = T * k;
    const int NB = kGateUp ? f / 256 : d / 512;
    TileSel ts;
    if (!select_tile(tiles, plan, offsets, E, nrows, NB, ts)) return;
    const int tid = threadIdx.x;
    if (tid < kBM) {
        const int r = ts.row0 + min(ts.m0 + tid, ts.ne - 1);
        if (kGateUp) {
            const int row = sorted_rows[r];
            a_rowidx[tid] = (unsigned)row < (unsigned)nrows ? row / k : 0;
        } else {
            a_rowidx[tid] = r;                      // h rows are expert-major
        }
    }
    __syncthreads();
    // the A operand's buffer: T (gate/up) or T * k (down) split rows
    const uint32_t a_bytes = (uint32_t)((kGateUp ? (size_t)T : (size_t)nrows) *
                                        (size_t)((kGateUp ? d : f) >> 7) * kStepBytes);
    const int rows = __builtin_amdgcn_readfirstlane(min(kBM, ts.ne - ts.m0));
    if (rows <= 16)
        gemm_tile<kGateUp, kSingle, 1>(aq, a_bytes, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else if (rows <= 32)
        gemm_tile<kGateUp, kSingle, 2>(aq, a_bytes, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else if (rows <= 64)
        gemm_tile<kGateUp, kSingle, 4>(aq, a_bytes, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else
        gemm_tile<kGateUp, kSingle, 8>(aq, a_bytes, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
}

// The operand-order ("packed") layout of one MXFP4 matrix [rows][K] per
// expert, rows % 16 == 0, K % 512 == 0, the same bytes as the canonical one:
//   codes: 1 KB block per (16-row tile t, K step s of 128), at
//     (t * (K / 128) + s) * 1024; in it lane l = r + 16 g (r < 16, g < 4)
//     holds, at 16 l, the 16 code bytes of row 16 t + r, K elements
//     128 s + 32 g .. + 31 -- the B operand of one lane of the scaled MFMA;
//   scales: 256 B block per (tile t, group G of 4 K steps), at
//     (t * (K / 512) + G) * 256; row r's 16 scale bytes (blocks 16 G ..
//     16 G + 15) at 16 r.
// One thread per 16-byte piece; grid.y = 0 codes, 1 scales.
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      uint8_t *__restrict__ pcodes,
                                                      uint8_t *__restrict__ pscales, int E,
                                                      int rows, int K) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t tiles = (size_t)(rows >> 4);
    if (blockIdx.y == 0) {
        const size_t S = (size_t)(K >> 7);
        const size_t n = (size_t)E * tiles * S * 64;
        if (i >= n) return;
        const size_t l = i & 63, blk = i >> 6;          // blk = (e * tiles + t) * S + s
        const size_t s = blk % S, et = blk / S;
        const size_t e = et / tiles, t = et - e * tiles;
        const size_t row = t * 16 + (l & 15), g = l >> 4;
        const size_t src = (e * (size_t)rows + row) * (size_t)(K >> 1) + 64 * s + 16 * g;
        reinterpret_cast<uint4 *>(pcodes)[i] = *reinterpret_cast<const uint4 *>(codes + src);
    } else {
        const size_t G = (size_t)(K >> 9);
        const size_t n = (size_t)E * tiles * G * 16;
        if (i >= n) return;
        const size_t r = i & 15, blk = i >> 4;          // blk = (e * tiles + t) * G + q
        const size_t q = blk % G, et = blk / G;
        const size_t e = et / tiles, t = et - e * tiles;
        const size_t row = t * 16 + r;
        const size_t src = (e * (size_t)rows + row) * (size_t)(K >> 5) + 16 * q;
        reinterpret_cast<uint4 *>(pscales)[i] = *reinterpret_cast<const uint4 *>(scales + src);
    }
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

bool g_attr_done = false;

hipError_t set_lds_attrs() {
    if (g_attr_done) return hipSuccess;
    const void *k[4] = {(const void *)ffn_mfma_kernel<true, false>,
                        (const void *)ffn_mfma_kernel<true, true>,
                        (const void *)ffn_mfma_kernel<false, false>,
                        (const void *)ffn_mfma_kernel<false, true>};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 4 && e == hipSuccess; ++i)
        e = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e == hipSuccess) g_attr_done = true;
    return e;
}

}  // namespace

// The split rows are addressed with 32-bit byte offsets.
bool mfma_shape_ok(int T, int d, int k, int f) {
    return d % 512 == 0 && f % 256 == 0 &&
           (double)T * (d / 128) * kStepBytes < 4294967296.0 &&
           (double)T * k * (f / 128) * kStepBytes < 4294967296.0;
}

size_t mx_split_bytes(int rows, int K) { return (size_t)rows * (K / 128) * kStepBytes; }

size_t mfma_ws_bytes(int T, int d, int E, int k, int f) {
    const size_t rows = (size_t)T * k;
    return al256(mx_split_bytes(T, d)) + al256(mx_split_bytes((int)rows, f)) +
           al256((size_t)(E + 1) * 4);
}

size_t mixed_ws_bytes(int T, int d, int E, int k, int f, int gemv_max) {
    // the scaled-MFMA scratch, the small experts' list and their fp32 h rows
    const size_t rows = (size_t)T * k;
    const size_t small_rows = gemv_max > 0 ? std::min(rows, (size_t)E * gemv_max) : 0;
    return al256(mfma_ws_bytes(T, d, E, k, f)) + al256((size_t)(E + 1) * 4) +
           al256(small_rows * f * 4);
}

hipError_t launch_mx_split_bf16(const uint16_t *in, int rows, int K, uint8_t *q, hipStream_t st) {
    const uint32_t items = (uint32_t)rows * (uint32_t)(K / 32);
    if (items == 0) return hipSuccess;
    (void)timed_launch("mx_split_x", mx_split_e2m3_kernel<uint16_t>, dim3((items + 255) / 256), dim3(256), 0, st, in, items, K, q);
    return hipGetLastError();
}

hipError_t launch_mx_split_f32(const float *in, int rows, int K, uint8_t *q, hipStream_t st) {
    const uint32_t items = (uint32_t)rows * (uint32_t)(K / 32);
    if (items == 0) return hipSuccess;
    mx_split_e2m3_kernel<float><<<(items + 255) / 256, 256, 0, st>>>(in, items, K, q);
    return hipGetLastError();
}

hipError_t launch_mx_round_bf16(const uint16_t *in, int rows, int K, uint16_t *out,
                                hipStream_t st) {
    const uint32_t items = (uint32_t)rows * (uint32_t)(K / 32);
    if (items == 0) return hipSuccess;
    return timed_launch("mx_round", mx_round_kernel<uint16_t>, dim3((items + 255) / 256),
                        dim3(256), 0, st, in, items, out);
}

hipError_t launch_mx_round_f32(const float *in, int rows, int K, float *out, hipStream_t st) {
    const uint32_t items = (uint32_t)rows * (uint32_t)(K / 32);
    if (items == 0) return hipSuccess;
    return timed_launch("mx_round", mx_round_kernel<float>, dim3((items + 255) / 256), dim3(256),
                        0, st, in, items, out);
}

hipError_t launch_mfma_ffn(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                           const int32_t *sorted_rows, const int32_t *plan, uint16_t *rows_out,
                           void *ws, int T, int d, int E, int k, int f, bool single,
                           hipStream_t s, bool packed, int gemv_max) {
    hipError_t e = set_lds_attrs();
    if (e != hipSuccess) return e;
    const size_t rows = (size_t)T * k;
    char *p = static_cast<char *>(ws);
    uint8_t *xq = reinterpret_cast<uint8_t *>(p);
    p += al256(mx_split_bytes(T, d));
    uint8_t *hq = reinterpret_cast<uint8_t *>(p);
    p += al256(mx_split_bytes((int)rows, f));
    int32_t *tiles = reinterpret_cast<int32_t *>(p);
    p += al256((size_t)(E + 1) * 4);
    // the mixed path's part of the scratch (mixed_ws_bytes)
    int32_t *small = reinterpret_cast<int32_t *>(p);
    p += al256((size_t)(E + 1) * 4);
    float *h_small = reinterpret_cast<float *>(p);
    const bool mixed = gemv_max > 0;

    {
        e = launch_mx_split_bf16(x, T, d, xq, s);
    }
    if (e != hipSuccess) return e;
    mfma_plan_kernel<<<1, 1024, 0, s>>>(offsets, plan, tiles, mixed ? small : nullptr, E,
                                        mixed ? gemv_max : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // experts with few rows: the grouped GEMVs (weights streamed once per
    // row), their h rows at small-expert index * gemv_max
    if (mixed) {
        e = launch_gemv_gate_up_small(x, w, offsets, sorted_rows, small, h_small, T, d, E, k, f,
                                      gemv_max, s);
        if (e != hipSuccess) return e;
    }
    // upper bound on the m-tiles: one partial tile per expert plus full tiles
    const long long mt_max = min(E, (int)rows) + (long long)((rows + kBM - 1) / kBM);
    {
        const long long blocks = 8 * ((mt_max * (f / 256) + 7) / 8);
        (void)timed_launch("gate_up_mfma",
                           single ? ffn_mfma_kernel<true, true> : ffn_mfma_kernel<true, false>,
                           dim3((unsigned)blocks), dim3(512), kLdsBytes, s, xq, w, offsets,
                           sorted_rows, plan, tiles, hq, nullptr, T, d, E, k, f, (int)packed);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mixed) {
        e = launch_gemv_down_small(h_small, w, offsets, small, rows_out, T, d, E, k, f,
                                   gemv_max, s);
        if (e != hipSuccess) return e;
    }
    {
        const long long blocks = 8 * ((mt_max * (d / 512) + 7) / 8);
        (void)timed_launch("down_mfma",
                           single ? ffn_mfma_kernel<false, true> : ffn_mfma_kernel<false, false>,
                           dim3((unsigned)blocks), dim3(512), kLdsBytes, s, hq, w, offsets,
                           sorted_rows, plan, tiles, nullptr, rows_out, T, d, E, k, f, (int)packed);
    }
    return hipGetLastError();
}

bool prepack_ok(int d, int f) { return d % 512 == 0 && f % 512 == 0; }

hipError_t launch_prepack(ExpertArgs src, ExpertArgs dst, int E, int d, int f, hipStream_t s) {
    // gate/up: rows 2f, K = d; down: rows d, K = f
    const int mats[2][2] = {{2 * f, d}, {d, f}};
    for (int m = 0; m < 2; ++m) {
        const int rows = mats[m][0], K = mats[m][1];
        const size_t n_codes = (size_t)E * rows * (K / 32);     // 16-byte pieces
        const size_t blocks = (n_codes + 255) / 256;             // >= the scale pieces' blocks
        if (blocks == 0) continue;
        prepack_kernel<<<dim3((unsigned)blocks, 2), 256, 0, s>>>(
            m == 0 ? src.gu_codes : src.dn_codes, m == 0 ? src.gu_scales : src.dn_scales,
            const_cast<uint8_t *>(m == 0 ? dst.gu_codes : dst.dn_codes),
            const_cast<uint8_t *>(m == 0 ? dst.gu_scales : dst.dn_scales), E, rows, K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe
