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

#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kStepBytes = 208;  // split bytes per row per K step
constexpr int kSlotsRow = 13;    // 16-byte pieces per row per K step

// ---------------------------------------------------------------------------
// MX E2M3 conversion (OCP MX v1.0): shared exponent X = floor(log2(amax)) - 2
// clamped to [-127, 127] (E8M0 code X + 127; an all-zero block gets code 0);
// elements v / 2^X rounded to nearest even onto the E2M3 grid (subnormals
// 0, 1/8, .., 7/8; then 1..1.875, 2..3.75, 4..7.5), saturating at 7.5, the
// sign kept (also on zero).  gfx950 converts and packs 32 such elements in
// one instruction, and decodes them back exactly.
// ---------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef unsigned u32x6_t __attribute__((ext_vector_type(6)));

__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.f)) return -127;
    int e;
    (void)frexpf(amax, &e);                       // amax = m 2^e, m in [0.5, 1)
    return min(max(e - 1 - 2, -127), 127);
}

// The scale 2^X as the conversions' fp32 operand: they read only its
// exponent field, which holds the E8M0 code (X = -127 gives +0.0f).
__device__ __forceinline__ float e8m0_operand(int X) {
    return __uint_as_float((uint32_t)(X + 127) << 23);
}

// Codes of 32 values, 6 bits each, element i at bits 6i of the 192 bits.
// The conversion puts its first operand's 16 values in the even slots and
// the second's in the odd ones.  It writes its first result registers
// before it has read all of its sources, so its destination must not
// overlap them: the empty asm keeps the sources live past the instruction
// (and, taking the result, cannot be hoisted above it), which keeps the
// register allocator from overlapping them.
__device__ __forceinline__ u32x6_t e2m3_pack32(const float (&v)[32], float scale) {
    f32x16_t ev, od;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        ev[m] = v[2 * m];
        od[m] = v[2 * m + 1];
    }
    u32x6_t c = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, scale);
    asm volatile("" : "+v"(c) : "v"(ev), "v"(od), "v"(scale));
    return c;
}

// The exact values of 32 packed codes under scale 2^X (same constraint).
__device__ __forceinline__ f32x32_t e2m3_unpack32(u32x6_t c, float scale) {
    f32x32_t v = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(c, scale);
    asm volatile("" : "+v"(v) : "v"(c), "v"(scale));
    return v;
}

__device__ __forceinline__ float amax32(const float (&v)[32]) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
    return a;
}

// Two-term split of one 32-element block held by one lane: hi = the block
// quantised, lo = the residual (exact in fp32) quantised with its own scale.
struct SplitBlock {
    u32x6_t hi, lo;
    uint32_t scales;                              // hi E8M0 | lo E8M0 << 8
};

__device__ __forceinline__ SplitBlock split_block32(const float (&v)[32]) {
    SplitBlock b;
    // a NaN element has no E2M3 code: the block's scales become the E8M0
    // NaN code 255, which the scaled MFMA carries into every product
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) nan |= v[i] != v[i];
    const int xh = mx_exponent(amax32(v));
    b.hi = e2m3_pack32(v, e8m0_operand(xh));
    const f32x32_t hd = e2m3_unpack32(b.hi, e8m0_operand(xh));
    float r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = v[i] - hd[i];
    const int xl = mx_exponent(amax32(r));
    b.lo = e2m3_pack32(r, e8m0_operand(xl));
    b.scales = nan ? 0xFFFFu : (uint32_t)(xh + 127) | ((uint32_t)(xl + 127) << 8);
    return b;
}

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
// Grouped GEMM block: 128 rows of one expert x 512 weight rows (gate/up:
// 256 gate + the matching 256 up rows; down: 512 output columns), K in steps
// of 128.  Four waves, one per SIMD, each owning all 128 rows x 128 weight
// rows: 8 x 8 MFMA tiles, 256 fp32 accumulators, two MFMAs (hi, lo) per
// tile and step.
//
// Data movement per step:
//   A (split activations, shared by the four waves): global -> LDS direct
//     loads into a ring of kNst stages, issued kNst - 1 steps ahead; each
//     wave waits for its own loads (vmcnt) and a barrier publishes them.
//     Fragment reads are explicit ds_read instructions so that the next
//     stages' loads stay in flight while a stage is read.
//   B (weights, private to a wave): global -> registers (see BRing).
// Every step issues the same number of loads (steps past the end re-load
// the last step), so the wait counts are constants.
// ---------------------------------------------------------------------------
constexpr int kNst = 4;                              // LDS stages
// Tile heights: MT m-tiles of 16 rows (MT = 1, 2, 4 or 8).  The A stage of
// MT * 16 rows x 13 pieces takes DMA(MT) direct loads per wave (4 waves).
template <int MT>
struct Tile {
    static constexpr int kDma = (MT * 16 * kSlotsRow + 255) / 256;   // 1, 2, 4, 7
    static constexpr int kStageBytes = 4 * kDma * 1024;              // pad loads overflow here
    static_assert(MT * 16 * kSlotsRow <= 4 * kDma * 64, "direct loads must cover the stage");
};
constexpr int kLdsBytes = kNst * Tile<8>::kStageBytes;  // 114688: the 128-row ring, and the
                                                        // gate/up epilogue's staging

// Global -> LDS direct load of 16 bytes per lane (lane l fills LDS bytes
// m0 + 16 l).  Written as inline asm so that the compiler's wait-count
// bookkeeping sees only the weight loads (all of one kind, hence exact
// waits); the direct loads are waited for explicitly with vmcnt.  m0 holds
// nothing else in these kernels (no other direct loads, GWS or messages).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void direct16(uint32_t voff, const uint8_t *sbase, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(sbase), "s"(lds_addr)
        : "memory", "m0");
}
#pragma clang diagnostic pop

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

// Weight loads.  Codes: the 64 bytes a step needs from a row are half of a
// 128-byte line, so steps are loaded in pairs (2p, 2p+1), first all tiles'
// step 2p then all tiles' step 2p+1 (the second touch of each line hits the
// L1), into a ring of two pair slots; pair p is issued at step 2p - 2.
// Scales: one 16-byte load per row covers four steps (4 blocks each); group
// G (steps 4G..4G+3) is issued at step 4G - 3 and each lane keeps its four
// bytes (block g of each step) packed in one register.
//
// Like the direct loads, these are inline asm, waited for by the one
// explicit vmcnt at the top of each step.  The destinations are tied
// ("+v"): a ring slot keeps one register for its whole life, so no copy of
// a register whose load is still in flight can exist (a codegen test checks
// that the main loop holds no vector register copies).
struct BRing {
    u32x4_t q[2][2][8];         // [pair slot][step in pair][tile]
    u32x4_t sraw[8];            // scale group in flight
    uint32_t spk[8];            // current group, this lane's byte per step
};

struct GemmArgs {
    i32x4_t bq, bs;             // buffer resources: this expert's codes / scales
    uint32_t boff, soff;        // this lane's offsets in its first B tile (codes, scales)
    uint32_t tq[8], ts[8];      // wave-uniform offsets of the 8 B tiles (codes, scales)
    uint32_t psel01;            // v_perm selector: byte g of two dwords
    uint32_t cstep, sgrp;       // bytes from one K step's codes to the next, one scale group's
    int nsteps;
};

// A raw buffer resource (base, byte size) in scalar registers.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = 0x00020000;
    return r;
}

__device__ __forceinline__ void buf_load16_async(u32x4_t &dst, const i32x4_t &rsrc, uint32_t voff,
                                                 uint32_t soff) {
    asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen"
                 : "+v"(dst)
                 : "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

// Vector memory instructions issued at a step with ring position R (= the
// step index mod 4), in this order: 7 direct loads; at even R 16 code loads
// (8 of the pair's first step, then 8 of its second); at R == 1 8 scale
// loads.
constexpr int kCodeLoads = 16, kScaleLoads = 8;
// The one wait at the top of step kk (ring position R): what must have
// landed is this wave's part of stage kk (issued at step kk - 3), the codes
// of step kk (issued at step kk - 2 for even R, kk - 3 for odd R) and, at
// R == 0, the scale group (issued at step kk - 3).  The count is the number
// of loads issued after the last of those.
//   R = 0: last needed = codes s0 of step kk-2; after it: s1 (8), A(kk+2)
//   R = 1: last needed = codes s1 of step kk-3; after: A(kk+1), A(kk+2), 16 codes
//   R = 2: last needed = codes s0 of step kk-2; after: s1 (8), A(kk+2), 8 scales
//   R = 3: last needed = codes s1 of step kk-3; after: A(kk+1), 8 scales,
//          A(kk+2), 16 codes
constexpr int step_top_vmcnt(int R, int dma) {
    return R == 0 ? 8 + dma
         : R == 1 ? dma + dma + kCodeLoads
         : R == 2 ? 8 + dma + kScaleLoads
         : dma + kScaleLoads + dma + kCodeLoads;
}
static_assert(step_top_vmcnt(0, 7) == 15 && step_top_vmcnt(1, 7) == 30 &&
                  step_top_vmcnt(2, 7) == 23 && step_top_vmcnt(3, 7) == 38 &&
                  step_top_vmcnt(3, 1) == 26,
              "wait counts (the largest, 38, fits the 6-bit vmcnt)");

template <int PS>
__device__ __forceinline__ void issue_codes(BRing &br, const GemmArgs &ga, int j) {
    const uint32_t j0 = (uint32_t)min(j, ga.nsteps - 1), j1 = (uint32_t)min(j + 1, ga.nsteps - 1);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) buf_load16_async(br.q[PS][0][nt], ga.bq, ga.boff, ga.tq[nt] + j0 * ga.cstep);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) buf_load16_async(br.q[PS][1][nt], ga.bq, ga.boff, ga.tq[nt] + j1 * ga.cstep);
}

__device__ __forceinline__ void issue_scales(BRing &br, const GemmArgs &ga, int G) {
    const uint32_t gg = (uint32_t)min(G, (ga.nsteps - 1) >> 2);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) buf_load16_async(br.sraw[nt], ga.bs, ga.soff, ga.ts[nt] + gg * ga.sgrp);
}

// After the last step some weight loads (the clamped re-loads past the end)
// may still be in flight into ring registers the compiler no longer needs.
// Waiting for them, then naming every ring register in an asm statement,
// keeps those registers from being reused before the data has landed.
__device__ __forceinline__ void drain_weight_loads(BRing &br) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
            asm volatile("" ::"v"(br.q[ps][sub][0]), "v"(br.q[ps][sub][1]), "v"(br.q[ps][sub][2]),
                         "v"(br.q[ps][sub][3]), "v"(br.q[ps][sub][4]), "v"(br.q[ps][sub][5]),
                         "v"(br.q[ps][sub][6]), "v"(br.q[ps][sub][7]));
    asm volatile("" ::"v"(br.sraw[0]), "v"(br.sraw[1]), "v"(br.sraw[2]), "v"(br.sraw[3]),
                 "v"(br.sraw[4]), "v"(br.sraw[5]), "v"(br.sraw[6]), "v"(br.sraw[7]));
}

// spk byte i = byte g of dword i of the group's 16 bytes.
__device__ __forceinline__ void pack_scales(BRing &br, const GemmArgs &ga) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const u32x4_t r = br.sraw[nt];
        const uint32_t t01 = __builtin_amdgcn_perm(r.y, r.x, ga.psel01);
        const uint32_t t23 = __builtin_amdgcn_perm(r.w, r.z, ga.psel01);
        br.spk[nt] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
}

template <int MT>
__device__ __forceinline__ void issue_a(uint32_t lds_addr, const uint8_t *aq,
                                        const uint32_t (&src)[Tile<MT>::kDma], int nsteps, int j,
                                        int wid) {
    const uint32_t jj = (uint32_t)min(j, nsteps - 1);
    const uint32_t stage = lds_addr + (uint32_t)((j & (kNst - 1)) * Tile<MT>::kStageBytes);
#pragma unroll
    for (int i = 0; i < Tile<MT>::kDma; ++i)
        direct16(src[i] + jj * (uint32_t)kStepBytes, aq,
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(stage + 1024u * (4 * i + wid))));
}

// The scale operand reads byte 0 of the register (bits above are ignored).
// kSingle: the activation-MX mode, the hi term alone.
template <int PS, int SUB, bool kSingle>
__device__ __forceinline__ void mfma_mt(f32x4_t (&acc)[8], const AFrag &a, const BRing &br,
                                        const uint32_t (&bsc)[8]) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const u32x4_t q = br.q[PS][SUB][nt];
        const i32x8_t b = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        acc[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.hi, b, acc[nt], 2, 4, 0,
                                                                   (int)a.sc, 0, (int)bsc[nt]);
        if constexpr (!kSingle)
            acc[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.lo, b, acc[nt], 2, 4, 1,
                                                                       (int)a.sc, 0, (int)bsc[nt]);
    }
}

// The MT m-tiles of one K step: m-tile I's fragment is waited for (the
// next one's five reads may still be in flight), its 8 x (1 or 2) MFMAs
// issued, and m-tile I + 2's reads queued into the freed fragment.
template <int I, int MT, int PS, int SUB, bool kSingle>
__device__ __forceinline__ void mt_chain(f32x4_t (&acc)[MT][8], AFrag (&f)[2], const BRing &br,
                                         const uint32_t (&bsc)[8], uint32_t a, uint32_t s) {
    if constexpr (I < MT) {
        afrag_ready<(I + 1 < MT) ? 5 : 0>(f[I & 1]);
        mfma_mt<PS, SUB, kSingle>(acc[I], f[I & 1], br, bsc);
        if constexpr (I + 2 < MT) read_afrag<I + 2>(f[I & 1], a, s);
        mt_chain<I + 1, MT, PS, SUB, kSingle>(acc, f, br, bsc, a, s);
    }
}

// One K step at ring position R = kk % 4: wait for stage kk, queue step
// kk + 3's activations (and, by R, a code pair or a scale group), then
// MT * 16 (or MT * 8) MFMAs (A fragments read one m-tile ahead).
template <int R, bool kSingle, int MT>
__device__ __forceinline__ void gemm_step(f32x4_t (&acc)[MT][8], BRing &br, const GemmArgs &ga,
                                          const uint8_t *aq,
                                          const uint32_t (&src)[Tile<MT>::kDma],
                                          uint32_t lds_addr, uint32_t a_lane, uint32_t s_lane,
                                          int kk, int wid, bool live) {
    constexpr int PS = (R >> 1) & 1;        // pair slot of steps kk (and kk ^ 1)
    constexpr int SUB = R & 1;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(step_top_vmcnt(R, Tile<MT>::kDma)));
    __builtin_amdgcn_s_barrier();                        // everyone's part; stage kk-1 free
    __builtin_amdgcn_sched_barrier(0);
    issue_a<MT>(lds_addr, aq, src, ga.nsteps, kk + 3, wid);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr ((R & 1) == 0) issue_codes<PS ^ 1>(br, ga, kk + 2);
    if constexpr (R == 1) issue_scales(br, ga, (kk + 3) >> 2);
    if constexpr (R == 0) pack_scales(br, ga);
    __builtin_amdgcn_sched_barrier(0);
    if (!live) return;
    const uint32_t st = lds_addr + (uint32_t)((kk & (kNst - 1)) * Tile<MT>::kStageBytes);
    const uint32_t a = st + a_lane, s = st + s_lane;
    uint32_t bsc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) bsc[nt] = br.spk[nt] >> (8 * R);
    AFrag f[2];
    read_afrag<0>(f[0], a, s);
    if constexpr (MT > 1) read_afrag<1>(f[1], a, s);
    mt_chain<0, MT, PS, SUB, kSingle>(acc, f, br, bsc, a, s);
}

// The block's tile: which expert, which 128 rows of it, which 512 weight
// rows.  Blocks are spread over the 8 XCDs (consecutive block ids go to
// consecutive XCDs) so that each XCD walks a contiguous range of the
// (m-tile, n-block) order: the n-blocks of one m-tile, and the m-tiles of
// one expert, meet in the same L2.
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
    const int mt = u / NB;
    ts.nb = u - mt * NB;
    const int nact = plan[0];
    const int a = find_expert(tiles, nact, mt);
    ts.e = plan[1 + a];
    if ((unsigned)ts.e >= (unsigned)E) return false;
    ts.row0 = offsets[ts.e];
    ts.ne = offsets[ts.e + 1] - ts.row0;
    if (ts.row0 < 0 || ts.ne <= 0 || ts.row0 + ts.ne > nrows) return false;
    ts.m0 = (mt - tiles[1 + a]) * kBM;
    return true;
}

// kGateUp: A = split x (token rows), out = hq, the split of h = silu(gate) *
//          up [rows][f] (expert-major rows), the down pass's A;
// else:    A = hq, out = rows_out bf16 [rows][d].
// packed: the weights are in the operand-order layout of prepack_kernel
// (K % 512 == 0): each code load of a 16-row tile and K step reads 1 KB
// contiguous, each scale load 256 B, instead of 16 rows x 64 B (16 B); the
// registers receive the same bytes either way.
// MT: the tile's height in 16-row m-tiles, the smallest of 1, 2, 4, 8 that
// holds its rows, so that an expert with few rows pays matrix work for
// those rows (rounded up to 16, 32 or 64) rather than for 128.
template <bool kGateUp, bool kSingle, int MT>
__device__ __forceinline__ void gemm_tile(const uint8_t *__restrict__ aq, const ExpertArgs &W,
                                          uint8_t *__restrict__ hq,
                                          uint16_t *__restrict__ rows_out, int d, int f,
                                          int packed, const TileSel &ts,
                                          const int *a_rowidx, uint8_t *lds) {
    constexpr int kDma = Tile<MT>::kDma;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = kGateUp ? d : f;
    GemmArgs ga;
    ga.nsteps = K >> 7;
    const uint32_t a_row_bytes = (uint32_t)ga.nsteps * kStepBytes;
    const uint32_t code_row = (uint32_t)K >> 1, nblk = (uint32_t)K >> 5;
    const uint32_t wrows = kGateUp ? 2u * (uint32_t)f : (uint32_t)d;
    const uint8_t *bq = (kGateUp ? W.gu_codes : W.dn_codes) + (size_t)ts.e * wrows * code_row;
    const uint8_t *bsb = (kGateUp ? W.gu_scales : W.dn_scales) + (size_t)ts.e * wrows * nblk;
    ga.bq = buffer_rsrc(bq, wrows * code_row);
    ga.bs = buffer_rsrc(bsb, wrows * nblk);
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int wr = kGateUp ? (nt < 4 ? ts.nb * 256 + 64 * wid + 16 * nt
                                         : f + ts.nb * 256 + 64 * wid + 16 * (nt - 4))
                               : ts.nb * 512 + 128 * wid + 16 * nt;
        // tile wr / 16 of the expert: (K / 128) code blocks of 1 KB and
        // (K / 512) scale groups of 256 B when packed
        ga.tq[nt] = packed ? (uint32_t)(wr >> 4) * (uint32_t)(K >> 7) * 1024u : (uint32_t)wr * code_row;
        ga.ts[nt] = packed ? (uint32_t)(wr >> 4) * (uint32_t)(K >> 9) * 256u : (uint32_t)wr * nblk;
    }
    ga.boff = packed ? 16u * (uint32_t)lane : (uint32_t)r16 * code_row + 16u * g;
    ga.soff = packed ? 16u * (uint32_t)r16 : (uint32_t)r16 * nblk;   // dword aligned
    ga.cstep = packed ? 1024u : 64u;
    ga.sgrp = packed ? 256u : 16u;
    ga.psel01 = (uint32_t)g | ((4u + (uint32_t)g) << 8);
    uint32_t src[kDma];                             // byte offsets into aq (< 4 GiB)
    constexpr int kRows = MT * 16;
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int sl = 64 * (4 * i + wid) + lane;
        const int r = sl < kRows * kSlotsRow ? sl / kSlotsRow : kRows - 1;
        const int pc = sl < kRows * kSlotsRow ? sl - r * kSlotsRow : kSlotsRow - 1;
        src[i] = (uint32_t)a_rowidx[r] * a_row_bytes + 16u * pc;
    }
    const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
    const uint32_t a_lane = (uint32_t)(r16 * kStepBytes + 48 * g);
    const uint32_t s_lane = (uint32_t)(r16 * kStepBytes + 192 + 2 * g);

    f32x4_t acc[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // prologue: the loads of steps -3, -2, -1 in the steady state's roles
    // (ring positions 1, 2, 3): A(0) + scale group 0, A(1) + codes of steps
    // 0 and 1, A(2)
    BRing br = {};
    issue_a<MT>(lds_addr, aq, src, ga.nsteps, 0, wid);
    __builtin_amdgcn_sched_barrier(0);
    issue_scales(br, ga, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_a<MT>(lds_addr, aq, src, ga.nsteps, 1, wid);
    __builtin_amdgcn_sched_barrier(0);
    issue_codes<0>(br, ga, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_a<MT>(lds_addr, aq, src, ga.nsteps, 2, wid);
    __builtin_amdgcn_sched_barrier(0);
    // four steps per turn of the register ring and no branch around any
    // load, wait or barrier (a step past the end only skips its MFMAs), so
    // the wait counts the compiler derives at the loop header are exact
    for (int kk = 0; kk < ga.nsteps; kk += 4) {
        gemm_step<0, kSingle, MT>(acc, br, ga, aq, src, lds_addr, a_lane, s_lane, kk, wid, true);
        gemm_step<1, kSingle, MT>(acc, br, ga, aq, src, lds_addr, a_lane, s_lane, kk + 1, wid,
                                  kk + 1 < ga.nsteps);
        gemm_step<2, kSingle, MT>(acc, br, ga, aq, src, lds_addr, a_lane, s_lane, kk + 2, wid,
                                  kk + 2 < ga.nsteps);
        gemm_step<3, kSingle, MT>(acc, br, ga, aq, src, lds_addr, a_lane, s_lane, kk + 3, wid,
                                  kk + 3 < ga.nsteps);
    }
    // drain the trailing (re-)loads before their registers or the block's
    // LDS can be reused
    drain_weight_loads(br);
    __builtin_amdgcn_sched_barrier(0);

    // epilogue: lane holds rows 4 (l / 16) + i, column l % 16 of each tile
    if (kGateUp) {
        // h = silu(gate) * up goes through LDS (the A ring is idle now) in
        // passes of up to 64 rows, then is split one 32-element block per
        // lane: the wave's 64 h columns hc0 .. hc0 + 63 are MX blocks gb0,
        // gb0 + 1 of down step hc0 / 128
        constexpr int kHs = 68;                          // floats per staged row
        constexpr int kPassMt = MT < 4 ? MT : 4;         // m-tiles per pass
        float *hs = reinterpret_cast<float *>(lds) + wid * 64 * kHs;
        const int hc0 = ts.nb * 256 + 64 * wid;
        const uint32_t hq_row = (uint32_t)(f >> 7) * kStepBytes;
        uint8_t *hq_step = hq + (size_t)(hc0 >> 7) * kStepBytes;
        const int gb0 = (hc0 & 127) >> 5;
        __syncthreads();                                 // every wave is done with the ring
#pragma unroll
        for (int pass = 0; pass < MT / kPassMt; ++pass) {
            const int left = ts.ne - ts.m0 - 64 * pass;   // rows of the tile from this pass on
            if (left <= 0) break;
#pragma unroll
            for (int m = 0; m < kPassMt; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const float gv = acc[kPassMt * pass + m][nt][i];
                        const float uv = acc[kPassMt * pass + m][nt + 4][i];
                        hs[(16 * m + 4 * g + i) * kHs + 16 * nt + r16] = gv / (1.0f + expf(-gv)) * uv;
                    }
            __syncthreads();
            // buffer stores drop offsets past the pass's live rows
            const uint32_t live_bytes = (uint32_t)min(left, 16 * kPassMt) * hq_row;
            const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
                hq_step + (size_t)(ts.row0 + ts.m0 + 64 * pass) * hq_row, 0, (int)live_bytes,
                0x00020000);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                if (it == 1 && (kPassMt < 4 || left <= 32)) break;
                const int item = 64 * it + lane, rl = item >> 1, blk = gb0 + (item & 1);
                float v[32];
                const float *src = hs + rl * kHs + 32 * (item & 1);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f32x4_t w = *reinterpret_cast<const f32x4_t *>(src + 4 * c);
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[4 * c + q] = w[q];
                }
                const SplitBlock sb = split_block32(v);
                u32x4_t w[3];
                split_words(sb, w);
                const uint32_t o = (uint32_t)rl * hq_row;
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    __builtin_amdgcn_raw_buffer_store_b128(w[c], out, o + 48u * blk + 16u * c, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sb.scales, out, o + 192u + 2u * blk,
                                                      0, 0);
            }
            __syncthreads();
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ts.m0 + mt * 16 + 4 * g + i;
                if (r < ts.ne) {
                    uint16_t *orow = rows_out + (size_t)(ts.row0 + r) * d + ts.nb * 512 + 128 * wid;
#pragma unroll
                    for (int nt = 0; nt < 8; ++nt) orow[16 * nt + r16] = f32_to_bf16_rne(acc[mt][nt][i]);
                }
            }
    }
}

// One block per (m-tile, n-block) unit of the tile plan; the tile's height
// is chosen from its rows (block-uniform, so the branch below and every
// barrier inside gemm_tile are taken by the whole block).
template <bool kGateUp, bool kSingle>
__global__ __launch_bounds__(256) void ffn_mfma_kernel(
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
    const int rows = __builtin_amdgcn_readfirstlane(min(kBM, ts.ne - ts.m0));
    if (rows <= 16)
        gemm_tile<kGateUp, kSingle, 1>(aq, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else if (rows <= 32)
        gemm_tile<kGateUp, kSingle, 2>(aq, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else if (rows <= 64)
        gemm_tile<kGateUp, kSingle, 4>(aq, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
    else
        gemm_tile<kGateUp, kSingle, 8>(aq, W, hq, rows_out, d, f, packed, ts, a_rowidx, lds);
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
                           dim3((unsigned)blocks), dim3(256), kLdsBytes, s, xq, w, offsets,
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
                           dim3((unsigned)blocks), dim3(256), kLdsBytes, s, hq, w, offsets,
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
