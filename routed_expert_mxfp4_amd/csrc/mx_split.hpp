// mx_split.hpp -- the two-term MX E2M3 split of 32-element blocks on gfx950
// (device helpers shared by the scaled-MFMA GEMM and the decode kernels).
#pragma once

#include "moe_internal.hpp"

namespace moe {

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

}  // namespace moe
