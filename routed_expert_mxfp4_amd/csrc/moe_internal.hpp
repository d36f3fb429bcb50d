// moe_internal.hpp -- device helpers and kernel-launch declarations shared
// by the gfx950 kernels of the routed MXFP4 MoE layer and its C ABI.
//
// Nothing here is visible through include/moe.h; the ABI file validates
// arguments and then calls the launch_* functions below, all of which queue
// work on the given stream and return the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

// ---------------------------------------------------------------------------
// Fixed limits of the library (checked on the host before any launch).
// ---------------------------------------------------------------------------
constexpr int kMaxExperts = 1024;   // top-k keeps <= 16 logits per lane
constexpr int kMaxTopK = 32;
constexpr int kMfmaMinT = 128;      // tokens from which the activation-MX mode and the
                                    // packed store take the scaled-MFMA expert path
// Per-expert path choice of the bf16 (W4A16) layer: in a call on the
// scaled-MFMA path, experts with at most kGemvMaxRows rows take the grouped
// GEMVs and the rest the MFMA tiles (the crossover measured on MI355X by
// bench.py --crossover); a diagnostic override may set 0..kGemvMaxRowsCap.
constexpr int kGemvMaxRows = 1;
constexpr int kGemvMaxRowsCap = 16;
constexpr int kRouteFilterMinT = 256; // tokens from which routing filters on bf16 MFMA logits

// ---------------------------------------------------------------------------
// Small device helpers.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// x * 2^(code - 127) for an E8M0 scale code; code 255 is NaN.  ldexp keeps
// the result exact down to fp32 subnormals (code 0 is 2^-127).
__device__ __forceinline__ float apply_e8m0(float x, uint32_t code) {
    return code == 255u ? __uint_as_float(0x7FC00000u) : ldexpf(x, (int)code - 127);
}

// Raw buffer loads: a wave-uniform resource (base, byte size) plus a 32-bit
// per-lane offset and a uniform offset.  Loads past the size return 0, so
// a malformed index can never fault; addresses need one VGPR, not two.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// Issue-order helpers: an empty asm statement that takes loaded values as
// operands makes every one of them complete at that point, so a batch of
// loads is issued back to back and waited for once (instead of each load
// being scheduled next to its single use, one memory round trip apiece).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t as_v4(uint4 v) { return __builtin_bit_cast(u32x4_t, v); }
__device__ __forceinline__ void loads_done(const uint4 (&b)[2]) {
    __asm__ volatile("" ::"v"(as_v4(b[0])), "v"(as_v4(b[1])));
}
__device__ __forceinline__ void loads_done(const uint4 (&b)[4]) {
    __asm__ volatile("" ::"v"(as_v4(b[0])), "v"(as_v4(b[1])), "v"(as_v4(b[2])), "v"(as_v4(b[3])));
}
__device__ __forceinline__ void loads_done(const uint4 (&b)[16]) {
    __asm__ volatile("" ::"v"(as_v4(b[0])), "v"(as_v4(b[1])), "v"(as_v4(b[2])), "v"(as_v4(b[3])),
                     "v"(as_v4(b[4])), "v"(as_v4(b[5])), "v"(as_v4(b[6])), "v"(as_v4(b[7])),
                     "v"(as_v4(b[8])), "v"(as_v4(b[9])), "v"(as_v4(b[10])), "v"(as_v4(b[11])),
                     "v"(as_v4(b[12])), "v"(as_v4(b[13])), "v"(as_v4(b[14])), "v"(as_v4(b[15])));
}

// DPP row_ror:n on a float (rotate right by n within each row of 16 lanes).
template <int N>
__device__ __forceinline__ float dpp_ror_f32(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a lane group (lanes 16g .. 16g+15); every lane of
// the group gets the sum (DPP rotations, no LDS traffic).
__device__ __forceinline__ float group16_sum_f32(float v) {
    v += dpp_ror_f32<8>(v);
    v += dpp_ror_f32<4>(v);
    v += dpp_ror_f32<2>(v);
    v += dpp_ror_f32<1>(v);
    return v;
}

// Sum over the wave (fixed order: rows 0+1, rows 2+3, then the two); the
// result is wave-uniform.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = group16_sum_f32(v);
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (a + b) + (c + d);
}

// Dot product of 8 E2M1 codes (one 32-bit word, element 2i in the low
// nibble of byte i) with 8 bf16 values (four bf16x2 words), fp32 accumulate.
__device__ __forceinline__ float dot8_fp4_bf16(uint32_t codes, uint4 xv, float acc) {
    bf16x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 0);
    bf16x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 1);
    bf16x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 2);
    bf16x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 3);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w0, __builtin_bit_cast(bf16x2_t, xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w1, __builtin_bit_cast(bf16x2_t, xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w2, __builtin_bit_cast(bf16x2_t, xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w3, __builtin_bit_cast(bf16x2_t, xv.w), acc, false);
    return acc;
}

// Dot product of 8 E2M1 codes with 8 fp32 values.
__device__ __forceinline__ float dot8_fp4_f32(uint32_t codes, float4 a, float4 b, float acc) {
    f32x2_t w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    f32x2_t w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    f32x2_t w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    f32x2_t w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    acc = fmaf(w0.x, a.x, acc); acc = fmaf(w0.y, a.y, acc);
    acc = fmaf(w1.x, a.z, acc); acc = fmaf(w1.y, a.w, acc);
    acc = fmaf(w2.x, b.x, acc); acc = fmaf(w2.y, b.y, acc);
    acc = fmaf(w3.x, b.z, acc); acc = fmaf(w3.y, b.w, acc);
    return acc;
}

// ---------------------------------------------------------------------------
// Diagnostics: while moe_diag_time_kernel(name) is active, a DiagScope named
// `name` records HIP events before and after the launches in its lifetime
// (defined in moe_abi.cpp; costs one atomic load when timing is off).
// ---------------------------------------------------------------------------
class DiagScope {
  public:
    DiagScope(const char *kernel, hipStream_t s);
    ~DiagScope();
    DiagScope(const DiagScope &) = delete;
    DiagScope &operator=(const DiagScope &) = delete;

  private:
    hipStream_t s_;
    hipEvent_t stop_ = nullptr;
};

// The same timing for one launch, taken at the kernel itself: when `kernel`
// is being timed, the next start/stop event pair, which the launch records
// at the kernel's start and end; both null otherwise.
void diag_launch_events(const char *kernel, hipEvent_t *start, hipEvent_t *stop);

// Launches `fn` on stream s, timed as `kernel` when that name is being timed
// (the launch records the events itself, so no dispatch gap is counted).
template <typename F, typename... Args>
inline hipError_t timed_launch(const char *kernel, F fn, dim3 grid, dim3 block, size_t shmem,
                               hipStream_t s, Args... args) {
    hipEvent_t a = nullptr, b = nullptr;
    diag_launch_events(kernel, &a, &b);
    hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)shmem, s, a, b, 0u, args...);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).  All pointers are device pointers.
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const uint16_t *x, const uint16_t *wr, const float *bias,
                                float *logits, int T, int d, int E, hipStream_t s);
hipError_t launch_topk_softmax(const float *logits, int32_t *ids, float *w, int T, int E,
                               int k, hipStream_t s);
// Many tokens: top-k + softmax of the canonical logits without computing all
// of them (bf16 MFMA filter, certified bounds, canonical refinement).
// zt: fp32 [T][E] scratch, nx: fp32 [T], nw: fp32 [E] scratch; cand: int32
// [T][kRouteCandMax] and ncand: int32 [T] scratch (each token's candidates).
constexpr int kRouteCandMax = 64;
bool route_filter_ok(int T, int d, int E);
hipError_t launch_route_filtered(const uint16_t *x, const uint16_t *wr, const float *bias,
                                 float *zt, float *nx, float *nw, int32_t *cand, int32_t *ncand,
                                 int32_t *ids, float *tw, int T, int d, int E, int k,
                                 hipStream_t s);

size_t permute_ws_bytes(int T, int E);
// plan (nullable): int32 [1 + E] = number of active experts, then their ids.
hipError_t launch_permute(const int32_t *ids, int32_t *counts, int32_t *offsets,
                          int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, int T,
                          int E, int k, void *ws, hipStream_t s);
hipError_t launch_plan(const int32_t *offsets, int32_t *plan, int E, hipStream_t s);
// T <= 16: top-k + softmax and the grouping (with the plan) in one launch.
bool topk_permute_fusable(int T, int E, int k);
hipError_t launch_topk_permute_small(const float *logits, int32_t *ids, float *tw,
                                     int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                                     int32_t *row_pos, int32_t *plan, int T, int E, int k,
                                     hipStream_t s);

struct ExpertArgs {
    const uint8_t *gu_codes, *gu_scales, *dn_codes, *dn_scales;
};

// h: fp32 [T*k][f], expert-major rows (the row order of sorted_rows).
// hb: h is stored as bf16 (h points at T*k*f bf16 values; needs
// gemv_bf16_h_ok, else hipErrorInvalidValue), for a down + combine that
// reads bf16 h; otherwise fp32.
bool gemv_bf16_h_ok(int T, int d, int f);
hipError_t launch_gemv_gate_up(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                               const int32_t *sorted_rows, const int32_t *plan, float *h,
                               int T, int d, int E, int k, int f, hipStream_t s, bool hb = false);
// One token: top-k, softmax and grouping inside the gate/up GEMV (writes
// ids, tw, counts, offsets, sorted_rows, row_pos and plan as the permute
// step would).  Needs gate_up_token_fusable.
bool gate_up_token_fusable(int T, int d, int E, int k, int f);
hipError_t launch_gate_up_token(const float *logits, const uint16_t *x, ExpertArgs w,
                                int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                int32_t *sorted_rows, int32_t *row_pos, int32_t *plan, float *h,
                                int d, int E, int k, int f, hipStream_t s, bool hb = false);
hipError_t launch_gemv_down(const float *h, ExpertArgs w, const int32_t *offsets,
                            const int32_t *plan, uint16_t *rows_out, int T, int d, int E,
                            int k, int f, hipStream_t s);

// Measured ceilings (peaks.hip): one streaming read of `bytes` (a multiple
// of 16, src 16-byte aligned) over `blocks` blocks of 256 threads, a checksum
// per block into out[blocks]; and `iters` x 4 independent matrix
// instructions per wave on `blocks` blocks of four waves, one sum per wave
// into out[4 blocks].  kind: 0 FP6 E2M3 x FP4, 1 FP8 E4M3 x FP4, 2 FP4 x FP4,
// 3 FP8 x FP8 (scaled 16x16x128), 4 bf16 (32x32x16), 5 FP6 x FP4 and 6 FP4
// x FP4 (scaled 32x32x64).
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks,
                              hipStream_t s);
hipError_t launch_mfma_rate(int kind, int blocks, int iters, float *out, hipStream_t s);
hipError_t launch_down_combine(const float *h, ExpertArgs w, const int32_t *ids,
                               const float *topk_w, const int32_t *row_pos, uint16_t *y,
                               int T, int d, int E, int k, int f, hipStream_t s, bool hb = false);
// The mixed path's small experts (at most gemv_max rows each, listed in
// small[]: count, then ids): the grouped GEMVs with their fp32 h rows at
// small-expert index * gemv_max of h_small.  Need gemv_small_ok(d, f).
bool gemv_small_ok(int d, int f);
hipError_t launch_gemv_gate_up_small(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                                     const int32_t *sorted_rows, const int32_t *small,
                                     float *h_small, int T, int d, int E, int k, int f,
                                     int gemv_max, hipStream_t s);
hipError_t launch_gemv_down_small(const float *h_small, ExpertArgs w, const int32_t *offsets,
                                  const int32_t *small, uint16_t *rows_out, int T, int d, int E,
                                  int k, int f, int gemv_max, hipStream_t s);
// Expert FFN on scaled MFMA (x and h as two-term MX E2M3, weights as
// stored; the gate/up pass writes h already split).  Needs d % 512 == 0,
// f % 256 == 0; ws of mfma_ws_bytes, or of mixed_ws_bytes with
// gemv_max > 0: then the experts with at most gemv_max rows take the
// grouped GEMVs instead (the per-expert path choice; needs gemv_small_ok).
bool mfma_shape_ok(int T, int d, int k, int f);
size_t mfma_ws_bytes(int T, int d, int E, int k, int f);
size_t mixed_ws_bytes(int T, int d, int E, int k, int f, int gemv_max);
// single: the activation-MX mode (one matrix pass with the hi terms).
hipError_t launch_mfma_ffn(const uint16_t *x, ExpertArgs w, const int32_t *offsets,
                           const int32_t *sorted_rows, const int32_t *plan, uint16_t *rows_out,
                           void *ws, int T, int d, int E, int k, int f, bool single,
                           hipStream_t s, bool packed = false, int gemv_max = 0);
// The operand-order layout of the MXFP4 store for the scaled-MFMA GEMM (same
// bytes; needs d % 512 == 0 and f % 512 == 0): dst = prepack(src), dst must
// not overlap src.
bool prepack_ok(int d, int f);
hipError_t launch_prepack(ExpertArgs src, ExpertArgs dst, int E, int d, int f, hipStream_t s);
// The activation-MX rounding of rows x K (K % 32 == 0): every 32-element
// block to its one-term MX E2M3 value (out may be in).
hipError_t launch_mx_round_bf16(const uint16_t *in, int rows, int K, uint16_t *out,
                                hipStream_t st);
hipError_t launch_mx_round_f32(const float *in, int rows, int K, float *out, hipStream_t st);
// rows x K (K % 128 == 0) -> two-term MX E2M3 split rows, 208 bytes per row
// and 128-element step (codes of both terms, then their E8M0 scales).
size_t mx_split_bytes(int rows, int K);
hipError_t launch_mx_split_bf16(const uint16_t *in, int rows, int K, uint8_t *q, hipStream_t st);
hipError_t launch_mx_split_f32(const float *in, int rows, int K, uint8_t *q, hipStream_t st);

// resid (bf16 [T][d]) and extra (fp32 [T][d], needs resid; either may be
// NULL): the pre-norm block's residual and shared-expert terms, added in the
// same pass.
hipError_t launch_combine(const uint16_t *rows_out, const int32_t *row_pos,
                          const float *topk_w, uint16_t *y, int T, int d, int k,
                          hipStream_t s, const uint16_t *resid = nullptr,
                          const float *extra = nullptr);

// ---- FP8 experts (ffn_fp8.hip) ---------------------------------------------------
// E4M3FN codes [E][rows][K], fp32 scales [E][rows/128][K/128].
struct Fp8Args {
    const uint8_t *gu_codes;
    const float *gu_scales;
    const uint8_t *dn_codes;
    const float *dn_scales;
};
// Grouped dequant-GEMVs for any T: h fp32 [T*k][f] (expert-major rows),
// rows_out bf16 [T*k][d].  Need d % 128 == 0, f % 128 == 0.
hipError_t launch_fp8_gate_up(const uint16_t *x, Fp8Args w, const int32_t *offsets,
                              const int32_t *sorted_rows, const int32_t *plan, float *h, int T,
                              int d, int E, int k, int f, hipStream_t s);
hipError_t launch_fp8_down(const float *h, Fp8Args w, const int32_t *offsets,
                           const int32_t *plan, uint16_t *rows_out, int T, int d, int E, int k,
                           int f, hipStream_t s);
// One token: gate/up + SwiGLU with the top-k and grouping inside (as
// launch_gate_up_token, writing ids, tw, counts, offsets, sorted_rows,
// row_pos and plan), h fp32 [k][f].  Needs fp8_gate_up_token_fusable.
bool fp8_gate_up_token_fusable(int T, int d, int E, int k, int f);
hipError_t launch_fp8_gate_up_token(const float *logits, const uint16_t *x, Fp8Args w,
                                    int32_t *ids, float *tw, int32_t *counts, int32_t *offsets,
                                    int32_t *sorted_rows, int32_t *row_pos, int32_t *plan,
                                    float *h, int d, int E, int k, int f, hipStream_t s);
// Few tokens (fp8_down_combine_ok: T <= 4): down + weighted combine in one
// pass, y bf16 [T][d] (fp32 expert outputs, summed in slot order).
bool fp8_down_combine_ok(int T, int d, int k, int f);
hipError_t launch_fp8_down_combine(const float *h, Fp8Args w, const int32_t *ids,
                                   const float *topk_w, const int32_t *row_pos, uint16_t *y,
                                   int T, int d, int E, int k, int f, hipStream_t s);
// Many tokens (fp8_mfma_ok): the bf16 matrix-core GEMMs of ffn_fp8_mfma.hip
// (codes converted exactly to bf16 in LDS, block scales applied per 128-K
// chunk in fp32): tiles int32 scratch of fp8_mfma_tiles_bytes, h bf16
// [T*k][f], rows_out bf16 [T*k][d], both expert-major.
bool fp8_mfma_ok(int T, int d, int E, int k, int f);
int fp8_mfma_max_tiles(int T, int E, int k);
size_t fp8_mfma_tiles_bytes(int T, int E, int k);
hipError_t launch_fp8_mfma_ffn(const uint16_t *x, Fp8Args w, const int32_t *offsets,
                               const int32_t *sorted_rows, int32_t *tiles, uint16_t *h,
                               uint16_t *rows_out, int T, int d, int E, int k, int f,
                               hipStream_t s);

// ---- MoE tail (tail.hip, shared_gemm.hip) --------------------------------------
// xn = bf16(RMSNorm(x) * gamma), canonical fp64 order, one wave per token.
hipError_t launch_rmsnorm(const uint16_t *x, const uint16_t *gamma, float eps, uint16_t *xn,
                          int T, int d, hipStream_t s);
// Few tokens (1 <= T <= kSharedGemvMaxT): shared expert GEMVs, the down pass
// writing out = bf16(xres + yr + shared(xn)); h: fp32 [T][fs] scratch.
constexpr int kSharedGemvMaxT = 8;
hipError_t launch_shared_gemv(const uint16_t *xn, const uint16_t *sgu, const uint16_t *sdn,
                              const uint16_t *xres, const uint16_t *yr, float *h, uint16_t *out,
                              int T, int d, int fs, hipStream_t s);
// Many tokens, on the bf16 matrix cores (shared_gemm.hip):
// h bf16 [T][fs] = bf16(silu(xn Wgu[:fs]^T) * (xn Wgu[fs:]^T)), and
// sx fp32 [T][d] = h Wdn^T.  Need d % 64 == 0, fs % 32 == 0.
hipError_t launch_shared_gate_up_gemm(const uint16_t *xn, const uint16_t *sgu, uint16_t *h, int T,
                                      int d, int fs, hipStream_t s);
hipError_t launch_shared_down_gemm(const uint16_t *h, const uint16_t *sdn, float *sx, int T,
                                   int d, int fs, hipStream_t s);

}  // namespace moe
