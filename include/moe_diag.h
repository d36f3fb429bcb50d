/*
 * moe_diag.h -- diagnostics of the routed MXFP4 MoE library: GPU time of
 * one named kernel, measured with HIP events recorded on the same stream as
 * the kernel's launches.  Not part of the layer's computation; a benchmark
 * uses it to time its dominant kernel inside the timed region.
 *
 * Kernel names: "router_logits", "topk_softmax", "permute", "topk_permute"
 * (the two fused, small T), "router_norms", "router_filter_gemm",
 * "router_select", "router_refine" (routing of many tokens; the refine
 * kernel also takes the top-k), "plan", "gemv_gate_up", "gemv_down",
 * "down_combine", "combine", "mfma_ffn" (the whole scaled-MFMA expert
 * FFN, with its small experts' GEMVs), its parts "mx_split_x",
 * "gate_up_mfma" (which also splits h) and "down_mfma", and "mx_round" (the activation-MX mode's
 * rounding of x and h on the GEMV paths); for FP8 experts "fp8_gate_up" and
 * "fp8_down" (GEMVs for few tokens, matrix-core GEMMs from 128 on) and
 * "fp8_plan" (the GEMMs' row tiles); "stream_read" and "mfma_rate" (the
 * measured ceilings below); for the pre-norm block "rmsnorm", "shared_gate_up",
 * "shared_down_add", "shared_gemm_gate_up" (which also applies the SwiGLU)
 * and "shared_gemm_down".
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_DIAG_H
#define ROUTED_EXPERT_MXFP4_MOE_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The activation split the scaled-MFMA expert path feeds to the matrix
 * cores, exposed for bit-exact checks: each row of `in` (rows x K, K a
 * multiple of 128; bf16 bits if in_is_bf16, else fp32; in and out 16-byte
 * aligned; the output under 4 GiB) is
 * cut into 32-element blocks and each block a into two OCP MX E2M3 terms,
 * hi = MX(a), lo = MX(a - hi): shared exponent X = floor(log2 max|.|) - 2
 * clamped to [-127, 127] (E8M0 code X + 127; all-zero block -> code 0),
 * elements rounded to nearest even and saturated at 7.5.  Output `out`,
 * rows x (K/128) x 208 bytes; per row and 128-element step:
 *   block g (0..3) at byte 48 g: [hi codes 0..15][lo codes 0..15]
 *                                [hi codes 16..23][lo codes 16..23]
 *   byte 192 + 2 g: E8M0 code of hi, 193 + 2 g: of lo; bytes 200..207 zero
 * where a term's "codes" are its 24-byte stream of 6-bit fields, element i
 * of the block at bits 6i..6i+5, little-endian.  Device pointers;
 * asynchronous on hip_stream.  Returns 0, or -1 on bad arguments or a
 * launch error. */
int moe_diag_mx_split_e2m3(const void *in, int in_is_bf16, int rows, int K, uint8_t *out,
                           void *hip_stream);

/* Start timing every launch of `kernel` (NULL or "" stops timing).  Creates
 * `capacity` event pairs up front (the only allocation); launches beyond
 * that many are not timed.  A single-kernel name is timed by events that
 * its launch itself records (hipExtLaunchKernel) and that skip the
 * system-scope fence; names covering several launches (permute, plan,
 * mfma_ffn, router_norms) by events recorded around them.  Drops any
 * earlier records.  Returns 0, or -1 if event creation failed or
 * capacity < 0. */
int moe_diag_time_kernel(const char *kernel, int capacity);

/* As moe_diag_time_kernel, but only the 1st, (every+1)-th, (2 every+1)-th,
 * ... launch of the kernel is timed (every >= 1), so that a long run of
 * short launches carries the events' own cost on a sample of them only.
 * Returns 0, or -1 as moe_diag_time_kernel or if every < 1. */
int moe_diag_time_kernel_every(const char *kernel, int capacity, int every);

/* Sum of the elapsed times (ms) of the recorded launches and their count.
 * Call only after the device has been synchronised.  Clears
 * the records (timing stays on).  Returns 0, or -1 on a HIP error. */
int moe_diag_kernel_time(double *total_ms, long long *launches);

/* The elapsed time (ms) of each recorded launch, in launch order: up to
 * `cap` of them into ms_out (host memory), their number into *launches.
 * Call only after the device has been synchronised.  Clears the records
 * like moe_diag_kernel_time.  Returns 0, or -1 on a HIP error or bad
 * arguments. */
int moe_diag_kernel_times(double *ms_out, int cap, long long *launches);

/* Measured ceilings, for reporting each kernel's fraction of what this GPU
 * sustains next to the published peaks.
 *
 * moe_diag_stream_read: one launch that reads `bytes` bytes at `src`
 * (device memory, 16-byte aligned, bytes a multiple of 16) with 16-byte
 * loads, eight in flight per thread, over `blocks` blocks of 256 threads,
 * and writes an XOR checksum per block to out[0 .. blocks-1] (device
 * memory).  Time it with events on hip_stream: bytes / time is the
 * streaming-read bandwidth a kernel reading the same bytes in one launch
 * can reach.
 *
 * moe_diag_mfma_rate: one launch of `blocks` blocks of four waves; each
 * wave issues iters x 4 matrix instructions (iters a multiple of 4) from
 * registers, in sixteen (16x16 shapes) or four (32x32 shapes) independent
 * accumulation chains, with no memory traffic, and writes one sum to
 * out[4 blocks] (device memory).
 * kind 0: scaled 16x16x128 with A FP6 E2M3, B FP4 E2M1 (the expert GEMMs'
 * split activations x weights); 1: A FP8 E4M3, B FP4; 2: FP4 x FP4;
 * 3: FP8 x FP8; 4: bf16 32x32x16 (the shared expert's GEMMs); 5: FP6 x
 * FP4 and 6: FP4 x FP4 in the 32x32x64 scaled shape.  Flops per
 * instruction: 2*16*16*128 for kinds 0-3, 2*32*32*16 for kind 4,
 * 2*32*32*64 for kinds 5 and 6.
 *
 * Both are asynchronous on hip_stream; return 0, or -1 on bad arguments or
 * a launch error. */
int moe_diag_stream_read(const void *src, size_t bytes, uint32_t *out, int blocks,
                         void *hip_stream);
int moe_diag_mfma_rate(int kind, int blocks, int iters, float *out, void *hip_stream);

/* The per-expert path choice of the bf16 layer: in a call on the
 * scaled-MFMA expert path, experts with at most this many rows take the
 * grouped dequant-GEMVs instead of 128-row MFMA tiles.  Set 0..16 to
 * override the built-in crossover for the calls that follow (0: every
 * expert on MFMA tiles), -1 to restore it; a benchmark sweeps it to measure
 * the crossover.  Process-wide; moe_workspace_bytes follows the setting, so
 * size workspaces after setting it.  Returns 0, or -1 outside -1..16. */
int moe_diag_set_gemv_max_rows(int rows);

/* The crossover in effect (the override if one is set). */
int moe_diag_gemv_max_rows(void);

#ifdef __cplusplus
}
#endif
#endif
