/*
 * moe_diag.h -- diagnostics of the routed MXFP4 MoE library: GPU time of
 * one named kernel, measured with HIP events recorded on the same stream as
 * the kernel's launches.  Not part of the layer's computation; a benchmark
 * uses it to time its dominant kernel inside the timed region.
 *
 * Kernel names: "router_logits", "topk_softmax", "permute", "topk_permute"
 * (the two fused, small T), "plan", "gemv_gate_up", "gemv_down",
 * "down_combine", "combine".
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_DIAG_H
#define ROUTED_EXPERT_MXFP4_MOE_DIAG_H

#ifdef __cplusplus
extern "C" {
#endif

/* Start timing every launch of `kernel` (NULL or "" stops timing).  Creates
 * `capacity` event pairs up front (the only allocation); launches beyond
 * that many are not timed.  Drops any earlier records.  Returns 0, or -1 if
 * event creation failed or capacity < 0. */
int moe_diag_time_kernel(const char *kernel, int capacity);

/* Sum of the elapsed times (ms) of the recorded launches and their count.
 * Call only after the streams they ran on have been synchronised.  Clears
 * the records (timing stays on).  Returns 0, or -1 on a HIP error. */
int moe_diag_kernel_time(double *total_ms, long long *launches);

#ifdef __cplusplus
}
#endif
#endif
