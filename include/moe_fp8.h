/*
 * moe_fp8.h -- C ABI of the routed MoE layer of moe.h with FP8 experts, for
 * AMD Instinct MI355X (gfx950).
 *
 * The pages' FP8 lane (Moonshine README, "GLM 5.3 Flash status") pairs an
 * exhaustive OCP E4M3FN oracle with a fused GEMV and a bounded BF16-dequant
 * prefill floor.  The layer is the one of moe.h (router, top-k, grouping,
 * SwiGLU experts, weighted combine, the same readings), with each expert
 * stored as:
 *   gu_codes  [E][2f][d]          E4M3FN codes of the gate/up matrix (K = d)
 *   gu_scales [E][2f/128][d/128]  fp32: one scale per 128 x 128 block
 *   dn_codes  [E][d][f]           E4M3FN codes of the down matrix (K = f)
 *   dn_scales [E][d/128][f/128]   fp32
 * weight = E4M3FN(code) * scale of its block; gate = rows [0, f), up =
 * rows [f, 2f).  E4M3FN is the OCP 8-bit E4M3 format (bias 7, no
 * infinities, S.1111.111 NaN, largest finite 448).  The pages do not print
 * the scale layout; the 128 x 128 fp32 block scale is the reading (the
 * layout of block-scaled official FP8 checkpoints).  3*d*f bytes of codes
 * per expert, twice the MXFP4 store.
 *
 * Below 128 tokens the experts run as grouped dequant-GEMVs (bf16 weights
 * exist only in registers, per tile in flight; each 16-element partial sum
 * is multiplied by its block scale in fp32).  From 128 tokens on they run
 * as grouped GEMMs on the bf16 matrix cores: each weight, converted exactly
 * from E4M3FN and multiplied by its block scale in fp32, is rounded once to
 * bf16 (relative error at most 2^-9) as the wave reads its fragment from
 * LDS; activations are used as given, accumulation is fp32, and h is
 * rounded to bf16 between the two GEMMs.  Conventions are those of moe.h (device pointers owned
 * by the caller, asynchronous on hip_stream, validation before any launch,
 * T == 0 a no-op, deterministic).  Also: d % 128 == 0, f % 128 == 0,
 * dims->act == MOE_ACT_BF16 (else MOE_ERR_UNSUPPORTED), codes and scales
 * 16-byte aligned.
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_FP8_H
#define ROUTED_EXPERT_MXFP4_MOE_FP8_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The FP8 expert store (struct in host memory, tensors on the device). */
typedef struct moe_fp8_experts {
    const uint8_t *gu_codes;
    const float *gu_scales;
    const uint8_t *dn_codes;
    const float *dn_scales;
} moe_fp8_experts;

/* Scratch bytes of moe_expert_ffn_fp8 (entry MOE_ENTRY_EXPERT_FFN) or
 * moe_layer_forward_fp8 (MOE_ENTRY_LAYER_FORWARD); (size_t)-1 for invalid
 * dims or another entry. */
size_t moe_fp8_workspace_bytes(const moe_dims *dims, int entry);

/* Expert FFN over grouped rows (step 4 of moe.h) with FP8 experts: offsets
 * and sorted_rows from moe_permute; rows_out bf16 [T*k][d], expert-major. */
moe_status moe_expert_ffn_fp8(const moe_dims *dims, const uint16_t *x,
                              const moe_fp8_experts *experts, const int32_t *offsets,
                              const int32_t *sorted_rows, uint16_t *rows_out, void *ws,
                              size_t ws_bytes, void *hip_stream);

/* The whole layer (steps 1-5 of moe.h) with FP8 experts. */
moe_status moe_layer_forward_fp8(const moe_dims *dims, const uint16_t *x,
                                 const uint16_t *router_w, const float *router_bias,
                                 const moe_fp8_experts *experts, uint16_t *y,
                                 int32_t *topk_ids_out, float *topk_w_out, void *ws,
                                 size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_MXFP4_MOE_FP8_H */
