/*
 * moe_packed.h -- the MXFP4 expert store of moe.h re-laid in the operand
 * order of the prefill GEMM, for AMD Instinct MI355X (gfx950).
 *
 * The store holds the same bytes as the canonical one (the page's
 * 17,547,264 B per expert: Moonshine README, GitHub mirror, "Expert-stream
 * compression"); only their order differs.  In the canonical store a
 * 16-row tile's K step is 16 rows x 64 code bytes; the scaled-MFMA GEMM
 * gives each lane one row's 16 bytes, so each of its code loads gathers 64
 * bytes from 16 rows.  Packed, those 1,024 bytes are contiguous in lane
 * order, and a 16-row tile's scales for 4 K steps are 256 contiguous bytes:
 *   codes  [E] then per matrix [rows/16][K/128] blocks of 1 KB; in a block,
 *          lane l = r + 16 g (r < 16, g < 4) holds at 16 l the codes of row
 *          16 t + r for K elements 128 s + 32 g .. 128 s + 32 g + 31;
 *   scales [E] then per matrix [rows/16][K/512] blocks of 256 B; row r's 16
 *          E8M0 codes (K blocks 16 G .. 16 G + 15) at 16 r;
 * for gate/up (rows 2f, K = d) and down (rows d, K = f) alike.  The struct
 * is moe_mxfp4_experts with its four arrays in this order and their
 * canonical sizes.  Needs d % 512 == 0 and f % 512 == 0.
 *
 * moe_layer_forward_packed serves prefill-sized calls (the scaled-MFMA
 * path of moe_layer_forward: T >= 128) and gives the same bits as
 * moe_layer_forward on the canonical store.  Conventions are those of
 * moe.h.
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_PACKED_H
#define ROUTED_EXPERT_MXFP4_MOE_PACKED_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dst = the packed layout of src (dims->E experts of shape d, f; T, k and
 * act are ignored but must be valid).  dst's arrays have src's sizes and
 * must not overlap src.  MOE_ERR_UNSUPPORTED unless d % 512 == 0 and
 * f % 512 == 0.  Asynchronous on hip_stream; a one-time conversion, run
 * before (not inside) the calls that use it. */
moe_status moe_prepack_experts(const moe_dims *dims, const moe_mxfp4_experts *src,
                               const moe_mxfp4_experts *dst, void *hip_stream);

/* moe_layer_forward with the experts in the packed layout.  Workspace: the
 * size moe_workspace_bytes(dims, MOE_ENTRY_LAYER_FORWARD) gives.
 * MOE_ERR_UNSUPPORTED unless T >= 128, d % 512 == 0 and f % 512 == 0. */
moe_status moe_layer_forward_packed(const moe_dims *dims, const uint16_t *x,
                                    const uint16_t *router_w, const float *router_bias,
                                    const moe_mxfp4_experts *packed, uint16_t *y,
                                    int32_t *topk_ids_out, float *topk_w_out, void *ws,
                                    size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_MXFP4_MOE_PACKED_H */
