/*
 * moe_tail.h -- C ABI of the MoE tail around the routed layer of moe.h: the
 * pre-norm block of a Kimi-K3-shaped MoE layer on AMD Instinct MI355X
 * (gfx950).
 *
 * The pages profile the model-shape MoE tail as the weighted reduction,
 * RMSNorm, the routed-up activation quantisation and the residual adds
 * (Moonshine README, "Run layer-major prefill"), and keep the shared experts
 * and norms in a bf16/Q8 static tier next to the routers, apart from the
 * MXFP4 routed experts (Moonshine README, "How the engine works", tier
 * diagram).  The block, per token t:
 *
 *   xn[t]  = RMSNorm(x[t]) * gamma                         (bf16)
 *   out[t] = x[t] + routed(xn[t]) + shared(xn[t])          (bf16)
 *
 * with routed() the layer of moe_layer_forward() on xn (router, top-k,
 * MXFP4 experts, weighted combine) and shared() one SwiGLU MLP of width fs
 * with bf16 weights, always applied with weight 1.
 *
 * Readings where the pages are silent (the CPU reference uses the same):
 *   - RMSNorm in a fixed fp64 order, so xn (and with it the routing) is
 *     reproducible bit for bit: ss = sum of x_i^2 over 64 equal chunks of d
 *     (each summed in ascending order) combined by the pairwise tree
 *     ((0,1),(2,3),... level by level); ms = ss / d; den = sqrt(ms + eps);
 *     xn_i = (x_i / den) * gamma_i, each one IEEE fp64 operation, rounded
 *     once from fp64 to bf16 (nearest even);
 *   - shared expert: gate = rows [0, fs) and up = rows [fs, 2fs) of
 *     shared_gu [2fs][d]; h = silu(gate) * up; shared_dn [d][fs]; no biases.
 *     fs = 0 (or NULL shared weights) means no shared expert;
 *   - out = x + y + s summed in fp32 (or fp64 by the reference) and rounded
 *     once to bf16.  On the GPU y, the routed sum, and h of the shared
 *     expert's second GEMM for many tokens are rounded to bf16 on the way.
 *
 * Conventions are those of moe.h: device pointers owned by the caller,
 * asynchronous on hip_stream, validation before any launch (a refused call
 * launches nothing and touches no output), T == 0 a no-op, no exception
 * crosses the boundary, identical inputs give identical bits.  The MoE
 * block also needs fs % 32 == 0, fs <= 16384, and 16-byte aligned gamma and
 * shared weights.  Like every entry point, the block allocates nothing: for
 * T <= 8 the shared expert runs as GEMVs, for T > 8 as two bf16
 * matrix-core GEMMs (SwiGLU fused into the first), all in this library.
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_TAIL_H
#define ROUTED_EXPERT_MXFP4_MOE_TAIL_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The tail's weights (struct in host memory, tensors on the device):
 *   norm_w     bf16 [d]       RMSNorm weight gamma
 *   eps        the norm's epsilon (>= 0, finite)
 *   fs         shared expert width (0: no shared expert)
 *   shared_gu  bf16 [2fs][d]  gate rows [0, fs), up rows [fs, 2fs)
 *   shared_dn  bf16 [d][fs]   */
typedef struct moe_tail_weights {
    const uint16_t *norm_w;
    float eps;
    int32_t fs;
    const uint16_t *shared_gu;
    const uint16_t *shared_dn;
} moe_tail_weights;

/* Scratch bytes moe_block_forward needs (the routed layer's workspace plus
 * the tail's); (size_t)-1 for invalid dims or tail shape. */
size_t moe_block_workspace_bytes(const moe_dims *dims, const moe_tail_weights *tail);

/* xn bf16 [T][d] = RMSNorm(x) * gamma in the fixed fp64 order above.
 *   x bf16 [T][d], gamma bf16 [d]; d % 64 == 0, d <= 32768 (dims->E, k, f
 *   and act are ignored but must be valid).  Bit-exact. */
moe_status moe_rmsnorm(const moe_dims *dims, const uint16_t *x, const uint16_t *gamma,
                       float eps, uint16_t *xn, void *hip_stream);

/* The whole pre-norm block on one stream, no host synchronisation.
 *   x            bf16 [T][d]  block input (the residual stream)
 *   tail         norm and shared expert weights
 *   router_w, router_bias, experts, dims->act: as for moe_layer_forward,
 *                applied to xn
 *   out          bf16 [T][d] out (must not alias x)
 *   topk_ids_out int32 [T][k] out or NULL; topk_w_out fp32 [T][k] or NULL */
moe_status moe_block_forward(const moe_dims *dims, const uint16_t *x,
                             const moe_tail_weights *tail, const uint16_t *router_w,
                             const float *router_bias, const moe_mxfp4_experts *experts,
                             uint16_t *out, int32_t *topk_ids_out, float *topk_w_out,
                             void *ws, size_t ws_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_MXFP4_MOE_TAIL_H */
