/*
 * moe.h -- C ABI of one routed Mixture-of-Experts FFN layer with MXFP4
 * experts, for AMD Instinct MI355X (gfx950).
 *
 * The layer, per token t of T:
 *   1. router logits  l[t][e] = sum_i x[t][i] * Wr[e][i] (+ b[e]) over E
 *      experts (the router runs on the requesting side, the routed expert FFN
 *      is the offloaded unit: MoonTail README, requester / volunteer table);
 *   2. top-k: k of E experts per token, 16 of 896 in the Kimi-K3 shape
 *      (Moonshine README, "How the engine works");
 *   3. group the T*k (token, slot) rows by expert before touching any weight
 *      ("groups all rows selecting each expert", a payload-free plan built
 *      from routing alone: Moonshine README, "How the engine works");
 *   4. per expert, gate/up GEMM with fused SwiGLU, then down GEMM, with the
 *      weights read once from their MXFP4 store (Moonshine README, GitHub
 *      mirror, "Expert-stream compression": 17,547,264 B per expert);
 *   5. weighted combine of each token's k expert outputs (the MoE tail's
 *      "weighted reduction": Moonshine README, "Run layer-major prefill").
 *
 * Readings where the pages are silent (the same ones the CPU reference uses):
 *   - canonical logit: split the d inputs into 64 equal chunks, sum each
 *     chunk in fp64 in ascending order, combine the chunk sums with a fixed
 *     pairwise tree ((0,1),(2,3),... level by level), add the bias in fp64,
 *     round once to fp32.  Expert selection is therefore bit-reproducible;
 *   - top-k order: descending logit; equal logits -> lower expert index first;
 *   - weights: softmax over the k selected logits, no extra scaling;
 *   - expert: h = silu(gate) * up, y_e = W_down h; no biases, no clamp;
 *   - gate = rows [0, f) of the gate/up matrix, up = rows [f, 2f);
 *     MXFP4 element 2i is the low nibble of byte i; one E8M0 scale per 32
 *     consecutive K elements (OCP Microscaling Formats v1.0).
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  "bf16" is the upper 16 bits of
 *     an IEEE binary32 in a uint16_t.  Arrays are row-major, densely packed.
 *   - `hip_stream` is a hipStream_t (NULL = the null stream).  Work is queued
 *     on it asynchronously; no call synchronises the host with the device.
 *   - Arguments are validated on the host BEFORE anything is launched.  On a
 *     non-zero status nothing has been launched and no output was touched.
 *     MOE_ERR_DEVICE reports a HIP launch error (work queued before it may
 *     have run).  No C++ exception crosses this boundary.
 *   - T == 0 is valid: the call returns MOE_OK and launches nothing.
 *   - Results are deterministic: identical inputs give identical bits.
 *   - Limits: d % 64 == 0, f % 32 == 0, 1 <= k <= min(E, 32), E <= 1024,
 *     T * k < 2^31, d <= 32768, f <= 16384.  Pointers to x, router_w, the
 *     expert tensors, rows_out, y and the workspace must be 16-byte aligned.
 *   - `ws` is scratch device memory of at least moe_workspace_bytes(dims,
 *     entry) bytes (may be NULL when that is 0).  It must not be shared by
 *     calls that can run concurrently.
 */
#ifndef ROUTED_EXPERT_MXFP4_MOE_H
#define ROUTED_EXPERT_MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

/* Activation modes of the expert GEMMs (moe_dims.act):
 *   MOE_ACT_BF16     x and h as computed (bf16 x, fp32 h): the layer's
 *                    W4A16 result; the prefill path gets there through a
 *                    two-term MX split (two matrix passes).
 *   MOE_ACT_MX_E2M3  the activation-MX mode: x and h are each rounded to
 *                    one OCP MX E2M3 term per 32 elements along K (shared
 *                    exponent floor(log2 amax) - 2, nearest-even elements
 *                    saturating at 7.5) before their GEMM, so the prefill
 *                    path makes one FP6 x FP4 matrix pass.  A different,
 *                    approximate result (a few % of max|y| away from W4A16
 *                    on the synthetic workloads).  The router always sees x
 *                    as given.  Like the pages' engine quantising the
 *                    routed-up activations ("Run layer-major prefill",
 *                    Moonshine README). */
#define MOE_ACT_BF16 0
#define MOE_ACT_MX_E2M3 1

/* Problem shape: T tokens, hidden size d, E experts, top-k, expert
 * intermediate size f; act: activation mode of moe_expert_ffn and
 * moe_layer_forward (MOE_ACT_*; the other entry points ignore it). */
typedef struct moe_dims {
    int32_t T, d, E, k, f;
    int32_t act;
} moe_dims;

/* The routed experts in their canonical MXFP4 store (device memory):
 *   gu_codes  [E][2f][d/2]   E2M1 codes of the gate/up matrix (K = d)
 *   gu_scales [E][2f][d/32]  E8M0 scale codes
 *   dn_codes  [E][d][f/2]    E2M1 codes of the down matrix (K = f)
 *   dn_scales [E][d][f/32]
 * 3*d*f*17/32 bytes per expert; the entry points here read these bytes as
 * they are (no dequantised or repacked copy).  moe_packed.h adds a one-time
 * re-layout of the same bytes for the prefill GEMM. */
typedef struct moe_mxfp4_experts {
    const uint8_t *gu_codes;
    const uint8_t *gu_scales;
    const uint8_t *dn_codes;
    const uint8_t *dn_scales;
} moe_mxfp4_experts;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                 */
    MOE_ERR_SHAPE = 2,       /* dims outside the limits above              */
    MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned           */
    MOE_ERR_WORKSPACE = 4,   /* ws_bytes < moe_workspace_bytes(...)        */
    MOE_ERR_UNSUPPORTED = 5, /* valid request the library does not serve   */
    MOE_ERR_DEVICE = 6,      /* HIP reported an error while launching      */
    MOE_ERR_SCRATCH = 7      /* moe_layer_forward_noalloc: the call needs
                                more than MOE_NOALLOC_SCRATCH_BYTES        */
} moe_status;

typedef enum moe_entry {
    MOE_ENTRY_ROUTE = 0,
    MOE_ENTRY_PERMUTE = 1,
    MOE_ENTRY_EXPERT_FFN = 2,
    MOE_ENTRY_COMBINE = 3,
    MOE_ENTRY_LAYER_FORWARD = 4
} moe_entry;

/* Scratch bytes an entry point needs for these dims (0 if none).  Returns
 * (size_t)-1 when dims are invalid or entry is unknown. */
size_t moe_workspace_bytes(const moe_dims *dims, int entry);

/* Static, human-readable text for a status code (never NULL). */
const char *moe_status_str(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

/* Router + top-k + softmax (steps 1-2).
 *   x           bf16 [T][d]
 *   router_w    bf16 [E][d]
 *   router_bias fp32 [E] or NULL (no bias)
 *   logits_out  fp32 [T][E] or NULL: the canonical logits, if wanted
 *   topk_ids    int32 [T][k] out: selected experts, descending logit
 *   topk_w      fp32 [T][k] out: softmax over the selected logits
 * Logits must come out finite; non-finite inputs give unspecified routing. */
moe_status moe_route(const moe_dims *dims, const uint16_t *x,
                     const uint16_t *router_w, const float *router_bias,
                     float *logits_out, int32_t *topk_ids, float *topk_w,
                     void *ws, size_t ws_bytes, void *hip_stream);

/* Group rows by expert (step 3).  Row r = t*k + j is (token t, slot j).
 *   topk_ids    int32 [T][k] in: distinct experts per token, each in [0, E)
 *   counts      int32 [E]    out: rows per expert
 *   offsets     int32 [E+1]  out: exclusive prefix sum of counts
 *   sorted_rows int32 [T*k]  out: rows ordered by (expert, token, slot)
 *   row_pos     int32 [T*k]  out: inverse of sorted_rows
 * Bit-exact integer work.  Ids that break the precondition (out of range
 * or repeated within a token) leave the outputs unspecified but in range
 * of their arrays. */
moe_status moe_permute(const moe_dims *dims, const int32_t *topk_ids,
                       int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                       int32_t *row_pos, void *ws, size_t ws_bytes,
                       void *hip_stream);

/* Expert FFN over the grouped rows (step 4).
 *   x           bf16 [T][d]
 *   experts     the MXFP4 store (struct in host memory, tensors on device)
 *   offsets     int32 [E+1] and sorted_rows int32 [T*k] from moe_permute
 *   rows_out    bf16 [T*k][d] out, expert-major: row p holds the output of
 *               expert e (offsets[e] <= p < offsets[e+1]) for token
 *               sorted_rows[p] / k.
 * fp32 accumulation; bf16 output. */
moe_status moe_expert_ffn(const moe_dims *dims, const uint16_t *x,
                          const moe_mxfp4_experts *experts,
                          const int32_t *offsets, const int32_t *sorted_rows,
                          uint16_t *rows_out, void *ws, size_t ws_bytes,
                          void *hip_stream);

/* Weighted combine (step 5): y[t] = sum_j topk_w[t][j] * rows_out[row_pos[t*k+j]]
 * accumulated in fp32 in slot order, rounded once to bf16 (RNE).
 *   rows_out bf16 [T*k][d], row_pos int32 [T*k], topk_w fp32 [T][k],
 *   y bf16 [T][d] out.  Each y element is written by exactly one thread:
 *   no atomics. */
moe_status moe_combine(const moe_dims *dims, const uint16_t *rows_out,
                       const int32_t *row_pos, const float *topk_w,
                       uint16_t *y, void *hip_stream);

/* The whole layer (steps 1-5) on one stream, no host synchronisation.
 *   y             bf16 [T][d] out
 *   topk_ids_out  int32 [T][k] out or NULL
 *   topk_w_out    fp32 [T][k] out or NULL
 * Small T takes a fused down + combine path that skips rows_out. */
moe_status moe_layer_forward(const moe_dims *dims, const uint16_t *x,
                             const uint16_t *router_w,
                             const float *router_bias,
                             const moe_mxfp4_experts *experts, uint16_t *y,
                             int32_t *topk_ids_out, float *topk_w_out,
                             void *ws, size_t ws_bytes, void *hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * exactly as moe_layer_forward computes it (same kernels, same bits), with
 * no workspace argument and no allocation of any kind.  Its scratch is one
 * static device array of MOE_NOALLOC_SCRATCH_BYTES, which the library holds
 * on every GPU it runs on until the process ends.
 *   - A call whose moe_workspace_bytes(dims, MOE_ENTRY_LAYER_FORWARD)
 *     exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH and
 *     launches nothing.  (The Kimi-K3 shape, d = 7168, 896 experts, top-16,
 *     f = 1536, fits up to 216 tokens.)
 *   - Every call on one GPU uses that GPU's one array: calls that can
 *     overlap on one GPU (other streams, other host threads) race on it and
 *     must be serialised by the caller.  The array keeps the last call's
 *     contents; no kernel reads a byte of it that the same call has not
 *     written first, so nothing needs clearing between calls.
 *   - hip_stream must belong to the calling thread's current device
 *     (MOE_ERR_UNSUPPORTED otherwise).  The first call on a device looks up
 *     that device's address of the array (hipGetSymbolAddress, which
 *     allocates nothing).
 * Arguments, outputs, validation and the other conventions are those of
 * moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_dims *dims, const uint16_t *x,
                                     const uint16_t *router_w,
                                     const float *router_bias,
                                     const moe_mxfp4_experts *experts, uint16_t *y,
                                     int32_t *topk_ids_out, float *topk_w_out,
                                     void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_MXFP4_MOE_H */
