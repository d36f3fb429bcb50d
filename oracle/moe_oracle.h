/*
 * moe_oracle.h -- plain, slow, fp64 CPU reference of one routed
 * Mixture-of-Experts FFN layer whose experts are stored as MXFP4.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant with the GPU library, and the GPU library
 * never calls it.
 *
 * Every array is row-major, host memory, owned by the caller.  "bf16" means
 * the upper 16 bits of an IEEE binary32, carried in a uint16_t.
 *
 * Expert weight layout (per expert e, K contiguous within a row):
 *   gu_codes  [E][2f][d/2]  E2M1 codes, element 2i in the low nibble of byte i
 *   gu_scales [E][2f][d/32] E8M0 codes, one per 32 consecutive K elements
 *   dn_codes  [E][d][f/2]
 *   dn_scales [E][d][f/32]
 *   gate = rows [0, f) of gu, up = rows [f, 2f).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar formats ---------------------------------------------------- */
double   orc_bf16_value(uint16_t bits);
double   orc_e2m1_value(unsigned code);            /* 4-bit code          */
double   orc_e8m0_value(unsigned code);            /* 8-bit code, 255=NaN */
uint16_t orc_round_to_bf16(double v);              /* RNE, fp64 -> bf16   */
double   orc_mxfp4_weight(const uint8_t *codes, const uint8_t *scales,
                          int K, int row, int col);

/* ---- router ------------------------------------------------------------ */
void orc_router_logits(int T, int d, int E, const uint16_t *x,
                       const uint16_t *router_w, const float *bias,
                       float *logits);
void orc_topk_softmax(int T, int E, int k, const float *logits,
                      int32_t *topk_ids, double *topk_w);

/* ---- grouping rows by expert ------------------------------------------- */
void orc_permute(int T, int E, int k, const int32_t *topk_ids,
                 int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                 int32_t *row_pos);

/* ---- one routed expert applied to one token row ------------------------ */
void orc_expert_row(int d, int f, const uint16_t *x_row,
                    const uint8_t *gu_codes, const uint8_t *gu_scales,
                    const uint8_t *dn_codes, const uint8_t *dn_scales,
                    double *h, double *o);

/* act = 1, the activation-MX mode: x and h each rounded to one MX E2M3 term
 * per 32 elements (orc_mx_round) before their products; h returns the
 * rounded values.  act = 0 is orc_expert_row. */
void orc_expert_row_act(int d, int f, int act, const uint16_t *x_row,
                        const uint8_t *gu_codes, const uint8_t *gu_scales,
                        const uint8_t *dn_codes, const uint8_t *dn_scales,
                        double *h, double *o);

/* ---- weighted combine of one token's k expert outputs ------------------ */
void orc_combine_token(int d, int k, const double *w, const double *o,
                       double *y64, uint16_t *y_bf16);

/* ---- whole layer, for configurations small enough to run in full ------- */
int orc_layer_forward(int T, int d, int E, int k, int f, const uint16_t *x,
                      const uint16_t *router_w, const float *bias,
                      const uint8_t *gu_codes, const uint8_t *gu_scales,
                      const uint8_t *dn_codes, const uint8_t *dn_scales,
                      float *logits, int32_t *topk_ids, double *topk_w,
                      double *y64, uint16_t *y_bf16, int n_threads);

/* The same layer with the expert rows in activation mode act (above). */
int orc_layer_forward_act(int T, int d, int E, int k, int f, int act, const uint16_t *x,
                          const uint16_t *router_w, const float *bias,
                          const uint8_t *gu_codes, const uint8_t *gu_scales,
                          const uint8_t *dn_codes, const uint8_t *dn_scales,
                          float *logits, int32_t *topk_ids, double *topk_w,
                          double *y64, uint16_t *y_bf16, int n_threads);

/* ---- MoE tail (pre-norm block around the routed layer) ---------------- */
/* xn = bf16((x / sqrt(ss/d + eps)) * gamma) with ss the canonical chunked
 * fp64 sum of squares (the router's order). */
void orc_rmsnorm(int T, int d, const uint16_t *x, const uint16_t *gamma, float eps,
                 uint16_t *xn);
/* SwiGLU shared expert of width fs, bf16 weights sgu [2fs][d], sdn [d][fs]. */
void orc_shared_expert_row(int d, int fs, const uint16_t *xn_row, const uint16_t *sgu,
                           const uint16_t *sdn, double *h, double *o);
/* out = x + routed(xn) + shared(xn) (sgu NULL: no shared expert). */
int orc_block_forward(int T, int d, int E, int k, int f, int fs, const uint16_t *x,
                      const uint16_t *gamma, float eps, const uint16_t *router_w,
                      const float *bias, const uint8_t *gu_codes, const uint8_t *gu_scales,
                      const uint8_t *dn_codes, const uint8_t *dn_scales, const uint16_t *sgu,
                      const uint16_t *sdn, uint16_t *xn_out, float *logits,
                      int32_t *topk_ids, double *topk_w, double *out64, uint16_t *out_bf16,
                      int n_threads);

/* ---- FP8 experts: E4M3FN codes, fp32 scale per 128 x 128 block ---------
 * gu codes [E][2f][d], gu scales [E][2f/128][d/128]; dn codes [E][d][f],
 * dn scales [E][d/128][f/128] (d % 128 == 0, f % 128 == 0). */
double orc_fp8_weight(const uint8_t *codes, const float *scales, int K, int row, int col);
void orc_expert_row_fp8(int d, int f, const uint16_t *x_row, const uint8_t *gu_codes,
                        const float *gu_scales, const uint8_t *dn_codes,
                        const float *dn_scales, double *h, double *o);
int orc_layer_forward_fp8(int T, int d, int E, int k, int f, const uint16_t *x,
                          const uint16_t *router_w, const float *bias, const uint8_t *gu_codes,
                          const float *gu_scales, const uint8_t *dn_codes,
                          const float *dn_scales, float *logits, int32_t *topk_ids,
                          double *topk_w, double *y64, uint16_t *y_bf16, int n_threads);

/* ---- OCP MX conversion model (element formats below) ------------------- */
enum { ORC_FMT_E4M3 = 0, ORC_FMT_E2M3 = 1, ORC_FMT_E2M1 = 2 };
double orc_elem_value(int fmt, unsigned code);
void   orc_mx_quantize_block(int fmt, const double *v, uint8_t *scale_code,
                             uint8_t *codes);
/* v[0..n) (n a multiple of 32) rounded in place, block by block, to one MX
 * term of element format fmt. */
void   orc_mx_round(int fmt, int n, double *v);
void   orc_mx_split_block(int fmt, const float *v, uint8_t *hi_scale,
                          uint8_t *hi_codes, uint8_t *lo_scale,
                          uint8_t *lo_codes);

#ifdef __cplusplus
}
#endif
#endif
