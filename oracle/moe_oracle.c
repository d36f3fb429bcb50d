/*
 * moe_oracle.c -- plain fp64 CPU reference of one routed MoE FFN layer with
 * MXFP4 experts.  TEST INFRASTRUCTURE ONLY (see moe_oracle.h).
 *
 * What the layer computes, and where it comes from:
 *   - A router on the requesting side scores every expert for each token and
 *     the routed expert FFN is the unit that runs elsewhere (MoonTail README,
 *     requester / volunteer table).
 *   - Each routed layer picks 16 of 896 experts per token (Moonshine README,
 *     "How the engine works"; MoonTail README, opening description).
 *   - Routed experts are stored as MXFP4; a decoded expert occupies
 *     16.734 MiB and the canonical store is 1,446,456,066,048 B for 82,432
 *     experts (Moonshine README, GitHub mirror, "Expert-stream compression",
 *     "MZG2 production store").  Both fix 17,547,264 B per expert, i.e.
 *     three d x f matrices at 4.25 bits per element.
 *   - Prefill groups all token rows that select each expert and reads each
 *     selected expert once (Moonshine README, "How the engine works").
 *   - The MoE tail ends in a weighted reduction of the expert outputs
 *     (Moonshine README, "Run layer-major prefill").
 *
 * The pages leave open the router's summation order, the top-k tie rule, the
 * softmax scope, the expert nonlinearity and the nibble order.  Readings:
 *   - logits: the canonical chunked fp64 sum of orc_router_logits();
 *   - top-k: descending logit, equal logits -> lower expert index first;
 *   - weights: softmax over the k selected logits, no extra scaling;
 *   - expert: SwiGLU, h = silu(gate) * up, no biases, no clamp;
 *   - gate = rows [0,f), up = rows [f,2f); element 2i = low nibble of byte i.
 *
 * Element and scale formats follow the OCP Microscaling Formats (MX) v1.0
 * specification (E2M1 / E2M3 / E4M3 element types, E8M0 scale type, and
 * its conversion of a block of 32 values to MX).
 *
 * Build: cc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include "moe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================= */
/* Scalar formats                                                           */
/* ======================================================================= */

/* bf16 is the upper half of an IEEE binary32: widen and reinterpret. */
double orc_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 (OCP MX v1.0 FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
 * bit.  Exponent field 0 is subnormal: value 0.5 * m.  Otherwise
 * 2^(e-1) * (1 + m/2).  Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Code 8 is
 * negative zero, which the Moonshine MZG2 store calls redundant and
 * canonicalises -- it has the value 0. */
double orc_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u;
    unsigned e = (code >> 1) & 3u;
    unsigned m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m
                          : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0 (OCP MX v1.0 scale): 2^(code - 127); code 255 is NaN. */
double orc_e8m0_value(unsigned code)
{
    if ((code & 0xFFu) == 255u)
        return NAN;
    return ldexp(1.0, (int)(code & 0xFFu) - 127);
}

/* Round an fp64 value to the nearest bf16, ties to even, directly from fp64
 * (no intermediate fp32 rounding).  bf16 keeps 8 significant bits, shares
 * fp32's exponent range, and its subnormals are spaced 2^-133 apart. */
uint16_t orc_round_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e;
    frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1)          */
    int qexp = e - 8;             /* spacing of 8-significant-bit values */
    if (qexp < -133)
        qexp = -133;              /* subnormal spacing                   */
    double q = ldexp(1.0, qexp);
    double r = nearbyint(a / q) * q;  /* a/q is exact; nearbyint is RNE   */
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r;          /* exact: r has <= 8 significant bits  */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* One dequantised MXFP4 weight: element (row, col) of a [rows][K] matrix
 * whose codes are packed two per byte (even column in the low nibble) and
 * whose E8M0 scale covers 32 consecutive columns.  The product is exact in
 * fp64. */
double orc_mxfp4_weight(const uint8_t *codes, const uint8_t *scales, int K,
                        int row, int col)
{
    uint8_t byte = codes[(size_t)row * (size_t)(K / 2) + (size_t)(col / 2)];
    unsigned code = (col & 1) ? (byte >> 4) : (byte & 0x0Fu);
    uint8_t sc = scales[(size_t)row * (size_t)(K / 32) + (size_t)(col / 32)];
    return orc_e2m1_value(code) * orc_e8m0_value(sc);
}

/* ======================================================================= */
/* Router                                                                   */
/* ======================================================================= */

/* Canonical router logit (the pages name the router but not its arithmetic;
 * this fixes one deterministic summation order so that expert selection can
 * be reproduced bit for bit):
 *   1. split the d inputs into 64 equal contiguous chunks;
 *   2. sum each chunk in fp64 in ascending k (every bf16*bf16 product is
 *      exact in fp64);
 *   3. combine the 64 chunk sums with a fixed pairwise tree, level by level:
 *      (0,1),(2,3),... then ((0,1),(2,3)),... ;
 *   4. add the bias (0 when absent) in fp64;
 *   5. round once to fp32 (round to nearest even).
 * Requires d % 64 == 0. */
void orc_router_logits(int T, int d, int E, const uint16_t *x,
                       const uint16_t *router_w, const float *bias,
                       float *logits)
{
    const int P = d / 64;
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double part[64];
            for (int c = 0; c < 64; ++c) {
                double s = 0.0;
                for (int i = 0; i < P; ++i) {
                    size_t kk = (size_t)c * P + (size_t)i;
                    double xv = orc_bf16_value(x[(size_t)t * d + kk]);
                    double wv = orc_bf16_value(router_w[(size_t)e * d + kk]);
                    s = s + xv * wv;
                }
                part[c] = s;
            }
            for (int width = 1; width < 64; width *= 2)
                for (int c = 0; c < 64; c += 2 * width)
                    part[c] = part[c] + part[c + width];
            double l = part[0] + (bias ? (double)bias[e] : 0.0);
            logits[(size_t)t * E + e] = (float)l;
        }
    }
}

/* Top-k and routing weights for each token.
 * Selection: repeatedly take the best remaining expert, where a larger logit
 * is better and, between equal logits, the lower expert index is better.
 * The k chosen experts come out in that order (descending logit).
 * Weights: softmax over the k selected logits in fp64,
 *   w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max),
 * with no further scaling.  Logits are assumed finite. */
void orc_topk_softmax(int T, int E, int k, const float *logits,
                      int32_t *topk_ids, double *topk_w)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;     /* strict '>' keeps the lower index on ties */
            }
            taken[best] = 1;
            topk_ids[(size_t)t * k + j] = best;
        }
        double lmax = (double)l[topk_ids[(size_t)t * k]];
        double denom = 0.0;
        for (int j = 0; j < k; ++j)
            denom += exp((double)l[topk_ids[(size_t)t * k + j]] - lmax);
        for (int j = 0; j < k; ++j)
            topk_w[(size_t)t * k + j] =
                exp((double)l[topk_ids[(size_t)t * k + j]] - lmax) / denom;
    }
    free(taken);
}

/* ======================================================================= */
/* Grouping rows by expert (layer-major plan)                               */
/* ======================================================================= */

/* Each (token t, slot j) pair is one row, numbered t*k + j.  Rows are grouped
 * by expert in ascending expert order, and inside an expert's group they keep
 * ascending row number -- a stable grouping.  counts[e] is the group size,
 * offsets[e] its start (offsets[E] = T*k), sorted_rows the grouped row
 * numbers and row_pos the inverse map (row number -> position). */
void orc_permute(int T, int E, int k, const int32_t *topk_ids,
                 int32_t *counts, int32_t *offsets, int32_t *sorted_rows,
                 int32_t *row_pos)
{
    int32_t n = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = n;
        int32_t c = 0;
        for (int t = 0; t < T; ++t) {
            for (int j = 0; j < k; ++j) {
                int32_t r = t * k + j;
                if (topk_ids[r] == e) {
                    sorted_rows[n] = r;
                    row_pos[r] = n;
                    ++n;
                    ++c;
                }
            }
        }
        counts[e] = c;
    }
    offsets[E] = n;
}

/* ======================================================================= */
/* One routed expert on one token row                                       */
/* ======================================================================= */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Each consecutive 32-element block of v[0..n) replaced, in place, by its
 * single-term MX value in element format fmt: the block quantised with
 * orc_mx_quantize_block and decoded exactly.  n is a multiple of 32. */
void orc_mx_round(int fmt, int n, double *v)
{
    for (int b = 0; b < n; b += 32) {
        uint8_t sc, codes[32];
        orc_mx_quantize_block(fmt, v + b, &sc, codes);
        double s = orc_e8m0_value(sc);
        for (int i = 0; i < 32; ++i)
            v[b + i] = orc_elem_value(fmt, codes[i]) * s;
    }
}

/* h[n] = silu(g_n) * u_n with g_n = sum_k x_k W_gu[n][k] and
 * u_n = sum_k x_k W_gu[f+n][k]; then o[m] = sum_n h_n W_dn[m][n].
 * All in fp64 with exact dequantised weights and exact bf16 inputs.
 * act = 1 (the activation-MX mode): x is rounded to one MX E2M3 term per
 * 32 elements before the gate/up products and h likewise before the down
 * products; h then returns the rounded values. */
static void expert_row_impl(int d, int f, int act, const uint16_t *x_row,
                            const uint8_t *gu_codes, const uint8_t *gu_scales,
                            const uint8_t *dn_codes, const uint8_t *dn_scales,
                            double *h, double *o)
{
    double *xv = (double *)malloc(sizeof(double) * (size_t)d);
    for (int kk = 0; kk < d; ++kk)
        xv[kk] = orc_bf16_value(x_row[kk]);
    if (act)
        orc_mx_round(ORC_FMT_E2M3, d, xv);
    for (int n = 0; n < f; ++n) {
        double g = 0.0, u = 0.0;
        for (int kk = 0; kk < d; ++kk) {
            g = g + xv[kk] * orc_mxfp4_weight(gu_codes, gu_scales, d, n, kk);
            u = u + xv[kk] * orc_mxfp4_weight(gu_codes, gu_scales, d, f + n, kk);
        }
        h[n] = silu(g) * u;
    }
    free(xv);
    if (act)
        orc_mx_round(ORC_FMT_E2M3, f, h);
    for (int m = 0; m < d; ++m) {
        double s = 0.0;
        for (int n = 0; n < f; ++n)
            s = s + h[n] * orc_mxfp4_weight(dn_codes, dn_scales, f, m, n);
        o[m] = s;
    }
}

void orc_expert_row(int d, int f, const uint16_t *x_row,
                    const uint8_t *gu_codes, const uint8_t *gu_scales,
                    const uint8_t *dn_codes, const uint8_t *dn_scales,
                    double *h, double *o)
{
    expert_row_impl(d, f, 0, x_row, gu_codes, gu_scales, dn_codes, dn_scales, h, o);
}

void orc_expert_row_act(int d, int f, int act, const uint16_t *x_row,
                        const uint8_t *gu_codes, const uint8_t *gu_scales,
                        const uint8_t *dn_codes, const uint8_t *dn_scales,
                        double *h, double *o)
{
    expert_row_impl(d, f, act, x_row, gu_codes, gu_scales, dn_codes, dn_scales, h, o);
}

/* ======================================================================= */
/* Weighted combine                                                         */
/* ======================================================================= */

/* y[m] = sum_j w_j * o_j[m] in fp64, in slot order j = 0..k-1, then rounded
 * once to bf16.  o is [k][d]. */
void orc_combine_token(int d, int k, const double *w, const double *o,
                       double *y64, uint16_t *y_bf16)
{
    for (int m = 0; m < d; ++m) {
        double s = 0.0;
        for (int j = 0; j < k; ++j)
            s = s + w[j] * o[(size_t)j * d + m];
        if (y64)
            y64[m] = s;
        if (y_bf16)
            y_bf16[m] = orc_round_to_bf16(s);
    }
}

/* ======================================================================= */
/* Whole layer                                                              */
/* ======================================================================= */

/* router -> top-k -> per-row expert FFN -> combine, token by token.
 * Returns 0, or -1 when the scratch allocation fails.  Rows are independent,
 * so they are spread over n_threads OpenMP threads (<= 0: runtime default).
 * act selects the expert rows' activation mode (see expert_row_impl); the
 * router always sees x as given. */
static int layer_forward_impl(int T, int d, int E, int k, int f, int act, const uint16_t *x,
                              const uint16_t *router_w, const float *bias,
                              const uint8_t *gu_codes, const uint8_t *gu_scales,
                              const uint8_t *dn_codes, const uint8_t *dn_scales,
                              float *logits, int32_t *topk_ids, double *topk_w,
                              double *y64, uint16_t *y_bf16, int n_threads)
{
    size_t gu_code_b = (size_t)2 * f * (d / 2), gu_sc_b = (size_t)2 * f * (d / 32);
    size_t dn_code_b = (size_t)d * (f / 2), dn_sc_b = (size_t)d * (f / 32);
    double *o = (double *)malloc(sizeof(double) * (size_t)T * k * d);
    if (!o)
        return -1;
    orc_router_logits(T, d, E, x, router_w, bias, logits);
    orc_topk_softmax(T, E, k, logits, topk_ids, topk_w);
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
    int rows = T * k;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int r = 0; r < rows; ++r) {
        double *h = (double *)malloc(sizeof(double) * (size_t)f);
        int t = r / k;
        size_t e = (size_t)topk_ids[r];
        expert_row_impl(d, f, act, x + (size_t)t * d, gu_codes + e * gu_code_b,
                        gu_scales + e * gu_sc_b, dn_codes + e * dn_code_b,
                        dn_scales + e * dn_sc_b, h, o + (size_t)r * d);
        free(h);
    }
    for (int t = 0; t < T; ++t)
        orc_combine_token(d, k, topk_w + (size_t)t * k, o + (size_t)t * k * d,
                          y64 ? y64 + (size_t)t * d : NULL,
                          y_bf16 ? y_bf16 + (size_t)t * d : NULL);
    free(o);
    return 0;
}

int orc_layer_forward(int T, int d, int E, int k, int f, const uint16_t *x,
                      const uint16_t *router_w, const float *bias,
                      const uint8_t *gu_codes, const uint8_t *gu_scales,
                      const uint8_t *dn_codes, const uint8_t *dn_scales,
                      float *logits, int32_t *topk_ids, double *topk_w,
                      double *y64, uint16_t *y_bf16, int n_threads)
{
    return layer_forward_impl(T, d, E, k, f, 0, x, router_w, bias, gu_codes, gu_scales,
                              dn_codes, dn_scales, logits, topk_ids, topk_w, y64, y_bf16,
                              n_threads);
}

int orc_layer_forward_act(int T, int d, int E, int k, int f, int act, const uint16_t *x,
                          const uint16_t *router_w, const float *bias,
                          const uint8_t *gu_codes, const uint8_t *gu_scales,
                          const uint8_t *dn_codes, const uint8_t *dn_scales,
                          float *logits, int32_t *topk_ids, double *topk_w,
                          double *y64, uint16_t *y_bf16, int n_threads)
{
    return layer_forward_impl(T, d, E, k, f, act, x, router_w, bias, gu_codes, gu_scales,
                              dn_codes, dn_scales, logits, topk_ids, topk_w, y64, y_bf16,
                              n_threads);
}

/* ======================================================================= */
/* OCP MX conversion model                                                  */
/* ======================================================================= */

/* Element formats of the OCP MX v1.0 specification used here:
 *   E4M3 (FP8): bias 7, largest normal exponent 8, max 448, no infinity;
 *   E2M3 (FP6): bias 1, largest normal exponent 2, max 7.5;
 *   E2M1 (FP4): bias 1, largest normal exponent 2, max 6.
 * All have subnormals (exponent field 0). */
typedef struct {
    int ebits, mbits, bias, emax;
    double maxval;
} orc_fmt;

static orc_fmt fmt_of(int fmt)
{
    orc_fmt F;
    switch (fmt) {
    case ORC_FMT_E4M3: F.ebits = 4; F.mbits = 3; F.bias = 7; F.emax = 8; F.maxval = 448.0; break;
    case ORC_FMT_E2M3: F.ebits = 2; F.mbits = 3; F.bias = 1; F.emax = 2; F.maxval = 7.5; break;
    default:           F.ebits = 2; F.mbits = 1; F.bias = 1; F.emax = 2; F.maxval = 6.0; break;
    }
    return F;
}

/* Value of an element code (no scale applied). */
double orc_elem_value(int fmt, unsigned code)
{
    orc_fmt F = fmt_of(fmt);
    unsigned nb = (unsigned)(1 + F.ebits + F.mbits);
    unsigned s = (code >> (nb - 1)) & 1u;
    unsigned e = (code >> F.mbits) & ((1u << F.ebits) - 1u);
    unsigned m = code & ((1u << F.mbits) - 1u);
    double frac = (double)m / (double)(1u << F.mbits);
    double mag = (e == 0) ? ldexp(frac, 1 - F.bias)
                          : ldexp(1.0 + frac, (int)e - F.bias);
    if (fmt == ORC_FMT_E4M3 && e == 15u && m == 7u)
        mag = NAN;               /* E4M3's only NaN encoding */
    return s ? -mag : mag;
}

/* Round r (already divided by the block scale) to the element format:
 * round to nearest, ties to even, with subnormals; magnitudes beyond the
 * format's largest value saturate to it.  The sign of the code is the sign
 * of r (so a negative value that rounds to zero gives negative zero). */
static unsigned encode_elem(const orc_fmt *F, double r)
{
    unsigned s = signbit(r) ? 1u : 0u;
    double a = fabs(r);
    int emin = 1 - F->bias;              /* smallest normal exponent */
    double v;
    if (a >= F->maxval) {
        v = F->maxval;
    } else {
        int e = emin;
        if (a > 0.0) {
            int fe;
            frexp(a, &fe);               /* a in [2^(fe-1), 2^fe) */
            e = fe - 1;
            if (e < emin)
                e = emin;
        }
        double q = ldexp(1.0, e - F->mbits);
        v = nearbyint(a / q) * q;     /* a < maxval, a grid point: v <= maxval */
    }
    unsigned field, mant;
    if (v < ldexp(1.0, emin)) {          /* subnormal (or zero) */
        field = 0;
        mant = (unsigned)(v / ldexp(1.0, emin - F->mbits));
    } else {
        int fe;
        frexp(v, &fe);
        int e = fe - 1;
        field = (unsigned)(e + F->bias);
        mant = (unsigned)((v / ldexp(1.0, e) - 1.0) * (double)(1u << F->mbits));
    }
    return (s << (F->ebits + F->mbits)) | (field << F->mbits) | mant;
}

/* OCP MX conversion of one block of 32 values: the shared exponent is
 * X = floor(log2(max |v_i|)) - emax_elem, clamped to [-127, 127] and stored
 * as the E8M0 code X + 127; every element is v_i / 2^X rounded to the
 * element format (round to nearest even, saturating).  An all-zero block
 * gets scale code 0 and zero elements.  Inputs must be finite. */
void orc_mx_quantize_block(int fmt, const double *v, uint8_t *scale_code,
                           uint8_t *codes)
{
    orc_fmt F = fmt_of(fmt);
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    int X = -127;
    if (amax > 0.0) {
        int fe;
        frexp(amax, &fe);                /* amax in [2^(fe-1), 2^fe) */
        X = (fe - 1) - F.emax;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    *scale_code = (uint8_t)(X + 127);
    for (int i = 0; i < 32; ++i)
        codes[i] = (uint8_t)encode_elem(&F, ldexp(v[i], -X));
}

/* Two-term split of a block: hi = MX(v), lo = MX(v - hi).  v - hi is exact
 * (it is formed in fp64 from fp32 inputs). */
void orc_mx_split_block(int fmt, const float *v, uint8_t *hi_scale,
                        uint8_t *hi_codes, uint8_t *lo_scale,
                        uint8_t *lo_codes)
{
    double a[32], r[32];
    for (int i = 0; i < 32; ++i)
        a[i] = (double)v[i];
    orc_mx_quantize_block(fmt, a, hi_scale, hi_codes);
    double s = orc_e8m0_value(*hi_scale);
    for (int i = 0; i < 32; ++i)
        r[i] = a[i] - orc_elem_value(fmt, hi_codes[i]) * s;
    orc_mx_quantize_block(fmt, r, lo_scale, lo_codes);
}

/* ======================================================================= */
/* MoE tail: RMSNorm before the router, the shared expert, residual add     */
/* ======================================================================= */

/* The pages' profile of the model-shape MoE tail names its steps: the
 * weighted reduction, RMSNorm, the routed-up activation quantisation and
 * the residual adds (Moonshine README, "Run layer-major prefill"); shared
 * experts and norms sit in the Q8/BF16 static tier next to the routers,
 * apart from the MXFP4 routed experts (Moonshine README, "How the engine
 * works", tier diagram).  Readings where the pages are silent:
 *   - pre-norm block: xn = RMSNorm(x) * gamma feeds both the router and the
 *     experts, out = x + routed(xn) + shared(xn);
 *   - RMSNorm: ss = sum of x_i^2 in the router's canonical order (64 equal
 *     chunks summed in ascending order, chunk sums combined by the fixed
 *     pairwise tree), ms = ss / d, den = sqrt(ms + eps), then
 *     xn_i = bf16((x_i / den) * gamma_i), every step one IEEE fp64 operation
 *     and the last rounding straight from fp64 to bf16 (RNE).  A fixed order
 *     makes xn, and hence the routing, reproducible bit for bit;
 *   - shared expert: one SwiGLU MLP of width fs with bf16 weights, gate =
 *     rows [0, fs) and up = rows [fs, 2fs) of sgu [2fs][d], down sdn [d][fs];
 *     always applied with weight 1, no biases;
 *   - out = x + y + s summed in fp64 (y the routed weighted sum, s the shared
 *     expert's output), rounded once to bf16. */
void orc_rmsnorm(int T, int d, const uint16_t *x, const uint16_t *gamma, float eps,
                 uint16_t *xn)
{
    const int P = d / 64;
    for (int t = 0; t < T; ++t) {
        const uint16_t *xr = x + (size_t)t * d;
        double part[64];
        for (int c = 0; c < 64; ++c) {
            double s = 0.0;
            for (int i = 0; i < P; ++i) {
                double v = orc_bf16_value(xr[(size_t)c * P + (size_t)i]);
                s = s + v * v;
            }
            part[c] = s;
        }
        for (int width = 1; width < 64; width *= 2)
            for (int c = 0; c < 64; c += 2 * width)
                part[c] = part[c] + part[c + width];
        double ms = part[0] / (double)d;
        double den = sqrt(ms + (double)eps);
        for (int i = 0; i < d; ++i) {
            double v = (orc_bf16_value(xr[i]) / den) * orc_bf16_value(gamma[i]);
            xn[(size_t)t * d + i] = orc_round_to_bf16(v);
        }
    }
}

/* The shared expert on one normalised row: h_n = silu(g_n) * u_n with
 * g_n = sum_k xn_k sgu[n][k], u_n = sum_k xn_k sgu[fs+n][k], then
 * o[m] = sum_n h_n sdn[m][n]; fp64 with exact bf16 weights. */
void orc_shared_expert_row(int d, int fs, const uint16_t *xn_row, const uint16_t *sgu,
                           const uint16_t *sdn, double *h, double *o)
{
    for (int n = 0; n < fs; ++n) {
        double g = 0.0, u = 0.0;
        for (int kk = 0; kk < d; ++kk) {
            double xv = orc_bf16_value(xn_row[kk]);
            g = g + xv * orc_bf16_value(sgu[(size_t)n * d + kk]);
            u = u + xv * orc_bf16_value(sgu[(size_t)(fs + n) * d + kk]);
        }
        h[n] = silu(g) * u;
    }
    for (int m = 0; m < d; ++m) {
        double s = 0.0;
        for (int n = 0; n < fs; ++n)
            s = s + h[n] * orc_bf16_value(sdn[(size_t)m * fs + n]);
        o[m] = s;
    }
}

/* The block: xn = RMSNorm(x) * gamma; the routed layer on xn (router, top-k,
 * experts, weighted combine, all as orc_layer_forward); the shared expert on
 * xn (skipped when sgu is NULL, i.e. s = 0); out = x + y + s in fp64, then
 * bf16.  xn_out, logits, topk_ids, topk_w and out64 are outputs as well.
 * Returns 0, or -1 when a scratch allocation fails. */
int orc_block_forward(int T, int d, int E, int k, int f, int fs, const uint16_t *x,
                      const uint16_t *gamma, float eps, const uint16_t *router_w,
                      const float *bias, const uint8_t *gu_codes, const uint8_t *gu_scales,
                      const uint8_t *dn_codes, const uint8_t *dn_scales, const uint16_t *sgu,
                      const uint16_t *sdn, uint16_t *xn_out, float *logits,
                      int32_t *topk_ids, double *topk_w, double *out64, uint16_t *out_bf16,
                      int n_threads)
{
    double *y = (double *)malloc(sizeof(double) * (size_t)T * d);
    if (!y)
        return -1;
    orc_rmsnorm(T, d, x, gamma, eps, xn_out);
    if (layer_forward_impl(T, d, E, k, f, 0, xn_out, router_w, bias, gu_codes, gu_scales,
                           dn_codes, dn_scales, logits, topk_ids, topk_w, y, NULL,
                           n_threads) != 0) {
        free(y);
        return -1;
    }
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int t = 0; t < T; ++t) {
        double *s = (double *)calloc((size_t)d, sizeof(double));
        double *h = (double *)malloc(sizeof(double) * (size_t)(fs > 0 ? fs : 1));
        if (!s || !h) {
#pragma omp atomic write
            failed = 1;
        } else {
            if (sgu)
                orc_shared_expert_row(d, fs, xn_out + (size_t)t * d, sgu, sdn, h, s);
            for (int m = 0; m < d; ++m) {
                size_t i = (size_t)t * d + m;
                double v = orc_bf16_value(x[i]) + y[i] + s[m];
                if (out64)
                    out64[i] = v;
                if (out_bf16)
                    out_bf16[i] = orc_round_to_bf16(v);
            }
        }
        free(s);
        free(h);
    }
    free(y);
    return failed ? -1 : 0;
}

/* ======================================================================= */
/* FP8 experts (E4M3FN codes, fp32 scale per 128 x 128 block)              */
/* ======================================================================= */

/* The pages' FP8 lane is an exhaustive OCP E4M3FN oracle, a fused GEMV and
 * a bounded BF16-dequant prefill floor (Moonshine README, "GLM 5.3 Flash
 * status").  They do not print the scale layout; the reading here is the
 * block-scaled layout of official FP8 checkpoints: one fp32 scale per
 * 128 x 128 block of each [rows][K] matrix, multiplying the decoded code.
 * E4M3FN is the OCP 8-bit E4M3 format (bias 7, no infinities, S.1111.111 is
 * NaN, largest finite 448): the E4M3 element type of orc_elem_value.
 *
 * Layout per expert (K contiguous):
 *   gu codes [2f][d], gu scales [2f/128][d/128]; dn codes [d][f],
 *   dn scales [d/128][f/128]; gate = rows [0, f), up = rows [f, 2f). */
double orc_fp8_weight(const uint8_t *codes, const float *scales, int K, int row, int col)
{
    double v = orc_elem_value(ORC_FMT_E4M3, codes[(size_t)row * K + col]);
    return v * (double)scales[(size_t)(row / 128) * (size_t)(K / 128) + (size_t)(col / 128)];
}

/* The SwiGLU expert of expert_row_impl with FP8 weights (fp64, exact
 * dequantised weights, exact bf16 inputs). */
void orc_expert_row_fp8(int d, int f, const uint16_t *x_row, const uint8_t *gu_codes,
                        const float *gu_scales, const uint8_t *dn_codes,
                        const float *dn_scales, double *h, double *o)
{
    for (int n = 0; n < f; ++n) {
        double g = 0.0, u = 0.0;
        for (int kk = 0; kk < d; ++kk) {
            double xv = orc_bf16_value(x_row[kk]);
            g = g + xv * orc_fp8_weight(gu_codes, gu_scales, d, n, kk);
            u = u + xv * orc_fp8_weight(gu_codes, gu_scales, d, f + n, kk);
        }
        h[n] = silu(g) * u;
    }
    for (int m = 0; m < d; ++m) {
        double s = 0.0;
        for (int n = 0; n < f; ++n)
            s = s + h[n] * orc_fp8_weight(dn_codes, dn_scales, f, m, n);
        o[m] = s;
    }
}

/* The layer of orc_layer_forward with FP8 experts: router, top-k, the FP8
 * expert rows, weighted combine.  Returns 0, or -1 when scratch allocation
 * fails. */
int orc_layer_forward_fp8(int T, int d, int E, int k, int f, const uint16_t *x,
                          const uint16_t *router_w, const float *bias, const uint8_t *gu_codes,
                          const float *gu_scales, const uint8_t *dn_codes,
                          const float *dn_scales, float *logits, int32_t *topk_ids,
                          double *topk_w, double *y64, uint16_t *y_bf16, int n_threads)
{
    size_t gu_code_b = (size_t)2 * f * d, gu_sc_n = (size_t)(2 * f / 128) * (d / 128);
    size_t dn_code_b = (size_t)d * f, dn_sc_n = (size_t)(d / 128) * (f / 128);
    double *o = (double *)malloc(sizeof(double) * (size_t)T * k * d);
    if (!o)
        return -1;
    orc_router_logits(T, d, E, x, router_w, bias, logits);
    orc_topk_softmax(T, E, k, logits, topk_ids, topk_w);
    int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
    int rows = T * k;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int r = 0; r < rows; ++r) {
        double *h = (double *)malloc(sizeof(double) * (size_t)f);
        if (!h) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        int t = r / k;
        size_t e = (size_t)topk_ids[r];
        orc_expert_row_fp8(d, f, x + (size_t)t * d, gu_codes + e * gu_code_b,
                           gu_scales + e * gu_sc_n, dn_codes + e * dn_code_b,
                           dn_scales + e * dn_sc_n, h, o + (size_t)r * d);
        free(h);
    }
    if (!failed)
        for (int t = 0; t < T; ++t)
            orc_combine_token(d, k, topk_w + (size_t)t * k, o + (size_t)t * k * d,
                              y64 ? y64 + (size_t)t * d : NULL,
                              y_bf16 ? y_bf16 + (size_t)t * d : NULL);
    free(o);
    return failed ? -1 : 0;
}
