/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU reference for the weight-only decode projections:
 * the MXFP4 gate/up matvec fused with SwiGLU and a per-row postscale, its
 * top-k routed-expert (MoE) variant with an MXFP4 down projection and a
 * weighted combine, and the grouped affine INT4 matvec.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product (the HIP library) never calls it and
 * shares no code, header, table or constant with it.
 *
 * Form: every weight is decoded from its bit fields by the format's own
 * definition, rounded once to fp32, and every dot product is taken naively,
 * products and sums in fp64, one row at a time.
 *
 * Sources (the pages are the ThinTensor developer logs):
 *   [DL4]  page kerbin.cskartikey.dev/@satvikhardat, "Dev Log #4 -- 91-96
 *          tok/s with Selective MXFP4", sections "Why this was not just normal
 *          quantization" (MXFP4 on gate/up, row postscale enabled) and "Where
 *          Blackwell helps" (the projection reads 4-bit codes under block
 *          scales, takes bf16 activations, sums without losing precision and
 *          multiplies each finished row sum by its postscale).
 *   [DL3]  same page, "Dev Log #3 -- SmolLM3-3B Results": the scaled FP8
 *          matvec snippet multiplies the full row sum by the row scale.
 *   [DL2]  same page, "Dev Log #2 -- Converting SafeTensors Into .thin":
 *          dense MLPs need a gated activation; MoE models use router and
 *          expert stages.
 *   [P2]   page stardance.hackclub.com/projects/29750: "ThinTensor
 *          Improvements" (INT4 and MXFP4 quantizers, exact routing),
 *          "numerical drift & speedups" (selected-expert MXFP4 matvec,
 *          dense INT4 Q/K/V/O), "Implemented a huge list of fixes" (affine
 *          INT4 with a partial last group).
 *   [OCP FP8] OCP 8-bit Floating Point Specification (OFP8): the E4M3
 *          encoding (bias 7, no infinities, S.1111.111 = NaN).  The pages
 *          say "FP8" only; E4M3 is the reading taken for weights.
 *   [OCP]  OCP Microscaling Formats (MX) Specification v1.0: the FP4 E2M1
 *          element (1 sign, 2 exponent bits with bias 1, 1 mantissa bit) and
 *          the E8M0 shared scale (2^(e-127), 0xFF = NaN), 32 elements per
 *          block.  The pages name MXFP4 but never spell the bit layout; this
 *          is the public definition of that name.
 *
 * Canonical (oracle-side) layouts, all row-major:
 *   MXFP4 matrix W[N][K]: codes u8[N][K/2] (element 2j in the low nibble of
 *     byte j, 2j+1 in the high nibble), scales u8[N][K/32] (E8M0, block b
 *     covers k in [32b, 32b+32)), postscale f32[N] (NULL = all ones).
 *   INT4 matrix W[N][K]: q u8[N][K/2] (same nibble order, values 0..15),
 *     s and z as IEEE binary16 bit patterns u16[N][G], G = ceil(K/group).
 *   Activations: bf16 bit patterns u16[B][K].
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes): E8M0 byte 0 is 2^-127 (not zero), 0xFF is NaN; code 8 is -0.0; the
 * postscale multiplies the full-K sum before the activation; the activation
 * is silu(gate)*up with no clamp; top-k ranks raw bf16 logits, ties to the
 * lower index, and the routing weights are the softmax of the k selected
 * logits; the routing weight multiplies each expert's down output; INT4 is
 * w = s*(q - z) over groups of consecutive k with a partial last group.
 */
#ifdef _OPENMP
#include <omp.h>
#endif
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element and scale formats                                           */
/* ------------------------------------------------------------------ */

/* FP4 E2M1 value of a 4-bit code [OCP]: bit 3 sign, bits 2..1 exponent
 * (bias 1), bit 0 mantissa; exponent field 0 is subnormal (0 or 0.5). */
double or_e2m1_value(int code)
{
    int sign = (code >> 3) & 1;
    int expo = (code >> 1) & 3;
    int mant = code & 1;
    double mag;
    if (expo == 0)
        mag = 0.5 * mant;
    else
        mag = ldexp(1.0 + 0.5 * mant, expo - 1);
    return sign ? -mag : mag;
}

/* E8M0 scale value [OCP]: 2^(e-127); the all-ones byte is NaN. */
double or_e8m0_value(int e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, e - 127);
}

/* One decoded MXFP4 weight: the exact product, rounded once to fp32. */
float or_mxfp4_weight(int code, int e)
{
    return (float)(or_e2m1_value(code) * or_e8m0_value(e));
}

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
double or_bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } c;
    c.u = (uint32_t)bits << 16;
    return (double)c.f;
}

/* IEEE binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits. */
double or_f16_value(uint16_t h)
{
    int sign = h >> 15;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + frac, expo - 25);
    return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even, and encode it. */
uint16_t or_f16_from_double(double v)
{
    uint16_t sign;
    double a, quantum, r;
    int ex, e;
    if (isnan(v))
        return 0x7E00;
    sign = signbit(v) ? 0x8000 : 0;
    a = fabs(v);
    /* 65504 is the largest finite value; the midpoint to the next step
     * (65536, which no longer fits) is 65520 and ties go to the even
     * neighbour, which is the overflow. */
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a == 0.0)
        return sign;
    frexp(a, &ex);          /* a in [2^(ex-1), 2^ex) */
    e = ex - 1;
    quantum = (e < -14) ? ldexp(1.0, -24) : ldexp(1.0, e - 10);
    r = rint(a / quantum) * quantum;   /* default mode: nearest, ties even */
    if (r == 0.0)
        return sign;
    frexp(r, &ex);
    e = ex - 1;
    if (e < -14)
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    return sign | (uint16_t)((e + 15) << 10)
                | (uint16_t)((int)(r / ldexp(1.0, e - 10)) - 1024);
}

/* ------------------------------------------------------------------ */
/* MXFP4 decode and matvec                                             */
/* ------------------------------------------------------------------ */

static int nibble(const uint8_t *row, int64_t k)
{
    uint8_t byte = row[k >> 1];
    return (k & 1) ? (byte >> 4) : (byte & 15);
}

/* Decode one row of an MXFP4 matrix to fp32. */
static void decode_mxfp4_row(const uint8_t *codes, const uint8_t *scales,
                             int64_t k, int64_t r, float *out)
{
    const uint8_t *crow = codes + r * (k / 2);
    const uint8_t *srow = scales + r * (k / 32);
    for (int64_t j = 0; j < k; ++j)
        out[j] = or_mxfp4_weight(nibble(crow, j), srow[j / 32]);
}

/* Decoded weights of a whole MXFP4 matrix, row-major fp32 [n][k]. */
void or_mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                         int64_t n, int64_t k, float *w)
{
    for (int64_t r = 0; r < n; ++r)
        decode_mxfp4_row(codes, scales, k, r, w + r * k);
}

/*
 * y[b][i] = ps[r] * sum_k w[r][k] * x[b][k] for r = rows[i] ([DL4]: block
 * scales inside the sum, the row postscale on the full sum, as the [DL3]
 * snippet does with its row scale).  S[b][i] = sum_k |ps[r] w[r][k] x[b][k]|
 * is the magnitude the tolerance is relative to.  rows == NULL means every
 * row (nrows must then be n).  S may be NULL.
 */
void or_mxfp4_gemv(const uint8_t *codes, const uint8_t *scales,
                   const float *ps, int64_t n, int64_t k,
                   const uint16_t *x, int64_t batch,
                   const int64_t *rows, int64_t nrows,
                   double *y, double *S)
{
    (void)n;
    /* Rows are independent; the timing build (-fopenmp) splits them over
     * threads, each row's sum keeping the same order, so both builds give
     * the same bits.  The plain build ignores the pragmas. */
#ifdef _OPENMP
#pragma omp parallel
#endif
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)k);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t r = rows ? rows[i] : i;
            double p = ps ? (double)ps[r] : 1.0;
            decode_mxfp4_row(codes, scales, k, r, w);
            for (int64_t b = 0; b < batch; ++b) {
                const uint16_t *xb = x + b * k;
                double acc = 0.0, mag = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    double t = (double)w[j] * or_bf16_value(xb[j]);
                    acc += t;
                    mag += fabs(t);
                }
                y[b * nrows + i] = p * acc;
                if (S)
                    S[b * nrows + i] = fabs(p) * mag;
            }
        }
        free(w);
    }
}

/* Threads the loops above run on (1 in the plain build). */
int or_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z)  ([DL2] gated activation). */
double or_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/*
 * Gate/up with SwiGLU: g = ps_g * (Wg x), u = ps_u * (Wu x), h = silu(g)*u,
 * for rows (output features) rows[i] of the intermediate dimension.
 * Outputs are [batch][nrows]; g, u, Sg, Su may be NULL.
 */
void or_mxfp4_gateup_swiglu(const uint8_t *g_codes, const uint8_t *g_scales,
                            const float *g_ps,
                            const uint8_t *u_codes, const uint8_t *u_scales,
                            const float *u_ps,
                            int64_t inter, int64_t hidden,
                            const uint16_t *x, int64_t batch,
                            const int64_t *rows, int64_t nrows,
                            double *h, double *g, double *u,
                            double *Sg, double *Su)
{
    size_t cnt = (size_t)(batch * nrows);
    double *gv = (double *)malloc(sizeof(double) * cnt);
    double *uv = (double *)malloc(sizeof(double) * cnt);
    double *sg = (double *)malloc(sizeof(double) * cnt);
    double *su = (double *)malloc(sizeof(double) * cnt);
    or_mxfp4_gemv(g_codes, g_scales, g_ps, inter, hidden, x, batch,
                  rows, nrows, gv, sg);
    or_mxfp4_gemv(u_codes, u_scales, u_ps, inter, hidden, x, batch,
                  rows, nrows, uv, su);
    for (size_t i = 0; i < cnt; ++i) {
        h[i] = or_silu(gv[i]) * uv[i];
        if (g) g[i] = gv[i];
        if (u) u[i] = uv[i];
        if (Sg) Sg[i] = sg[i];
        if (Su) Su[i] = su[i];
    }
    free(gv); free(uv); free(sg); free(su);
}

/* ------------------------------------------------------------------ */
/* Routed experts                                                      */
/* ------------------------------------------------------------------ */

/*
 * Top-k routing for one token per row of logits[batch][n_exp] (bf16):
 * repeatedly take the largest remaining logit, the lower index winning a
 * tie; the weights are the softmax of the k selected logits (the full
 * softmax renormalised over the selection -- the same numbers).
 */
void or_moe_route_topk(const uint16_t *logits, int64_t batch, int64_t n_exp,
                       int64_t topk, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)n_exp);
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *lb = logits + b * n_exp;
        double sel[64];
        double mx, den = 0.0;
        memset(taken, 0, (size_t)n_exp);
        for (int64_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < n_exp; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || or_bf16_value(lb[e]) > or_bf16_value(lb[best]))
                    best = e;
            }
            taken[best] = 1;
            ids[b * topk + j] = (int32_t)best;
            sel[j] = or_bf16_value(lb[best]);
        }
        mx = sel[0];
        for (int64_t j = 1; j < topk; ++j)
            if (sel[j] > mx) mx = sel[j];
        for (int64_t j = 0; j < topk; ++j)
            den += exp(sel[j] - mx);
        for (int64_t j = 0; j < topk; ++j)
            w[b * topk + j] = exp(sel[j] - mx) / den;
    }
    free(taken);
}

/*
 * Expert gate/up: for token b and slot j, h[b][j][:] is the gate/up SwiGLU
 * of expert ids[b][j] applied to x[b] ([P2] selected-expert matvec fused
 * with SwiGLU).  Banks hold n_exp experts back to back in the canonical
 * layout.  An id outside [0, n_exp) gives a NaN row.  Outputs are
 * [batch][topk][nrows]; Sg, Su may be NULL.
 */
void or_moe_gateup_swiglu(const uint8_t *g_codes, const uint8_t *g_scales,
                          const float *g_ps,
                          const uint8_t *u_codes, const uint8_t *u_scales,
                          const float *u_ps,
                          int64_t n_exp, int64_t inter, int64_t hidden,
                          const uint16_t *x, int64_t batch,
                          const int32_t *ids, int64_t topk,
                          const int64_t *rows, int64_t nrows,
                          double *h, double *Sg, double *Su)
{
    int64_t cstride = inter * (hidden / 2), sstride = inter * (hidden / 32);
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t j = 0; j < topk; ++j) {
            int64_t e = ids[b * topk + j];
            size_t o = (size_t)((b * topk + j) * nrows);
            if (e < 0 || e >= n_exp) {
                for (int64_t i = 0; i < nrows; ++i) {
                    h[o + i] = NAN;
                    if (Sg) Sg[o + i] = NAN;
                    if (Su) Su[o + i] = NAN;
                }
                continue;
            }
            or_mxfp4_gateup_swiglu(
                g_codes + e * cstride, g_scales + e * sstride,
                g_ps ? g_ps + e * inter : NULL,
                u_codes + e * cstride, u_scales + e * sstride,
                u_ps ? u_ps + e * inter : NULL,
                inter, hidden, x + b * hidden, 1, rows, nrows,
                h + o, NULL, NULL, Sg ? Sg + o : NULL, Su ? Su + o : NULL);
        }
    }
}

/*
 * Expert down projection and combine:
 *   y[b][r] = sum_j w[b][j] * ps_d[e][r] * sum_k Wd[e][r][k] * h[b][j][k],
 * e = ids[b][j], j taken in order.  h is [batch][topk][inter] (the values
 * the caller feeds the device path, converted exactly to double).
 * S[b][r] = sum_j |w[b][j]| * sum_k |ps_d Wd h|.  An id outside [0, n_exp)
 * makes the whole output row NaN.  Outputs are [batch][nrows].
 */
void or_moe_down_combine(const uint8_t *d_codes, const uint8_t *d_scales,
                         const float *d_ps,
                         int64_t n_exp, int64_t hidden, int64_t inter,
                         const double *h, const int32_t *ids, const double *w,
                         int64_t batch, int64_t topk,
                         const int64_t *rows, int64_t nrows,
                         double *y, double *S)
{
    int64_t cstride = hidden * (inter / 2), sstride = hidden * (inter / 32);
    float *wr = (float *)malloc(sizeof(float) * (size_t)inter);
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t r = rows ? rows[i] : i;
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < topk; ++j) {
                int64_t e = ids[b * topk + j];
                const double *hb = h + (b * topk + j) * inter;
                double wj = w[b * topk + j], p, dot = 0.0, dm = 0.0;
                if (e < 0 || e >= n_exp) {
                    acc = NAN;
                    mag = NAN;
                    continue;
                }
                p = d_ps ? (double)d_ps[e * hidden + r] : 1.0;
                decode_mxfp4_row(d_codes + e * cstride, d_scales + e * sstride,
                                 inter, r, wr);
                for (int64_t k = 0; k < inter; ++k) {
                    double t = (double)wr[k] * hb[k];
                    dot += t;
                    dm += fabs(t);
                }
                acc += wj * (p * dot);
                mag += fabs(wj) * fabs(p) * dm;
            }
            y[b * nrows + i] = acc;
            if (S)
                S[b * nrows + i] = mag;
        }
    }
    free(wr);
}

/* ------------------------------------------------------------------ */
/* FP8 row-scaled matvec                                               */
/* ------------------------------------------------------------------ */

/* FP8 E4M3 value of a byte [OCP FP8, the E4M3 encoding without
 * infinities]: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN. */
double or_fp8e4m3_value(int code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 15;
    int mant = code & 7;
    double mag;
    if (expo == 15 && mant == 7)
        return NAN;
    if (expo == 0)
        mag = ldexp(mant / 8.0, -6);
    else
        mag = ldexp(1.0 + mant / 8.0, expo - 7);
    return sign ? -mag : mag;
}

/*
 * Row-scaled FP8 matvec ([DL3], the scaled FP8 matvec of the quality FP8
 * profile: the row's sum of weight * activation, activations and scale in
 * fp32, times the row scale):
 *   y[b][r] = scale[r] * sum_k w[r][k] * x[b][k]
 * w: E4M3 bytes [n][k]; scale f32 [n] (NULL = ones); x: bf16 bit patterns
 * (x_f32 = 0) or fp32 (x_f32 = 1) [batch][k].  Products and sums in fp64,
 * one row at a time.  rows (NULL = all n) selects output rows; y and S are
 * [batch][nrows], S = |scale| * sum |w x| (the error scale of the sum).
 */
void or_fp8_gemv(const uint8_t *w, const float *scale, int64_t n, int64_t k,
                 const void *x, int x_f32, int64_t batch, const int64_t *rows,
                 int64_t nrows, double *y, double *S)
{
    int64_t m = rows ? nrows : n;
    double *xv = (double *)malloc((size_t)(batch * k) * sizeof(double));
    for (int64_t i = 0; i < batch * k; ++i)
        xv[i] = x_f32 ? (double)((const float *)x)[i]
                      : or_bf16_value(((const uint16_t *)x)[i]);
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t i = 0; i < m; ++i) {
            int64_t r = rows ? rows[i] : i;
            double sc = scale ? (double)scale[r] : 1.0, acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                double p = or_fp8e4m3_value(w[r * k + j]) * xv[b * k + j];
                acc += p;
                mag += fabs(p);
            }
            y[b * m + i] = sc * acc;
            if (S)
                S[b * m + i] = fabs(sc) * mag;
        }
    }
    free(xv);
}

/* ------------------------------------------------------------------ */
/* Single-token GQA attention                                          */
/* ------------------------------------------------------------------ */

/*
 * Single-token grouped-query attention over a bf16 KV cache ([DL3]: each
 * query head h reads kv head h / (hq / hkv); a score is the key . query dot
 * product times the scale; the attention output is the softmax-weighted sum
 * of the values over the T cached positions):
 *   s_t     = scale * sum_d K[g][t][d] q[h][d],    g = h / (hq / hkv)
 *   p_t     = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
 *   o[h][d] = sum_t p_t V[g][t][d]
 * q: bf16 [hq][d]; K, V: bf16, row t of kv head g at ((g * tcap) + t) * d;
 * everything in fp64.  out [hq][d]; A (NULL allowed) [hq][d] =
 * sum_t p_t |V[g][t][d]|; Smax (NULL allowed) [hq] = max_t scale *
 * sum_d |K q| (the error scales of the output and of the scores).
 */
void or_gqa_attention(const uint16_t *q, const uint16_t *K, const uint16_t *V,
                      int64_t hq, int64_t hkv, int64_t d, int64_t tcap,
                      int64_t T, double scale, double *out, double *A,
                      double *Smax)
{
    double *s = (double *)malloc((size_t)T * sizeof(double));
    double *mag = (double *)malloc((size_t)T * sizeof(double));
    for (int64_t h = 0; h < hq; ++h) {
        int64_t g = h / (hq / hkv);
        double m = -INFINITY, den = 0.0, smax = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const uint16_t *kr = K + (g * tcap + t) * d;
            double acc = 0.0, a = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                double pr = or_bf16_value(kr[j]) * or_bf16_value(q[h * d + j]);
                acc += pr;
                a += fabs(pr);
            }
            s[t] = scale * acc;
            mag[t] = fabs(scale) * a;
            if (s[t] > m)
                m = s[t];
            if (mag[t] > smax)
                smax = mag[t];
        }
        for (int64_t t = 0; t < T; ++t)
            den += exp(s[t] - m);
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0, a = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double p = exp(s[t] - m) / den;
                double v = or_bf16_value(V[(g * tcap + t) * d + j]);
                acc += p * v;
                a += p * fabs(v);
            }
            out[h * d + j] = acc;
            if (A)
                A[h * d + j] = a;
        }
        if (Smax)
            Smax[h] = smax;
    }
    free(s);
    free(mag);
}

/* ------------------------------------------------------------------ */
/* MXFP4 quantizer                                                     */
/* ------------------------------------------------------------------ */

/* Nearest E2M1 code (magnitude index 0..7) of a >= 0: ties go to the even
 * index, magnitudes at or above 6 clamp to 6 [OCP, conversion of a vector
 * of scalars to an MX block: round to nearest even, clamp to the largest
 * normal element]. */
static int e2m1_nearest_index(double a)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (a >= 6.0)
        return 7;
    for (int i = 0; i < 7; ++i) {
        if (a < grid[i + 1]) {
            double below = a - grid[i], above = grid[i + 1] - a;
            if (below < above)
                return i;
            if (above < below)
                return i + 1;
            return (i % 2 == 0) ? i : i + 1;
        }
    }
    return 7;
}

/*
 * MXFP4 quantizer [OCP]: per block of 32 consecutive k of a row, the shared
 * scale is X = 2^(floor(log2(max |V|)) - 2) -- 2 being the exponent of the
 * largest normal E2M1 magnitude, 6 = 1.5 * 2^2 -- with the exponent clamped
 * to the E8M0 range [-127, 127] (an all-zero block takes 2^-127, byte 0);
 * each element is V / X rounded to the nearest E2M1 value, ties to the even
 * code, magnitudes above 6 clamped to 6, the sign kept (a negative value
 * that rounds to zero is -0, code 8).
 *
 * Then, when ps is not NULL, the row postscale: the pages apply one per
 * quantized row but do not say how it is chosen; the reading taken is the
 * least-squares fit of the row, ps = <w, d> / <d, d> over the decoded row d
 * (exact products code * X), fp64 sums in k order, rounded to fp32; 1 when
 * d is all zero.
 *
 * Returns 0, or -1 (nothing written) when an input is not finite.
 */
int or_mxfp4_quantize(const float *w, int64_t n, int64_t k, uint8_t *codes,
                      uint8_t *scales, float *ps)
{
    int64_t nb = k / 32;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(w[i]))
            return -1;
    memset(codes, 0, (size_t)(n * (k / 2)));
    for (int64_t r = 0; r < n; ++r) {
        double wd = 0.0, dd = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const float *v = w + r * k + 32 * b;
            double amax = 0.0;
            int e;
            for (int j = 0; j < 32; ++j)
                if (fabs((double)v[j]) > amax)
                    amax = fabs((double)v[j]);
            if (amax == 0.0) {
                e = -127;
            } else {
                int ex;
                frexp(amax, &ex);      /* amax = m * 2^ex, m in [0.5, 1) */
                e = (ex - 1) - 2;      /* floor(log2(amax)) - 2 */
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
            }
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; ++j) {
                double x = ldexp((double)v[j], -e);   /* exact */
                int idx = e2m1_nearest_index(fabs(x));
                int code = idx | (signbit(x) ? 8 : 0);
                int64_t kk = 32 * b + j;
                codes[r * (k / 2) + kk / 2] |= (uint8_t)((kk & 1) ? code << 4 : code);
                if (ps) {
                    double d = or_e2m1_value(code) * ldexp(1.0, e);
                    wd += (double)v[j] * d;
                    dd += d * d;
                }
            }
        }
        if (ps)
            ps[r] = dd == 0.0 ? 1.0f : (float)(wd / dd);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Grouped affine INT4                                                 */
/* ------------------------------------------------------------------ */

static double clamp_0_15(double v)
{
    return v < 0.0 ? 0.0 : (v > 15.0 ? 15.0 : v);
}

/*
 * Affine INT4 quantizer, one group of consecutive k per (row, group), the
 * last group holding what is left of K ([P2] "correct affine INT4
 * partial-group quantization").  Per group, over its valid elements only:
 *   lo = min(0, min w), hi = max(0, max w)
 *   s  = binary16(round-nearest-even((hi - lo) / 15)); s = 1 if it is 0
 *   z  = clamp(rne(-lo / s), 0, 15)
 *   q  = clamp(rne(w / s) + z, 0, 15)
 * all in fp64 from the fp32 inputs, s held as the binary16 value.  q is
 * written as packed nibbles, s and z as binary16 bit patterns.
 * Returns 0, or -1 when s overflows binary16.
 */
int or_int4_quantize(const float *w, int64_t n, int64_t k, int64_t group,
                     uint8_t *q, uint16_t *s16, uint16_t *z16)
{
    int64_t G = (k + group - 1) / group;
    memset(q, 0, (size_t)(n * (k / 2)));
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < G; ++g) {
            int64_t k0 = g * group, k1 = k0 + group < k ? k0 + group : k;
            double lo = 0.0, hi = 0.0, s, z;
            uint16_t sb;
            for (int64_t j = k0; j < k1; ++j) {
                double v = (double)w[r * k + j];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            sb = or_f16_from_double((hi - lo) / 15.0);
            if ((sb & 0x7C00) == 0x7C00)
                return -1;
            s = or_f16_value(sb);
            if (s == 0.0) {
                sb = 0x3C00;
                s = 1.0;
            }
            z = clamp_0_15(rint(-lo / s));
            s16[r * G + g] = sb;
            z16[r * G + g] = or_f16_from_double(z);
            for (int64_t j = k0; j < k1; ++j) {
                int qv = (int)clamp_0_15(rint((double)w[r * k + j] / s) + z);
                q[r * (k / 2) + j / 2] |= (uint8_t)((j & 1) ? qv << 4 : qv);
            }
        }
    }
    return 0;
}

/* Decoded INT4 row: w = (q - z) * s, rounded once to fp32 (exact). */
static void decode_int4_row(const uint8_t *q, const uint16_t *s16,
                            const uint16_t *z16, int64_t k, int64_t group,
                            int64_t r, float *out)
{
    int64_t G = (k + group - 1) / group;
    const uint8_t *qrow = q + r * (k / 2);
    for (int64_t j = 0; j < k; ++j) {
        int64_t g = j / group;
        double s = or_f16_value(s16[r * G + g]);
        double z = or_f16_value(z16[r * G + g]);
        out[j] = (float)(((double)nibble(qrow, j) - z) * s);
    }
}

void or_int4_dequantize(const uint8_t *q, const uint16_t *s16,
                        const uint16_t *z16, int64_t n, int64_t k,
                        int64_t group, float *w)
{
    for (int64_t r = 0; r < n; ++r)
        decode_int4_row(q, s16, z16, k, group, r, w + r * k);
}

/* y[b][i] = sum_k w[r][k] * x[b][k], r = rows[i]; S as for MXFP4. */
void or_int4_gemv(const uint8_t *q, const uint16_t *s16, const uint16_t *z16,
                  int64_t n, int64_t k, int64_t group,
                  const uint16_t *x, int64_t batch,
                  const int64_t *rows, int64_t nrows,
                  double *y, double *S)
{
    float *w = (float *)malloc(sizeof(float) * (size_t)k);
    (void)n;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        decode_int4_row(q, s16, z16, k, group, r, w);
        for (int64_t b = 0; b < batch; ++b) {
            const uint16_t *xb = x + b * k;
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                double t = (double)w[j] * or_bf16_value(xb[j]);
                acc += t;
                mag += fabs(t);
            }
            y[b * nrows + i] = acc;
            if (S)
                S[b * nrows + i] = mag;
        }
    }
    free(w);
}
