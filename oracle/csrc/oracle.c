/*
 * oracle.c -- plain C CPU oracle for the int4 MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, smoke() and the bench's
 * cpu_baseline leg, never by the product library. It shares no code with it.
 *
 * Two things live here, both written as the plainest loops:
 *
 *  1. oracle_quantize_int4: the int4 group quantizer printed as
 *     int4_row_quantize on the discosf.com page "1 卡跑通 Llama 4", section
 *     "FP8 / Int4 混合量化". Per group of `group` consecutive fp32 weights:
 *     scale = max(max|w|, 1e-6f) / 8, code = clamp(round_half_even(w / scale),
 *     -8, 7). fp32 division (IEEE, correctly rounded) and rintf under the
 *     default round-to-nearest-even mode. Built with -ffp-contract=off and
 *     without fast-math.
 *
 *  2. oracle_moe_token: the MoE layer for ONE token, as a per-token loop
 *     (discosf.com page, section "混合专家路由"): router logits, top-k
 *     (ties to the lower expert id), sigmoid gates, and for each chosen expert
 *     the SwiGLU FFN (docs.ifdog.com page "Llama 开源模型系列", section
 *     "SwiGLU：门控激活的数学") weighted by its gate, then plus the shared
 *     expert. Everything in double; logits rounded to float before the top-k
 *     choice (the choice is taken in fp32). Routed weights are dequantized
 *     on the fly as code * scale, one weight at a time.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- quantizer */

void oracle_quantize_int4(const float *w, int64_t rows, int64_t K, int64_t group,
                          int8_t *codes, float *scales)
{
    const int64_t ngroups = K / group;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < ngroups; ++g) {
            const float *src = w + r * K + g * group;
            int8_t *dst = codes + r * K + g * group;
            float m = 0.0f;
            for (int64_t i = 0; i < group; ++i) {
                float a = fabsf(src[i]);
                if (a > m) m = a;
            }
            float s = (m < 1e-6f ? 1e-6f : m) / 8.0f;
            scales[r * ngroups + g] = s;
            for (int64_t i = 0; i < group; ++i) {
                float q = rintf(src[i] / s);
                if (q < -8.0f) q = -8.0f;
                if (q > 7.0f) q = 7.0f;
                dst[i] = (int8_t)q;
            }
        }
    }
}

/* ------------------------------------------------------------------ helpers */

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

static double silu(double z) { return z * sigmoid(z); }

/* w_hat[row][j] of an int4 matrix with `cols` columns */
static double dq(const int8_t *c, const float *s, int64_t cols, int64_t group,
                 int64_t row, int64_t j)
{
    return (double)c[row * cols + j] * (double)s[row * (cols / group) + j / group];
}

/* One SwiGLU expert with int4 weights on one token:
 *   a[n] = sum_j x[j] W1[n][j],  b[n] = sum_j x[j] W3[n][j]   (W1, W3: [h, d])
 *   u[n] = silu(a[n]) * b[n]
 *   o[m] = sum_n u[n] W2[m][n]                                  (W2: [d, h]) */
void oracle_swiglu_int4_token(const double *x, int64_t d, int64_t h, int64_t group,
                              const int8_t *c1, const float *s1,
                              const int8_t *c3, const float *s3,
                              const int8_t *c2, const float *s2,
                              double *u, double *o)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < h; ++n) {
        double a = 0.0, b = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            a += x[j] * dq(c1, s1, d, group, n, j);
            b += x[j] * dq(c3, s3, d, group, n, j);
        }
        u[n] = silu(a) * b;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int64_t n = 0; n < h; ++n)
            acc += u[n] * dq(c2, s2, h, group, m, n);
        o[m] = acc;
    }
}

/* The same expert with bf16 weights (the shared expert). */
void oracle_swiglu_bf16_token(const double *x, int64_t d, int64_t h,
                              const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              double *u, double *o)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < h; ++n) {
        double a = 0.0, b = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            a += x[j] * bf16_to_double(w1[n * d + j]);
            b += x[j] * bf16_to_double(w3[n * d + j]);
        }
        u[n] = silu(a) * b;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < d; ++m) {
        double acc = 0.0;
        for (int64_t n = 0; n < h; ++n)
            acc += u[n] * bf16_to_double(w2[m * h + n]);
        o[m] = acc;
    }
}

/* logits[e] = (float)(sum_j x[j] Wr[e][j] + b[e]), accumulated in double */
void oracle_router_token(const double *x, const float *wr, const float *bias,
                         int64_t E, int64_t d, float *logits)
{
    for (int64_t e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int64_t j = 0; j < d; ++j)
            acc += x[j] * (double)wr[e * d + j];
        if (bias) acc += (double)bias[e];
        logits[e] = (float)acc;
    }
}

/* k rounds of "largest remaining logit, lower id on ties" */
void oracle_topk_token(const float *logits, int64_t E, int32_t k, int32_t *ids)
{
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            int taken = 0;
            for (int32_t i = 0; i < j; ++i)
                if (ids[i] == (int32_t)e) taken = 1;
            if (taken) continue;
            if (best < 0 || logits[e] > logits[best]) best = (int32_t)e;
        }
        ids[j] = best;
    }
}

/*
 * The whole layer for one token. Expert e's weights are c1[e], s1[e], ...;
 * an expert the token does not choose may be NULL. If forced_ids is not NULL
 * it replaces the top-k choice. Returns 0, or -1 if a chosen expert is NULL
 * or an id is out of range.
 *   y[m] = sum_j gate_j * expert_{id_j}(x)[m]  +  shared(x)[m]
 * scratch: u [h] and o [d] doubles.
 */
int oracle_moe_token(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                     int64_t group, const float *wr, const float *bias,
                     const int8_t *const *c1, const float *const *s1,
                     const int8_t *const *c3, const float *const *s3,
                     const int8_t *const *c2, const float *const *s2,
                     const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                     const int32_t *forced_ids,
                     float *logits, int32_t *ids, double *gates,
                     double *u, double *o, double *y)
{
    oracle_router_token(x, wr, bias, E, d, logits);
    if (forced_ids)
        for (int32_t j = 0; j < k; ++j) ids[j] = forced_ids[j];
    else
        oracle_topk_token(logits, E, k, ids);

    for (int64_t m = 0; m < d; ++m) y[m] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t e = ids[j];
        if (e < 0 || e >= E || !c1[e] || !c3[e] || !c2[e]) return -1;
        gates[j] = sigmoid((double)logits[e]);
        oracle_swiglu_int4_token(x, d, h, group, c1[e], s1[e], c3[e], s3[e],
                                 c2[e], s2[e], u, o);
        for (int64_t m = 0; m < d; ++m) y[m] += gates[j] * o[m];
    }
    oracle_swiglu_bf16_token(x, d, h, sh1, sh3, sh2, u, o);
    for (int64_t m = 0; m < d; ++m) y[m] += o[m];
    return 0;
}

/*
 * oracle_moe_token with bf16 routed experts: the pure-bf16 path, which the
 * lshu.cn page (section "三条推理路径差异") lists as the accuracy baseline.
 * Expert e's weights are w1[e], w3[e], w2[e] (bf16 bits, widened exactly);
 * everything else as in oracle_moe_token.
 */
int oracle_moe_token_bf16(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                          const float *wr, const float *bias,
                          const uint16_t *const *w1, const uint16_t *const *w3,
                          const uint16_t *const *w2,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                          const int32_t *forced_ids,
                          float *logits, int32_t *ids, double *gates,
                          double *u, double *o, double *y)
{
    oracle_router_token(x, wr, bias, E, d, logits);
    if (forced_ids)
        for (int32_t j = 0; j < k; ++j) ids[j] = forced_ids[j];
    else
        oracle_topk_token(logits, E, k, ids);

    for (int64_t m = 0; m < d; ++m) y[m] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t e = ids[j];
        if (e < 0 || e >= E || !w1[e] || !w3[e] || !w2[e]) return -1;
        gates[j] = sigmoid((double)logits[e]);
        oracle_swiglu_bf16_token(x, d, h, w1[e], w3[e], w2[e], u, o);
        for (int64_t m = 0; m < d; ++m) y[m] += gates[j] * o[m];
    }
    oracle_swiglu_bf16_token(x, d, h, sh1, sh3, sh2, u, o);
    for (int64_t m = 0; m < d; ++m) y[m] += o[m];
    return 0;
}

/* ------------------------------------------------------------ fp8 row-wise */
/*
 * The fp8_mixed path of the lshu.cn page "Llama 4 单卡量化推理与选型指南"
 * (sections "三条推理路径差异" and "量化环节"): activations quantized per
 * row to fp8 with an upper bound on the row scale, fp8 weights with one scale
 * per row, the fp8 x fp8 product scaled by both row scales and returned in
 * bf16. fp8 is OCP E4M3 (bias 7, 3 mantissa bits, largest finite 448,
 * subnormal spacing 2^-9); conversion rounds to nearest, ties to even.
 * A row's scale is min(max(max|v|, 1e-12), ub) / 448 (ub <= 0: no bound) and
 * its codes are fp8(clamp(v / scale, -448, 448)), fp32 arithmetic.
 * The same readings as the numpy form in fp8.py, written as plain loops.
 */

/* nearest E4M3 value to v, |v| <= 448: in the binade [2^e, 2^(e+1)) the
 * spacing is 2^(e-3); below 2^-6 (subnormals) it is 2^-9 */
static double fp8_round_value(double v)
{
    double a = fabs(v);
    if (a == 0.0) return v;
    int ex;
    (void)frexp(a, &ex);  /* a = f * 2^ex with f in [0.5, 1): binade 2^(ex-1) */
    int e = ex - 1;
    if (e < -6) e = -6;
    double spacing = ldexp(1.0, e - 3);
    return copysign(nearbyint(a / spacing) * spacing, v);
}

/* bit pattern of an E4M3 value */
static uint8_t fp8_bits(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a < ldexp(1.0, -6))                       /* exponent field 0 */
        return (uint8_t)(sign | (uint8_t)(a / ldexp(1.0, -9)));
    int ex;
    double f = frexp(a, &ex);                     /* a = (2f) * 2^(ex-1), 2f in [1, 2) */
    int mant = (int)((2.0 * f - 1.0) * 8.0);
    return (uint8_t)(sign | (uint8_t)(((ex - 1 + 7) << 3) | mant));
}

/* value of an E4M3 bit pattern; exponent and mantissa fields all ones (0x7F,
 * 0xFF) encode NaN, the format having no infinities */
double oracle_fp8_value(uint8_t c)
{
    if ((c & 0x7F) == 0x7F) return NAN;
    int ef = (c >> 3) & 15, m = c & 7;
    double v = ef == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ef - 7);
    return (c & 0x80) ? -v : v;
}

static void quantize_fp8_row(const float *v, int64_t K, float ub, uint8_t *q, float *scale)
{
    float m = 0.0f;
    for (int64_t i = 0; i < K; ++i) {
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    if (m < 1e-12f) m = 1e-12f;
    if (ub > 0.0f && m > ub) m = ub;
    float s = m / 448.0f;
    *scale = s;
    for (int64_t i = 0; i < K; ++i) {
        float t = v[i] / s;
        if (t > 448.0f) t = 448.0f;
        if (t < -448.0f) t = -448.0f;
        q[i] = fp8_bits(fp8_round_value((double)t));
    }
}

void oracle_quantize_fp8_rows(const float *w, int64_t rows, int64_t K, float ub,
                              uint8_t *q, float *scales)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        quantize_fp8_row(w + r * K, K, ub, q + r * K, scales + r);
}

/* nearest bf16 value (ties to even) of the fp32 rounding of v */
static double bf16_round_value(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* oracle_fp8_value of every code, filled once before the parallel loops
 * (a lookup of the same values, so the products below are unchanged) */
static double fp8_value_table[256];
static int fp8_value_table_ready;

static void fp8_table_init(void)
{
    if (fp8_value_table_ready) return;
    for (int c = 0; c < 256; ++c) fp8_value_table[c] = oracle_fp8_value((uint8_t)c);
    fp8_value_table_ready = 1;
}

/* bf16(sum_j fp8(a[j]) fp8(w[row][j]) * sa * sw[row]): the products are exact
 * and so is their fp64 sum (every term is a multiple of 2^-18 below 2^18) */
static double fp8_row_product(const uint8_t *a, float sa, const uint8_t *w, const float *sw,
                              int64_t K, int64_t row)
{
    double acc = 0.0;
    for (int64_t j = 0; j < K; ++j)
        acc += fp8_value_table[a[j]] * fp8_value_table[w[row * K + j]];
    return bf16_round_value(acc * (double)sa * (double)sw[row]);
}

/* One fp8 expert on one token (x: values of bf16 activations):
 *   xq, sx = quantize(x);  a1[n] = bf16(xq.W1[n] sx s1[n]);  a3 likewise (W3)
 *   u[n] = bf16(silu(a1[n]) a3[n]);  uq, su = quantize(u)
 *   o[m] = bf16(uq.W2[m] su s2[m]) */
void oracle_swiglu_fp8_token(const double *x, int64_t d, int64_t h,
                             const uint8_t *q1, const float *s1,
                             const uint8_t *q3, const float *s3,
                             const uint8_t *q2, const float *s2, float ub,
                             float *f32, uint8_t *codes, double *u, double *o)
{
    float sx, su;
    fp8_table_init();
    for (int64_t j = 0; j < d; ++j) f32[j] = (float)x[j];
    quantize_fp8_row(f32, d, ub, codes, &sx);
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < h; ++n) {
        double a1 = fp8_row_product(codes, sx, q1, s1, d, n);
        double a3 = fp8_row_product(codes, sx, q3, s3, d, n);
        u[n] = bf16_round_value(silu(a1) * a3);
    }
    for (int64_t n = 0; n < h; ++n) f32[n] = (float)u[n];
    quantize_fp8_row(f32, h, ub, codes, &su);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < d; ++m)
        o[m] = fp8_row_product(codes, su, q2, s2, h, m);
}

/*
 * oracle_moe_token with fp8 routed experts: expert e's codes q1[e], q3[e]
 * ([h, d] row-major), q2[e] ([d, h]) and row scales s1[e], s3[e] [h],
 * s2[e] [d]; ub bounds the activation row scales. Router, gates and the bf16
 * shared expert as in oracle_moe_token. scratch: f32 and codes of
 * max(d, h) entries, u [h], o [d].
 */
int oracle_moe_token_fp8(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                         const float *wr, const float *bias,
                         const uint8_t *const *q1, const float *const *s1,
                         const uint8_t *const *q3, const float *const *s3,
                         const uint8_t *const *q2, const float *const *s2, float ub,
                         const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                         const int32_t *forced_ids,
                         float *logits, int32_t *ids, double *gates,
                         float *f32, uint8_t *codes, double *u, double *o, double *y)
{
    oracle_router_token(x, wr, bias, E, d, logits);
    if (forced_ids)
        for (int32_t j = 0; j < k; ++j) ids[j] = forced_ids[j];
    else
        oracle_topk_token(logits, E, k, ids);

    for (int64_t m = 0; m < d; ++m) y[m] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t e = ids[j];
        if (e < 0 || e >= E || !q1[e] || !q3[e] || !q2[e]) return -1;
        gates[j] = sigmoid((double)logits[e]);
        oracle_swiglu_fp8_token(x, d, h, q1[e], s1[e], q3[e], s3[e], q2[e], s2[e], ub,
                                f32, codes, u, o);
        for (int64_t m = 0; m < d; ++m) y[m] += gates[j] * o[m];
    }
    oracle_swiglu_bf16_token(x, d, h, sh1, sh3, sh2, u, o);
    for (int64_t m = 0; m < d; ++m) y[m] += o[m];
    return 0;
}
