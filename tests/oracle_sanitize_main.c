/*
 * oracle_sanitize_main.c -- drives every entry point of the C oracle
 * (oracle/csrc/oracle.c) on small edge-case layers, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py).
 *
 * Every buffer is allocated at exactly the size the oracle's documentation
 * states, so a read or write one element past it is reported. The layers
 * cover the three group sizes, one expert, top_k = E, all-zero weight groups
 * (the scale clamp), huge and tiny weights, a NULL weight pointer for an
 * expert no token chooses, forced expert ids, an out-of-range forced id
 * (which must return -1), and a quantizer call with no rows. Outputs must be
 * finite. Exit status 0 means every call ran clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_quantize_int4(const float *w, int64_t rows, int64_t K, int64_t group,
                          int8_t *codes, float *scales);
int oracle_moe_token(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                     int64_t group, const float *wr, const float *bias,
                     const int8_t *const *c1, const float *const *s1,
                     const int8_t *const *c3, const float *const *s3,
                     const int8_t *const *c2, const float *const *s2,
                     const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                     const int32_t *forced_ids,
                     float *logits, int32_t *ids, double *gates,
                     double *u, double *o, double *y);
int oracle_moe_token_bf16(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                          const float *wr, const float *bias,
                          const uint16_t *const *w1, const uint16_t *const *w3,
                          const uint16_t *const *w2,
                          const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                          const int32_t *forced_ids,
                          float *logits, int32_t *ids, double *gates,
                          double *u, double *o, double *y);
void oracle_quantize_fp8_rows(const float *w, int64_t rows, int64_t K, float ub,
                              uint8_t *codes, float *scales);
double oracle_fp8_value(uint8_t c);
int oracle_moe_token_fp8(const double *x, int64_t d, int64_t h, int64_t E, int32_t k,
                         const float *wr, const float *bias,
                         const uint8_t *const *q1, const float *const *s1,
                         const uint8_t *const *q3, const float *const *s3,
                         const uint8_t *const *q2, const float *const *s2, float ub,
                         const uint16_t *sh1, const uint16_t *sh3, const uint16_t *sh2,
                         const int32_t *forced_ids,
                         float *logits, int32_t *ids, double *gates,
                         float *f32, uint8_t *codes, double *u, double *o, double *y);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* uniform in [-1, 1) from a 64-bit linear congruential generator */
static float uniform(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void *checked_malloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* bf16 bits of a float (round to nearest even; finite inputs) */
static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* weights of `rows` x `K` with the layer's edge cases mixed in */
static float *weights(int64_t rows, int64_t K, int64_t group)
{
    float *w = checked_malloc((size_t)(rows * K) * sizeof(float));
    for (int64_t i = 0; i < rows * K; ++i) w[i] = 0.05f * uniform();
    if (rows > 0) {
        for (int64_t i = 0; i < group && i < K; ++i) w[i] = 0.0f;       /* all-zero group */
        if (K >= 2 * group) w[group] = 3.0e4f;                          /* huge weight */
        if (rows > 1) w[K] = 1.0e-30f;                                  /* tiny weight */
    }
    return w;
}

static int check_finite(const double *v, int64_t n, const char *what)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) {
            fprintf(stderr, "%s[%lld] is not finite\n", what, (long long)i);
            return 1;
        }
    return 0;
}

/* one layer: d, h, E experts, top-k, int4 group */
static int run_layer(int64_t d, int64_t h, int64_t E, int32_t k, int64_t group)
{
    int bad = 0;
    const int64_t nd = d / group, nh = h / group;
    const float ub = 1200.0f;
    int8_t **c1 = checked_malloc(E * sizeof(*c1)), **c3 = checked_malloc(E * sizeof(*c3));
    int8_t **c2 = checked_malloc(E * sizeof(*c2));
    float **s1 = checked_malloc(E * sizeof(*s1)), **s3 = checked_malloc(E * sizeof(*s3));
    float **s2 = checked_malloc(E * sizeof(*s2));
    uint16_t **b1 = checked_malloc(E * sizeof(*b1)), **b3 = checked_malloc(E * sizeof(*b3));
    uint16_t **b2 = checked_malloc(E * sizeof(*b2));
    uint8_t **q1 = checked_malloc(E * sizeof(*q1)), **q3 = checked_malloc(E * sizeof(*q3));
    uint8_t **q2 = checked_malloc(E * sizeof(*q2));
    float **f1 = checked_malloc(E * sizeof(*f1)), **f3 = checked_malloc(E * sizeof(*f3));
    float **f2 = checked_malloc(E * sizeof(*f2));
    for (int64_t e = 0; e < E; ++e) {
        float *w1 = weights(h, d, group), *w3 = weights(h, d, group), *w2 = weights(d, h, group);
        c1[e] = checked_malloc((size_t)(h * d));
        c3[e] = checked_malloc((size_t)(h * d));
        c2[e] = checked_malloc((size_t)(d * h));
        s1[e] = checked_malloc((size_t)(h * nd) * sizeof(float));
        s3[e] = checked_malloc((size_t)(h * nd) * sizeof(float));
        s2[e] = checked_malloc((size_t)(d * nh) * sizeof(float));
        oracle_quantize_int4(w1, h, d, group, c1[e], s1[e]);
        oracle_quantize_int4(w3, h, d, group, c3[e], s3[e]);
        oracle_quantize_int4(w2, d, h, group, c2[e], s2[e]);
        for (int64_t i = 0; i < h * d; ++i)
            if (c1[e][i] < -8 || c1[e][i] > 7) bad = 1;
        b1[e] = checked_malloc((size_t)(h * d) * 2);
        b3[e] = checked_malloc((size_t)(h * d) * 2);
        b2[e] = checked_malloc((size_t)(d * h) * 2);
        for (int64_t i = 0; i < h * d; ++i) {
            b1[e][i] = to_bf16(w1[i]);
            b3[e][i] = to_bf16(w3[i]);
            b2[e][i] = to_bf16(w2[i]);
        }
        q1[e] = checked_malloc((size_t)(h * d));
        q3[e] = checked_malloc((size_t)(h * d));
        q2[e] = checked_malloc((size_t)(d * h));
        f1[e] = checked_malloc((size_t)h * sizeof(float));
        f3[e] = checked_malloc((size_t)h * sizeof(float));
        f2[e] = checked_malloc((size_t)d * sizeof(float));
        oracle_quantize_fp8_rows(w1, h, d, ub, q1[e], f1[e]);
        oracle_quantize_fp8_rows(w3, h, d, ub, q3[e], f3[e]);
        oracle_quantize_fp8_rows(w2, d, h, ub, q2[e], f2[e]);
        free(w1);
        free(w3);
        free(w2);
    }
    uint16_t *sh1 = checked_malloc((size_t)(h * d) * 2), *sh3 = checked_malloc((size_t)(h * d) * 2);
    uint16_t *sh2 = checked_malloc((size_t)(d * h) * 2);
    for (int64_t i = 0; i < h * d; ++i) {
        sh1[i] = to_bf16(0.05f * uniform());
        sh3[i] = to_bf16(0.05f * uniform());
        sh2[i] = to_bf16(0.05f * uniform());
    }
    float *wr = checked_malloc((size_t)(E * d) * sizeof(float));
    float *bias = checked_malloc((size_t)E * sizeof(float));
    for (int64_t i = 0; i < E * d; ++i) wr[i] = 0.1f * uniform();
    for (int64_t e = 0; e < E; ++e) bias[e] = 0.01f * uniform();

    double *x = checked_malloc((size_t)d * sizeof(double));
    float *logits = checked_malloc((size_t)E * sizeof(float));
    int32_t *ids = checked_malloc((size_t)k * sizeof(int32_t));
    int32_t *forced = checked_malloc((size_t)k * sizeof(int32_t));
    double *gates = checked_malloc((size_t)k * sizeof(double));
    double *u = checked_malloc((size_t)h * sizeof(double));
    double *o = checked_malloc((size_t)d * sizeof(double));
    double *y = checked_malloc((size_t)d * sizeof(double));
    const int64_t mx = d > h ? d : h;
    float *f32 = checked_malloc((size_t)mx * sizeof(float));
    uint8_t *codes = checked_malloc((size_t)mx);

    for (int token = 0; token < 3; ++token) {
        for (int64_t i = 0; i < d; ++i) x[i] = (double)(0.5f * uniform());
        if (token == 2) x[0] = 2.0e3;  /* one large activation: the fp8 ub clamp */
        if (oracle_moe_token(x, d, h, E, k, group, wr, bias, (const int8_t *const *)c1,
                             (const float *const *)s1, (const int8_t *const *)c3,
                             (const float *const *)s3, (const int8_t *const *)c2,
                             (const float *const *)s2, sh1, sh3, sh2, NULL, logits, ids, gates,
                             u, o, y) != 0)
            bad = 1;
        bad |= check_finite(y, d, "int4 y");
        if (oracle_moe_token_bf16(x, d, h, E, k, wr, bias, (const uint16_t *const *)b1,
                                  (const uint16_t *const *)b3, (const uint16_t *const *)b2,
                                  sh1, sh3, sh2, NULL, logits, ids, gates, u, o, y) != 0)
            bad = 1;
        bad |= check_finite(y, d, "bf16 y");
        if (oracle_moe_token_fp8(x, d, h, E, k, wr, bias, (const uint8_t *const *)q1,
                                 (const float *const *)f1, (const uint8_t *const *)q3,
                                 (const float *const *)f3, (const uint8_t *const *)q2,
                                 (const float *const *)f2, ub, sh1, sh3, sh2, NULL, logits,
                                 ids, gates, f32, codes, u, o, y) != 0)
            bad = 1;
        bad |= check_finite(y, d, "fp8 y");
    }

    /* forced ids: the last k experts, with expert 0's weights withdrawn when
       it is not among them (an expert no token chooses may be NULL) */
    for (int32_t j = 0; j < k; ++j) forced[j] = (int32_t)(E - k + j);
    int8_t *keep = c1[0];
    if (E - k > 0) c1[0] = NULL;
    if (oracle_moe_token(x, d, h, E, k, group, wr, bias, (const int8_t *const *)c1,
                         (const float *const *)s1, (const int8_t *const *)c3,
                         (const float *const *)s3, (const int8_t *const *)c2,
                         (const float *const *)s2, sh1, sh3, sh2, forced, logits, ids, gates, u,
                         o, y) != 0)
        bad = 1;
    bad |= check_finite(y, d, "forced y");
    c1[0] = keep;
    /* an out-of-range forced id is refused */
    forced[0] = (int32_t)E;
    if (oracle_moe_token(x, d, h, E, k, group, wr, bias, (const int8_t *const *)c1,
                         (const float *const *)s1, (const int8_t *const *)c3,
                         (const float *const *)s3, (const int8_t *const *)c2,
                         (const float *const *)s2, sh1, sh3, sh2, forced, logits, ids, gates, u,
                         o, y) != -1)
        bad = 1;

    for (int64_t e = 0; e < E; ++e) {
        free(c1[e]); free(c3[e]); free(c2[e]); free(s1[e]); free(s3[e]); free(s2[e]);
        free(b1[e]); free(b3[e]); free(b2[e]);
        free(q1[e]); free(q3[e]); free(q2[e]); free(f1[e]); free(f3[e]); free(f2[e]);
    }
    free(c1); free(c3); free(c2); free(s1); free(s3); free(s2);
    free(b1); free(b3); free(b2); free(q1); free(q3); free(q2); free(f1); free(f3); free(f2);
    free(sh1); free(sh3); free(sh2); free(wr); free(bias);
    free(x); free(logits); free(ids); free(forced); free(gates); free(u); free(o); free(y);
    free(f32); free(codes);
    if (bad) fprintf(stderr, "layer d=%lld h=%lld E=%lld k=%d group=%lld failed\n", (long long)d,
                     (long long)h, (long long)E, k, (long long)group);
    return bad;
}

int main(void)
{
    int bad = 0;
    /* a quantizer call with no rows touches nothing */
    oracle_quantize_int4(NULL, 0, 128, 128, NULL, NULL);
    /* every fp8 code decodes to a finite value or NaN, never past 448 */
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_fp8_value((uint8_t)c);
        if (!isnan(v) && fabs(v) > 448.0) bad = 1;
    }
    bad |= run_layer(128, 128, 1, 1, 128);  /* one expert */
    bad |= run_layer(256, 384, 4, 2, 64);   /* groups of 64, h not a power of two */
    bad |= run_layer(128, 256, 5, 5, 32);   /* groups of 32, top_k = E */
    bad |= run_layer(256, 128, 6, 1, 128);  /* h < d */
    if (!bad) printf("oracle sanitize run: all calls clean\n");
    return bad;
}
