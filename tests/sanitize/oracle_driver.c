/* Drives every entry point of the CPU oracle on small, exactly sized heap
 * buffers, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any read or write past a buffer, use of uninitialized shape arithmetic that
 * overflows, or other undefined behaviour aborts the run.  Exits 0 when every
 * call returned what its header promises. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

static int failures = 0;
#define EXPECT(c)                                                     \
    do {                                                              \
        if (!(c)) {                                                   \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                               \
        }                                                             \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* xorshift64*, in [0, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static double normal(void) {
    double u = uniform(), v = uniform();
    if (u < 1e-300) u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static uint16_t *bf16_rows(int rows, int64_t k, double scale) {
    uint16_t *x = xmalloc(sizeof(uint16_t) * (size_t)rows * (size_t)k);
    for (int64_t i = 0; i < rows * k; ++i) x[i] = nvo_bf16_from_double(normal() * scale);
    return x;
}

static void codecs(void) {
    for (unsigned c = 0; c < 16; ++c) EXPECT(nvo_e2m1_encode((float)nvo_e2m1_value(c)) == (c == 8 ? 8u : c) ||
                                             nvo_e2m1_value(c) == 0.0);
    for (unsigned b = 0; b < 256; ++b) {
        const float v = nvo_e4m3_value(b);
        if (!isnan(v)) EXPECT(nvo_e4m3_value(nvo_e4m3_encode(v)) == v);
        EXPECT(!isnan(nvo_e8m0_value(b)) || b == 255);
    }
    const float specials[] = {0.0f, -0.0f, 1e-45f, 1e-30f, 0.25f, 5.9f, 6.1f, 448.0f, 465.0f, 1e30f, INFINITY,
                              -INFINITY, NAN};
    for (size_t i = 0; i < sizeof specials / sizeof *specials; ++i) {
        if (!isnan(specials[i])) (void)nvo_e2m1_encode(specials[i]);   /* its domain: not NaN */
        (void)nvo_e4m3_encode(specials[i]);
        (void)nvo_bf16_from_double(specials[i]);
    }
    for (unsigned h = 0; h < 65536; h += 7) {
        (void)nvo_bf16_value((uint16_t)h);
        (void)nvo_f16_value((uint16_t)h);
    }
}

static void nvfp4(int64_t n, int64_t k) {
    float *W = xmalloc(sizeof(float) * (size_t)(n * k));
    for (int64_t i = 0; i < n * k; ++i) W[i] = (float)(normal() * 0.02);
    for (int64_t i = 0; i < 16 && i < k; ++i) W[i] = 0.0f;   /* a zero group */
    uint8_t *codes = xmalloc((size_t)(n * k / 2)), *scales = xmalloc((size_t)(n * k / 16));
    float sg = 0.0f;
    EXPECT(nvo_quantize(W, n, k, codes, scales, &sg) == 0);
    EXPECT(nvo_quantize(W, n, k + 8, codes, scales, &sg) == -1);
    float *D = xmalloc(sizeof(float) * (size_t)(n * k));
    nvo_dequant(codes, scales, sg, n, k, D);
    int64_t sel[3] = {0, n / 2, n - 1};
    for (int rows = 0; rows <= NVO_MAX_ROWS + 1; rows += (rows < 9 ? 1 : 28)) {
        uint16_t *x = bf16_rows(rows ? rows : 1, k, 1.0);
        const int64_t ns = rows % 2 ? 3 : n;
        const int64_t *s = rows % 2 ? sel : NULL;
        const size_t out = (size_t)(rows ? rows : 1) * (size_t)ns;
        double *y = xmalloc(sizeof(double) * out), *a = xmalloc(sizeof(double) * out);
        double *g = xmalloc(sizeof(double) * out), *u = xmalloc(sizeof(double) * out);
        double *ag = xmalloc(sizeof(double) * out), *au = xmalloc(sizeof(double) * out);
        uint16_t *yb = xmalloc(sizeof(uint16_t) * out);
        float *y32 = xmalloc(sizeof(float) * out);
        const int want = rows >= 1 && rows <= NVO_MAX_ROWS ? 0 : -1;
        EXPECT(nvo_gemv(codes, scales, sg, n, k, x, rows, s, ns, y, a, yb) == want);
        EXPECT(nvo_gemv_f32seq(codes, scales, sg, n, k, x, rows, s, ns, y32, yb) == want);
        EXPECT(nvo_gemv_dual_silu(codes, scales, sg, codes, scales, sg, n, k, x, rows, s, ns, y, g, u, ag, au, yb) ==
               want);
        free(x), free(y), free(a), free(g), free(u), free(ag), free(au), free(yb), free(y32);
    }
    W[3] = NAN;
    EXPECT(nvo_quantize(W, n, k, codes, scales, &sg) == -2);
    free(W), free(codes), free(scales), free(D);
}

static void dense_and_norm(void) {
    const int64_t n = 7, k = 80;
    const int rows = 3;
    uint16_t *W = bf16_rows((int)n, k, 0.05), *x = bf16_rows(rows, k, 1.0);
    double *y = xmalloc(sizeof(double) * rows * n), *a = xmalloc(sizeof(double) * rows * n);
    uint16_t *yb = xmalloc(sizeof(uint16_t) * rows * n);
    nvo_dense_gemv(W, n, k, x, rows, NULL, n, y, a, yb);
    uint16_t *r = bf16_rows(rows, k, 2.0), *h = bf16_rows(rows, k, 1.0), *w = bf16_rows(1, k, 0.1);
    uint16_t *ro = xmalloc(sizeof(uint16_t) * rows * k), *xo = xmalloc(sizeof(uint16_t) * rows * k);
    double *inv = xmalloc(sizeof(double) * rows);
    for (int gemma = 0; gemma < 2; ++gemma) {
        nvo_residual_rmsnorm(r, h, w, k, rows, 1e-6, gemma, ro, xo, inv);
        nvo_residual_rmsnorm(r, h, w, k, rows, 0.0, gemma, ro, xo, NULL);
    }
    free(W), free(x), free(y), free(a), free(yb), free(r), free(h), free(w), free(ro), free(xo), free(inv);
}

static void formats(void) {
    const int64_t n = 5, k = 96;
    const int rows = 2;
    float *W = xmalloc(sizeof(float) * (size_t)(n * k));
    for (int64_t i = 0; i < n * k; ++i) W[i] = (float)(normal() * 0.02);
    uint8_t *mc = xmalloc((size_t)(n * k / 2)), *ms = xmalloc((size_t)(n * k / 32));
    int8_t *wc = xmalloc((size_t)(n * k));
    uint16_t *ws = xmalloc(sizeof(uint16_t) * (size_t)(n * k / 32));
    double *deq = xmalloc(sizeof(double) * (size_t)(n * k));
    uint16_t *x = bf16_rows(rows, k, 1.0), *yb = xmalloc(sizeof(uint16_t) * rows * n);
    double *y = xmalloc(sizeof(double) * rows * n), *a = xmalloc(sizeof(double) * rows * n);
    EXPECT(nvo_mx_quantize(W, n, k, mc, ms) == 0);
    nvo_mx_dequant(mc, ms, n, k, deq);
    nvo_mx_gemv(mc, ms, n, k, x, rows, NULL, n, y, a, yb);
    EXPECT(nvo_w8_quantize(W, n, k, wc, ws) == 0);
    nvo_w8_dequant(wc, ws, n, k, deq);
    nvo_w8_gemv(wc, ws, n, k, x, rows, NULL, n, y, a, yb);
    free(W), free(mc), free(ms), free(wc), free(ws), free(deq), free(x), free(yb), free(y), free(a);
}

int main(void) {
    nvo_set_num_threads(1);
    codecs();
    nvfp4(3, 48);
    nvfp4(70, 272);
    dense_and_norm();
    formats();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: ok\n");
    return 0;
}
