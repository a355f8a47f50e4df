/*
 * nvfp4_oracle.c -- plain CPU oracle for weight-only NVFP4 projection GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see nvfp4_oracle.h).  Compiled with
 * -O2 -ffp-contract=off and no fast-math, so every float expression below is
 * evaluated exactly as written: one IEEE rounding per operation, in the
 * precision the operands have (float stays float on x86-64 SSE).
 *
 * Rounding-to-nearest-even is done with rint(), which follows the current
 * rounding mode; the default mode (round to nearest, ties to even) is never
 * changed by this library.
 *
 * Readings of points the pages leave open (the pages name "nvfp4/g16" with a
 * bf16 activation on the Qwen3.8-27B-NVFP4 blueprint page, "Precision" table,
 * and give no arithmetic):
 *   R1  a group is 16 consecutive k of one output row;
 *   R2  element 2j sits in the low nibble of byte j;
 *   R3  E2M1 rounds to nearest, ties to the code with mantissa bit 0;
 *   R4  |v| > 6 saturates to +-6 (E2M1 has no Inf/NaN);
 *   R5  a negative value that rounds to zero keeps its sign (code 0x8);
 *   R6  E4M3 (OCP) rounds to nearest even, saturates to 448, keeps
 *       subnormals, never produces NaN;
 *   R7  s_g = amax / 2688 (= 448*6) in fp32, stored as the dequant multiplier;
 *   R8  group scale code = E4M3((a / 6) / s_g), two fp32 divisions;
 *   R9  elements are divided by the decoded scale S = e4m3(code) * s_g (fp32);
 *   R10 a group whose S is 0 gets every code 0x0;
 *   R11 an all-zero tensor gets s_g = 0, every scale 0x00, every code 0x0;
 *   R12 a non-finite weight is an error.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0 ---- */

double nvo_e2m1_value(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
    return s ? -mag : mag;
}

/* magnitude value -> 3-bit magnitude code; values are the E2M1 grid */
static unsigned e2m1_mag_code(double r)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (unsigned c = 0; c < 8; ++c)
        if (grid[c] == r) return c;
    abort(); /* unreachable: r is always a grid point */
}

/* R3/R4/R5: round |v| to the E2M1 grid as a floating-point format does: the
 * quantum is 2^(e-1) for unbiased exponent e clamped to [0, 2] (e = 0 also
 * covers the subnormal 0.5), ties go to the even multiple (= mantissa 0). */
unsigned nvo_e2m1_encode(float v)
{
    unsigned sign = signbit(v) ? 8u : 0u;
    double a = fabs((double)v);
    if (a >= 6.0) return sign | 7u;
    int ex;
    frexp(a, &ex);               /* a = f * 2^ex, f in [0.5, 1); 0 gives ex = 0 */
    int ue = ex - 1;
    if (ue < 0) ue = 0;
    if (ue > 2) ue = 2;
    double q = ldexp(1.0, ue - 1);
    double r = rint(a / q) * q;  /* exact: scaling by a power of two */
    if (r > 6.0) r = 6.0;
    return sign | e2m1_mag_code(r);
}

/* ---- OCP E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0 ---- */

float nvo_e4m3_value(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else        mag = ldexp(1.0 + m / 8.0, (int)e - 7);
    return (float)(s ? -mag : mag);
}

/* R6: round to nearest even on the E4M3 grid, saturate at 448, never NaN. */
unsigned nvo_e4m3_encode(float v)
{
    unsigned sign = signbit(v) ? 0x80u : 0u;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7Eu;   /* also +-Inf */
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int ue = ex - 1;                       /* a = 1.f * 2^ue */
    if (ue < -6) ue = -6;                  /* subnormals share the 2^-9 quantum */
    double r = rint(a / ldexp(1.0, ue - 3));   /* integer in [0, 16] */
    if (r >= 16.0) { r = 8.0; ue += 1; }
    if (r < 8.0) return sign | (unsigned)r;    /* subnormal (ue == -6) or zero */
    return sign | ((unsigned)(ue + 7) << 3) | ((unsigned)r - 8u);
}

/* ---- bf16 ---- */

double nvo_bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* round a double to bf16 (8 significant bits, 8 exponent bits), nearest even */
uint16_t nvo_bf16_from_double(double v)
{
    if (isnan(v)) return 0x7FC0u;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80u;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int ue = ex - 1;
    if (ue < -126) ue = -126;              /* bf16 subnormal quantum 2^-133 */
    double q = ldexp(1.0, ue - 7);
    double r = rint(a / q) * q;
    if (r >= 0x1p128) return sign | 0x7F80u;
    float f = (float)r;                    /* exact: <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)((u >> 16) & 0x7FFFu);
}

/* ---- quantizer (R1, R7..R12) ---- */

int nvo_quantize(const float *W, int64_t n, int64_t k, uint8_t *codes,
                 uint8_t *scales, float *global_scale)
{
    if (n <= 0 || k <= 0 || k % 16 != 0) return -1;
    float amax = 0.0f;
    for (int64_t i = 0; i < n * k; ++i) {
        float a = fabsf(W[i]);
        if (!isfinite(a)) return -2;
        if (a > amax) amax = a;
    }
    const float s_g = amax / 2688.0f;
    *global_scale = s_g;
    const int64_t ng = k / 16;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const float *w = W + r * k + 16 * g;
            float a = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(w[i]) > a) a = fabsf(w[i]);
            unsigned e = 0;
            if (s_g != 0.0f) {
                float t = (a / 6.0f) / s_g;
                e = nvo_e4m3_encode(t);
            }
            scales[r * ng + g] = (uint8_t)e;
            const float S = nvo_e4m3_value(e) * s_g;
            for (int i = 0; i < 16; i += 2) {
                unsigned lo = (S == 0.0f) ? 0u : nvo_e2m1_encode(w[i] / S);
                unsigned hi = (S == 0.0f) ? 0u : nvo_e2m1_encode(w[i + 1] / S);
                codes[r * (k / 2) + 8 * g + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* ---- dequantization: D = fp32(fp32(e2m1 * e4m3) * s_g) ---- */

static float dequant_one(const uint8_t *codes, const uint8_t *scales, float s_g,
                         int64_t k, int64_t r, int64_t c)
{
    unsigned byte = codes[r * (k / 2) + c / 2];
    unsigned code = (c & 1) ? (byte >> 4) : (byte & 15u);
    /* the product has at most 6 significant bits: exact in double and float */
    float cs = (float)(nvo_e2m1_value(code) * (double)nvo_e4m3_value(scales[r * (k / 16) + c / 16]));
    return cs * s_g;
}

void nvo_dequant(const uint8_t *codes, const uint8_t *scales, float global_scale,
                 int64_t n, int64_t k, float *D)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            D[r * k + c] = dequant_one(codes, scales, global_scale, k, r, c);
}

/* ---- projection: y = sum_k D[n][k] x[r][k] in fp64, ascending k ---- */

static void gemv_row(const uint8_t *codes, const uint8_t *scales, float s_g,
                     int64_t k, int64_t feat, const uint16_t *x, int rows,
                     float *drow, double *yv, double *av)
{
    for (int64_t c = 0; c < k; ++c)
        drow[c] = dequant_one(codes, scales, s_g, k, feat, c);
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            double p = (double)drow[c] * nvo_bf16_value(x[r * k + c]);
            acc += p;
            aacc += fabs(p);
        }
        yv[r] = acc;
        av[r] = aacc;
    }
}

int nvo_gemv(const uint8_t *codes, const uint8_t *scales, float global_scale,
             int64_t n, int64_t k, const uint16_t *x, int rows,
             const int64_t *sel, int64_t nsel,
             double *y, double *absdot, uint16_t *y_bf16)
{
    if (rows < 1 || rows > NVO_MAX_ROWS || n < 1 || k < 16 || k % 16) return -1;
    if (!sel) nsel = n;
#pragma omp parallel
    {
        float *drow = (float *)malloc(sizeof(float) * (size_t)k);
        double yv[NVO_MAX_ROWS], av[NVO_MAX_ROWS];
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nsel; ++j) {
            int64_t feat = sel ? sel[j] : j;
            gemv_row(codes, scales, global_scale, k, feat, x, rows, drow, yv, av);
            for (int r = 0; r < rows; ++r) {
                if (y) y[r * nsel + j] = yv[r];
                if (absdot) absdot[r * nsel + j] = av[r];
                if (y_bf16) y_bf16[r * nsel + j] = nvo_bf16_from_double(yv[r]);
            }
        }
        free(drow);
    }
    return 0;
}

/* ---- projection as the plain fp32 definition: dequantize, then
 * y32 = sum_k D[n][k] * x[r][k] with one fp32 rounding per multiply and per
 * add, starting from +0.0f, ascending k; y16 = bf16 RNE of y32 ---- */
int nvo_gemv_f32seq(const uint8_t *codes, const uint8_t *scales, float global_scale,
                    int64_t n, int64_t k, const uint16_t *x, int rows,
                    const int64_t *sel, int64_t nsel, float *y32, uint16_t *y_bf16)
{
    if (rows < 1 || rows > NVO_MAX_ROWS || n < 1 || k < 16 || k % 16) return -1;
    if (!sel) nsel = n;
#pragma omp parallel
    {
        float *drow = (float *)malloc(sizeof(float) * (size_t)k);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nsel; ++j) {
            int64_t feat = sel ? sel[j] : j;
            for (int64_t c = 0; c < k; ++c)
                drow[c] = dequant_one(codes, scales, global_scale, k, feat, c);
            for (int r = 0; r < rows; ++r) {
                float acc = 0.0f;
                for (int64_t c = 0; c < k; ++c) {
                    float p = drow[c] * (float)nvo_bf16_value(x[r * k + c]);
                    acc = acc + p;
                }
                if (y32) y32[r * nsel + j] = acc;
                if (y_bf16) y_bf16[r * nsel + j] = nvo_bf16_from_double((double)acc);
            }
        }
        free(drow);
    }
    return 0;
}

/* ---- gate/up pair: o = silu(g) * u = g / (1 + exp(-g)) * u, fp64 ---- */

int nvo_gemv_dual_silu(const uint8_t *g_codes, const uint8_t *g_scales, float g_global,
                       const uint8_t *u_codes, const uint8_t *u_scales, float u_global,
                       int64_t n, int64_t k, const uint16_t *x, int rows,
                       const int64_t *sel, int64_t nsel,
                       double *o, double *g, double *u, double *abs_g, double *abs_u,
                       uint16_t *o_bf16)
{
    if (rows < 1 || rows > NVO_MAX_ROWS || n < 1 || k < 16 || k % 16) return -1;
    if (!sel) nsel = n;
#pragma omp parallel
    {
        float *drow = (float *)malloc(sizeof(float) * (size_t)k);
        double gv[NVO_MAX_ROWS], ga[NVO_MAX_ROWS], uv[NVO_MAX_ROWS], ua[NVO_MAX_ROWS];
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nsel; ++j) {
            int64_t feat = sel ? sel[j] : j;
            gemv_row(g_codes, g_scales, g_global, k, feat, x, rows, drow, gv, ga);
            gemv_row(u_codes, u_scales, u_global, k, feat, x, rows, drow, uv, ua);
            for (int r = 0; r < rows; ++r) {
                double ov = gv[r] / (1.0 + exp(-gv[r])) * uv[r];
                size_t at = (size_t)(r * nsel + j);
                if (o) o[at] = ov;
                if (g) g[at] = gv[r];
                if (u) u[at] = uv[r];
                if (abs_g) abs_g[at] = ga[r];
                if (abs_u) abs_u[at] = ua[r];
                if (o_bf16) o_bf16[at] = nvo_bf16_from_double(ov);
            }
        }
        free(drow);
    }
    return 0;
}

void nvo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int nvo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- dense bf16 projection (the lm head's weights stay bf16: the
 * Qwen3.8-27B-NVFP4 blueprint page, "Precision" table, bf16 x bf16 nodes, and
 * its kernel table, gemv::dense_gemv_bf16):
 * y[r][j] = sum_k W[j][k] x[r][k] in fp64, ascending k ---- */
void nvo_dense_gemv(const uint16_t *W, int64_t n, int64_t k, const uint16_t *x, int rows,
                    const int64_t *sel, int64_t nsel,
                    double *y, double *absdot, uint16_t *y_bf16)
{
    if (!sel) nsel = n;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nsel; ++j) {
        const int64_t feat = sel ? sel[j] : j;
        for (int r = 0; r < rows; ++r) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double p = nvo_bf16_value(W[feat * k + c]) * nvo_bf16_value(x[(int64_t)r * k + c]);
                acc += p;
                aacc += fabs(p);
            }
            if (y) y[r * nsel + j] = acc;
            if (absdot) absdot[r * nsel + j] = aacc;
            if (y_bf16) y_bf16[r * nsel + j] = nvo_bf16_from_double(acc);
        }
    }
}

/* ---- residual add + RMSNorm, the step before a projection (the blueprint
 * page's kernel table: norm::residual_add_rms_norm; kern's gemma_rms_norm is
 * the variant with the Gemma offset).  Per row: v = bf16(r + h) is the new
 * residual stream; x = bf16(v * w' / sqrt(mean(v^2) + eps)) with w' = w, or
 * 1 + w with the offset; fp64 throughout. ---- */
void nvo_residual_rmsnorm(const uint16_t *r, const uint16_t *h, const uint16_t *w, int64_t k, int rows,
                          double eps, int gemma_offset, uint16_t *r_out, uint16_t *x_out, double *inv_rms)
{
    for (int row = 0; row < rows; ++row) {
        const uint16_t *rr = r + (int64_t)row * k, *hh = h + (int64_t)row * k;
        uint16_t *ro = r_out + (int64_t)row * k, *xo = x_out + (int64_t)row * k;
        double ss = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            ro[j] = nvo_bf16_from_double(nvo_bf16_value(rr[j]) + nvo_bf16_value(hh[j]));
            double v = nvo_bf16_value(ro[j]);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / (double)k + eps);
        if (inv_rms) inv_rms[row] = inv;
        for (int64_t j = 0; j < k; ++j) {
            double wj = nvo_bf16_value(w[j]);
            if (gemma_offset) wj += 1.0;
            xo[j] = nvo_bf16_from_double(nvo_bf16_value(ro[j]) * inv * wj);
        }
    }
}

/* ---- MXFP4 (the OCP microscaling format: E2M1 elements, one E8M0
 * power-of-two scale per 32 consecutive k of a row, no tensor scale).  The
 * pages only name it (gpu_mxfp4 kernels in the kern build listing); the
 * readings: the block's shared exponent is floor(log2(amax)) - 2 (2 is
 * E2M1's largest exponent), clamped to E8M0's -127..127; elements are
 * V / 2^X rounded as E2M1 everywhere else here (nearest, ties to the even
 * mantissa, saturating at +-6, sign of zero kept); an all-zero block gets
 * scale byte 127 (2^0) and zero codes; E8M0 byte 255 (NaN) is never
 * produced. ---- */
double nvo_e8m0_value(unsigned b)
{
    return b == 255u ? NAN : ldexp(1.0, (int)b - 127);
}

int nvo_mx_quantize(const float *W, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales)
{
    if (k % 32 != 0) return -1;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(W[i])) return -2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 32; ++b) {
            const float *v = W + r * k + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
            uint8_t *c = codes + r * (k / 2) + b * 16;
            if (amax == 0.0f) {
                scales[r * (k / 32) + b] = 127;
                for (int j = 0; j < 16; ++j) c[j] = 0;
                continue;
            }
            int ex;
            frexp((double)amax, &ex);          /* amax = m 2^ex, 0.5 <= m < 1: floor(log2) = ex - 1 */
            int X = ex - 1 - 2;
            if (X < -127) X = -127;
            if (X > 127) X = 127;
            scales[r * (k / 32) + b] = (uint8_t)(X + 127);
            for (int j = 0; j < 32; j += 2) {
                unsigned lo = nvo_e2m1_encode((float)ldexp((double)v[j], -X));
                unsigned hi = nvo_e2m1_encode((float)ldexp((double)v[j + 1], -X));
                c[j / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    return 0;
}

void nvo_mx_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, double *out)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            unsigned byte = codes[r * (k / 2) + c / 2];
            unsigned code = (c & 1) ? byte >> 4 : byte & 15u;
            out[r * k + c] = nvo_e2m1_value(code) * nvo_e8m0_value(scales[r * (k / 32) + c / 32]);
        }
}

void nvo_mx_gemv(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, const uint16_t *x, int rows,
                 const int64_t *sel, int64_t nsel, double *y, double *absdot, uint16_t *y_bf16)
{
    if (!sel) nsel = n;
#pragma omp parallel
    {
        double *drow = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nsel; ++j) {
            const int64_t feat = sel ? sel[j] : j;
            nvo_mx_dequant(codes + feat * (k / 2), scales + feat * (k / 32), 1, k, drow);
            for (int r = 0; r < rows; ++r) {
                double acc = 0.0, aacc = 0.0;
                for (int64_t c = 0; c < k; ++c) {
                    double p = drow[c] * nvo_bf16_value(x[(int64_t)r * k + c]);
                    acc += p;
                    aacc += fabs(p);
                }
                if (y) y[r * nsel + j] = acc;
                if (absdot) absdot[r * nsel + j] = aacc;
                if (y_bf16) y_bf16[r * nsel + j] = nvo_bf16_from_double(acc);
            }
        }
        free(drow);
    }
}

/* ---- W8G32_F16S (the pages name this encoding for the DFlash2 drafter's
 * matrices and give nothing else): signed 8-bit weights with one fp16 scale
 * per 32 consecutive k of a row, symmetric (no zero point).  Readings: the
 * quantizer takes scale = fp16(amax / 127) (nearest even) and code =
 * rint(w / scale) (ties to even) clamped to +-127; a group whose scale is 0
 * gets codes 0; the weight is code * scale (exact in fp32). ---- */
/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double nvo_f16_value(uint16_t h)
{
    const double sign = (h & 0x8000u) ? -1.0 : 1.0;
    const int e = (h >> 10) & 31, m = h & 1023;
    if (e == 31) return m ? NAN : sign * INFINITY;
    if (e == 0) return sign * ldexp((double)m, -24);
    return sign * ldexp((double)(1024 + m), e - 25);
}

/* float -> binary16, nearest with ties to even (rint in the default mode) */
static uint16_t f16_from_float(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
    const double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);      /* the halfway point above 65504 rounds to even: inf */
    if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)rint(ldexp(a, 24)));   /* subnormal (1024 = 2^-14) */
    int e;
    frexp(a, &e);                                             /* a = m 2^e, 0.5 <= m < 1 */
    double q = rint(ldexp(a, 11 - e));                        /* 1024 .. 2048 */
    if (q == 2048.0) {
        q = 1024.0;
        ++e;
    }
    const int E = e - 1 + 15;
    if (E >= 31) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024));
}

int nvo_w8_quantize(const float *W, int64_t n, int64_t k, int8_t *codes, uint16_t *scales)
{
    if (k % 32 != 0) return -1;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(W[i])) return -2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 32; ++b) {
            const float *v = W + r * k + b * 32;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
            const uint16_t sh = f16_from_float(amax / 127.0f);
            scales[r * (k / 32) + b] = sh;
            const double S = nvo_f16_value(sh);
            for (int j = 0; j < 32; ++j) {
                double q = (S == 0.0 || !isfinite(S)) ? 0.0 : rint((double)v[j] / S);
                if (q > 127.0) q = 127.0;
                if (q < -127.0) q = -127.0;
                codes[r * k + b * 32 + j] = (int8_t)q;
            }
        }
    return 0;
}

void nvo_w8_dequant(const int8_t *codes, const uint16_t *scales, int64_t n, int64_t k, double *out)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            out[r * k + c] = (double)codes[r * k + c] * nvo_f16_value(scales[r * (k / 32) + c / 32]);
}

void nvo_w8_gemv(const int8_t *codes, const uint16_t *scales, int64_t n, int64_t k, const uint16_t *x, int rows,
                 const int64_t *sel, int64_t nsel, double *y, double *absdot, uint16_t *y_bf16)
{
    if (!sel) nsel = n;
#pragma omp parallel
    {
        double *drow = (double *)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < nsel; ++j) {
            const int64_t feat = sel ? sel[j] : j;
            nvo_w8_dequant(codes + feat * k, scales + feat * (k / 32), 1, k, drow);
            for (int r = 0; r < rows; ++r) {
                double acc = 0.0, aacc = 0.0;
                for (int64_t c = 0; c < k; ++c) {
                    double p = drow[c] * nvo_bf16_value(x[(int64_t)r * k + c]);
                    acc += p;
                    aacc += fabs(p);
                }
                if (y) y[r * nsel + j] = acc;
                if (absdot) absdot[r * nsel + j] = aacc;
                if (y_bf16) y_bf16[r * nsel + j] = nvo_bf16_from_double(acc);
            }
        }
        free(drow);
    }
}
