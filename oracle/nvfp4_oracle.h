/*
 * nvfp4_oracle.h -- CPU oracle for weight-only NVFP4 projection GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this code; only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg do.  It shares no
 * source with the HIP path.
 *
 * What it computes (plain loops, host pointers, no blocking or fusion):
 *   - E2M1 element codes and OCP E4M3 group scales (encode + decode);
 *   - the NVFP4 "g16" quantizer: FP32 tensor scale amax/(448*6), one E4M3
 *     scale per 16 consecutive weights of a row, E2M1 round-to-nearest-even;
 *   - dequantization D = fp32(fp32(e2m1 * e4m3) * s_g);
 *   - the projection y[r][n] = sum_k D[n][k] * x[r][k] in fp64 (an FP64
 *     reference per projection class, as the TensorFold issue #603 thread asks
 *     for), with sum_k |D*x| for tolerances and a bf16 round-to-nearest-even copy;
 *   - the same projection as the plain fp32 definition (dequantize, then a
 *     sequential fp32 dot product in ascending k);
 *   - the gate/up pair o = silu(g) * u in fp64 (the SwiGLU FFN of the
 *     Qwen3.8-27B-NVFP4 blueprint page, "w4a16_gemv_dual" kernels).
 *
 * Format source: the Qwen3.8-27B-NVFP4 blueprint page, "Precision" table
 * (weights nvfp4/g16, activations bf16) and its "Kernels" table (w4a16_gemv
 * family).  The pages name the format but never define its arithmetic; the
 * definition used here (E2M1 set {0,+-0.5,+-1,+-1.5,+-2,+-3,+-4,+-6}, OCP
 * E4M3 group scale, FP32 tensor scale amax/(448*6), RNE) is the format's
 * standard one.  Every choice the definition leaves open is listed as a
 * "reading" in the comments of nvfp4_oracle.c.
 *
 * Layouts (canonical, row-major):
 *   codes  [n][k/2]  byte j of row r holds element 2j in its low nibble and
 *                    element 2j+1 in its high nibble;
 *   scales [n][k/16] one OCP E4M3 byte per group of 16 consecutive k;
 *   x      [rows][k] bf16 bit patterns (uint16);
 *   y      [rows][nsel] (nsel = n when sel == NULL).
 * k must be a positive multiple of 16.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

double   nvo_e2m1_value(unsigned code);
unsigned nvo_e2m1_encode(float v);   /* v not NaN (the quantizer rejects non-finite weights first) */
float    nvo_e4m3_value(unsigned byte);
unsigned nvo_e4m3_encode(float v);
double   nvo_bf16_value(uint16_t h);
uint16_t nvo_bf16_from_double(double v);

/* returns 0, or -1 for bad shape, -2 for a non-finite weight */
int  nvo_quantize(const float *W, int64_t n, int64_t k, uint8_t *codes,
                  uint8_t *scales, float *global_scale);
void nvo_dequant(const uint8_t *codes, const uint8_t *scales, float global_scale,
                 int64_t n, int64_t k, float *D);
/* Projections take 1..NVO_MAX_ROWS activation rows and return 0, or -1 (and
 * compute nothing) for rows outside that range or a bad shape. */
#define NVO_MAX_ROWS 64
int  nvo_gemv(const uint8_t *codes, const uint8_t *scales, float global_scale,
              int64_t n, int64_t k, const uint16_t *x, int rows,
              const int64_t *sel, int64_t nsel,
              double *y, double *absdot, uint16_t *y_bf16);
/* The same projection as the plain fp32 definition: D in fp32, then
 * sum_k D*x with one fp32 rounding per multiply and add, ascending k from
 * +0.0f; y32 fp32 and its bf16 RNE copy, [rows][nsel]. */
int  nvo_gemv_f32seq(const uint8_t *codes, const uint8_t *scales, float global_scale,
                     int64_t n, int64_t k, const uint16_t *x, int rows,
                     const int64_t *sel, int64_t nsel, float *y32, uint16_t *y_bf16);
int  nvo_gemv_dual_silu(const uint8_t *g_codes, const uint8_t *g_scales, float g_global,
                        const uint8_t *u_codes, const uint8_t *u_scales, float u_global,
                        int64_t n, int64_t k, const uint16_t *x, int rows,
                        const int64_t *sel, int64_t nsel,
                        double *o, double *g, double *u, double *abs_g, double *abs_u,
                        uint16_t *o_bf16);
int  nvo_num_threads(void);
void nvo_set_num_threads(int n);   /* OpenMP threads of the projections (results do not depend on it) */

/* Dense bf16 projection: W bf16 [n][k], x bf16 [rows][k]; y, |D.x| sums and a
 * bf16 copy of y for the selected features (sel NULL: all), [rows][nsel]. */
void nvo_dense_gemv(const uint16_t *W, int64_t n, int64_t k, const uint16_t *x, int rows,
                    const int64_t *sel, int64_t nsel,
                    double *y, double *absdot, uint16_t *y_bf16);

/* Residual add + RMSNorm per row: r_out = bf16(r + h), x = bf16(r_out * w' /
 * sqrt(mean(r_out^2) + eps)), w' = w or 1 + w (gemma_offset); inv_rms
 * (optional) receives 1 / sqrt(mean + eps) per row. */
void nvo_residual_rmsnorm(const uint16_t *r, const uint16_t *h, const uint16_t *w, int64_t k, int rows,
                          double eps, int gemma_offset, uint16_t *r_out, uint16_t *x_out, double *inv_rms);

/* MXFP4: E2M1 codes [n][k/2] (low nibble first) + E8M0 scales [n][k/32]. */
double nvo_e8m0_value(unsigned b);
int nvo_mx_quantize(const float *W, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales);
void nvo_mx_dequant(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, double *out);
void nvo_mx_gemv(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, const uint16_t *x, int rows,
                 const int64_t *sel, int64_t nsel, double *y, double *absdot, uint16_t *y_bf16);

/* W8G32_F16S: int8 codes [n][k] + fp16 scale bits [n][k/32], symmetric. */
double nvo_f16_value(uint16_t h);
int nvo_w8_quantize(const float *W, int64_t n, int64_t k, int8_t *codes, uint16_t *scales);
void nvo_w8_dequant(const int8_t *codes, const uint16_t *scales, int64_t n, int64_t k, double *out);
void nvo_w8_gemv(const int8_t *codes, const uint16_t *scales, int64_t n, int64_t k, const uint16_t *x, int rows,
                 const int64_t *sel, int64_t nsel, double *y, double *absdot, uint16_t *y_bf16);

#ifdef __cplusplus
}
#endif
#endif
