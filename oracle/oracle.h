/*
 * oracle.h - CPU parity oracle for the block-scaled (MXFP4 A4W4 and PTPC FP8
 * A8W8) linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test-suite, the package smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header, table
 * or helper with the HIP library.
 *
 * Plain C11, no fast-math, no FP contraction.  Every function is written from
 * the definition of the format it handles, not for speed:
 *   - MXFP4 storage contract: "Kimi-K3 DSpark O-Proj-only MXFP4", section
 *     "Exact quantization coverage" (E2M1 elements, E8M0 scale per 32
 *     consecutive input-channel values, weight (7168, 8192), scale (7168, 256),
 *     dynamic MXFP4 activations with A4W4 dispatch).
 *   - PTPC FP8 contract: "Kimi-K3-DSpark-FP8-PTPC", section "Phase 1 FP8 PTPC
 *     Quantization" (E4M3 weights, FP32 per-output-channel scale of shape
 *     (out_features, 1), dynamic per-token FP8 activations computed online).
 *   - "OCP MXFP4" is the standard named by "Kimi-K3-Quark-MXFP4-AttnFP8",
 *     sections "Model Overview" and "Model Quantization"; the numeric rules the
 *     pages leave open (shared exponent floor(log2 amax) - 2, round to nearest
 *     even, saturation, NaN/zero handling, nibble order) are the readings listed
 *     beside each function below.
 *
 * Layouts (all row-major, contiguous):
 *   activations X [rows, K]; weights W [N, K] (out x in); output Y [M, N],
 *   Y = X . W^T, no bias.
 *   MXFP4 codes [rows, K/2] bytes: element 2j in the low nibble of byte j,
 *   element 2j+1 in the high nibble.  E8M0 scales [rows, K/32] bytes.
 *   E4M3 codes [rows, K] bytes; FP32 scales [rows].
 *
 * Return codes: 0 ok; ORC_EARG bad argument; ORC_EINEXACT the exactness
 * condition of the FP64 block sum does not hold for some output (see
 * orc_gemm_a4w4_at).
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EINEXACT (-2)

/* ---- element and scale decoders (exact in FP64) ---- */
double orc_e2m1_value(unsigned code);   /* code 0..15: sign<<3 | exp<<1 | man  */
double orc_e8m0_value(unsigned code);   /* 2^(code-127); 0xFF is NaN          */
double orc_e4m3fn_value(unsigned code); /* OCP E4M3 "fn": max 448, no Inf     */
double orc_bf16_value(uint16_t bits);   /* upper half of an IEEE binary32     */

/* ---- element encoders (round to nearest, ties to even, saturating) ---- */
unsigned orc_e2m1_encode(double t);      /* |t| already divided by the scale */
unsigned orc_e4m3fn_encode(double r);

/* ---- MX quantization of one 32-element block ---- */
void orc_mx_block(const double v[32], uint8_t codes[32], uint8_t *scale);

/* ---- row quantizers ---- */
int orc_mx_quant_bf16(const uint16_t *x, int64_t rows, int64_t K,
                      uint8_t *q, uint8_t *s, int nthreads);
int orc_mx_quant_f32(const float *x, int64_t rows, int64_t K,
                     uint8_t *q, uint8_t *s, int nthreads);
int orc_ptpc_quant_bf16(const uint16_t *x, int64_t rows, int64_t K,
                        uint8_t *q, float *s, int nthreads);
int orc_ptpc_quant_f32(const float *x, int64_t rows, int64_t K,
                       uint8_t *q, float *s, int nthreads);

/* ---- exact GEMMs on a grid of selected outputs ----
 * For every i < n_rows and j < n_cols, with m = rows[i] and n = cols[j]:
 *   y[i*n_cols + j]      = exact value of Y[m, n] (one final FP64 rounding)
 *   absdot[i*n_cols + j] = sum over k of |a_k * w_k| with a, w the dequantized
 *                          operands (scales included)
 * absdot may be NULL.  max_span (may be NULL) receives the largest exponent
 * span seen by the A4W4 exactness check. */
int orc_gemm_a4w4_at(const uint8_t *qa, const uint8_t *sa,
                     const uint8_t *qw, const uint8_t *sw,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows,
                     const int64_t *cols, int64_t n_cols,
                     double *y, double *absdot, int *max_span, int nthreads);
int orc_gemm_a8w8_at(const uint8_t *qa, const float *sa,
                     const uint8_t *qw, const float *sw,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t n_rows,
                     const int64_t *cols, int64_t n_cols,
                     double *y, double *absdot, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
