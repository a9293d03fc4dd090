/*
 * qvref.h -- plain CPU oracle for the W4A4 Hadamard-rotated, smoothed, int4-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or call this library:
 * only tests, the package smoke check and the benchmark's CPU-baseline leg do. It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * Sources (cited by page title and section; the text of the pages, not their line numbers):
 *   [P4] "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com) -- a translation of the QuantVGGT
 *        paper's method.  Sections used: 训练后量化（PTQ） (the symmetric N-bit quantizer),
 *        双平滑细粒度量化（DSFQ） > 预全局旋转 (Hadamard rotation and matmul invariance),
 *        > 后局部平滑 (per-channel smoothing with alpha, taken from the rotated distribution),
 *        > 细粒度量化粒度 (granularity; truncated on the page).
 *   [P3] the lsdiaocha.cn write-up of "Quantized Visual Geometry Grounded Transformer"
 *        (arXiv:2509.21302): W4A4 / W8A8 settings, rotate-then-scale ablation.
 * The equations themselves were stripped from [P4]; where a step is left open, the reading taken
 * is stated at the function that implements it.
 *
 * Conventions: row-major arrays, leading dimension in elements; all pointers are host pointers
 * owned by the caller.  Every function returns 0 on success and a negative code on bad arguments
 * (-1) or on an int32 overflow of the accumulator (-2).
 */
#ifndef QVREF_H
#define QVREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sylvester-order Hadamard matrix by its closed form H[i][j] = (-1)^popcount(i & j). d = 2^n. */
int qvref_hadamard_closed_form(int64_t d, int8_t* H);
/* The same matrix by the Sylvester recursion H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]. */
int qvref_hadamard_sylvester(int64_t d, int8_t* H);

/* Y[m][:] = X[m][:] . H_d / sqrt(d) in fp64 by the explicit matrix product ([P4] 预全局旋转). */
int qvref_rotate_explicit(const double* X, int64_t M, int64_t d, int64_t ldx, double* Y);
/* The same rotation by an in-place scalar fast Walsh-Hadamard transform in fp64. */
int qvref_rotate_fwht(const double* X, int64_t M, int64_t d, int64_t ldx, double* Y);

/* Per-row symmetric quantization of rotated rows ([P4] 训练后量化（PTQ）), decided in fp32:
 *   xs = fl32(Xhat); xt = fl32(xs * mult[k]); a = max_k |xt|; s = fl32(a / (2^(bits-1) - 1));
 *   if s is zero or subnormal: s = 0 and every code is 0;
 *   else q = clamp(rne(fl32(xt / s)), -2^(bits-1), 2^(bits-1) - 1).
 * mult may be NULL (all ones).  bits in {2..8}. */
int qvref_quantize_rows(const double* Xhat, int64_t M, int64_t K, const float* mult, int bits,
                        int8_t* q, float* scale);

/* Two's-complement nibble packing: byte i of a row = (q[2i] & 0xF) | ((q[2i+1] & 0xF) << 4). */
int qvref_pack_int4(const int8_t* q, int64_t rows, int64_t K, uint8_t* packed);
int qvref_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, int8_t* q);

/* acc[m][n] = sum_k qa[m][k] * qw[n][k], accumulated in int64; -2 if any sum leaves int32. */
int qvref_gemm_int(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K, int32_t* acc);

/* Y[m][n] = acc[m][n] * sa[m] * sw[n] (+ bias[n]) in fp64; epi = 1 applies the erf GELU. */
int qvref_dequant(const int32_t* acc, const float* sa, const float* sw, const float* bias,
                  int64_t M, int64_t N, int epi, double* Y);
/* GELU(y) = y * Phi(y), evaluated as 0.5 * y * erfc(-y / sqrt(2)). */
double qvref_gelu(double y);

/* Smoothing factors from the rotated statistics ([P4] 后局部平滑):
 *   s_k = (max_m |Xhat[m][k]|)^alpha / (max_n |What[n][k]|)^(1 - alpha), s_k = 1 if either max is 0;
 *   s is stored as fp32 and inv_s[k] = fl32(1 / s_k). */
int qvref_smoothing(const double* Xhat, int64_t Mc, const double* What, int64_t N, int64_t K,
                    double alpha, float* s, float* inv_s);

/* Whole steps, mirroring the HIP library's entry points.  rot_mode 0 = explicit matrix, 1 = FWHT. */
int qvref_hadamard_smooth_quant(const double* X, int64_t M, int64_t K, int64_t ldx,
                                const float* inv_smooth, int rot_mode, uint8_t* Xq, float* x_scale);
int qvref_pack_weights(const double* W, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                       int rot_mode, uint8_t* Wq, float* w_scale);
int qvref_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                    const float* bias, int64_t M, int64_t N, int64_t K, int epi, double* Y,
                    int32_t* acc_out);
int qvref_w4a4_linear(const double* X, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                      const uint8_t* Wq, const float* w_scale, const float* bias, int64_t N, int epi,
                      int rot_mode, double* Y);

/* Group-wise granularity ([P4] 细粒度量化粒度; the subsection is truncated, see the reading in the
 * implementation): Y[m][n] = sum_g (sum_{k in group g} qa[m][k] qw[n][k]) * sa[m][g] * sw[n][g]
 * (+ bias[n]) in fp64, then the erf GELU when epi = 1.  qa [M][K], qw [N][K] int8 codes;
 * sa [M][K/group], sw [N][K/group]; group divides K. */
int qvref_dequant_grouped(const int8_t* qa, const int8_t* qw, const float* sa, const float* sw,
                          const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, int epi,
                          double* Y);

#ifdef __cplusplus
}
#endif
#endif
