/*
 * qvref.c -- plain, slow CPU oracle for the W4A4 Hadamard-rotated quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY (see qvref.h).  Written for readability against the pages, not speed:
 * the rotation is an explicit fp64 matrix product (or, as an independent second evaluation, a
 * scalar fp64 butterfly transform), the contraction is a triple loop in int64, and the
 * quantization follows the symmetric quantizer step by step.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC qvref.c -lm
 * (-ffp-contract=off keeps every fp32 product and quotient a separately rounded IEEE operation.)
 *
 * Readings of the pages taken here (the equations are missing from [P4]):
 *  - the Hadamard matrix is in Sylvester order and normalised by 1/sqrt(d), so that H H^T = I
 *    ([P4] 预全局旋转 says the matrix times its transpose is the identity);
 *  - the scale of the symmetric quantizer is absmax / (2^(N-1) - 1) and "round" is round half to
 *    even ([P4] 训练后量化（PTQ） gives q = clamp(round(x / s), -2^(N-1), 2^(N-1) - 1));
 *  - the rotated value is held in fp32 before the smoothing multiply and the quantization
 *    decision, because fp32 is the precision the kernel decides the code in;
 *  - a row whose fp32 scale is zero or subnormal quantizes to scale 0 and all-zero codes;
 *  - the smoothing factor is SmoothQuant's form with alpha applied to the rotated statistics
 *    ([P4] 后局部平滑: alpha balances activation and weight difficulty, usually 0.5).
 */
#include "qvref.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static int is_pow2(int64_t d) { return d >= 1 && (d & (d - 1)) == 0; }

static int popcount_u64(uint64_t v) {
    int c = 0;
    while (v) {
        v &= v - 1;
        ++c;
    }
    return c;
}

int qvref_hadamard_closed_form(int64_t d, int8_t* H) {
    if (!H || !is_pow2(d)) return -1;
    for (int64_t i = 0; i < d; ++i)
        for (int64_t j = 0; j < d; ++j)
            H[i * d + j] = (popcount_u64((uint64_t)(i & j)) & 1) ? -1 : 1;
    return 0;
}

int qvref_hadamard_sylvester(int64_t d, int8_t* H) {
    if (!H || !is_pow2(d)) return -1;
    H[0] = 1;
    /* Grow the top-left n x n block to 2n x 2n in place: [[H, H], [H, -H]]. */
    for (int64_t n = 1; n < d; n *= 2) {
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t j = 0; j < n; ++j) {
                int8_t h = H[i * d + j];
                H[i * d + (j + n)] = h;
                H[(i + n) * d + j] = h;
                H[(i + n) * d + (j + n)] = (int8_t)-h;
            }
        }
    }
    return 0;
}

int qvref_rotate_explicit(const double* X, int64_t M, int64_t d, int64_t ldx, double* Y) {
    if ((!X && M > 0) || (!Y && M > 0) || !is_pow2(d) || ldx < d || M < 0) return -1;
    int8_t* H = (int8_t*)malloc((size_t)(d * d));
    if (!H) return -1;
    qvref_hadamard_closed_form(d, H);
    const double norm = 1.0 / sqrt((double)d);
    for (int64_t m = 0; m < M; ++m) {
        const double* x = X + m * ldx;
        double* y = Y + m * d;
        for (int64_t j = 0; j < d; ++j) y[j] = 0.0;
        /* y_j = sum_i x_i H[i][j]; accumulate row by row of H for cache-friendliness. */
        for (int64_t i = 0; i < d; ++i) {
            const double xi = x[i];
            const int8_t* h = H + i * d;
            for (int64_t j = 0; j < d; ++j) y[j] += xi * (double)h[j];
        }
        for (int64_t j = 0; j < d; ++j) y[j] *= norm;
    }
    free(H);
    return 0;
}

int qvref_rotate_fwht(const double* X, int64_t M, int64_t d, int64_t ldx, double* Y) {
    if ((!X && M > 0) || (!Y && M > 0) || !is_pow2(d) || ldx < d || M < 0) return -1;
    const double norm = 1.0 / sqrt((double)d);
    for (int64_t m = 0; m < M; ++m) {
        double* y = Y + m * d;
        memcpy(y, X + m * ldx, (size_t)d * sizeof(double));
        /* Butterflies on index bit h: (u, v) -> (u + v, u - v) with u at the lower index. */
        for (int64_t h = 1; h < d; h *= 2) {
            for (int64_t base = 0; base < d; base += 2 * h) {
                for (int64_t i = base; i < base + h; ++i) {
                    const double u = y[i], v = y[i + h];
                    y[i] = u + v;
                    y[i + h] = u - v;
                }
            }
        }
        for (int64_t j = 0; j < d; ++j) y[j] *= norm;
    }
    return 0;
}

int qvref_quantize_rows(const double* Xhat, int64_t M, int64_t K, const float* mult, int bits,
                        int8_t* q, float* scale) {
    if (M < 0 || K <= 0 || bits < 2 || bits > 8) return -1;
    if (M == 0) return 0;
    if (!Xhat || !q || !scale) return -1;
    const int qmax = (1 << (bits - 1)) - 1;
    const int qmin = -(1 << (bits - 1));
    float* xt = (float*)malloc((size_t)K * sizeof(float));
    if (!xt) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const double* xh = Xhat + m * K;
        /* Smoothed rotated value in fp32, and the row's absolute maximum. */
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float xs = (float)xh[k];
            const float mk = mult ? mult[k] : 1.0f;
            xt[k] = xs * mk;
            const float ax = fabsf(xt[k]);
            if (ax > amax) amax = ax;
        }
        /* Symmetric scale: the row maximum maps to the largest positive code. */
        float s = amax / (float)qmax;
        if (!(s >= FLT_MIN)) s = 0.0f; /* zero or subnormal scale: the row is all zeros */
        scale[m] = s;
        int8_t* qm = q + m * K;
        for (int64_t k = 0; k < K; ++k) {
            if (s == 0.0f) {
                qm[k] = 0;
                continue;
            }
            const float t = xt[k] / s;
            float r = rintf(t); /* round half to even in the default rounding mode */
            if (r > (float)qmax) r = (float)qmax;
            if (r < (float)qmin) r = (float)qmin;
            qm[k] = (int8_t)r;
        }
    }
    free(xt);
    return 0;
}

int qvref_pack_int4(const int8_t* q, int64_t rows, int64_t K, uint8_t* packed) {
    if (rows < 0 || K <= 0 || (K & 1)) return -1;
    if (rows == 0) return 0;
    if (!q || !packed) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < K / 2; ++i) {
            const int lo = q[r * K + 2 * i], hi = q[r * K + 2 * i + 1];
            if (lo < -8 || lo > 7 || hi < -8 || hi > 7) return -1;
            packed[r * (K / 2) + i] = (uint8_t)((lo & 0xF) | ((hi & 0xF) << 4));
        }
    }
    return 0;
}

int qvref_unpack_int4(const uint8_t* packed, int64_t rows, int64_t K, int8_t* q) {
    if (rows < 0 || K <= 0 || (K & 1)) return -1;
    if (rows == 0) return 0;
    if (!q || !packed) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < K / 2; ++i) {
            const int b = packed[r * (K / 2) + i];
            int lo = b & 0xF, hi = (b >> 4) & 0xF;
            if (lo >= 8) lo -= 16; /* two's-complement nibble */
            if (hi >= 8) hi -= 16;
            q[r * K + 2 * i] = (int8_t)lo;
            q[r * K + 2 * i + 1] = (int8_t)hi;
        }
    }
    return 0;
}

int qvref_gemm_int(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!qa || !qw || !acc) return -1;
    int overflow = 0;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return overflow ? -2 : 0;
}

double qvref_gelu(double y) { return 0.5 * y * erfc(-y / sqrt(2.0)); }

int qvref_dequant(const int32_t* acc, const float* sa, const float* sw, const float* bias,
                  int64_t M, int64_t N, int epi, double* Y) {
    if (M < 0 || N < 0 || (epi != 0 && epi != 1)) return -1;
    if (M == 0 || N == 0) return 0;
    if (!acc || !sa || !sw || !Y) return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double y = (double)acc[m * N + n] * (double)sa[m] * (double)sw[n];
            if (bias) y += (double)bias[n];
            if (epi == 1) y = qvref_gelu(y);
            Y[m * N + n] = y;
        }
    }
    return 0;
}

int qvref_smoothing(const double* Xhat, int64_t Mc, const double* What, int64_t N, int64_t K,
                    double alpha, float* s, float* inv_s) {
    if (Mc < 0 || N < 0 || K <= 0 || !(alpha >= 0.0 && alpha <= 1.0)) return -1;
    if (!s || !inv_s || (Mc > 0 && !Xhat) || (N > 0 && !What)) return -1;
    for (int64_t k = 0; k < K; ++k) {
        double ax = 0.0, aw = 0.0;
        for (int64_t m = 0; m < Mc; ++m) ax = fmax(ax, fabs(Xhat[m * K + k]));
        for (int64_t n = 0; n < N; ++n) aw = fmax(aw, fabs(What[n * K + k]));
        double sk = 1.0;
        if (ax > 0.0 && aw > 0.0) sk = pow(ax, alpha) / pow(aw, 1.0 - alpha);
        s[k] = (float)sk;
        inv_s[k] = (float)(1.0 / (double)s[k]);
    }
    return 0;
}

static int rotate(const double* X, int64_t M, int64_t K, int64_t ld, int rot_mode, double* Y) {
    if (rot_mode == 0) return qvref_rotate_explicit(X, M, K, ld, Y);
    if (rot_mode == 1) return qvref_rotate_fwht(X, M, K, ld, Y);
    return -1;
}

/* Rotate, smooth, quantize to 4 bits and pack, one row at a time (bounded memory). */
static int rotate_quant_pack(const double* X, int64_t M, int64_t K, int64_t ld, const float* mult,
                             int rot_mode, uint8_t* out, float* scale) {
    if (M < 0 || K <= 0 || (K & 1) || ld < K || rot_mode < 0 || rot_mode > 1) return -1;
    if (M == 0) return 0;
    if (!X || !out || !scale) return -1;
    double* xh = (double*)malloc((size_t)K * sizeof(double));
    int8_t* q = (int8_t*)malloc((size_t)K);
    int rc = (xh && q) ? 0 : -1;
    for (int64_t m = 0; m < M && rc == 0; ++m) {
        rc = rotate(X + m * ld, 1, K, ld, rot_mode, xh);
        if (rc == 0) rc = qvref_quantize_rows(xh, 1, K, mult, 4, q, scale + m);
        if (rc == 0) rc = qvref_pack_int4(q, 1, K, out + m * (K / 2));
    }
    free(xh);
    free(q);
    return rc;
}

int qvref_hadamard_smooth_quant(const double* X, int64_t M, int64_t K, int64_t ldx,
                                const float* inv_smooth, int rot_mode, uint8_t* Xq, float* x_scale) {
    return rotate_quant_pack(X, M, K, ldx, inv_smooth, rot_mode, Xq, x_scale);
}

int qvref_pack_weights(const double* W, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                       int rot_mode, uint8_t* Wq, float* w_scale) {
    return rotate_quant_pack(W, N, K, ldw, smooth, rot_mode, Wq, w_scale);
}

int qvref_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                    const float* bias, int64_t M, int64_t N, int64_t K, int epi, double* Y,
                    int32_t* acc_out) {
    if (M < 0 || N < 0 || K <= 0 || (K & 1)) return -1;
    if (M == 0 || N == 0) return 0;
    int8_t* qa = (int8_t*)malloc((size_t)(M * K));
    int8_t* qw = (int8_t*)malloc((size_t)(N * K));
    int32_t* acc = acc_out ? acc_out : (int32_t*)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = (qa && qw && acc) ? 0 : -1;
    if (rc == 0) rc = qvref_unpack_int4(Xq, M, K, qa);
    if (rc == 0) rc = qvref_unpack_int4(Wq, N, K, qw);
    if (rc == 0) rc = qvref_gemm_int(qa, qw, M, N, K, acc);
    if (rc == 0) rc = qvref_dequant(acc, x_scale, w_scale, bias, M, N, epi, Y);
    free(qa);
    free(qw);
    if (!acc_out) free(acc);
    return rc;
}

int qvref_w4a4_linear(const double* X, int64_t M, int64_t K, int64_t ldx, const float* inv_smooth,
                      const uint8_t* Wq, const float* w_scale, const float* bias, int64_t N, int epi,
                      int rot_mode, double* Y) {
    if (M < 0 || K <= 0 || (K & 1)) return -1;
    if (M == 0) return 0;
    uint8_t* xq = (uint8_t*)malloc((size_t)(M * (K / 2)));
    float* xs = (float*)malloc((size_t)M * sizeof(float));
    int rc = (xq && xs) ? 0 : -1;
    if (rc == 0) rc = qvref_hadamard_smooth_quant(X, M, K, ldx, inv_smooth, rot_mode, xq, xs);
    if (rc == 0) rc = qvref_w4a4_gemm(xq, xs, Wq, w_scale, bias, M, N, K, epi, Y, NULL);
    free(xq);
    free(xs);
    return rc;
}

/* Group-wise granularity ([P4] 双平滑细粒度量化（DSFQ） > 细粒度量化粒度, truncated on the page;
 * reading: each row of activations and of weights carries one scale per group of `group`
 * consecutive channels of the rotated, smoothed row, and the product sums the groups' integer dot
 * products, each dequantized by its own pair of scales):
 *   Y[m][n] = sum_g (sum_{k in g} qa[m][k] qw[n][k]) * sa[m][g] * sw[n][g] (+ bias[n]), in fp64,
 *   then the erf GELU when epi = 1.  sa is [M][K/group], sw is [N][K/group], both row-major. */
int qvref_dequant_grouped(const int8_t* qa, const int8_t* qw, const float* sa, const float* sw,
                          const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, int epi,
                          double* Y) {
    if (M < 0 || N < 0 || K <= 0 || group <= 0 || K % group != 0 || (epi != 0 && epi != 1)) return -1;
    if (M == 0 || N == 0) return 0;
    if (!qa || !qw || !sa || !sw || !Y) return -1;
    const int64_t groups = K / group;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double y = 0.0;
            for (int64_t g = 0; g < groups; ++g) {
                int64_t acc = 0;
                for (int64_t k = g * group; k < (g + 1) * group; ++k)
                    acc += (int64_t)qa[m * K + k] * qw[n * K + k];
                if (acc > INT32_MAX || acc < INT32_MIN) return -2;
                y += (double)acc * (double)sa[m * groups + g] * (double)sw[n * groups + g];
            }
            if (bias != NULL) y += (double)bias[n];
            if (epi == 1) y = qvref_gelu(y);
            Y[m * N + n] = y;
        }
    }
    return 0;
}
