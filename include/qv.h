/*
 * qv.h -- C ABI of libqv, an MI355X (gfx950) library for the W4A4 Hadamard-rotated, smoothed,
 * int4-quantized linear layer of QuantVGGT (and, at the end of this file, its W8A8 variant and a
 * variant with group-wise scales).
 *
 * Sources, cited by page title and section:
 *   [P4] "十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), a translation of the QuantVGGT
 *        paper's method:  训练后量化（PTQ） -- the symmetric N-bit quantizer
 *        q = clamp(round(x / s), -2^(N-1), 2^(N-1) - 1);  双平滑细粒度量化（DSFQ） > 预全局旋转 --
 *        rotate activations and weights by a Hadamard matrix (H H^T = I keeps the product);
 *        > 后局部平滑 -- per-channel smoothing factors with alpha (usually 0.5) taken from the
 *        rotated distribution, divided out of activations and folded into weights.
 *   [P3] the lsdiaocha.cn write-up of the paper: W4A4 (4-bit weights and activations).
 *
 * What one linear computes (rows of X are tokens, K is the input width and the Hadamard width):
 *   Xhat = X . H_K / sqrt(K)                       (Sylvester-order Hadamard, K in {1024, 4096})
 *   Xt[m][k] = Xhat[m][k] * inv_smooth[k]
 *   x_scale[m] = max_k |Xt[m][k]| / 7,  Xq[m][k] = clamp(rne(Xt[m][k] / x_scale[m]), -8, 7)
 *   acc[m][n] = sum_k Xq[m][k] * Wq[n][k]           (exact, int32)
 *   Y[m][n] = acc[m][n] * x_scale[m] * w_scale[n] (+ bias[n]),  optionally GELU(y) = y * Phi(y)
 * and the offline weight step applies the same rotation to the rows of W, multiplies by smooth[k]
 * and quantizes per output channel.  Scales are fp32; the quantization decision is taken in fp32.
 * A row whose fp32 scale would be zero or subnormal gets scale 0 and all-zero codes.
 *
 * Packed int4 layout (Xq, Wq): row-major, K/2 bytes per row, byte i of a row holds the
 * two's-complement code of element 2i in its low nibble and of element 2i+1 in its high nibble.
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers, allocated and owned by the caller.  The library allocates
 *     nothing, frees nothing and keeps no pointer after returning.
 *   - hip_stream is a hipStream_t passed as void* (NULL = the default stream).  Every call is
 *     asynchronous and ordered on that stream; the library never synchronizes.  A call only
 *     launches kernels (no allocation, memset, copy or synchronization), so calls may be recorded
 *     into a HIP graph by stream capture and replayed.
 *   - All argument checks run on the host before any HIP call; a failed check returns its status and
 *     launches nothing.  M == 0 (or N == 0) is a valid no-op returning QV_OK.
 *   - Leading dimensions are in elements.  Base pointers must be 16-byte aligned and every row
 *     stride a multiple of 16 bytes.
 *   - Inputs must be finite; results for rows holding Inf or NaN are unspecified.
 *   - Kernels use no atomics on the hot path; results are deterministic run to run.
 *   - Nothing throws across the ABI.  A HIP launch error is returned as QV_ERR_HIP.
 */
#ifndef QV_H
#define QV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QV_OK = 0,
  QV_ERR_NULL = 1,        /* a required pointer is NULL */
  QV_ERR_SHAPE = 2,       /* a size is negative, unsupported, or a leading dimension is too small */
  QV_ERR_UNSUPPORTED = 3, /* the request is well formed but outside what the kernels implement */
  QV_ERR_ALIGN = 4,       /* a pointer or row stride is not 16-byte aligned */
  QV_ERR_DTYPE = 5,       /* unknown dtype or epilogue value */
  QV_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the matching *_linear_workspace_size() */
  QV_ERR_HIP = 7,         /* the HIP runtime reported an error when launching */
  QV_ERR_INTERNAL = 8     /* an unexpected internal error */
} qv_status;

typedef enum { QV_F32 = 0, QV_BF16 = 1 } qv_dtype;

typedef enum { QV_EPI_NONE = 0, QV_EPI_GELU = 1 } qv_epilogue;

/* Human-readable name of a status code (static storage; never NULL). */
const char* qv_status_string(qv_status s);

/*
 * qv_hadamard_smooth_quant -- online activation step ([P4] 预全局旋转, 后局部平滑, 训练后量化（PTQ）).
 *   X          [M][ldx] fp32 or bf16 (x_dtype), row-major; only the first K columns are read.
 *   K          Hadamard width = row width, 1024 or 4096 (else QV_ERR_UNSUPPORTED).
 *   inv_smooth [K] fp32 per-channel multiplier applied after the rotation (1 / smoothing factor);
 *              NULL means all ones (rotation only).
 *   Xq         [M][K/2] packed int4 codes (output).
 *   x_scale    [M] fp32 per-token scales (output).
 */
qv_status qv_hadamard_smooth_quant(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const float* inv_smooth, uint8_t* Xq, float* x_scale,
                                   void* hip_stream);

/*
 * qv_pack_weights -- offline weight step ([P4] 预全局旋转: weights are rotated by the same H;
 * 后局部平滑: the smoothing factor is folded into the weights).  The same kernel as the activation
 * step, with smooth[k] as the per-channel multiplier and one output channel per row.
 *   W       [N][ldw] fp32 or bf16 (w_dtype): row n holds output channel n over the K inputs.
 *   K       1024 or 4096.
 *   smooth  [K] fp32 smoothing factors s_k (NULL = ones).
 *   Wq      [N][K/2] packed int4 codes (output);  w_scale [N] fp32 per-channel scales (output).
 */
qv_status qv_pack_weights(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                          const float* smooth, uint8_t* Wq, float* w_scale, void* hip_stream);

/*
 * qv_w4a4_gemm -- int4 x int4 contraction with int32 accumulation and a fused dequantization
 * epilogue ([P3]: W4A4;  [P4] 训练后量化（PTQ）: symmetric scales make dequantization one product).
 *   Xq [M][K/2], x_scale [M], Wq [N][K/2], w_scale [N] as produced by the two calls above.
 *   bias [N] fp32 or NULL.
 *   K  multiple of 128 in [128, 65536] (the accumulator stays exact);  N multiple of 128;  M >= 0.
 *   epi QV_EPI_NONE or QV_EPI_GELU (GELU(y) = 0.5 y erfc(-y / sqrt 2), applied after the bias).
 *   Y  [M][ldy] fp32 or bf16 (y_dtype, bf16 rounded to nearest even), ldy >= N, and a row of
 *      ldy outputs below 2^24 bytes (else QV_ERR_UNSUPPORTED).
 */
qv_status qv_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                       const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                       qv_dtype y_dtype, int64_t ldy, void* hip_stream);

/* Bytes of workspace qv_w4a4_linear needs for M rows of width K: the packed codes and the scales,
 * each region rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t qv_w4a4_linear_workspace_size(int64_t M, int64_t K);

/*
 * qv_w4a4_linear -- the whole online layer: qv_hadamard_smooth_quant into the caller's workspace,
 * then qv_w4a4_gemm.  Arguments as for those two calls; workspace is a device buffer of at least
 * qv_w4a4_linear_workspace_size(M, K) bytes, 256-byte aligned, reused freely by later calls.
 */
qv_status qv_w4a4_linear(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const uint8_t* Wq, const float* w_scale,
                         const float* bias, int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of workspace qv_w4a4_gemm_requant needs for M rows: one counter per 128-row stripe,
 * rounded up to 256 bytes (0 for invalid sizes). */
size_t qv_w4a4_gemm_requant_workspace_size(int64_t M);

/*
 * qv_w4a4_gemm_requant -- qv_w4a4_gemm with bf16 outputs that also prepares the next linear's
 * input: every output row is rotated, smoothed and quantized exactly as qv_hadamard_smooth_quant
 * would do to Y, without a second pass over Y in HBM.  This is the MLP's fc1 -> GELU -> H_4096 ->
 * int4 step ([P4] 预全局旋转 and 后局部平滑 applied to the next layer's input, 训练后量化（PTQ）; the
 * intermediate is bf16, rounded to nearest even, as qv_w4a4_gemm stores it).
 *   Xq, x_scale, Wq, w_scale, bias, M, K, epi   as for qv_w4a4_gemm.
 *   N               1024 or 4096: the output width, which is the next layer's Hadamard width.
 *   Y               [M][ldy] bf16 outputs, as qv_w4a4_gemm writes them (they are also read back).
 *   inv_smooth_next [N] fp32 factors of the next layer (1 / smoothing), NULL = ones.
 *   Xq_next         [M][N/2] packed int4 codes;  x_scale_next [M] fp32 per-row scales (outputs),
 *                   identical to qv_hadamard_smooth_quant(Y, bf16, M, N, ldy, inv_smooth_next, ...).
 *   workspace       at least qv_w4a4_gemm_requant_workspace_size(M) bytes, 256-byte aligned, cleared
 *                   by the call itself (a fill kernel) and reused freely by later calls.
 * The tiles of a 128-row stripe finish in any order; the block that finishes a stripe's last
 * tile quantizes the stripe's rows after an agent-scope acquire that pairs with every tile's
 * release.  No block waits for another.
 */
qv_status qv_w4a4_gemm_requant(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                               const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                               int64_t ldy, const float* inv_smooth_next, uint8_t* Xq_next, float* x_scale_next,
                               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of the static device scratch array behind qv_w4a4_linear_noalloc, one copy per GPU. */
#define QV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * qv_w4a4_linear_noalloc -- qv_w4a4_linear for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Arguments,
 * rules and results are those of qv_w4a4_linear; the packed codes and per-row scales go to a
 * static device array inside the library instead of a caller workspace.
 *   Limit: qv_w4a4_linear_workspace_size(M, K) <= QV_NOALLOC_SCRATCH_BYTES (32 MiB), i.e. up to
 *   65027 rows at K = 1024 and 16352 rows at K = 4096; larger calls return QV_ERR_WORKSPACE and
 *   launch nothing.
 *   The call allocates and frees nothing.  Each GPU the library runs on holds its own copy of the
 *   array until the process ends; the first call on a device looks up that copy's device address
 *   (hipGetSymbolAddress) and caches it.
 *   Every call on one GPU uses that GPU's one array, which keeps the last call's contents (the
 *   codes and scales are fully rewritten before they are read, so nothing needs clearing).  Calls
 *   on one stream are ordered and safe; calls that overlap in time on one GPU (several streams,
 *   several host threads) race on the array and give undefined results.
 */
qv_status qv_w4a4_linear_noalloc(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 const float* inv_smooth, const uint8_t* Wq, const float* w_scale,
                                 const float* bias, int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype,
                                 int64_t ldy, void* hip_stream);

/*
 * qv_smooth_calibrate -- smoothing factors from rotated statistics ([P4] 后局部平滑: the factor is
 * computed from the distribution after the Hadamard rotation, alpha balances the two sides):
 *   s_k = (max_m |Xhat_c[m][k]|)^alpha / (max_n |What[n][k]|)^(1 - alpha),  s_k = 1 if either max is 0,
 *   inv_smooth[k] = 1 / s_k,
 * where Xhat_c are the rotated calibration rows Xc [Mc][ldx] and What the rotated weight rows
 * W [N][ldw] (both fp32 or bf16, width K in {1024, 4096}).  alpha in [0, 1].
 *   smooth, inv_smooth  [K] fp32 outputs; both are also used as scratch by the call.
 * Mc >= 1 and N >= 1.
 */
qv_status qv_smooth_calibrate(const void* Xc, qv_dtype xc_dtype, int64_t Mc, int64_t ldx, const void* W,
                              qv_dtype w_dtype, int64_t N, int64_t ldw, int64_t K, float alpha,
                              float* smooth, float* inv_smooth, void* hip_stream);

/*
 * W8A8: the pages' second setting ([P3]: W8A8 next to W4A4;  [P4] 训练后量化（PTQ） with N = 8).
 * The same rotation, smoothing and per-token / per-output-channel scales, with
 *   scale = max |Xt| / 127,  q = clamp(rne(Xt / scale), -128, 127),
 * one two's-complement int8 code per byte, row-major, K bytes per row (Xq8, Wq8).
 *
 * qv_hadamard_smooth_quant8 / qv_pack_weights8 -- as qv_hadamard_smooth_quant / qv_pack_weights
 *   (same arguments and rules), writing int8 codes [M][K] / [N][K].
 */
qv_status qv_hadamard_smooth_quant8(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                    const float* inv_smooth, int8_t* Xq8, float* x_scale, void* hip_stream);
qv_status qv_pack_weights8(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                           const float* smooth, int8_t* Wq8, float* w_scale, void* hip_stream);

/*
 * qv_w8a8_gemm -- int8 x int8 contraction (int32 accumulation, exact) with the epilogue of
 * qv_w4a4_gemm.  Xq8 [M][K], Wq8 [N][K] int8;  K a multiple of 64 in [64, 65536];  N a multiple of
 * 128;  other arguments and rules as for qv_w4a4_gemm.
 */
qv_status qv_w8a8_gemm(const int8_t* Xq8, const float* x_scale, const int8_t* Wq8, const float* w_scale,
                       const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                       qv_dtype y_dtype, int64_t ldy, void* hip_stream);

/* Workspace of qv_w8a8_linear: M*K code bytes and 4*M scale bytes, each rounded up to 256 bytes
 * (0 for invalid sizes). */
size_t qv_w8a8_linear_workspace_size(int64_t M, int64_t K);

/* qv_w8a8_linear -- qv_hadamard_smooth_quant8 into the workspace, then qv_w8a8_gemm; arguments and
 * workspace rules as for qv_w4a4_linear. */
qv_status qv_w8a8_linear(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const int8_t* Wq8, const float* w_scale,
                         const float* bias, int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype,
                         int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Group-wise granularity ([P4] 双平滑细粒度量化（DSFQ） > 细粒度量化粒度; the subsection is truncated on
 * the page).  Reading: the rotation and smoothing are unchanged (pre-global, over the whole row);
 * each row of activations and of weights is quantized in groups of `group` consecutive channels
 * of the rotated, smoothed row, each group with its own symmetric scale:
 *   scale[r][g] = max_{k in group g} |Xt[r][k]| / 7,  q = clamp(rne(Xt / scale[r][g]), -8, 7)
 * (a zero or subnormal group scale gives scale 0 and zero codes), and the product sums the groups'
 * integer dot products, each dequantized by its own pair of scales:
 *   Y[m][n] = sum_g (sum_{k in g} qa[m][k] qw[n][k]) * x_scale[m][g] * w_scale[n][g] (+ bias[n])
 * (+ GELU), accumulated in fp32.  Codes use the int4 layout above; scales are row-major
 * [rows][K / group] fp32.  group is 128, 256 or 512 and divides K, with K / group <= 32.
 *
 * qv_hadamard_smooth_quant_grouped / qv_pack_weights_grouped -- as qv_hadamard_smooth_quant /
 *   qv_pack_weights (same arguments and rules, K in {1024, 4096}), writing x_scale [M][K / group]
 *   / w_scale [N][K / group].  An unsupported group returns QV_ERR_UNSUPPORTED.
 */
qv_status qv_hadamard_smooth_quant_grouped(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                           const float* inv_smooth, int64_t group, uint8_t* Xq, float* x_scale,
                                           void* hip_stream);
qv_status qv_pack_weights_grouped(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                                  const float* smooth, int64_t group, uint8_t* Wq, float* w_scale,
                                  void* hip_stream);

/*
 * qv_w4a4_gemm_grouped -- the int4 x int4 contraction with group-wise dequantization: each
 * group's int32 dot products (exact) times x_scale[m][g] w_scale[n][g], summed over the groups in
 * fp32, then bias and GELU as in qv_w4a4_gemm.  x_scale [M][K / group], w_scale [N][K / group];
 * other arguments and rules as for qv_w4a4_gemm.
 */
qv_status qv_w4a4_gemm_grouped(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                               const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, qv_epilogue epi,
                               void* Y, qv_dtype y_dtype, int64_t ldy, void* hip_stream);

/* Workspace of qv_w4a4_linear_grouped: M*K/2 code bytes and 4*M*(K/group) scale bytes, each
 * rounded up to 256 bytes (0 for invalid sizes). */
size_t qv_w4a4_linear_grouped_workspace_size(int64_t M, int64_t K, int64_t group);

/* qv_w4a4_linear_grouped -- qv_hadamard_smooth_quant_grouped into the workspace, then
 * qv_w4a4_gemm_grouped; arguments and workspace rules as for qv_w4a4_linear. */
qv_status qv_w4a4_linear_grouped(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 const float* inv_smooth, int64_t group, const uint8_t* Wq, const float* w_scale,
                                 const float* bias, int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype,
                                 int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* QV_H */
