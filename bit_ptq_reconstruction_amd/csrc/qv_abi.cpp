// qv_abi.cpp -- the C ABI of libqv (declared in include/qv.h): host-side argument checks, then the
// kernel launches on the caller's stream.  Every check runs before the first HIP call, so a
// rejected call launches nothing and touches no device state.
#include "qv.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qv_internal.h"

namespace {

constexpr int64_t kAlign = 16;
// Largest row count or leading dimension accepted (2^40): far beyond any device memory, and small
// enough that every byte count formed from them below stays inside int64 / size_t.
constexpr int64_t kMaxDim = int64_t{1} << 40;

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

int64_t dtype_bytes(qv_dtype t) { return t == QV_BF16 ? 2 : 4; }

bool valid_dtype(qv_dtype t) { return t == QV_F32 || t == QV_BF16; }

// Shared checks of the rotate-quantize step (activation or weight side).
qv_status check_rotate_quant(const void* X, qv_dtype dt, int64_t rows, int64_t K, int64_t ld, const float* mult,
                             const void* q, const float* scale) {
  if (!valid_dtype(dt)) return QV_ERR_DTYPE;
  if (rows < 0 || K <= 0 || rows > kMaxDim) return QV_ERR_SHAPE;
  if (K != 1024 && K != 4096) return QV_ERR_UNSUPPORTED;
  if (ld < K || ld > kMaxDim) return QV_ERR_SHAPE;
  if (rows == 0) return QV_OK;
  if (!X || !q || !scale) return QV_ERR_NULL;
  if (!aligned(X) || !aligned(q) || !aligned(scale) || !aligned(mult) || ((ld * dtype_bytes(dt)) % kAlign) != 0)
    return QV_ERR_ALIGN;
  return QV_OK;
}

// k_step: 128 for packed int4 operands (one 64-byte stage), 64 for int8 operands.
qv_status check_gemm(const void* Xq, const float* xs, const void* Wq, const float* ws, const float* bias,
                     int64_t M, int64_t N, int64_t K, qv_epilogue epi, const void* Y, qv_dtype yt, int64_t ldy,
                     int64_t k_step = 128) {
  if (!valid_dtype(yt) || (epi != QV_EPI_NONE && epi != QV_EPI_GELU)) return QV_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || M > kMaxDim || N > kMaxDim) return QV_ERR_SHAPE;
  if ((K % k_step) != 0 || K > 65536 || (N % 128) != 0) return QV_ERR_UNSUPPORTED;
  if (ldy < N) return QV_ERR_SHAPE;
  // output rows below 16 MiB: the epilogue addresses a tile's rows with 32-bit offsets
  if (ldy >= (int64_t{1} << 24) / dtype_bytes(yt)) return QV_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QV_OK;
  if (!Xq || !xs || !Wq || !ws || !Y) return QV_ERR_NULL;
  if (!aligned(Xq) || !aligned(xs) || !aligned(Wq) || !aligned(ws) || !aligned(bias) || !aligned(Y) ||
      ((ldy * dtype_bytes(yt)) % kAlign) != 0)
    return QV_ERR_ALIGN;
  return QV_OK;
}

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Group sizes of the group-wise variant: 128, 256 or 512 channels, dividing K, at most
// qv::kMaxGroups groups per row.
qv_status check_group(int64_t K, int64_t group) {
  if (group != 128 && group != 256 && group != 512) return QV_ERR_UNSUPPORTED;
  if (K <= 0 || (K % group) != 0 || K / group > qv::kMaxGroups) return QV_ERR_UNSUPPORTED;
  return QV_OK;
}

qv_status hip_status(hipError_t e) { return e == hipSuccess ? QV_OK : QV_ERR_HIP; }

}  // namespace

extern "C" {

const char* qv_status_string(qv_status s) {
  switch (s) {
    case QV_OK: return "QV_OK";
    case QV_ERR_NULL: return "QV_ERR_NULL: a required pointer is NULL";
    case QV_ERR_SHAPE: return "QV_ERR_SHAPE: negative size or leading dimension smaller than the row";
    case QV_ERR_UNSUPPORTED: return "QV_ERR_UNSUPPORTED: size outside what the kernels implement";
    case QV_ERR_ALIGN: return "QV_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case QV_ERR_DTYPE: return "QV_ERR_DTYPE: unknown dtype or epilogue";
    case QV_ERR_WORKSPACE: return "QV_ERR_WORKSPACE: workspace missing or too small";
    case QV_ERR_HIP: return "QV_ERR_HIP: HIP runtime error at launch";
    case QV_ERR_INTERNAL: return "QV_ERR_INTERNAL: unexpected internal error";
  }
  return "unknown qv_status";
}

qv_status qv_hadamard_smooth_quant(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const float* inv_smooth, uint8_t* Xq, float* x_scale, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, Xq, x_scale);
    if (st != QV_OK || M == 0) return st;
    return hip_status(qv::launch_rotate_quant(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth, Xq, x_scale, 4,
                                              static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_pack_weights(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                          uint8_t* Wq, float* w_scale, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(W, w_dtype, N, K, ldw, smooth, Wq, w_scale);
    if (st != QV_OK || N == 0) return st;
    return hip_status(qv::launch_rotate_quant(W, w_dtype == QV_BF16, N, K, ldw, smooth, Wq, w_scale, 4,
                                              static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                       const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                       qv_dtype y_dtype, int64_t ldy, void* hip_stream) {
  try {
    qv_status st = check_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, Y, y_dtype, ldy);
    if (st != QV_OK || M == 0 || N == 0) return st;
    return hip_status(qv::launch_w4a4_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y,
                                           y_dtype == QV_BF16, ldy, static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

size_t qv_w4a4_linear_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K <= 0 || (K % 2) != 0 || M > kMaxDim || K > kMaxDim) return 0;
  return round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2)) + round256(static_cast<size_t>(M) * 4);
}

qv_status qv_w4a4_linear(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const uint8_t* Wq, const float* w_scale, const float* bias,
                         int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  try {
    // Validate both steps up front so that nothing is launched when either would be rejected.
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, reinterpret_cast<uint8_t*>(16),
                                      reinterpret_cast<float*>(16));
    if (st != QV_OK) return st;
    st = check_gemm(reinterpret_cast<uint8_t*>(16), reinterpret_cast<float*>(16), Wq, w_scale, bias, M, N, K, epi,
                    Y, y_dtype, ldy);
    if (st != QV_OK) return st;
    if (M == 0 || N == 0) return QV_OK;
    const size_t need = qv_w4a4_linear_workspace_size(M, K);
    if (!workspace || workspace_bytes < need) return QV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % 256) != 0) return QV_ERR_ALIGN;
    uint8_t* xq = static_cast<uint8_t*>(workspace);
    float* xs = reinterpret_cast<float*>(xq + round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2)));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = hip_status(qv::launch_rotate_quant(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth, xq, xs, 4, s));
    if (st != QV_OK) return st;
    return hip_status(
        qv::launch_w4a4_gemm(xq, xs, Wq, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y, y_dtype == QV_BF16, ldy, s));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_w4a4_linear_noalloc(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 const float* inv_smooth, const uint8_t* Wq, const float* w_scale, const float* bias,
                                 int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype, int64_t ldy,
                                 void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, reinterpret_cast<uint8_t*>(16),
                                      reinterpret_cast<float*>(16));
    if (st != QV_OK) return st;
    st = check_gemm(reinterpret_cast<uint8_t*>(16), reinterpret_cast<float*>(16), Wq, w_scale, bias, M, N, K, epi,
                    Y, y_dtype, ldy);
    if (st != QV_OK) return st;
    if (M == 0 || N == 0) return QV_OK;
    // The codes and scales must fit the static array (checked on the host, before any HIP call).
    const size_t need = qv_w4a4_linear_workspace_size(M, K);
    if (need == 0 || need > QV_NOALLOC_SCRATCH_BYTES) return QV_ERR_WORKSPACE;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    st = hip_status(qv::noalloc_scratch(&ws, &ws_bytes));
    if (st != QV_OK) return st;
    if (ws_bytes < need) return QV_ERR_WORKSPACE;
    uint8_t* xq = static_cast<uint8_t*>(ws);
    float* xs = reinterpret_cast<float*>(xq + round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2)));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = hip_status(qv::launch_rotate_quant(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth, xq, xs, 4, s));
    if (st != QV_OK) return st;
    return hip_status(
        qv::launch_w4a4_gemm(xq, xs, Wq, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y, y_dtype == QV_BF16, ldy, s));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

size_t qv_w4a4_gemm_requant_workspace_size(int64_t M) {
  if (M < 0 || M > kMaxDim) return 0;
  return round256(static_cast<size_t>((M + 127) / 128) * 4);
}

qv_status qv_w4a4_gemm_requant(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                               const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                               int64_t ldy, const float* inv_smooth_next, uint8_t* Xq_next, float* x_scale_next,
                               void* workspace, size_t workspace_bytes, void* hip_stream) {
  try {
    qv_status st = check_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, Y, QV_BF16, ldy);
    if (st != QV_OK) return st;
    if (N != 1024 && N != 4096) return QV_ERR_UNSUPPORTED;  // the next layer's Hadamard width
    if (M == 0) return QV_OK;
    if (!Xq_next || !x_scale_next) return QV_ERR_NULL;
    if (!aligned(Xq_next) || !aligned(x_scale_next) || !aligned(inv_smooth_next)) return QV_ERR_ALIGN;
    const size_t need = qv_w4a4_gemm_requant_workspace_size(M);
    if (!workspace || workspace_bytes < need) return QV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % 256) != 0) return QV_ERR_ALIGN;
    return hip_status(qv::launch_w4a4_gemm_requant(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y,
                                                   ldy, inv_smooth_next, Xq_next, x_scale_next,
                                                   static_cast<unsigned*>(workspace),
                                                   static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_smooth_calibrate(const void* Xc, qv_dtype xc_dtype, int64_t Mc, int64_t ldx, const void* W,
                              qv_dtype w_dtype, int64_t N, int64_t ldw, int64_t K, float alpha, float* smooth,
                              float* inv_smooth, void* hip_stream) {
  try {
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return QV_ERR_SHAPE;
    if (Mc < 1 || N < 1) return QV_ERR_SHAPE;
    qv_status st = check_rotate_quant(Xc, xc_dtype, Mc, K, ldx, nullptr, reinterpret_cast<uint8_t*>(16),
                                      reinterpret_cast<float*>(16));
    if (st != QV_OK) return st;
    st = check_rotate_quant(W, w_dtype, N, K, ldw, nullptr, reinterpret_cast<uint8_t*>(16),
                            reinterpret_cast<float*>(16));
    if (st != QV_OK) return st;
    if (!smooth || !inv_smooth) return QV_ERR_NULL;
    if (!aligned(smooth) || !aligned(inv_smooth)) return QV_ERR_ALIGN;
    return hip_status(qv::launch_smooth_calibrate(Xc, xc_dtype == QV_BF16, Mc, ldx, W, w_dtype == QV_BF16, N, ldw, K,
                                                  alpha, smooth, inv_smooth, static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_hadamard_smooth_quant8(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                    const float* inv_smooth, int8_t* Xq8, float* x_scale, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, Xq8, x_scale);
    if (st != QV_OK || M == 0) return st;
    return hip_status(qv::launch_rotate_quant(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth,
                                              reinterpret_cast<uint8_t*>(Xq8), x_scale, 8,
                                              static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_pack_weights8(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, const float* smooth,
                           int8_t* Wq8, float* w_scale, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(W, w_dtype, N, K, ldw, smooth, Wq8, w_scale);
    if (st != QV_OK || N == 0) return st;
    return hip_status(qv::launch_rotate_quant(W, w_dtype == QV_BF16, N, K, ldw, smooth,
                                              reinterpret_cast<uint8_t*>(Wq8), w_scale, 8,
                                              static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_w8a8_gemm(const int8_t* Xq8, const float* x_scale, const int8_t* Wq8, const float* w_scale,
                       const float* bias, int64_t M, int64_t N, int64_t K, qv_epilogue epi, void* Y,
                       qv_dtype y_dtype, int64_t ldy, void* hip_stream) {
  try {
    qv_status st = check_gemm(Xq8, x_scale, Wq8, w_scale, bias, M, N, K, epi, Y, y_dtype, ldy, 64);
    if (st != QV_OK || M == 0 || N == 0) return st;
    return hip_status(qv::launch_w8a8_gemm(Xq8, x_scale, Wq8, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y,
                                           y_dtype == QV_BF16, ldy, static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

size_t qv_w8a8_linear_workspace_size(int64_t M, int64_t K) {
  if (M < 0 || K <= 0 || M > kMaxDim || K > kMaxDim) return 0;
  return round256(static_cast<size_t>(M) * static_cast<size_t>(K)) + round256(static_cast<size_t>(M) * 4);
}

qv_status qv_w8a8_linear(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                         const float* inv_smooth, const int8_t* Wq8, const float* w_scale, const float* bias,
                         int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype, int64_t ldy, void* workspace,
                         size_t workspace_bytes, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, reinterpret_cast<uint8_t*>(16),
                                      reinterpret_cast<float*>(16));
    if (st != QV_OK) return st;
    st = check_gemm(reinterpret_cast<int8_t*>(16), reinterpret_cast<float*>(16), Wq8, w_scale, bias, M, N, K, epi, Y,
                    y_dtype, ldy, 64);
    if (st != QV_OK) return st;
    if (M == 0 || N == 0) return QV_OK;
    const size_t need = qv_w8a8_linear_workspace_size(M, K);
    if (!workspace || workspace_bytes < need) return QV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % 256) != 0) return QV_ERR_ALIGN;
    int8_t* xq = static_cast<int8_t*>(workspace);
    float* xs = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) +
                                         round256(static_cast<size_t>(M) * static_cast<size_t>(K)));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = hip_status(qv::launch_rotate_quant(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth,
                                            reinterpret_cast<uint8_t*>(xq), xs, 8, s));
    if (st != QV_OK) return st;
    return hip_status(
        qv::launch_w8a8_gemm(xq, xs, Wq8, w_scale, bias, M, N, K, epi == QV_EPI_GELU, Y, y_dtype == QV_BF16, ldy, s));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

// ------------------------------------------------------------------ group-wise granularity

qv_status qv_hadamard_smooth_quant_grouped(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                           const float* inv_smooth, int64_t group, uint8_t* Xq, float* x_scale,
                                           void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, Xq, x_scale);
    if (st == QV_OK) st = check_group(K, group);
    if (st != QV_OK || M == 0) return st;
    return hip_status(qv::launch_rotate_quant_grouped(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth, group, Xq,
                                                      x_scale, static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_pack_weights_grouped(const void* W, qv_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                                  const float* smooth, int64_t group, uint8_t* Wq, float* w_scale,
                                  void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(W, w_dtype, N, K, ldw, smooth, Wq, w_scale);
    if (st == QV_OK) st = check_group(K, group);
    if (st != QV_OK || N == 0) return st;
    return hip_status(qv::launch_rotate_quant_grouped(W, w_dtype == QV_BF16, N, K, ldw, smooth, group, Wq, w_scale,
                                                      static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

qv_status qv_w4a4_gemm_grouped(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                               const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, qv_epilogue epi,
                               void* Y, qv_dtype y_dtype, int64_t ldy, void* hip_stream) {
  try {
    qv_status st = check_gemm(Xq, x_scale, Wq, w_scale, bias, M, N, K, epi, Y, y_dtype, ldy);
    if (st == QV_OK) st = check_group(K, group);
    if (st != QV_OK || M == 0 || N == 0) return st;
    return hip_status(qv::launch_w4a4_gemm_grouped(Xq, x_scale, Wq, w_scale, bias, M, N, K, group,
                                                   epi == QV_EPI_GELU, Y, y_dtype == QV_BF16, ldy,
                                                   static_cast<hipStream_t>(hip_stream)));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

size_t qv_w4a4_linear_grouped_workspace_size(int64_t M, int64_t K, int64_t group) {
  if (M < 0 || M > kMaxDim || check_group(K, group) != QV_OK) return 0;
  return round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2)) +
         round256(static_cast<size_t>(M) * static_cast<size_t>(K / group) * 4);
}

qv_status qv_w4a4_linear_grouped(const void* X, qv_dtype x_dtype, int64_t M, int64_t K, int64_t ldx,
                                 const float* inv_smooth, int64_t group, const uint8_t* Wq, const float* w_scale,
                                 const float* bias, int64_t N, qv_epilogue epi, void* Y, qv_dtype y_dtype,
                                 int64_t ldy, void* workspace, size_t workspace_bytes, void* hip_stream) {
  try {
    qv_status st = check_rotate_quant(X, x_dtype, M, K, ldx, inv_smooth, reinterpret_cast<uint8_t*>(16),
                                      reinterpret_cast<float*>(16));
    if (st == QV_OK) st = check_group(K, group);
    if (st != QV_OK) return st;
    st = check_gemm(reinterpret_cast<uint8_t*>(16), reinterpret_cast<float*>(16), Wq, w_scale, bias, M, N, K, epi,
                    Y, y_dtype, ldy);
    if (st != QV_OK) return st;
    if (M == 0 || N == 0) return QV_OK;
    const size_t need = qv_w4a4_linear_grouped_workspace_size(M, K, group);
    if (!workspace || workspace_bytes < need) return QV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) % 256) != 0) return QV_ERR_ALIGN;
    uint8_t* xq = static_cast<uint8_t*>(workspace);
    float* xs = reinterpret_cast<float*>(xq + round256(static_cast<size_t>(M) * static_cast<size_t>(K / 2)));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    st = hip_status(qv::launch_rotate_quant_grouped(X, x_dtype == QV_BF16, M, K, ldx, inv_smooth, group, xq, xs, s));
    if (st != QV_OK) return st;
    return hip_status(qv::launch_w4a4_gemm_grouped(xq, xs, Wq, w_scale, bias, M, N, K, group, epi == QV_EPI_GELU, Y,
                                                   y_dtype == QV_BF16, ldy, s));
  } catch (...) {
    return QV_ERR_INTERNAL;
  }
}

}  // extern "C"
