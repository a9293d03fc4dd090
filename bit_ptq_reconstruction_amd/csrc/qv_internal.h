// qv_internal.h -- launchers shared between the kernels' translation units and the C ABI layer.
// Arguments are validated by the ABI layer (qv_abi.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qv {

// Rotate (Hadamard width K in {1024, 4096}), multiply by mult[k] (NULL = 1), quantize each row to
// `bits` in {4, 8} with scale absmax / (2^(bits-1) - 1): int4 codes packed two per byte (even k in
// the low nibble), int8 codes one per byte.  The activation step and, with the smoothing factors as
// mult, the weight step.
hipError_t launch_rotate_quant(const void* X, bool bf16, int64_t M, int64_t K, int64_t ld, const float* mult,
                               uint8_t* q, float* scale, int bits, hipStream_t st);

// Int4 x int4 GEMM (N % 128 == 0, K % 128 == 0) with dequantization epilogue.
hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                            const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out,
                            int64_t ldy, hipStream_t st);

// The int4 GEMM with bf16 outputs (N in {1024, 4096}) that also rotates, smooths (mult_next [N])
// and quantizes every finished row stripe of its output for the next linear: q_next [M][N / 2],
// scale_next [M].  counters: ceil(M / 128) unsigned of scratch, cleared by the call.
hipError_t launch_w4a4_gemm_requant(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                                    const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y,
                                    int64_t ldy, const float* mult_next, uint8_t* q_next, float* scale_next,
                                    unsigned* counters, hipStream_t st);

// Group-wise variant of the rotate-quantize step: one scale per row and group of `group` in
// {128, 256, 512} channels, scale[row][K / group].
hipError_t launch_rotate_quant_grouped(const void* X, bool bf16, int64_t M, int64_t K, int64_t ld, const float* mult,
                                       int64_t group, uint8_t* q, float* scale, hipStream_t st);

// Int4 x int4 GEMM with group-wise scales (xs [M][K / group], ws [N][K / group], group in
// {128, 256, 512}, K / group <= kMaxGroups): each group's integer dot products dequantized by its
// own pair of scales and summed in fp32, then the same epilogue.
constexpr int kMaxGroups = 32;
hipError_t launch_w4a4_gemm_grouped(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                                    const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, bool gelu,
                                    void* Y, bool bf16_out, int64_t ldy, hipStream_t st);

// Int8 x int8 GEMM (N % 128 == 0, K % 64 == 0) with the same epilogue.
hipError_t launch_w8a8_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                            const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out,
                            int64_t ldy, hipStream_t st);

// Device address (on the current device) and size of the library's static scratch array, used
// by qv_w4a4_linear_noalloc in place of a caller workspace.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Smoothing factors from rotated column maxima of calibration rows and weight rows.
hipError_t launch_smooth_calibrate(const void* Xc, bool xbf16, int64_t Mc, int64_t ldx, const void* W, bool wbf16,
                                   int64_t N, int64_t ldw, int64_t K, float alpha, float* smooth,
                                   float* inv_smooth, hipStream_t st);

}  // namespace qv
