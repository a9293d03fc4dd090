// rotate_quant.hip -- fused Hadamard rotation, per-channel smoothing, per-row symmetric int4
// quantization and nibble packing (one HBM read of X, one write of the codes and scales).
//
// Method ("十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com)):
//   双平滑细粒度量化（DSFQ） > 预全局旋转: rows are rotated by the Hadamard matrix, X . H / sqrt(K);
//   > 后局部平滑: the rotated value is multiplied by a per-channel factor (1/s for activations,
//     s for weights, folded offline);
//   训练后量化（PTQ）: symmetric quantization q = clamp(round(x / s), -8, 7) with N = 4.
// The scale is absmax / 7 per row (per token for activations, per output channel for weights),
// rounding is to nearest even, and the decision is taken in fp32: x / s is evaluated as
// x * fl(1/s) rounded once to an integer (a fused multiply-add onto 1.5 * 2^23 + 8).  That differs
// from a correctly rounded quotient only when x / s lies within a few ulp of a half-integer.
//
// Work split: K = 1024 puts one row on 16 lanes (4 rows per wave), K = 4096 one row per wave;
// every lane holds 64 values (fwht_regs.h).  Loads are 16-byte per lane and each 16-lane row
// group covers 256 contiguous bytes; every lane writes one packed dword per 8 elements.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "fwht_regs.h"
#include "qv_internal.h"

namespace qv {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kMagic = 12582920.0f;  // 1.5 * 2^23 + 8: its low mantissa byte holds rne(t) + 8

// Load the 64 values of a lane's share of one row into v (fp32 or bf16 source).
template <int K, typename In>
__device__ __forceinline__ void load_row(const In* __restrict__ row, int lane, bool valid, float (&v)[8][8]) {
  constexpr int C = RowLayout<K>::kChunks;
  const int c = load_chunk<K>(lane);
  if constexpr (sizeof(In) == 2) {
    u32x4 raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      raw[j] = valid ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 8 * (c + C * j)))
                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w[4] = {raw[j][0], raw[j][1], raw[j][2], raw[j][3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = __builtin_bit_cast(float, w[i] << 16);
        v[j][2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
      }
    }
  } else {
    f32x4 raw[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x4* p = reinterpret_cast<const f32x4*>(row + 8 * (c + C * j));
      raw[2 * j] = valid ? __builtin_nontemporal_load(p) : f32x4{0.f, 0.f, 0.f, 0.f};
      raw[2 * j + 1] = valid ? __builtin_nontemporal_load(p + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[j][e] = raw[2 * j][e];
        v[j][4 + e] = raw[2 * j + 1][e];
      }
    }
  }
}

// Eight codes (already offset by +8 in the low byte of the magic-rounded floats) -> one dword of
// two's-complement nibbles, element 2i in the low nibble of byte i.
__device__ __forceinline__ uint32_t pack8(const uint32_t (&m)[8]) {
  const uint32_t p01 = (m[1] << 4) + m[0];  // low byte: (q1 + 8) << 4 | (q0 + 8)
  const uint32_t p23 = (m[3] << 4) + m[2];
  const uint32_t p45 = (m[5] << 4) + m[4];
  const uint32_t p67 = (m[7] << 4) + m[6];
  const uint32_t lo = __builtin_amdgcn_perm(p23, p01, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(p67, p45, 0x0c0c0400u);
  return (lo | (hi << 16)) ^ 0x88888888u;  // (q + 8) ^ 8 == q & 0xF for q in [-8, 7]
}

template <int K, typename In>
__global__ __launch_bounds__(kThreads) void rotate_quant_kernel(const In* __restrict__ X, int64_t M, int64_t ldx,
                                                               const float* __restrict__ mult,
                                                               uint8_t* __restrict__ Xq,
                                                               float* __restrict__ x_scale) {
  using L = RowLayout<K>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / L::kLanesPerRow;  // row inside the wave

  // Per-lane multiplier: fold sign * 1/sqrt(K) * smoothing multiplier of the channels this lane
  // owns after the transform (exact: the first two factors are a signed power of two).
  float cm[8][8];
  const float base = fold_sign(lane) * L::kNorm;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k0 = 8 * dword_index<K>(lane, j);
    if (mult) {
      const float4 a = *reinterpret_cast<const float4*>(mult + k0);
      const float4 b = *reinterpret_cast<const float4*>(mult + k0 + 4);
      cm[j][0] = base * a.x; cm[j][1] = base * a.y; cm[j][2] = base * a.z; cm[j][3] = base * a.w;
      cm[j][4] = base * b.x; cm[j][5] = base * b.y; cm[j][6] = base * b.z; cm[j][7] = base * b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) cm[j][e] = base;
    }
  }

  const int64_t groups = (M + L::kRowsPerWave - 1) / L::kRowsPerWave;
  const int64_t wave_stride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wave; g < groups; g += wave_stride) {
    const int64_t row = g * L::kRowsPerWave + sub;
    const bool valid = row < M;
    float v[8][8];
    load_row<K, In>(X + (valid ? row : 0) * ldx, lane, valid, v);

    fwht_row_regs<K>(v, lane);

    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[j][e] *= cm[j][e];
        amax = fmaxf(amax, fabsf(v[j][e]));
      }
    }
    amax = row_max<K>(amax);
    float s = amax / 7.0f;
    if (!(s >= 1.17549435e-38f)) s = 0.0f;  // zero or subnormal scale: all-zero row
    const float r = (s > 0.0f) ? 1.0f / s : 0.0f;

    if (valid) {
      uint32_t* out = reinterpret_cast<uint32_t*>(Xq + row * (K / 2));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = __builtin_bit_cast(uint32_t, __builtin_fmaf(v[j][e], r, kMagic));
        out[dword_index<K>(lane, j)] = pack8(m);
      }
      if ((lane & (L::kLanesPerRow - 1)) == 0) x_scale[row] = s;
    }
  }
}

// Column-wise maximum of |rotated value| over rows (calibration statistics).  Each lane keeps the
// running maxima of the 64 channels it owns; non-negative floats order like their bit patterns,
// so the cross-block combine is an integer atomic max (order-independent, deterministic).
template <int K, typename In>
__global__ __launch_bounds__(kThreads) void rotated_colmax_kernel(const In* __restrict__ X, int64_t M, int64_t ld,
                                                                 unsigned* __restrict__ colmax) {
  using L = RowLayout<K>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / L::kLanesPerRow;
  float mx[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[j][e] = 0.0f;

  const int64_t groups = (M + L::kRowsPerWave - 1) / L::kRowsPerWave;
  const int64_t wave_stride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wave; g < groups; g += wave_stride) {
    const int64_t row = g * L::kRowsPerWave + sub;
    const bool valid = row < M;
    float v[8][8];
    load_row<K, In>(X + (valid ? row : 0) * ld, lane, valid, v);
    fwht_row_regs<K>(v, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[j][e] = fmaxf(mx[j][e], fabsf(v[j][e]) * L::kNorm);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k0 = 8 * dword_index<K>(lane, j);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (mx[j][e] > 0.0f) atomicMax(colmax + k0 + e, __builtin_bit_cast(unsigned, mx[j][e]));
    }
  }
}

// s_k = ax^alpha / aw^(1 - alpha) (1 where either maximum is 0), inv = 1 / s, written over the
// two statistics buffers.
__global__ void smoothing_finalize_kernel(float* __restrict__ s_io, float* __restrict__ inv_io, int64_t K,
                                          float alpha) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const float ax = s_io[k], aw = inv_io[k];
  float s = 1.0f;
  if (ax > 0.0f && aw > 0.0f) s = powf(ax, alpha) / powf(aw, 1.0f - alpha);
  s_io[k] = s;
  inv_io[k] = 1.0f / s;
}

__global__ void zero_kernel(unsigned* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int grid_for_rows(int64_t M, int rows_per_wave) {
  const int64_t groups = (M + rows_per_wave - 1) / rows_per_wave;
  const int64_t blocks = (groups + (kThreads / 64) - 1) / (kThreads / 64);
  const int64_t cap = 256 * 8;  // enough resident waves to cover HBM latency; rows loop beyond
  return (int)(blocks < cap ? blocks : cap);
}

template <int K, typename In>
hipError_t launch_rq(const void* X, int64_t M, int64_t ld, const float* mult, uint8_t* q, float* scale,
                     hipStream_t st) {
  const int grid = grid_for_rows(M, RowLayout<K>::kRowsPerWave);
  hipLaunchKernelGGL((rotate_quant_kernel<K, In>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const In*>(X), M, ld, mult, q, scale);
  return hipGetLastError();
}

template <int K, typename In>
hipError_t launch_colmax(const void* X, int64_t M, int64_t ld, unsigned* colmax, hipStream_t st) {
  const int grid = grid_for_rows(M, RowLayout<K>::kRowsPerWave);
  hipLaunchKernelGGL((rotated_colmax_kernel<K, In>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const In*>(X), M, ld, colmax);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const void* X, bool bf16, int64_t M, int64_t K, int64_t ld, const float* mult,
                               uint8_t* q, float* scale, hipStream_t st) {
  if (K == 1024) {
    return bf16 ? launch_rq<1024, uint16_t>(X, M, ld, mult, q, scale, st)
                : launch_rq<1024, float>(X, M, ld, mult, q, scale, st);
  }
  return bf16 ? launch_rq<4096, uint16_t>(X, M, ld, mult, q, scale, st)
              : launch_rq<4096, float>(X, M, ld, mult, q, scale, st);
}

hipError_t launch_smooth_calibrate(const void* Xc, bool xbf16, int64_t Mc, int64_t ldx, const void* W, bool wbf16,
                                   int64_t N, int64_t ldw, int64_t K, float alpha, float* smooth,
                                   float* inv_smooth, hipStream_t st) {
  unsigned* ax = reinterpret_cast<unsigned*>(smooth);
  unsigned* aw = reinterpret_cast<unsigned*>(inv_smooth);
  const int zb = (int)((K + 255) / 256);
  hipLaunchKernelGGL(zero_kernel, dim3(zb), dim3(256), 0, st, ax, K);
  hipLaunchKernelGGL(zero_kernel, dim3(zb), dim3(256), 0, st, aw, K);
  hipError_t e;
  if (K == 1024) {
    e = xbf16 ? launch_colmax<1024, uint16_t>(Xc, Mc, ldx, ax, st) : launch_colmax<1024, float>(Xc, Mc, ldx, ax, st);
    if (e != hipSuccess) return e;
    e = wbf16 ? launch_colmax<1024, uint16_t>(W, N, ldw, aw, st) : launch_colmax<1024, float>(W, N, ldw, aw, st);
  } else {
    e = xbf16 ? launch_colmax<4096, uint16_t>(Xc, Mc, ldx, ax, st) : launch_colmax<4096, float>(Xc, Mc, ldx, ax, st);
    if (e != hipSuccess) return e;
    e = wbf16 ? launch_colmax<4096, uint16_t>(W, N, ldw, aw, st) : launch_colmax<4096, float>(W, N, ldw, aw, st);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(smoothing_finalize_kernel, dim3(zb), dim3(256), 0, st, smooth, inv_smooth, K, alpha);
  return hipGetLastError();
}

}  // namespace qv
