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
// Two kernels.  The butterfly kernel (rotate_quant_kernel) runs every log2(K) stage on the vector
// ALU: K = 1024 puts one row on 16 lanes (4 rows per wave), K = 4096 one row per wave, and every
// lane holds 64 values (fwht_regs.h).  The matrix-core kernel (rotate_quant_mfma_kernel), used for
// bf16 rows of width 4096 with one scale per row, forms the first five stages as an exact-operand
// bf16 MFMA product with H_32 and the rest as butterflies (see its comment).  In both, loads are
// 16-byte per lane over contiguous 256-byte or larger runs, and every lane writes one packed dword
// per 8 elements.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include <atomic>

#include "fwht_regs.h"
#include "qv_internal.h"
#include "rq_mfma.h"

namespace qv {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Waves per SIMD the K = 4096 kernel is compiled for: 5 (96 registers, no spills) measured 2 %
// faster than 4 (116 registers); the K = 1024 kernel fits 96 registers at the default.
#ifndef QV_RQ_WAVES
#define QV_RQ_WAVES 5
#endif
#ifndef QV_RQM_WAVES
#define QV_RQM_WAVES 3  // waves per SIMD of the width-4096 matrix-core kernel (134 registers with the prefetch)
#endif
#ifndef QV_RQ_MFMA
#define QV_RQ_MFMA 1  // 1: bf16 rows of width 4096 with one scale per row use the matrix-core kernel
#endif
#ifndef QV_RQM_LANES_1024
// a-values per DPP row of the width-1024 matrix-core kernel: 8 (2 rows per wave, 32 values per
// lane, 96 registers, 5 waves) measured 5 % faster than the butterfly kernel; 4 (4 rows per wave,
// 64 values, 151 registers, 3 waves) measured level with it, and 16 (one row per wave, 16 values,
// 64 registers, 8 waves) 4-6 % slower than 8.
#define QV_RQM_LANES_1024 8
#endif
#ifndef QV_RQM_WAVES_1024
#define QV_RQM_WAVES_1024 (QV_RQM_LANES_1024 == 8 ? 5 : 3)
#endif
#ifndef QV_RQ_MFMA_1024
#define QV_RQ_MFMA_1024 1  // 1: bf16 rows of width 1024 with one scale per row use the matrix-core kernel
#endif
#ifndef QV_RQ_PREFETCH
#define QV_RQ_PREFETCH 0  // 1: keep the next row group's raw data in registers (3 waves/SIMD instead of 4)
#endif

constexpr int kThreads = 256;

// Raw 16-byte chunks of a lane's share of one row: 8 chunks for bf16, 16 for fp32.
template <typename In>
struct RawRow {
  static constexpr int kChunks = (sizeof(In) == 2) ? 8 : 16;
  u32x4 c[kChunks];
};

template <int K, typename In>
__device__ __forceinline__ void load_raw(const In* __restrict__ row, int lane, RawRow<In>& r) {
  constexpr int C = RowLayout<K>::kChunks;
  const int c = load_chunk<K>(lane);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row + 8 * (c + C * j));
    if constexpr (sizeof(In) == 2) {
      r.c[j] = __builtin_nontemporal_load(p);
    } else {
      r.c[2 * j] = __builtin_nontemporal_load(p);
      r.c[2 * j + 1] = __builtin_nontemporal_load(p + 1);
    }
  }
}

template <typename In>
__device__ __forceinline__ void unpack_raw(const RawRow<In>& r, float (&v)[8][8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (sizeof(In) == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = r.c[j][i];
        v[j][2 * i] = __builtin_bit_cast(float, w << 16);
        v[j][2 * i + 1] = __builtin_bit_cast(float, w & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // Copy each element to a scalar before reinterpreting it: a bit-cast applied directly to
        // a vector element reads the vector's first element.
        const uint32_t lo = r.c[2 * j][i], hi = r.c[2 * j + 1][i];
        v[j][i] = __builtin_bit_cast(float, lo);
        v[j][4 + i] = __builtin_bit_cast(float, hi);
      }
    }
  }
}

template <int K, typename In>
__device__ __forceinline__ void load_row(const In* __restrict__ row, int lane, float (&v)[8][8]) {
  RawRow<In> r;
  load_raw<K, In>(row, lane, r);
  unpack_raw<In>(r, v);
}

// Per-lane multiplier table in LDS: row p holds, for the lanes at DPP-row position p (K = 1024) or
// lane p (K = 4096), the 64 factors fold_sign * 1/sqrt(K) * mult[k] of the channels that lane owns
// after the transform, in v[j][e] order (rows padded to kCmStride floats).

template <int K>
__device__ __forceinline__ void fill_multiplier_table(const float* __restrict__ mult, float* cm) {
  using L = RowLayout<K>;
  constexpr int kRows = (K == 1024) ? 16 : 64;
  for (int idx = threadIdx.x; idx < kRows * 64; idx += kThreads) {
    const int p = idx >> 6, r = idx & 63, j = r >> 3, e = r & 7;
    const int k = 8 * dword_index<K>(p, j) + e;
    cm[p * kCmStride + r] = fold_sign(p) * L::kNorm * (mult ? mult[k] : 1.0f);
  }
}

// Maximum over the 16 lanes of a DPP row.
__device__ __forceinline__ float lanes16_max(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true)));
  return x;
}

// Group-wise scales (kGroup = 128, 256 or 512 channels; 0 = one scale per row).  After the
// transform register group j of a lane holds 8 consecutive channels 8 dword_index(lane, j) + 0..7,
// and the 16 lanes of a DPP row hold the 16 chunks of one aligned 128-channel block, so a
// 128-channel group is one j across a DPP row; 256 channels pair j with j ^ 1 and 512 channels
// join j, j ^ 1, j ^ 2 (dword_index(lane, j) / 16 steps by one with j bit 0 and by two with j bit 1,
// for both widths).  A group's maximum is therefore an in-lane max over those j and a max over the
// DPP row, and its index is 8 dword_index / kGroup.
template <int K, int kGroup>
__device__ __forceinline__ int group_of(int lane, int j) {
  return 8 * dword_index<K>(lane & ~15, j) / kGroup;
}

template <int K, typename In, int kBits, int kGroup>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(K == 4096 ? QV_RQ_WAVES : 4))) void rotate_quant_kernel(const In* __restrict__ X, int64_t M, int64_t ldx,
                                                               const float* __restrict__ mult,
                                                               uint8_t* __restrict__ Xq,
                                                               float* __restrict__ x_scale) {
  static_assert(kGroup == 0 || kGroup == 128 || kGroup == 256 || kGroup == 512, "group size");
  static_assert(kGroup == 0 || kBits == 4, "group-wise scales are built for 4-bit codes");
  constexpr int kJoin = kGroup == 512 ? 3 : (kGroup == 256 ? 1 : 0);  // j bits joined in a group
  using L = RowLayout<K>;
  __shared__ __attribute__((aligned(16))) float cm_lds[(K == 1024 ? 16 : 64) * kCmStride];
  const int lane = threadIdx.x & 63;
  // The wave index, hence the row group, is uniform; readfirstlane keeps the group's addresses in
  // scalar registers, and each lane adds a 32-bit offset.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane / L::kLanesPerRow;  // row inside the wave
  const float* cm_row = cm_lds + (K == 1024 ? (lane & 15) : lane) * kCmStride;

  const int64_t groups = (M + L::kRowsPerWave - 1) / L::kRowsPerWave;
  const int64_t wave_stride = (int64_t)gridDim.x * (kThreads / 64);
  int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wave;

  // Rows past the end are clamped to the last row (loaded, transformed, never stored), so every
  // load is unconditional and no lane diverges before the stores.
  // The lane's row as (uniform first row of the group) + (row inside the group, clamped).
  auto row_ptr = [&](int64_t grp) {
    const int64_t r0 = grp * L::kRowsPerWave;
    const int64_t r = r0 + sub < M ? r0 + sub : M - 1;
    return X + r0 * ldx + (uint32_t)((r - r0) * ldx);
  };
#if QV_RQ_PREFETCH
  RawRow<In> next;
  if (g < groups) load_raw<K, In>(row_ptr(g), lane, next);
#endif

  fill_multiplier_table<K>(mult, cm_lds);
  __syncthreads();

  for (; g < groups; g += wave_stride) {
    const int64_t row = g * L::kRowsPerWave + sub;
    float v[8][8];
#if QV_RQ_PREFETCH
    unpack_raw<In>(next, v);
    // Prefetch the next row group while this one is transformed.
    if (g + wave_stride < groups) load_raw<K, In>(row_ptr(g + wave_stride), lane, next);
#else
    load_row<K, In>(row_ptr(g), lane, v);
#endif

    fwht_row_regs<K>(v, lane);

    float gmax[8];  // per register group j: the maximum of |smoothed value| over its channels
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 c0 = *reinterpret_cast<const float4*>(cm_row + 8 * j);
      const float4 c1 = *reinterpret_cast<const float4*>(cm_row + 8 * j + 4);
      const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      gmax[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[j][e] *= c[e];
        gmax[j] = fmaxf(gmax[j], fabsf(v[j][e]));
      }
    }
    // Scale and reciprocal of each register group's quantization group (the whole row, or one
    // group of channels).
    float sg[8], rg[8];
    constexpr float kQmax = (float)((1 << (kBits - 1)) - 1);
    if constexpr (kGroup == 0) {
      float amax = gmax[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) amax = fmaxf(amax, gmax[j]);
      amax = row_max<K>(amax);
      float s = amax / kQmax;
      if (!(s >= 1.17549435e-38f)) s = 0.0f;  // zero or subnormal scale: all-zero row
      const float r = (s > 0.0f) ? 1.0f / s : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) { sg[j] = s; rg[j] = r; }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((j & kJoin) == 0) {  // the group's first register group computes, the others copy
          float a = gmax[j];
          if constexpr (kJoin & 1) a = fmaxf(a, gmax[j | 1]);
          if constexpr (kJoin & 2) a = fmaxf(fmaxf(a, gmax[j | 2]), gmax[j | 3]);
          a = lanes16_max(a);
          float s = a / kQmax;
          if (!(s >= 1.17549435e-38f)) s = 0.0f;  // zero or subnormal scale: all-zero group
          sg[j] = s;
          rg[j] = (s > 0.0f) ? 1.0f / s : 0.0f;
        } else {
          sg[j] = sg[j & ~kJoin];
          rg[j] = rg[j & ~kJoin];
        }
      }
    }

    if (row < M) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = __builtin_bit_cast(uint32_t, __builtin_fmaf(v[j][e], rg[j], kMagic<kBits>));
        // the lane's eight codes of group j are k = 8 dword_index + 0..7
        uint8_t* const qrow = Xq + g * L::kRowsPerWave * (K * kBits / 8) + (uint32_t)(sub * (K * kBits / 8));
        if constexpr (kBits == 4) {
          reinterpret_cast<uint32_t*>(qrow)[dword_index<K>(lane, j)] = pack8(m);
        } else {
          reinterpret_cast<uint2*>(qrow)[dword_index<K>(lane, j)] = pack8_int8(m);
        }
      }
      if constexpr (kGroup == 0) {
        if ((lane & (L::kLanesPerRow - 1)) == 0) x_scale[row] = sg[0];
      } else {
        // the first lane of each DPP row writes the scales of the groups its row holds
        constexpr int kGroups = K / kGroup;
        if ((lane & 15) == 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if ((j & kJoin) == 0) x_scale[row * kGroups + group_of<K, kGroup>(lane, j)] = sg[j];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// bf16 rows with one scale per row: the first five index bits on the matrix cores (rq_mfma.h).

// Waves per SIMD the register allocation must allow.  The 8-bit width-1024 instance needs a few
// more registers (two dwords of codes per 8 channels) and would spill at 5.
template <int K, int kBits, int LA>
constexpr int mfma_waves() {
  return K == 1024 ? (kBits == 8 && QV_RQM_WAVES_1024 > 4 ? 4 : QV_RQM_WAVES_1024) : QV_RQM_WAVES;
}

template <int K, int kBits, int LA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(mfma_waves<K, kBits, LA>()))) void rotate_quant_mfma_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, const float* __restrict__ mult,
    uint8_t* __restrict__ Xq, float* __restrict__ x_scale) {
  using RQ = MfmaRowQuant<K, kBits, LA>;
  using L = typename RQ::L;
  __shared__ __attribute__((aligned(16))) float cm_lds[L::kTableRows * kCmStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const RQ rq(lane);
  const float* cm_row = rq.table_row(cm_lds);

  const int64_t groups = (M + L::kRowsPerWave - 1) / L::kRowsPerWave;
  const int64_t wave_stride = (int64_t)gridDim.x * (kThreads / 64);
  int64_t grp = (int64_t)blockIdx.x * (kThreads / 64) + wave;

  // The first row group is requested before the factor table is built, and each next one as soon
  // as the matrix cores have read the current tiles, so its loads are in flight during the
  // butterflies, the quantization and the stores.
  rq_u32x4 raw[RQ::T];
  if (grp < groups) rq.load(X, ldx, grp * L::kRowsPerWave, M, raw);
  fill_mfma_table<K, LA, kThreads>(mult, cm_lds);
  __syncthreads();

  for (; grp < groups; grp += wave_stride) {
    float v[RQ::T][8];
    rq.transform_b(raw, v);
    if (grp + wave_stride < groups) rq.load(X, ldx, (grp + wave_stride) * L::kRowsPerWave, M, raw);
    rq.finish(v, cm_row, grp * L::kRowsPerWave, M, Xq, x_scale);
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
    int64_t row = g * L::kRowsPerWave + sub;
    if (row >= M) row = M - 1;  // a repeated row does not change a maximum
    float v[8][8];
    load_row<K, In>(X + row * ld, lane, v);
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

// Resident blocks per CU for a kernel (queried once per kernel and device) times the CU count:
// the streaming kernels loop over row groups with the next group prefetched, and their grid is a
// small multiple of this (grid_for_rows).  The cache holds one entry per
// kernel instance (the template argument) and device below 16; callers on several host threads may
// fill an entry concurrently, each storing the same value.  Higher device ordinals query every time.
template <auto kKernel>
int resident_grid() {
  static std::atomic<int> cached[16];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cacheable = dev >= 0 && dev < 16;
  if (cacheable) {
    const int hit = cached[dev].load(std::memory_order_relaxed);
    if (hit > 0) return hit;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kKernel, kThreads, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int grid = per_cu * cus;
  if (cacheable) cached[dev].store(grid, std::memory_order_relaxed);
  return grid;
}

// Grid of the streaming kernels: at most twice the resident blocks.  Each block loops over row
// groups; with two blocks per resident slot every block does about half the rounds, and a slot whose
// block finishes early takes another, so the last round is shorter.  On 137400-row launches this
// measured 2-3 % faster than one block per slot (K = 1024: 62.7-63.3 against 64.1-65.4 us; K = 4096:
// 265.5-265.8 against 269.1-271.7 us); one block per row group, with no loop and no prefetch of the
// next group, was 25-40 % slower.
int grid_for_rows(int64_t M, int rows_per_wave, int resident) {
  const int64_t groups = (M + rows_per_wave - 1) / rows_per_wave;
  const int64_t blocks = (groups + (kThreads / 64) - 1) / (kThreads / 64);
  return (int)(blocks < 2 * (int64_t)resident ? blocks : 2 * (int64_t)resident);
}

template <int K, typename In, int kBits, int kGroup = 0>
hipError_t launch_rq(const void* X, int64_t M, int64_t ld, const float* mult, uint8_t* q, float* scale,
                     hipStream_t st) {
  const int grid =
      grid_for_rows(M, RowLayout<K>::kRowsPerWave, resident_grid<rotate_quant_kernel<K, In, kBits, kGroup>>());
  hipLaunchKernelGGL((rotate_quant_kernel<K, In, kBits, kGroup>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const In*>(X), M, ld, mult, q, scale);
  return hipGetLastError();
}

template <int K, int kBits>
hipError_t launch_rq_mfma(const void* X, int64_t M, int64_t ld, const float* mult, uint8_t* q, float* scale,
                          hipStream_t st) {
  constexpr int LA = K == 1024 ? QV_RQM_LANES_1024 : 16;
  const int grid = grid_for_rows(M, MfmaLayout<K, LA>::kRowsPerWave,
                                 resident_grid<rotate_quant_mfma_kernel<K, kBits, LA>>());
  hipLaunchKernelGGL((rotate_quant_mfma_kernel<K, kBits, LA>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(X), M, ld, mult, q, scale);
  return hipGetLastError();
}

template <int K, int kGroup>
hipError_t launch_rq_grouped(const void* X, bool bf16, int64_t M, int64_t ld, const float* mult, uint8_t* q,
                             float* scale, hipStream_t st) {
  return bf16 ? launch_rq<K, uint16_t, 4, kGroup>(X, M, ld, mult, q, scale, st)
              : launch_rq<K, float, 4, kGroup>(X, M, ld, mult, q, scale, st);
}

template <int K, typename In>
hipError_t launch_colmax(const void* X, int64_t M, int64_t ld, unsigned* colmax, hipStream_t st) {
  const int grid = grid_for_rows(M, RowLayout<K>::kRowsPerWave, resident_grid<rotated_colmax_kernel<K, In>>());
  hipLaunchKernelGGL((rotated_colmax_kernel<K, In>), dim3(grid), dim3(kThreads), 0, st,
                     static_cast<const In*>(X), M, ld, colmax);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const void* X, bool bf16, int64_t M, int64_t K, int64_t ld, const float* mult,
                               uint8_t* q, float* scale, int bits, hipStream_t st) {
  if constexpr (QV_RQ_MFMA) {
    if (bf16 && K == 4096)
      return bits == 8 ? launch_rq_mfma<4096, 8>(X, M, ld, mult, q, scale, st)
                       : launch_rq_mfma<4096, 4>(X, M, ld, mult, q, scale, st);
  }
  if constexpr (QV_RQ_MFMA_1024) {
    if (bf16 && K == 1024)
      return bits == 8 ? launch_rq_mfma<1024, 8>(X, M, ld, mult, q, scale, st)
                       : launch_rq_mfma<1024, 4>(X, M, ld, mult, q, scale, st);
  }
  if (bits == 8) {
    if (K == 1024) {
      return bf16 ? launch_rq<1024, uint16_t, 8>(X, M, ld, mult, q, scale, st)
                  : launch_rq<1024, float, 8>(X, M, ld, mult, q, scale, st);
    }
    return bf16 ? launch_rq<4096, uint16_t, 8>(X, M, ld, mult, q, scale, st)
                : launch_rq<4096, float, 8>(X, M, ld, mult, q, scale, st);
  }
  if (K == 1024) {
    return bf16 ? launch_rq<1024, uint16_t, 4>(X, M, ld, mult, q, scale, st)
                : launch_rq<1024, float, 4>(X, M, ld, mult, q, scale, st);
  }
  return bf16 ? launch_rq<4096, uint16_t, 4>(X, M, ld, mult, q, scale, st)
              : launch_rq<4096, float, 4>(X, M, ld, mult, q, scale, st);
}

hipError_t launch_rotate_quant_grouped(const void* X, bool bf16, int64_t M, int64_t K, int64_t ld, const float* mult,
                                       int64_t group, uint8_t* q, float* scale, hipStream_t st) {
  if (K == 1024) {
    if (group == 128) return launch_rq_grouped<1024, 128>(X, bf16, M, ld, mult, q, scale, st);
    if (group == 256) return launch_rq_grouped<1024, 256>(X, bf16, M, ld, mult, q, scale, st);
    return launch_rq_grouped<1024, 512>(X, bf16, M, ld, mult, q, scale, st);
  }
  if (group == 128) return launch_rq_grouped<4096, 128>(X, bf16, M, ld, mult, q, scale, st);
  if (group == 256) return launch_rq_grouped<4096, 256>(X, bf16, M, ld, mult, q, scale, st);
  return launch_rq_grouped<4096, 512>(X, bf16, M, ld, mult, q, scale, st);
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
