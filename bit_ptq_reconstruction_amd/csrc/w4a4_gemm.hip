// w4a4_gemm.hip -- int4 x int4 contraction on the gfx950 int8 matrix cores with int32
// accumulation and a fused dequantization (+ bias) (+ GELU) epilogue.
//
// Method: W4A4 linear layers (4-bit weights and activations; the lsdiaocha.cn write-up of the
// QuantVGGT paper) with symmetric per-token / per-output-channel scales ("十亿参数的三维重建模型，
// 能塞进手机吗？" (gslzct.com), 训练后量化（PTQ）), so y = acc * x_scale[m] * w_scale[n].
//
// Block tile BN (weight rows n) x BM (token rows m) over a WGN x WGM grid of waves (2 x 2 by
// default); each wave owns a (BN/WGN) x (BM/WGM) sub-tile of v_mfma_i32_32x32x32_i8 fragments whose
// int32 accumulators stay in registers.  Per stage of 128 codes (64 bytes of every tile row):
//   * each wave issues LDS-DMA loads (buffer_load_dwordx4 ... lds, the stage offset in a scalar
//     register) for its share of both packed tiles (no registers, no LDS store instructions) into
//     a ring of STAGES buffers, STAGES - 1 stages ahead; the
//     16-byte units of a 64-byte tile row are stored XOR-swizzled (unit u of row r at
//     u ^ ((r ^ r >> 2) & 3)) so the fragment reads hit distinct banks;
//   * a fragment is two ds_read_b128 per lane (32 + 32 packed codes), feeding four MFMAs;
//   * codes are widened to int8 with two masks: (p & 0xF0F0F0F0) keeps the odd-k nibbles as 16 q
//     and ((p << 4) & 0xF0F0F0F0) the even-k ones (one 64-bit shift serves two dwords).  Both
//     operands carry the factor 16, so the accumulator holds 256 * acc (exact: |256 acc| <=
//     256 * 64 * 65536 < 2^31); the epilogue folds the 2^-8 into the row scale.  A and B are
//     widened the same way, so every k is paired with itself and the order of the terms inside a
//     fragment does not matter;
//   * the widening of the next operands is interleaved with the MFMAs (the compiler's schedule),
//     so the unpack runs on the vector ALU while the matrix core is busy; the K loop is unrolled
//     by the ring depth, so a stage's LDS read addresses are instruction offsets.
// The tile's row and column scales are fetched into LDS by LDS-DMA when the tile starts, so the
// epilogue does not wait on global memory.  With group-wise scales (kGS > 0) each group's int32
// accumulators are dequantized into fp32 accumulators after the group's last stage.
// MFMA operand roles: A = weight tile (output rows i = n), B = activation tile (columns j = m): a
// lane owns runs of four consecutive n of one m; the epilogue stages each wave's outputs in LDS and
// writes whole 128-byte row segments with 16-byte buffer stores whose range ends at the last row
// below M.  With int8 operands (kW8) there is no widening; a stage holds 64 codes (64 bytes per
// row) on the 128 x 256 tiles of bf16 outputs, and 128 where K allows on the 128 x 128 tiles of fp32
// outputs.  Tiles are assigned XCD-major: the
// hardware deals blocks round-robin over the 8 XCDs, and the block -> tile map gives each XCD a
// contiguous run of tiles sharing activation rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "qv_internal.h"
#include "rq_mfma.h"

namespace qv {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#ifndef QV_STAGES
#define QV_STAGES 2  // LDS ring depth of the GEMM main loop, 128 int4 codes per stage
#endif
#ifndef QV_RB128
#define QV_RB128 0
#endif
#ifndef QV_DMA
#define QV_DMA 1  // 1: LDS-DMA stage loads; 0: loads through registers and ds_write_b128
#endif
#ifndef QV_STAGES_128
#define QV_STAGES_128 2  // ring depth with 256 codes per stage
#endif

constexpr int kXcds = 8;

#ifndef QV_BUF_DMA
#define QV_BUF_DMA 1  // 1: stage loads through buffer resources (scalar stage offset); 0: global addresses
#endif
// Word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format, no swizzle).
[[maybe_unused]] constexpr int kBufDword3 = 0x00020000;

// Position inside an XCD's run -> offset in the run's canonical (row-major over tiles) order.
// G = 0 keeps the canonical order: the blocks in flight share a few activation rows and sweep every
// weight tile, which suits weights that stay in L2.  G > 0 walks each chunk of G tile rows column by
// column, so the blocks in flight cover G activation rows and a few weight tiles, and each weight
// tile is fetched once per chunk; a last chunk of fewer whole rows is transposed the same way and any
// final partial row keeps the canonical order.
__device__ __forceinline__ int64_t run_offset(int64_t local, int64_t cnt, int64_t tiles_n, int64_t G) {
  if (G == 0) return local;
  const int64_t chunk = G * tiles_n;
  const int64_t c0 = (local / chunk) * chunk;
  const int64_t rows = (cnt - c0 < chunk ? cnt - c0 : chunk) / tiles_n;  // whole rows in this chunk
  const int64_t j = local - c0;
  if (j >= rows * tiles_n) return local;  // partial last row
  return c0 + (j % rows) * tiles_n + j / rows;
}

// Tile rows per chunk of run_offset.  int4 weights (2 MB for the widest layer) stay in an XCD's
// 4 MB L2 in the canonical order.  A 4096 x 1024 int8 weight fills it, and is re-fetched for every
// few activation rows unless chunks of 16 rows (16 activation tiles of 128 x 1024 bytes, 2 MB)
// bound the sweep.  With 4096-byte rows 16 activation tiles no longer fit either, and the canonical
// order, which reuses the activation tile, fetches less.
template <bool kW8>
__device__ __forceinline__ int64_t chunk_rows(int64_t tile_bytes) {
  return (kW8 && 16 * tile_bytes <= (2 << 20)) ? 16 : 0;
}

// XOR swizzle of the 16-byte units of a tile row (U units per row): conflict-free fragment reads
// whether the LDS serves 8 lanes per 128 bytes or 16 lanes per 256 bytes.
template <int U>
__device__ __forceinline__ int swz(int r) {
  return (U == 4) ? ((r ^ (r >> 2)) & 3) : ((r ^ (r >> 3)) & 7);
}

// The even-k nibbles of both packed dwords are shifted by one 64-bit shift (the bits carried from
// p0 into p1's low nibble are masked off with the rest); written directly, because the compiler
// splits a 64-bit shift whose carried bits are masked into two 32-bit shifts.
__device__ __forceinline__ v4i widen(uint32_t p0, uint32_t p1) {
  uint64_t w = (((uint64_t)p1) << 32) | p0;
  asm("v_lshlrev_b64 %0, 4, %1" : "=v"(w) : "v"(w));
  v4i o;
  o[0] = (int)((uint32_t)w & 0xF0F0F0F0u);
  o[1] = (int)(p0 & 0xF0F0F0F0u);
  o[2] = (int)((uint32_t)(w >> 32) & 0xF0F0F0F0u);
  o[3] = (int)(p1 & 0xF0F0F0F0u);
  return o;
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// GELU(y) = y Phi(y) = max(y, 0) - |y| Q(|y|), Q(x) = Phi(-x) = erfc(x / sqrt 2) / 2 (for y >= 0,
// y Phi(y) = y - y Q(y); for y < 0 it is y Q(-y)).  Q is evaluated as t 2^(P(t) - x^2 log2(e) / 2)
// with t = 1 / (1 + 0.35 x): the factor exp(-x^2/2) is exact in form, and P, a degree-5 polynomial
// in t, carries log2 of the remaining slowly varying ratio.  The coefficients are a minimax fit of
// log2(Q(x) / t) + x^2 log2(e) / 2 over x in [0, 13.5] (beyond that |y| Q(|y|) is below the fp32
// normal range); in fp32 the largest relative error of the GELU is 1.4e-5 down to the smallest
// normal output.  P's constant term carries +8, so 2^(...) stays normal wherever the output is.
// The kernel evaluates P in t' = t / 256 = 1 / (256 + 89.6 x) with coefficients c_i 256^i, so the
// product x t' carries the 2^-8 that undoes the +8.  (A degree-3 fit, 1.9e-4, saves two
// multiply-adds; it moves ~1 % of bf16 outputs by an ulp, against 0.05 % here, and that shows up
// downstream as extra code flips in the next layer's quantization.)
__device__ __forceinline__ float gelu(float y) {
  const float x = fabsf(y);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(89.5999984741211f, x, 256.0f));
  float p = 366175256576.0f;
  p = __builtin_fmaf(p, t, -4510181376.0f);
  p = __builtin_fmaf(p, t, 12373395.0f);
  p = __builtin_fmaf(p, t, 22816.5234375f);
  p = __builtin_fmaf(p, t, 377.2472839355469f);
  p = __builtin_fmaf(p, t, 5.157796859741211f);
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x * -0.72134752044448170f, x, p));
  return __builtin_fmaf(-(x * t), e, fmaxf(y, 0.0f));
}

// LDS of a block: the stage ring (reused for output staging in the epilogue), then the tile's BN
// bias values (when a bias is given), BN weight scales and BM activation scales, fetched by LDS-DMA
// when the tile starts.
template <int BN, int BM, int WGN, int WGM, int RB, int STAGES, bool kBF16Out, bool kBias>
struct GemmLds {
  static constexpr size_t kStage = (size_t)STAGES * (BN + BM) * RB;
  static constexpr size_t kOut =
      (size_t)WGN * WGM * (BM / WGM) * ((BN / WGN) * (kBF16Out ? 2 : 4) + (kBF16Out ? 8 : 16));
  static constexpr size_t kBiasOffset = kStage > kOut ? kStage : kOut;
  static constexpr size_t kScaleOffset = kBiasOffset + (kBias ? 4 * (size_t)BN : 0);
  static constexpr size_t kTotal = kScaleOffset + 4 * (size_t)(BN + BM);
};

// Waves per SIMD the register allocation must allow (at most 128 registers per lane for 4, 168
// for 3): 64 x 64 wave tiles (64 accumulators per lane) with a 2-deep ring of 64-byte stages fit
// four 4-wave or two 8-wave blocks per CU; a 3-deep ring leaves room for three 4-wave blocks;
// 64 x 96 wave tiles (96 accumulators) allow three; 64 x 128 wave tiles and the 128-byte stages
// allow two.
template <int BN, int BM, int WGN, int WGM, int RB, int STAGES, int kGS = 0>
constexpr int waves_per_eu() {
  if (kGS > 0) return 2;  // group-wise scales: an fp32 accumulator beside the int32 one
  constexpr int kAcc = (BN / WGN) * (BM / WGM) / 64;
  if (RB == 128 || kAcc > 96) return 2;
  if (kAcc > 64) return 3;
  return (WGN * WGM == 8 || STAGES == 2) ? 4 : 3;
}

typedef float v16f __attribute__((ext_vector_type(16)));

// Next-layer quantization fused into the GEMM (kReq = N, the next layer's Hadamard width, 1024 or
// 4096; 0 = none): the bf16 output rows are also rotated, smoothed and quantized for the next
// linear ([P4] 预全局旋转 / 后局部平滑 / 训练后量化（PTQ） applied to this layer's output).  A row
// needs all N outputs, which span the N / BN tiles of its row stripe.  Every block, after storing
// its tile, makes its stores visible device-wide (agent-scope release) and increments the
// stripe's counter; the block that brings the counter to N / BN -- the last tile of the stripe to
// finish -- acquires and runs the rotate-quantize over the stripe's rows, reading them back
// (mostly from the caches).  No block ever waits on another.
struct NextQuant {
  const float* mult;     // [N] per-channel factor of the next layer (1 / smoothing), or NULL
  uint8_t* q;            // [M][N / 2] packed int4 codes of the next layer's input
  float* scale;          // [M] per-row scales
  unsigned* counters;    // [ceil(M / BM)] tile counts per row stripe, zero at launch
};

// kW8: int8 operands (one code per byte, no widening, the accumulator is acc itself) instead of
// packed int4.  kGS > 0: group-wise scales, one per row and group of 128 kGS channels (kGS stages
// of 128 codes): x_scale is [M][K / (128 kGS)], w_scale [N][K / (128 kGS)], and each group's int32
// accumulator is dequantized into an fp32 accumulator when the group's last stage is done.
template <int BN, int BM, int WGN, int WGM, int RB, int STAGES, bool kBF16Out, bool kGelu, bool kBias, bool kW8,
          int kGS = 0, int kReq = 0>
__global__ __launch_bounds__(64 * WGN * WGM)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<BN, BM, WGN, WGM, RB, STAGES, kGS>()))) void w4a4_gemm_kernel(const uint8_t* __restrict__ Xq,
                                                            const float* __restrict__ x_scale,
                                                            const uint8_t* __restrict__ Wq,
                                                            const float* __restrict__ w_scale,
                                                            const float* __restrict__ bias, int64_t M,
                                                            int64_t N, int64_t K, void* __restrict__ Y,
                                                            int64_t ldy, NextQuant nq) {
  constexpr int kWaves = WGN * WGM, kThr = 64 * kWaves;
  constexpr int WN = BN / WGN, WM = BM / WGM;  // wave sub-tile
  constexpr int FN = WN / 32, FM = WM / 32;
  constexpr int kRowBytes = RB;   // bytes of one tile row per stage (2 RB int4 or RB int8 codes)
  constexpr int U = RB / 16;      // 16-byte units per tile row and stage
  constexpr int kSub = kW8 ? RB / 32 : RB / 16;  // K32 MFMA sub-steps per stage
  constexpr int kReads = RB / 32; // ds_read_b128 per fragment per stage
  constexpr int kUnits = (BN + BM) * U;  // 16-byte units per stage
  constexpr int kLoads = kUnits / kThr;                  // LDS-direct loads per lane per stage
  constexpr int kStageBytes = (BN + BM) * kRowBytes;
  static_assert(kUnits % kThr == 0, "tile must split evenly over the waves");
  static_assert(STAGES >= 2 && (STAGES - 2) * kLoads < 64, "pipeline depth");
  static_assert(kGS == 0 || (!kW8 && RB == 64), "group-wise scales: int4 operands, 128-code stages");
  static_assert((BN + BM) % 64 == 0 && BN % 64 == 0, "whole waves of scale and bias loads");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform; readfirstlane keeps it (and the LDS-DMA addresses derived from it)
  // in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WGN, wm = wave / WGN;

  // XCD-major tile order.
  const int64_t tiles_n = N / BN;
  const int64_t tiles = tiles_n * ((M + BM - 1) / BM);
  const int64_t b = blockIdx.x;
  const int64_t per = tiles / kXcds, rem = tiles % kXcds;
  const int64_t xcd = b % kXcds, local = b / kXcds;
  const int64_t cnt = per + (xcd < rem ? 1 : 0);
  const int64_t tile = xcd * per + (xcd < rem ? xcd : rem) +
                       run_offset(local, cnt, tiles_n, chunk_rows<kW8>(BM * (kW8 ? K : K / 2)));
  const int64_t tile_n = tile % tiles_n;
  const int64_t tile_m = tile / tiles_n;
  const int64_t n0 = tile_n * BN;
  const int64_t m0 = tile_m * BM;
  const int64_t row_bytes = kW8 ? K : K / 2;  // bytes of one operand row

  // Source of each of this lane's loads; LDS unit P = 64 * (kWaves i + wave) + lane of the stage
  // buffer.
  // Each load instruction covers 16 whole tile rows, so it reads either the weight tile or the
  // activation tile: a uniform base (that tile's first row) plus a per-lane 32-bit offset.
  static_assert((BN * U) % 64 == 0, "a load instruction stays inside one operand tile");
  const uint8_t* sbase[kLoads];
  uint32_t soff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int P = 64 * (kWaves * i + wave) + lane;
    const int r = P / U;  // row inside the combined A|B tile
    if (64 * (kWaves * i + wave) < BN * U) {
      sbase[i] = Wq + n0 * row_bytes;
      soff[i] = (uint32_t)(r * row_bytes + 16 * ((P % U) ^ swz<U>(r)));
    } else {
      const int rb = r - BN;
      int64_t mr = m0 + rb;
      if (mr > M - 1) mr = M - 1;  // ragged tail: repeat the last row; its outputs are not stored
      sbase[i] = Xq + m0 * row_bytes;
      soff[i] = (uint32_t)((mr - m0) * row_bytes + 16 * ((P % U) ^ swz<U>(rb)));
    }
  }
  auto src_at = [&](int i, int64_t kb) { return sbase[i] + kb + soff[i]; };
  // Buffer resources over the two operand tiles (raw, byte-addressed): a stage's loads then take
  // the lane offset in a vector register and the stage's byte offset kb in a scalar one, so no
  // vector instruction advances an address from stage to stage.
  // (The host pass does not know the buffer-resource type; it compiles the global-address form.)
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t rsrc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const bool isA = 64 * (kWaves * i + wave) < BN * U;
    rsrc[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sbase[i]), (short)0,
                                                (int)((isA ? BN : BM) * row_bytes), kBufDword3);
  }
  constexpr bool kBufDma = QV_BUF_DMA;
#else
  constexpr bool kBufDma = false;
#endif
  // Stage loads.  With LDS-DMA (global_load_lds_dwordx4) the 16 bytes of lane l land at unit
  // 64 * (kWaves i + wave) + l of the stage buffer directly; otherwise they are fetched into registers
  // (fetch_stage) and written to the same units with ds_write_b128 (store_stage).
  u32x4 staged[kLoads];
  auto fetch_stage = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) staged[i] = *reinterpret_cast<const u32x4*>(src_at(i, kb));
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      *reinterpret_cast<u32x4*>(lds + buf * kStageBytes + 1024 * (kWaves * i + wave) + 16 * lane) = staged[i];
  };
  auto issue_stage = [&](int buf, int64_t kb) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      uint8_t* dst = lds + buf * kStageBytes + 1024 * (kWaves * i + wave);
      auto* ldst = reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(dst));
      if constexpr (kBufDma) {
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc[i], ldst, 16, soff[i], (unsigned)kb, 0, 0);
#endif
      } else {
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src_at(i, kb)), ldst, 16, 0, 0);
      }
    }
  };
  (void)fetch_stage; (void)store_stage; (void)issue_stage;

  v16i acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int c = 0; c < FM; ++c) acc[a][c] = v16i{};

  const int r32 = lane & 31;
  const int h = lane >> 5;
  const int nk = (int)(kW8 ? K / kRowBytes : K / (2 * kRowBytes));

  // The tile's scales: scale slot i holds w_scale[n0 + i] (i < BN) or x_scale[m0 + i - BN] (rows
  // past M repeat the last row); thread t fetches slots t, t + kThr, ...  Issued before the stage
  // loads, so the first iteration's vmcnt wait covers them.
  // Group-wise scales: the same for every group g, into slots g (BN + BM) + i, from column g of the
  // [rows][groups] scale matrices.
  using Lds = GemmLds<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kBias>;
  float* const scales = reinterpret_cast<float*>(lds + Lds::kScaleOffset);
  float* const bias_lds = reinterpret_cast<float*>(lds + Lds::kBiasOffset);
  const int groups = kGS > 0 ? (int)(K / (128 * kGS)) : 1;  // groups of 128 kGS channels
  for (int g = 0; g < groups; ++g) {
#pragma unroll
    for (int r = 0; r < (BN + BM + kThr - 1) / kThr; ++r) {
      const int i = tid + kThr * r;
      if (kThr * r + 64 * wave >= BN + BM) break;  // wave-uniform
      const float* sp;
      if (i < BN) {
        sp = w_scale + (n0 + i) * groups + g;
      } else {
        const int64_t mr = m0 + (i - BN);
        sp = x_scale + (mr < M ? mr : M - 1) * groups + g;
      }
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(sp),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(scales + g * (BN + BM) + 64 * (wave + kWaves * r))),
                                       4, 0, 0);
    }
  }
  if constexpr (kBias) {
    // The tile's BN bias values, so the epilogue reads them from LDS (no per-lane global addresses
    // held across the K loop).
#pragma unroll
    for (int r = 0; r < (BN + kThr - 1) / kThr; ++r) {
      if (kThr * r + 64 * wave >= BN) break;  // wave-uniform
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(bias + n0 + tid + kThr * r),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(
                                           reinterpret_cast<uintptr_t>(bias_lds + 64 * (wave + kWaves * r))),
                                       4, 0, 0);
    }
  }
  (void)bias_lds;
  if constexpr (QV_DMA) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue_stage(s, (int64_t)s * kRowBytes);
  } else {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) {
        fetch_stage((int64_t)s * kRowBytes);
        store_stage(s);
      }
  }

  // One stage: wait for stage kt, refill the ring, read and widen the fragments, 16 MFMAs.  A
  // "fresh" stage starts its accumulators from zero (the first stage of a group of channels).
  auto stage_step = [&](int kt, auto fresh, int buf) {  // buf = kt % STAGES
    constexpr bool kFresh = decltype(fresh)::value;
    if constexpr (QV_DMA) {
      // Stage kt has landed once at most STAGES - 2 later stages are still in flight.
      if (kt + STAGES - 2 < nk) wait_vmcnt<(STAGES - 2) * kLoads>();
      else wait_vmcnt<0>();
    }
    __syncthreads();  // every wave's share of stage kt is in LDS; stage kt - 1 is consumed
    const bool refill = kt + STAGES - 1 < nk;
    const int rbuf = buf == 0 ? STAGES - 1 : buf - 1;  // (kt + STAGES - 1) % STAGES
    if constexpr (QV_DMA) {
      if (refill) issue_stage(rbuf, (int64_t)(kt + STAGES - 1) * kRowBytes);
    } else {
      if (refill) fetch_stage((int64_t)(kt + STAGES - 1) * kRowBytes);
    }

    const uint8_t* As = lds + buf * kStageBytes;
    const uint8_t* Bs = As + BN * kRowBytes;
    u32x4 pa[FN][kReads], pb[FM][kReads];
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int r = wn * WN + 32 * a + r32;
#pragma unroll
      for (int q = 0; q < kReads; ++q)
        pa[a][q] = *reinterpret_cast<const u32x4*>(As + r * kRowBytes + 16 * ((2 * q + h) ^ swz<U>(r)));
    }
#pragma unroll
    for (int c = 0; c < FM; ++c) {
      const int r = wm * WM + 32 * c + r32;
#pragma unroll
      for (int q = 0; q < kReads; ++q)
        pb[c][q] = *reinterpret_cast<const u32x4*>(Bs + r * kRowBytes + 16 * ((2 * q + h) ^ swz<U>(r)));
    }
    if constexpr (kW8) {
      // int8: read q is the whole MFMA operand of sub-step q (16 codes per lane, the other 16 of the
      // K32 block in the lane 32 apart).
#pragma unroll
      for (int q = 0; q < kSub; ++q)
#pragma unroll
        for (int c = 0; c < FM; ++c)
#pragma unroll
          for (int a = 0; a < FN; ++a)
            acc[a][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(v4i, pa[a][q]),
                                                              __builtin_bit_cast(v4i, pb[c][q]), acc[a][c], 0, 0, 0);
    } else {
      // K32 sub-steps: sub-step s uses dwords 2(s&1), 2(s&1)+1 of read q = s >> 1.
#pragma unroll
      for (int s = 0; s < kSub; ++s) {
        v4i fa[FN];
#pragma unroll
        for (int a = 0; a < FN; ++a) {
          const uint32_t p0 = pa[a][s >> 1][2 * (s & 1)], p1 = pa[a][s >> 1][2 * (s & 1) + 1];
          fa[a] = widen(p0, p1);
        }
#pragma unroll
        for (int c = 0; c < FM; ++c) {
          const uint32_t p0 = pb[c][s >> 1][2 * (s & 1)], p1 = pb[c][s >> 1][2 * (s & 1) + 1];
          const v4i fb = widen(p0, p1);
#pragma unroll
          for (int a = 0; a < FN; ++a) acc[a][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb, (kFresh && s == 0) ? v16i{} : acc[a][c], 0, 0, 0);
        }
      }
    }
    if constexpr (!QV_DMA) {
      // The buffer of stage kt + STAGES - 1 held stage kt - 1, which every wave finished reading
      // before this iteration's barrier.
      if (refill) store_stage(rbuf);
    }
  };

  v16f facc[kGS > 0 ? FN : 1][kGS > 0 ? FM : 1];
  if constexpr (kGS > 0) {
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int c = 0; c < FM; ++c) facc[a][c] = v16f{};
  }
  (void)facc;
  if constexpr (kGS == 0) {
    // Whole turns of the ring first, so each step's buffer index is a constant and its LDS
    // addresses become instruction offsets; then the remaining stages.
    int kt = 0;
    for (; kt + STAGES <= nk; kt += STAGES) {
#pragma unroll
      for (int b = 0; b < STAGES; ++b) stage_step(kt + b, std::false_type{}, b);
    }
    for (; kt < nk; ++kt) stage_step(kt, std::false_type{}, kt % STAGES);
  } else {
    // Groups of kGS stages; after each, acc (256 x the group's integer dot products) is
    // dequantized with the group's scales into facc: the row scale carries the 2^-8.
    for (int kt0 = 0; kt0 < nk; kt0 += kGS) {
      stage_step(kt0, std::true_type{}, kt0 % STAGES);
#pragma unroll
      for (int st = 1; st < kGS; ++st) stage_step(kt0 + st, std::false_type{}, (kt0 + st) % STAGES);
      const float* sg = scales + (kt0 / kGS) * (BN + BM);
#pragma unroll
      for (int c = 0; c < FM; ++c) {
        const float sa = sg[BN + wm * WM + 32 * c + r32] * 0.00390625f;
#pragma unroll
        for (int a = 0; a < FN; ++a) {
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const float4 sw4 = *reinterpret_cast<const float4*>(sg + wn * WN + 32 * a + 8 * vg + 4 * h);
            const float sw[4] = {sw4.x, sw4.y, sw4.z, sw4.w};
#pragma unroll
            for (int v = 0; v < 4; ++v)
              facc[a][c][4 * vg + v] = __builtin_fmaf((float)acc[a][c][4 * vg + v] * sa, sw[v], facc[a][c][4 * vg + v]);
          }
        }
      }
    }
  }

  // Epilogue.  The lane holds, for fragment (a, c) and register group vg, outputs
  // m = wm*WM + 32c + r32 and n = wn*WN + 32a + 8vg + 4h + (0..3) of the tile.  They are dequantized
  // (+ bias) (+ GELU), converted, and staged in LDS as the wave's WM x WN output block (rows padded
  // by 8 or 16 bytes so the staging writes spread over the banks); the block is then written with
  // 16-byte non-temporal stores, each group of lanes covering whole contiguous row segments.
  using OutT = typename std::conditional<kBF16Out, uint16_t, float>::type;
  // int4: row scales carry the 2^-8 of the accumulator (256 acc converts to fp32 exactly, |256 acc|
  // < 2^26 with its low 8 bits zero); a row scale below 2^-118 becomes subnormal and keeps at least
  // 16 significant bits.  int8: the accumulator is acc.
  float sa[FM];
#pragma unroll
  for (int c = 0; c < FM; ++c) sa[c] = scales[BN + wm * WM + 32 * c + r32] * (kW8 ? 1.0f : 0.00390625f);
  // y for fragment (a, c) and register group vg: the lane's four consecutive columns
  // n = wn*WN + 32a + 8vg + 4h + (0..3) of row m = wm*WM + 32c + r32, dequantized (+ bias) (+ GELU).
  // The lane's weight scales are read once, before the staging passes, so the passes' LDS writes
  // and reads do not wait behind scale reads.
  float4 sw4[FN][4];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int vg = 0; vg < 4; ++vg)
      if constexpr (kGS == 0) sw4[a][vg] = *reinterpret_cast<const float4*>(scales + wn * WN + 32 * a + 8 * vg + 4 * h);
  (void)sw4;
  auto outputs = [&](int a, int c, int vg, float (&y)[4]) {
    float sw[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kGS == 0) { sw[0] = sw4[a][vg].x; sw[1] = sw4[a][vg].y; sw[2] = sw4[a][vg].z; sw[3] = sw4[a][vg].w; }
    float bb[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kBias) {
      const float4 b4 = *reinterpret_cast<const float4*>(bias_lds + wn * WN + 32 * a + 8 * vg + 4 * h);
      bb[0] = b4.x; bb[1] = b4.y; bb[2] = b4.z; bb[3] = b4.w;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (kGS > 0) {
        y[v] = facc[a][c][4 * vg + v];
      } else {
        y[v] = (float)acc[a][c][4 * vg + v] * sa[c] * sw[v];
      }
      if constexpr (kBias) y[v] += bb[v];
      if constexpr (kGelu) y[v] = gelu(y[v]);
    }
  };
  constexpr int kChunksPerRow = WN * (int)sizeof(OutT) / 16;  // 16-byte chunks per row
  constexpr int kRowsPerPass = 64 / kChunksPerRow;            // rows one wave-wide read covers

  // Output stores.  The wave's block of rows m0 + wm*WM + (0..WM-1) is written through a buffer
  // resource that starts at the block's first output and ends after its last row below M: a store
  // to a row at or past M falls outside the range and is dropped, so the lanes need no bounds test
  // and no 64-bit address.  The range check covers the vector offset (plus the instruction
  // offset) only -- the scalar offset is added after it -- so the row of a pass goes into the
  // vector offset too.  The host admits output rows below 2^24 bytes, so the block's WM <= 128 rows
  // span less than 2^31 bytes.
  static_assert(WM <= 128, "32-bit output offsets");
  const int64_t row_stride = ldy * (int64_t)sizeof(OutT);
  const int64_t rows_left = M - (m0 + wm * WM);
  const int rows = rows_left < 0 ? 0 : (rows_left > WM ? WM : (int)rows_left);
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<OutT*>(Y) + (m0 + wm * WM) * ldy + n0 + wn * WN, (short)0, (int)(rows * row_stride), kBufDword3);
  const uint32_t lane_off = (uint32_t)((lane / kChunksPerRow) * row_stride) + 16u * (uint32_t)(lane % kChunksPerRow);
#endif
  // Row ru + lane / kChunksPerRow of the block (ru uniform), chunk lane % kChunksPerRow.
  auto store_out = [&](int ru, const u32x4& v) {
#if defined(__HIP_DEVICE_COMPILE__)
    // non-temporal, except where the next-layer quantization reads the rows back
    __builtin_amdgcn_raw_buffer_store_b128(v, yrsrc, lane_off + (uint32_t)(ru * row_stride), 0, kReq ? 0 : 2);
#else
    (void)ru; (void)v; (void)rows; (void)row_stride; (void)Y;  // the host pass compiles no kernel code
#endif
  };

  // bf16 outputs are staged without a block barrier: after the last stage's barrier no wave reads
  // any ring buffer but the last stage's (every LDS-DMA has landed, no refill follows), so buffer
  // nk % STAGES is free.  Each wave stages its block in 32-row passes (one fragment row c at a
  // time) through a 4 KB slice of that buffer, rows of exactly WN outputs with 16-byte chunks
  // XOR-swizzled by the row.  Other blocks synchronize and stage over the whole ring, rows padded.
  constexpr int kPassBytes = 32 * WN * (int)sizeof(OutT);
  constexpr bool kFreeStaging = kBF16Out && WN * (int)sizeof(OutT) == 128 && kWaves * kPassBytes <= kStageBytes;
  if constexpr (kFreeStaging) {
    uint8_t* const stage_out = lds + (nk % STAGES) * kStageBytes + wave * kPassBytes;
#pragma unroll
    for (int c = 0; c < FM; ++c) {
#pragma unroll
      for (int a = 0; a < FN; ++a) {
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          float y[4];
          outputs(a, c, vg, y);
          const bf16x2 lo = __builtin_convertvector((f32x2{y[0], y[1]}), bf16x2);
          const bf16x2 hi = __builtin_convertvector((f32x2{y[2], y[3]}), bf16x2);
          // row r32, chunk 4a + vg swizzled by the row, half h of the chunk
          *reinterpret_cast<uint2*>(stage_out + r32 * 128 + 16 * ((4 * a + vg) ^ (r32 & 7)) + 8 * h) =
              make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // wave-local: read back by this wave
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int pass = 0; pass < 32 / kRowsPerPass; ++pass) {
        const int ml = pass * kRowsPerPass + lane / kChunksPerRow;
        const int ch = lane % kChunksPerRow;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage_out + ml * 128 + 16 * (ch ^ (ml & 7)));
        store_out(32 * c + pass * kRowsPerPass, v);
      }
      // the next pass rewrites this slice after the reads above
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  } else {
    constexpr int kOutRowBytes = WN * (int)sizeof(OutT) + (kBF16Out ? 8 : 16);
    __syncthreads();  // every wave is done with the stage buffers
    uint8_t* const stage_out = lds + wave * (WM * kOutRowBytes);
#pragma unroll
    for (int a = 0; a < FN; ++a) {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
#pragma unroll
        for (int c = 0; c < FM; ++c) {
          float y[4];
          outputs(a, c, vg, y);
          const int nl = 32 * a + 8 * vg + 4 * h;
          uint8_t* dst = stage_out + (32 * c + r32) * kOutRowBytes + nl * (int)sizeof(OutT);
          if constexpr (kBF16Out) {
            const bf16x2 lo = __builtin_convertvector((f32x2{y[0], y[1]}), bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2{y[2], y[3]}), bf16x2);
            *reinterpret_cast<uint2*>(dst) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
          }
        }
      }
    }
    // Wave-local: the block written above is read back by the same wave only.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int pass = 0; pass < WM / kRowsPerPass; ++pass) {
      const int ml = pass * kRowsPerPass + lane / kChunksPerRow;
      const int ch = lane % kChunksPerRow;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage_out + ml * kOutRowBytes + 16 * ch);
      store_out(pass * kRowsPerPass, v);
    }
  }

  if constexpr (kReq > 0) {
    static_assert(kBF16Out && !kW8 && kGS == 0 && (kReq == 1024 || kReq == 4096), "fused requantization: bf16 rows");
    constexpr int LA = kReq == 1024 ? 8 : 16;
    using RQ = MfmaRowQuant<kReq, 4, LA>;
    using RL = typename RQ::L;
    static_assert(RL::kTableRows * kCmStride * 4 <= (int)GemmLds<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kBias>::kScaleOffset,
                  "factor table fits the stage ring");
    static_assert(BM % (kWaves * RL::kRowsPerWave) == 0, "whole row groups per wave");
    // Every wave's output stores are complete and visible at agent scope, then one increment per block.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    int* const flag = reinterpret_cast<int*>(lds + GemmLds<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kBias>::kScaleOffset);
    if (tid == 0) {
      const unsigned done = __hip_atomic_fetch_add(nq.counters + tile_m, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = (done == (unsigned)(tiles_n - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;  // uniform over the block
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the other tiles' stores of this stripe are visible

    // This block finished the stripe: rotate-quantize its rows m0 .. min(m0 + BM, M) - 1.
    float* const cm = reinterpret_cast<float*>(lds);
    fill_mfma_table<kReq, LA, kThr>(nq.mult, cm);
    __syncthreads();
    const RQ rq(lane);
    const float* cm_row = rq.table_row(cm);
    const uint16_t* const Yb = static_cast<const uint16_t*>(Y);
    const int64_t m_end = (m0 + BM < M) ? m0 + BM : M;
    constexpr int kGroupRows = kWaves * RL::kRowsPerWave;  // rows per step of the whole block
    // At width 1024 the next row group's loads are issued before the current one is finished; at
    // width 4096 (64 values per lane) that would not fit the GEMM's 128 registers.
    constexpr bool kPrefetch = kReq == 1024;
    rq_u32x4 raw[RQ::T];
    int64_t r0 = m0 + wave * RL::kRowsPerWave;
    if (kPrefetch && r0 < m_end) rq.load(Yb, ldy, r0, m_end, raw);
    for (; r0 < m_end; r0 += kGroupRows) {
      float v[RQ::T][8];
      if (!kPrefetch) rq.load(Yb, ldy, r0, m_end, raw);
      rq.transform_b(raw, v);
      if (kPrefetch && r0 + kGroupRows < m_end) rq.load(Yb, ldy, r0 + kGroupRows, m_end, raw);
      rq.finish(v, cm_row, r0, m_end, nq.q, nq.scale);
    }
  }
}

template <int BN, int BM, int WGN, int WGM, int RB, int STAGES, bool kBF16Out, bool kGelu, bool kBias, bool kW8,
          int kGS = 0, int kReq = 0>
hipError_t launch_t(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                    int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, hipStream_t st, NextQuant nq = {}) {
  using Lds = GemmLds<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kBias>;
  // Group-wise scales take one (BN + BM)-float slot per group, at most kMaxGroups of them.
  const size_t lds = kGS > 0 ? Lds::kScaleOffset + 4 * (size_t)(BN + BM) * (size_t)(K / (128 * kGS)) : Lds::kTotal;
  constexpr size_t kLdsMax = kGS > 0 ? Lds::kScaleOffset + 4 * (size_t)(BN + BM) * kMaxGroups : Lds::kTotal;
  // Allow more than 64 KB of dynamic LDS, once per kernel instance and device below 16 (every
  // call on higher device ordinals).  Concurrent first calls from several host threads each set
  // the same attribute.
  static std::atomic<bool> attr_set[16];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cacheable = dev >= 0 && dev < 16;
  if (!cacheable || !attr_set[dev].load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&w4a4_gemm_kernel<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kGelu, kBias, kW8, kGS, kReq>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
    if (e != hipSuccess) return e;
    if (cacheable) attr_set[dev].store(true, std::memory_order_relaxed);
  }
  const int64_t blocks = (N / BN) * ((M + BM - 1) / BM);
  hipLaunchKernelGGL((w4a4_gemm_kernel<BN, BM, WGN, WGM, RB, STAGES, kBF16Out, kGelu, kBias, kW8, kGS, kReq>),
                     dim3((unsigned)blocks), dim3(64 * WGN * WGM), lds, st, Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, nq);
  return hipGetLastError();
}

// Tile configurations (block tile BN x BM, wave grid WGN x WGM):
//   0: 128 x 128, 2 x 2 waves of 64 x 64: 128 registers and 36 KB of LDS, four blocks per CU, so
//      one block's barrier, prologue and epilogue overlap the others' MFMAs;
//   1: 256 x 256, 2 x 4 waves of 128 x 64; 2: 256 x 256, 4 x 2 waves of 64 x 128 (one block per
//      CU, half the LDS-DMA bytes per MFMA);
//   3: 256 x 128, 4 x 2 waves of 64 x 64; 4: 128 x 256, 2 x 4 waves of 64 x 64;
//   5: 128 x 256, 2 x 2 waves of 64 x 128: each wave widens 2 weight and 4 activation fragments per
//      8 MFMAs (3.75 vector instructions per MFMA for the int4 widening instead of 5), at two waves
//      per SIMD (~200 registers; two blocks per CU).  On the 100-frame layers (M = 137400) it
//      measured 1-5 % faster than configuration 0 on every linear (proj 4.5 %, fc2 2.6 %, qkv 1.9 %,
//      fc1 1.0 %); a 3-deep ring or 256-code stages on the same tile did not help.
//   6: 128 x 192, 2 x 2 waves of 64 x 96: 4.17 widening instructions per MFMA, ~152 registers,
//      three blocks per CU (3 x 41.5 KB of LDS).  It does 12-14 % more MFMA work per clock than
//      configuration 5, but draws more power, so the power-limited clock settles 8-10 % lower
//      (1.58-1.81 against 1.72-1.98 GHz).  Net, in GEMM-only runs with the two alternating on the
//      100-frame layers, it was 2-5 % faster on every linear on two boxes (e.g. qkv 379-392 against
//      396-400 us, proj 126-130 against 134-136, fc1 633-641 against 655-661, fc2 430 against
//      438-440) and 3-4 % slower on a third; the outputs are identical.
// A configuration whose BN does not divide N, and every fp32-output launch, uses configuration 0,
// and so do int8 operands with configurations 5 and 6 (int8 operands with bf16 outputs have their
// own tile, QV_W8_TILE_CFG).
#ifndef QV_TILE_CFG
#define QV_TILE_CFG 6
#endif
// int8 operands with bf16 outputs: 5 = 128 x 256 tiles with 64-code stages (below), 0 = the
// 128 x 128 tiles with 128-code stages of the other int8 launches.
#ifndef QV_W8_TILE_CFG
#define QV_W8_TILE_CFG 5
#endif

template <int BN, int BM, int WGN, int WGM, bool kBF16Out, bool kGelu, bool kBias, bool kW8>
hipError_t launch_cfg(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                      int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, hipStream_t st) {
  // int4: 128 codes (64 bytes of every row) per stage; a 256-code stage variant is kept selectable
  // for measurements (it halves the barriers but its 64 KB ring leaves two blocks per CU).
  // int8 on 128 x 128 tiles: 128 codes (128 bytes) per stage where K allows; 64-byte stages would
  // carry half the MFMA work per barrier, and measured 5 % slower on the block despite the four
  // blocks per CU.
  if constexpr (kW8) {
    if ((K % 128) == 0)
      return launch_t<BN, BM, WGN, WGM, 128, QV_STAGES_128, kBF16Out, kGelu, kBias, kW8>(Xq, xs, Wq, ws, bias, M, N, K,
                                                                                      Y, ldy, st);
  }
  if constexpr (QV_RB128 && !kW8) {
    if ((K % 256) == 0)
      return launch_t<BN, BM, WGN, WGM, 128, QV_STAGES_128, kBF16Out, kGelu, kBias, kW8>(Xq, xs, Wq, ws, bias, M, N, K,
                                                                                      Y, ldy, st);
  }
  return launch_t<BN, BM, WGN, WGM, 64, QV_STAGES, kBF16Out, kGelu, kBias, kW8>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy,
                                                                              st);
}

template <bool kBF16Out, bool kGelu, bool kBias, bool kW8>
hipError_t launch_k(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                    int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, hipStream_t st) {
#define QV_LAUNCH(BN, BM, WGN, WGM) \
  launch_cfg<BN, BM, WGN, WGM, kBF16Out, kGelu, kBias, kW8>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st)
  if constexpr (!kBF16Out) {
    // fp32 outputs: the 256-wide tiles' output staging would not fit in LDS
    return QV_LAUNCH(128, 128, 2, 2);
  } else if constexpr (kW8 && QV_W8_TILE_CFG == 5) {
    // int8 operands with bf16 outputs: 128 x 256 tiles (4 waves of 64 x 128) with 64-code stages,
    // two blocks per CU (2 x 49.5 KB of LDS, ~172 registers).  On the 100-frame layers this
    // measured 3-5 % faster than 128 x 128 tiles with 128-code stages on the K = 1024 linears (qkv
    // 500 against 524-547 us, proj 170-180 against 179-185, fc1 795-842 against 836-865; GEMM-only,
    // alternating, two boxes) and level on fc2; a 3-deep ring, 128 x 192 and 256 x 128 tiles were
    // no better.
    return launch_t<128, 256, 2, 2, 64, QV_STAGES, kBF16Out, kGelu, kBias, kW8>(Xq, xs, Wq, ws, bias, M, N, K, Y,
                                                                               ldy, st);
  } else if constexpr (QV_TILE_CFG == 1) {
    if (N % 256 == 0) return QV_LAUNCH(256, 256, 2, 4);
  } else if constexpr (QV_TILE_CFG == 2) {
    if (N % 256 == 0) return QV_LAUNCH(256, 256, 4, 2);
  } else if constexpr (QV_TILE_CFG == 3) {
    if (N % 256 == 0) return QV_LAUNCH(256, 128, 4, 2);
  } else if constexpr (QV_TILE_CFG == 4) {
    return QV_LAUNCH(128, 256, 2, 4);
  } else if constexpr (QV_TILE_CFG == 5 && !kW8) {
    // int8 operands keep configuration 0: their 128-byte stages would leave one block per CU here
    return QV_LAUNCH(128, 256, 2, 2);
  } else if constexpr (QV_TILE_CFG == 6 && !kW8) {
    return QV_LAUNCH(128, 192, 2, 2);
  }
  return QV_LAUNCH(128, 128, 2, 2);
#undef QV_LAUNCH
}

}  // namespace

namespace {

template <bool kW8>
hipError_t launch_gemm(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                       int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out, int64_t ldy,
                       hipStream_t st) {
#define QV_K(B, G, BIAS) launch_k<B, G, BIAS, kW8>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st)
  if (bias) {
    if (bf16_out) return gelu ? QV_K(true, true, true) : QV_K(true, false, true);
    return gelu ? QV_K(false, true, true) : QV_K(false, false, true);
  }
  if (bf16_out) return gelu ? QV_K(true, true, false) : QV_K(true, false, false);
  return gelu ? QV_K(false, true, false) : QV_K(false, false, false);
#undef QV_K
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                            const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out,
                            int64_t ldy, hipStream_t st) {
  return launch_gemm<false>(Xq, xs, Wq, ws, bias, M, N, K, gelu, Y, bf16_out, ldy, st);
}

namespace {

template <int kGS>
hipError_t launch_grouped(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                          int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out, int64_t ldy,
                          hipStream_t st) {
#define QV_G(B, G, BIAS) \
  launch_t<128, 128, 2, 2, 64, QV_STAGES, B, G, BIAS, false, kGS>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st)
  if (bias) {
    if (bf16_out) return gelu ? QV_G(true, true, true) : QV_G(true, false, true);
    return gelu ? QV_G(false, true, true) : QV_G(false, false, true);
  }
  if (bf16_out) return gelu ? QV_G(true, true, false) : QV_G(true, false, false);
  return gelu ? QV_G(false, true, false) : QV_G(false, false, false);
#undef QV_G
}

}  // namespace

hipError_t launch_w4a4_gemm_grouped(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                                    const float* bias, int64_t M, int64_t N, int64_t K, int64_t group, bool gelu,
                                    void* Y, bool bf16_out, int64_t ldy, hipStream_t st) {
  if (group == 128) return launch_grouped<1>(Xq, xs, Wq, ws, bias, M, N, K, gelu, Y, bf16_out, ldy, st);
  if (group == 256) return launch_grouped<2>(Xq, xs, Wq, ws, bias, M, N, K, gelu, Y, bf16_out, ldy, st);
  return launch_grouped<4>(Xq, xs, Wq, ws, bias, M, N, K, gelu, Y, bf16_out, ldy, st);
}

namespace {

__global__ void zero_counters_kernel(unsigned* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int kReq, bool kGelu, bool kBias>
hipError_t launch_requant_t(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                            int64_t M, int64_t K, void* Y, int64_t ldy, NextQuant nq, hipStream_t st) {
  const int64_t stripes = (M + 127) / 128;
  hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)((stripes + 255) / 256)), dim3(256), 0, st, nq.counters,
                     stripes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_t<128, 128, 2, 2, 64, QV_STAGES, true, kGelu, kBias, false, 0, kReq>(Xq, xs, Wq, ws, bias, M, kReq,
                                                                                   K, Y, ldy, st, nq);
}

}  // namespace

hipError_t launch_w4a4_gemm_requant(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                                    const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y,
                                    int64_t ldy, const float* mult_next, uint8_t* q_next, float* scale_next,
                                    unsigned* counters, hipStream_t st) {
  const NextQuant nq{mult_next, q_next, scale_next, counters};
#define QV_R(W, G, B) launch_requant_t<W, G, B>(Xq, xs, Wq, ws, bias, M, K, Y, ldy, nq, st)
  if (N == 4096) {
    if (bias) return gelu ? QV_R(4096, true, true) : QV_R(4096, false, true);
    return gelu ? QV_R(4096, true, false) : QV_R(4096, false, false);
  }
  if (bias) return gelu ? QV_R(1024, true, true) : QV_R(1024, false, true);
  return gelu ? QV_R(1024, true, false) : QV_R(1024, false, false);
#undef QV_R
}

hipError_t launch_w8a8_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                            const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out,
                            int64_t ldy, hipStream_t st) {
  return launch_gemm<true>(reinterpret_cast<const uint8_t*>(Xq), xs, reinterpret_cast<const uint8_t*>(Wq), ws, bias,
                           M, N, K, gelu, Y, bf16_out, ldy, st);
}

}  // namespace qv
