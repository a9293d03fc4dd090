// fwht_regs.h -- in-register Walsh-Hadamard transform of one row per 16 lanes (K = 1024) or per
// wave (K = 4096) on gfx950, used by the rotate-quantize and calibration kernels.
//
// The rotation is X . H_K / sqrt(K) with H_K the Sylvester-order Hadamard matrix
// ("十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com), 双平滑细粒度量化（DSFQ） > 预全局旋转).
// H_K is the tensor product of log2(K) two-point transforms, one per index bit, so the rotation is
// log2(K) butterfly stages in any order; this file never materialises H.
//
// Register layout.  Every lane holds 64 elements of its row in v[j][e] (j, e in 0..7):
//     k = e + 8 * (chunk + C * j),   C = 16 (K = 1024) or 64 (K = 4096),
// so a lane's 8 consecutive elements (one 16-byte bf16 load, two fp32 loads, one packed-int4 dword)
// share a chunk.  Index bits held by e and j are transformed inside the lane (6 stages).
// Chunk bits 0-3 live in the lane's position inside its 16-lane DPP row.  Lane p holds chunk
// bits b = chunk_of_lane16(p), chosen so that the butterfly partner along chunk bit b is lane
// p ^ kDppMask[b] with kDppMask = {1, 2, 8, 15}: each such stage is one DPP-sourced v_fmac_f32
// (quad_perm for 1 and 2, row_ror:8 for 8, row_mirror for 15).  The fmac computes
// self + sigma * partner with sigma = -1 on the lane holding the upper element, which yields the
// negated difference there; the negations of all stages multiply into a fixed sign per chunk,
// (-1)^popcount(chunk & 15), which the caller folds into its per-channel multiplier.
// For K = 4096, chunk bits 4 and 5 are lane bits 4 and 5 (across DPP rows).  Those two stages
// swap the lane bit with register bit j0 (resp. j1) by v_permlane16_swap (v_permlane32_swap) and
// then run as ordinary in-lane butterflies; afterwards register j holds chunk bits 4, 5 = j0, j1 and
// j bits 0, 1 = lane bits 4, 5 (see dword_index()).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qv {

// Chunk held by lane p of a 16-lane DPP row: the inverse of lane(c) = c0*1 ^ c1*2 ^ c2*8 ^ c3*15.
__device__ __forceinline__ int chunk_of_lane16(int p) {
  const int l0 = p & 1, l1 = (p >> 1) & 1, l2 = (p >> 2) & 1, l3 = (p >> 3) & 1;
  return (l0 ^ l2) | ((l1 ^ l2) << 1) | ((l3 ^ l2) << 2) | (l2 << 3);
}

template <int K>
struct RowLayout {
  static_assert(K == 1024 || K == 4096, "Hadamard width must be 1024 or 4096");
  static constexpr int kLanesPerRow = (K == 1024) ? 16 : 64;
  static constexpr int kRowsPerWave = 64 / kLanesPerRow;
  static constexpr int kChunks = kLanesPerRow;  // C in the layout above
  static constexpr int kLog2K = (K == 1024) ? 10 : 12;
  static constexpr float kNorm = (K == 1024) ? 0.03125f : 0.015625f;  // 1/sqrt(K), exact
};

// Chunk index this lane loads for its row (before the transform).
template <int K>
__device__ __forceinline__ int load_chunk(int lane) {
  const int low = chunk_of_lane16(lane & 15);
  return (K == 1024) ? low : (low | (lane & 48));
}

// Index (in units of 8 elements) of the 8 elements register group j holds AFTER the transform.
template <int K>
__device__ __forceinline__ int dword_index(int lane, int j) {
  const int low = chunk_of_lane16(lane & 15);
  if (K == 1024) return low + 16 * j;
  const int chunk = low | ((j & 3) << 4);
  const int slab = ((lane >> 4) & 3) | (j & 4);
  return chunk + 64 * slab;
}

// Sign the transform leaves on this lane's elements: (-1)^popcount(chunk & 15).
__device__ __forceinline__ float fold_sign(int lane) {
  return (__builtin_popcount(chunk_of_lane16(lane & 15)) & 1) ? -1.0f : 1.0f;
}

// Butterfly sign for the DPP stage on chunk bit b: +1 on the lower element, -1 on the upper.
__device__ __forceinline__ float stage_sigma(int lane, int b) {
  return ((chunk_of_lane16(lane & 15) >> b) & 1) ? -1.0f : 1.0f;
}

// One DPP stage over 16 registers.  v_fmac_f32 is not merged with a DPP move by the compiler, so
// the stage is written directly; s_nop 1 before the block covers the VALU-write -> DPP-read hazard
// on the first registers, and s_nop 1 after it covers any DPP read the compiler emits next.
#define QV_DPP16(CTRL, R, S)                                                                         \
  asm volatile(                                                                                      \
      "s_nop 1\n\t"                                                                                  \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                           \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                         \
      "s_nop 1"                                                                                      \
      : "+v"(R[0]), "+v"(R[1]), "+v"(R[2]), "+v"(R[3]), "+v"(R[4]), "+v"(R[5]), "+v"(R[6]),          \
        "+v"(R[7]), "+v"(R[8]), "+v"(R[9]), "+v"(R[10]), "+v"(R[11]), "+v"(R[12]), "+v"(R[13]),     \
        "+v"(R[14]), "+v"(R[15])                                                                     \
      : "v"(S))

template <int STAGE>
__device__ __forceinline__ void dpp_stage(float* r, float sigma) {
  // r points at 64 consecutive floats (v[0][0] .. v[7][7]).
  if constexpr (STAGE == 0) {
    QV_DPP16("quad_perm:[1,0,3,2]", (r + 0), sigma);
    QV_DPP16("quad_perm:[1,0,3,2]", (r + 16), sigma);
    QV_DPP16("quad_perm:[1,0,3,2]", (r + 32), sigma);
    QV_DPP16("quad_perm:[1,0,3,2]", (r + 48), sigma);
  } else if constexpr (STAGE == 1) {
    QV_DPP16("quad_perm:[2,3,0,1]", (r + 0), sigma);
    QV_DPP16("quad_perm:[2,3,0,1]", (r + 16), sigma);
    QV_DPP16("quad_perm:[2,3,0,1]", (r + 32), sigma);
    QV_DPP16("quad_perm:[2,3,0,1]", (r + 48), sigma);
  } else if constexpr (STAGE == 2) {
    QV_DPP16("row_ror:8", (r + 0), sigma);
    QV_DPP16("row_ror:8", (r + 16), sigma);
    QV_DPP16("row_ror:8", (r + 32), sigma);
    QV_DPP16("row_ror:8", (r + 48), sigma);
  } else {
    QV_DPP16("row_mirror", (r + 0), sigma);
    QV_DPP16("row_mirror", (r + 16), sigma);
    QV_DPP16("row_mirror", (r + 32), sigma);
    QV_DPP16("row_mirror", (r + 48), sigma);
  }
}

// Unnormalised, sign-folded transform of the 64 values of this lane's row share (see top).
template <int K>
__device__ __forceinline__ void fwht_row_regs(float (&v)[8][8], int lane) {
  // Element bits 0-2 (e): in-lane butterflies.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((e & h) == 0) {
          const float a = v[j][e], b = v[j][e + h];
          v[j][e] = a + b;
          v[j][e + h] = a - b;
        }
      }
    }
  }
  // Slab bits (j): in-lane butterflies.
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & h) == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = v[j][e], b = v[j + h][e];
          v[j][e] = a + b;
          v[j + h][e] = a - b;
        }
      }
    }
  }
  // Chunk bits 0-3: DPP stages inside the 16-lane row.
  float* r = &v[0][0];
  dpp_stage<0>(r, stage_sigma(lane, 0));
  dpp_stage<1>(r, stage_sigma(lane, 1));
  dpp_stage<2>(r, stage_sigma(lane, 2));
  dpp_stage<3>(r, stage_sigma(lane, 3));
  if constexpr (K == 4096) {
    // Chunk bit 4 (lane bit 4) <-> register bit j0, then in-lane butterflies.
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const auto s = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v[j][e]),
                                                        __builtin_bit_cast(unsigned, v[j + 1][e]), false, false);
        // Copy the two halves to scalars before reinterpreting them: a bit-cast applied directly
        // to an element of the returned pair reads the pair's first element.
        const unsigned s0 = s[0], s1 = s[1];
        const float a = __builtin_bit_cast(float, s0), b = __builtin_bit_cast(float, s1);
        v[j][e] = a + b;
        v[j + 1][e] = a - b;
      }
    }
    // Chunk bit 5 (lane bit 5) <-> register bit j1.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j & 2) == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[j][e]),
                                                          __builtin_bit_cast(unsigned, v[j + 2][e]), false, false);
          const unsigned s0 = s[0], s1 = s[1];
          const float a = __builtin_bit_cast(float, s0), b = __builtin_bit_cast(float, s1);
          v[j][e] = a + b;
          v[j + 2][e] = a - b;
        }
      }
    }
  }
}

// Maximum over the lanes that share a row (16 lanes for K = 1024, the whole wave for K = 4096).
template <int K>
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true)));
  if constexpr (K == 4096) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
  }
  return x;
}

}  // namespace qv
