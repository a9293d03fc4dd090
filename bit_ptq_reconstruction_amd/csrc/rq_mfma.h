// rq_mfma.h -- rotate-smooth-quantize of bf16 rows with one scale per row, the first five Hadamard
// stages on the matrix cores: the per-wave row step shared by the standalone rotate-quantize kernel
// (rotate_quant.hip) and the GEMM that quantizes its own output for the next layer (w4a4_gemm.hip).
//
// Method ("十亿参数的三维重建模型，能塞进手机吗？" (gslzct.com)): 双平滑细粒度量化（DSFQ） > 预全局旋转 (rows
// times the Hadamard matrix, H / sqrt(K)); > 后局部平滑 (a per-channel factor on the rotated value);
// 训练后量化（PTQ） (symmetric per-row quantization, q = clamp(round(x / s), -8, 7) for N = 4).
//
// With k = 32 a + b, the Sylvester-order H_K is H_{K/32} (x) H_32, so the rotation is the 32-point
// transform over b followed by the (K/32)-point transform over a.  bf16 inputs and the +-1 entries
// of H_32 are exact MFMA operands, so v_mfma_f32_16x16x32_bf16 forms the b-transform with fp32
// accumulation and no unpacking: the loaded data is the B operand (k = b, column n = one of 16
// a-values held by the 16 lanes of a DPP row), a constant slice of H_32 the A operand (16 of the 32
// output indices b'), and two MFMAs (q = 0, 1) give all 32 b'.  Output row m = 4 (l / 16) + r of
// MFMA q is assigned b' = r + 4 q + 8 (l / 16), so a lane ends with the 8 consecutive channels
// b' = 8 (l / 16) + e, e = 4 q + r: one packed dword.  The a-transform remains: with LA a-values
// of each row on the 16 lanes of a DPP row (DPP-row position p = LA t + pp for row t of the wave's
// 16 / LA, a = LA J + a_lo(pp)), the a_lo bits are DPP butterflies (as in fwht_regs.h) and the tile
// index J is in registers.
//   K = 1024, LA = 8: two rows per wave, 32 values per lane, 3 DPP and 2 in-lane stages;
//   K = 4096, LA = 16: one row per wave, 64 values per lane, 4 DPP and 3 in-lane stages.
// Every element of the MFMA sum is an exact product and the fp32 accumulation of the 32 terms
// stays within the rounding error of the five butterfly stages it replaces.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwht_regs.h"

namespace qv {

typedef unsigned rq_u32x4 __attribute__((ext_vector_type(4)));
typedef float rq_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 1.5 * 2^23 + 2^(bits-1): fma(x, 1/s, magic) rounds once to nearest-even, and the low mantissa
// byte of the result is rne(x / s) + 2^(bits-1) (|x / s| <= 2^(bits-1) - 1 keeps it in the byte).
template <int kBits>
constexpr float kMagic = 12582912.0f + (float)(1 << (kBits - 1));

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

// Eight 8-bit codes (low bytes q + 128) -> two dwords of two's-complement bytes, k ascending.
__device__ __forceinline__ uint2 pack8_int8(const uint32_t (&m)[8]) {
  const uint32_t a = __builtin_amdgcn_perm(m[1], m[0], 0x0c0c0400u);  // bytes: q0 q1 0 0
  const uint32_t b = __builtin_amdgcn_perm(m[3], m[2], 0x0c0c0400u);
  const uint32_t c = __builtin_amdgcn_perm(m[5], m[4], 0x0c0c0400u);
  const uint32_t d = __builtin_amdgcn_perm(m[7], m[6], 0x0c0c0400u);
  return make_uint2((a | (b << 16)) ^ 0x80808080u, (c | (d << 16)) ^ 0x80808080u);
}

// Rows of the per-lane factor tables in LDS are padded to 68 floats, so that the 16-byte reads of
// 16 different rows fall in different banks.
constexpr int kCmStride = 68;

// LA a-values per row on the 16 lanes of a DPP row (4, 8 or 16), so 16 / LA rows per wave and
// K / (32 LA) tiles J per row in registers.
template <int K, int LA>
struct MfmaLayout {
  static_assert(LA == 4 || LA == 8 || LA == 16, "a-values per DPP row");
  static constexpr int kRowsPerWave = 16 / LA;
  static constexpr int kTiles = K / (32 * LA);
  static constexpr int kValues = 8 * kTiles;  // per lane and row
  static constexpr int kTableRows = 4 * LA;
  static constexpr int kDppStages = LA == 4 ? 2 : (LA == 8 ? 3 : 4);
  static constexpr float kNorm = (K == 1024) ? 0.03125f : 0.015625f;  // 1/sqrt(K), exact
  static_assert(kTiles * 32 * LA == K && kValues <= 64, "layout");
};

// a_lo held by position pp = p % LA of a row's lanes.  The map is chosen so that the butterfly
// partner along a_lo bit s is lane pp ^ {1, 2, 7 or 8, 15}[s]: quad_perm for bits 0 and 1,
// row_half_mirror (LA = 8) or row_ror:8 (LA = 16) for bit 2, row_mirror for bit 3.  The DPP
// butterflies leave the sign (-1)^popcount(a_lo) on a lane's elements; the factor table folds it in.
template <int LA>
__device__ __forceinline__ int mfma_alo(int pp) {
  if constexpr (LA == 4) return pp;
  if constexpr (LA == 8) return ((pp ^ (pp >> 2)) & 1) | ((((pp >> 1) ^ (pp >> 2)) & 1) << 1) | (pp & 4);
  return chunk_of_lane16(pp);
}

// One DPP butterfly stage over N registers: self + sigma * partner (see fwht_regs.h).
template <int LA, int S, int N>
__device__ __forceinline__ void mfma_dpp_stage(float* r, float sigma) {
#pragma unroll
  for (int i = 0; i < N; i += 16) {
    if constexpr (S == 0) QV_DPP16("quad_perm:[1,0,3,2]", (r + i), sigma);
    if constexpr (S == 1) QV_DPP16("quad_perm:[2,3,0,1]", (r + i), sigma);
    if constexpr (S == 2 && LA == 8) QV_DPP16("row_half_mirror", (r + i), sigma);
    if constexpr (S == 2 && LA == 16) QV_DPP16("row_ror:8", (r + i), sigma);
    if constexpr (S == 3) QV_DPP16("row_mirror", (r + i), sigma);
  }
}

// Factor table: row g LA + pp holds, for J < kTiles and e < 8, the factor
// sign * 1/sqrt(K) * mult[k'] of channel k' = 8 g + e + 32 (LA J + a_lo(pp)).  Filled by the
// kThr threads of a block.
template <int K, int LA, int kThr>
__device__ __forceinline__ void fill_mfma_table(const float* __restrict__ mult, float* cm) {
  using L = MfmaLayout<K, LA>;
  for (int idx = threadIdx.x; idx < L::kTableRows * L::kValues; idx += kThr) {
    const int row = idx / L::kValues, je = idx % L::kValues, J = je >> 3, e = je & 7;
    const int g = row / LA, alo = mfma_alo<LA>(row % LA);
    const int k = 8 * g + e + 32 * (LA * J + alo);
    const float sign = (__builtin_popcount(alo) & 1) ? -1.0f : 1.0f;
    cm[row * kCmStride + je] = sign * L::kNorm * (mult ? mult[k] : 1.0f);
  }
}

// The per-wave row step: a wave rotates, smooths and quantizes 16 / LA rows at a time.
template <int K, int kBits, int LA>
struct MfmaRowQuant {
  using L = MfmaLayout<K, LA>;
  static constexpr int T = L::kTiles;
  int lane, g, t, alo;
  uint32_t lane_off;  // element offset of the lane's 16-byte share inside tile J = 0 of its row
  bf16x8 hq[2];
  float sigma[4];

  __device__ __forceinline__ explicit MfmaRowQuant(int lane_) : lane(lane_) {
    const int p = lane & 15;
    g = lane >> 4;
    t = p / LA;  // row of the lane inside the wave's group
    alo = mfma_alo<LA>(p % LA);
    lane_off = (uint32_t)(32 * alo + 8 * g);
    // A operands: lane l holds row m = l % 16 and k = 8 (l / 16) + j of the 16 x 32 slice; row m of
    // slice q is output b' = (m % 4) + 4 q + 8 (m / 4), so entry j is (-1)^popcount(b' & (8 g + j)).
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int bp = (p & 3) + 4 * q + 8 * (p >> 2);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (__builtin_popcount(bp & (8 * g + 2 * i)) & 1) ? 0xBF80u : 0x3F80u;
        const uint32_t hi = (__builtin_popcount(bp & (8 * g + 2 * i + 1)) & 1) ? 0xBF80u : 0x3F80u;
        w[i] = lo | (hi << 16);
      }
      hq[q] = __builtin_bit_cast(bf16x8, (rq_u32x4){w[0], w[1], w[2], w[3]});
    }
    // DPP butterfly signs: +1 on the lower element of a pair, -1 on the upper.
#pragma unroll
    for (int s = 0; s < 4; ++s) sigma[s] = ((alo >> s) & 1) ? -1.0f : 1.0f;
  }

  // The factor-table row this lane reads.
  __device__ __forceinline__ const float* table_row(const float* cm) const {
    return cm + (g * LA + (lane & 15) % LA) * kCmStride;
  }

  // Lane's 16-byte share of every tile J of its row r0 + t: elements 32 (LA J + a_lo) + 8 g + 0..7.
  // Rows past the end are clamped to the last row: loaded and transformed, never stored.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ldx, int64_t r0, int64_t M,
                                       rq_u32x4 (&raw)[T]) const {
    const int64_t row = r0 + t;
    const uint16_t* xrow = X + r0 * ldx + (uint32_t)(((row < M ? row : M - 1) - r0) * ldx) + lane_off;
#pragma unroll
    for (int J = 0; J < T; ++J)
      raw[J] = __builtin_nontemporal_load(reinterpret_cast<const rq_u32x4*>(xrow + 32 * LA * J));
  }

  // The b-transform on the matrix cores (raw may be reloaded once this returns).
  __device__ __forceinline__ void transform_b(const rq_u32x4 (&raw)[T], float (&v)[T][8]) const {
#pragma unroll
    for (int J = 0; J < T; ++J) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, raw[J]);
      const rq_f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hq[0], b, (rq_f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const rq_f32x4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hq[1], b, (rq_f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // copy each element to a scalar first: a bit-cast of a vector element reads element 0
        const float x0 = d0[r], x1 = d1[r];
        v[J][r] = x0;
        v[J][4 + r] = x1;
      }
    }
  }

  // The a-transform (low bits across the DPP row, then the tile bits in-lane), the factors, the row
  // maximum, and the codes and scale of row r0 + t (stored when it is below M).
  __device__ __forceinline__ void finish(float (&v)[T][8], const float* __restrict__ cm_row, int64_t r0, int64_t M,
                                         uint8_t* __restrict__ Xq, float* __restrict__ x_scale) const {
    float* vr = &v[0][0];
    mfma_dpp_stage<LA, 0, 8 * T>(vr, sigma[0]);
    mfma_dpp_stage<LA, 1, 8 * T>(vr, sigma[1]);
    if constexpr (L::kDppStages > 2) mfma_dpp_stage<LA, 2, 8 * T>(vr, sigma[2]);
    if constexpr (L::kDppStages > 3) mfma_dpp_stage<LA, 3, 8 * T>(vr, sigma[3]);
#pragma unroll
    for (int h = 1; h < T; h <<= 1) {
#pragma unroll
      for (int J = 0; J < T; ++J) {
        if ((J & h) == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float a = v[J][e], b = v[J + h][e];
            v[J][e] = a + b;
            v[J + h][e] = a - b;
          }
        }
      }
    }

    float amax = 0.0f;
#pragma unroll
    for (int J = 0; J < T; ++J) {
      const float4 c0 = *reinterpret_cast<const float4*>(cm_row + 8 * J);
      const float4 c1 = *reinterpret_cast<const float4*>(cm_row + 8 * J + 4);
      const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[J][e] *= c[e];
        amax = fmaxf(amax, fabsf(v[J][e]));
      }
    }
    // Row maximum: over the row's LA lanes of each DPP row, then over the four DPP rows.
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, true)));
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0x4E, 0xF, 0xF, true)));
    if constexpr (LA == 8) {
      amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0x141, 0xF, 0xF, true)));
    } else if constexpr (LA == 16) {
      amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0x128, 0xF, 0xF, true)));
      amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, amax), 0x140, 0xF, 0xF, true)));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    constexpr float kQmax = (float)((1 << (kBits - 1)) - 1);
    float s = amax / kQmax;
    if (!(s >= 1.17549435e-38f)) s = 0.0f;  // zero or subnormal scale: all-zero row
    const float rs = (s > 0.0f) ? 1.0f / s : 0.0f;

    const int64_t row = r0 + t;
    if (row < M) {
      uint8_t* const qrow = Xq + r0 * (K * kBits / 8) + (uint32_t)(t * (K * kBits / 8));
#pragma unroll
      for (int J = 0; J < T; ++J) {
        uint32_t m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = __builtin_bit_cast(uint32_t, __builtin_fmaf(v[J][e], rs, kMagic<kBits>));
        // channels 8 g + 32 a + 0..7, a = LA J + a_lo
        const int idx = g + 4 * (LA * J + alo);
        if constexpr (kBits == 4) {
          reinterpret_cast<uint32_t*>(qrow)[idx] = pack8(m);
        } else {
          reinterpret_cast<uint2*>(qrow)[idx] = pack8_int8(m);
        }
      }
      if ((lane & (0x30 | (LA - 1))) == 0) x_scale[row] = s;
    }
  }
};

}  // namespace qv
