// w4a4_gemm.hip -- int4 x int4 contraction on the gfx950 int8 matrix cores with int32
// accumulation and a fused dequantization (+ bias) (+ GELU) epilogue.
//
// Method: W4A4 linear layers (4-bit weights and activations; the lsdiaocha.cn write-up of the
// QuantVGGT paper) with symmetric per-token / per-output-channel scales ("十亿参数的三维重建模型，
// 能塞进手机吗？" (gslzct.com), 训练后量化（PTQ）), so y = acc * x_scale[m] * w_scale[n].
//
// Data path.  Packed int4 tiles of Wq (rows n) and Xq (rows m) go global -> registers -> LDS
// (double buffered, XOR-swizzled at 8-byte granularity so the fragment reads spread over the banks).
// Each wave reads 8 packed bytes per lane per 16 x 64 operand fragment and widens them to int8 with
// two masks: (p & 0xF0F0F0F0) keeps the odd-k nibbles as 16 * q and ((p << 4) & 0xF0F0F0F0) the
// even-k ones.  Both operands carry the factor 16, so the int32 accumulator holds 256 * acc (exact:
// |256 * acc| <= 256 * 64 * 65536 < 2^31) and an arithmetic shift by 8 recovers acc.  Because A
// and B are widened identically, the order of k inside a fragment is the same for both, and a dot
// product does not depend on the order of its terms.
// Operand roles: the MFMA A operand is the weight tile (output rows i = n) and B the activation
// tile (output columns j = m); a lane then owns four consecutive n of one m and stores them with
// one 16-byte (fp32) or 8-byte (bf16) write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qv_internal.h"

namespace qv {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileN = 128;         // weight rows per block
constexpr int kTileM = 128;         // token rows per block
constexpr int kTileKBytes = 64;     // 128 int4 codes per row per stage
constexpr int kWaveN = 64, kWaveM = 64;
constexpr int kFragN = kWaveN / 16, kFragM = kWaveM / 16;

// Byte offset of 8-byte unit u of tile row r inside an LDS tile (64 bytes per row).
__device__ __forceinline__ int lds_off(int r, int u) { return r * kTileKBytes + 8 * (u ^ ((r >> 1) & 7)); }

__device__ __forceinline__ v4i widen(uint2 p) {
  v4i o;
  o[0] = (int)((p.x << 4) & 0xF0F0F0F0u);
  o[1] = (int)(p.x & 0xF0F0F0F0u);
  o[2] = (int)((p.y << 4) & 0xF0F0F0F0u);
  o[3] = (int)(p.y & 0xF0F0F0F0u);
  return o;
}

__device__ __forceinline__ float gelu(float y) { return 0.5f * y * erfcf(-0.70710678118654752f * y); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // Round to nearest even (finite inputs).
  uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
  ua = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
  ub = (ub + 0x7FFFu + ((ub >> 16) & 1u)) & 0xFFFF0000u;
  return ua | ub;
}

template <bool kBF16Out, bool kGelu>
__global__ __launch_bounds__(kThreads) void w4a4_gemm_kernel(const uint8_t* __restrict__ Xq,
                                                            const float* __restrict__ x_scale,
                                                            const uint8_t* __restrict__ Wq,
                                                            const float* __restrict__ w_scale,
                                                            const float* __restrict__ bias, int64_t M,
                                                            int64_t N, int64_t K, void* __restrict__ Y,
                                                            int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileN * kTileKBytes];  // [buf][A/B][...]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;

  const int64_t tiles_n = N / kTileN;
  const int64_t tile_n = blockIdx.x % tiles_n;
  const int64_t tile_m = blockIdx.x / tiles_n;
  const int64_t n0 = tile_n * kTileN;
  const int64_t m0 = tile_m * kTileM;
  const int64_t row_bytes = K / 2;

  // Global -> register staging: each thread moves two 16-byte chunks of each tile per stage.
  const uint8_t* gA[2];
  const uint8_t* gB[2];
  int lrow[2], lunit[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + kThreads * i;  // 512 chunks of 16 bytes per tile
    lrow[i] = c >> 2;
    lunit[i] = (c & 3) * 2;
    gA[i] = Wq + (n0 + lrow[i]) * row_bytes + (c & 3) * 16;
    int64_t mr = m0 + lrow[i];
    if (mr > M - 1) mr = M - 1;  // ragged tail: duplicate the last row; its outputs are not stored
    gB[i] = Xq + mr * row_bytes + (c & 3) * 16;
  }
  uint4 stA[2], stB[2];
  auto gload = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      stA[i] = *reinterpret_cast<const uint4*>(gA[i] + kb);
      stB[i] = *reinterpret_cast<const uint4*>(gB[i] + kb);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint8_t* a = &lds[buf][0][0];
      uint8_t* b = &lds[buf][1][0];
      *reinterpret_cast<uint2*>(a + lds_off(lrow[i], lunit[i])) = make_uint2(stA[i].x, stA[i].y);
      *reinterpret_cast<uint2*>(a + lds_off(lrow[i], lunit[i] + 1)) = make_uint2(stA[i].z, stA[i].w);
      *reinterpret_cast<uint2*>(b + lds_off(lrow[i], lunit[i])) = make_uint2(stB[i].x, stB[i].y);
      *reinterpret_cast<uint2*>(b + lds_off(lrow[i], lunit[i] + 1)) = make_uint2(stB[i].z, stB[i].w);
    }
  };

  v4i acc[kFragN][kFragM];
#pragma unroll
  for (int a = 0; a < kFragN; ++a)
#pragma unroll
    for (int b = 0; b < kFragM; ++b) acc[a][b] = v4i{0, 0, 0, 0};

  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int nk = (int)(K / (2 * kTileKBytes));

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * kTileKBytes);
    const uint8_t* As = &lds[cur][0][0];
    const uint8_t* Bs = &lds[cur][1][0];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int u = 4 * s + g;  // 8-byte unit of this lane inside the 64-byte row chunk
      v4i fa[kFragN], fb[kFragM];
#pragma unroll
      for (int a = 0; a < kFragN; ++a)
        fa[a] = widen(*reinterpret_cast<const uint2*>(As + lds_off(wn * kWaveN + 16 * a + r16, u)));
#pragma unroll
      for (int b = 0; b < kFragM; ++b)
        fb[b] = widen(*reinterpret_cast<const uint2*>(Bs + lds_off(wm * kWaveM + 16 * b + r16, u)));
#pragma unroll
      for (int a = 0; a < kFragN; ++a)
#pragma unroll
        for (int b = 0; b < kFragM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane owns n = n0 + wn*64 + 16a + 4g + (0..3), m = m0 + wm*64 + 16b + r16.
#pragma unroll
  for (int b = 0; b < kFragM; ++b) {
    const int64_t m = m0 + wm * kWaveM + 16 * b + r16;
    if (m >= M) continue;
    const float sa = x_scale[m];
#pragma unroll
    for (int a = 0; a < kFragN; ++a) {
      const int64_t n = n0 + wn * kWaveN + 16 * a + 4 * g;
      const float4 sw = *reinterpret_cast<const float4*>(w_scale + n);
      float y[4];
      const float swv[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) y[v] = (float)(acc[a][b][v] >> 8) * sa * swv[v];
      if (bias) {
        const float4 bv = *reinterpret_cast<const float4*>(bias + n);
        y[0] += bv.x; y[1] += bv.y; y[2] += bv.z; y[3] += bv.w;
      }
      if constexpr (kGelu) {
#pragma unroll
        for (int v = 0; v < 4; ++v) y[v] = gelu(y[v]);
      }
      if constexpr (kBF16Out) {
        uint16_t* out = static_cast<uint16_t*>(Y) + m * ldy + n;
        *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      } else {
        float* out = static_cast<float*>(Y) + m * ldy + n;
        *reinterpret_cast<float4*>(out) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  }
}

template <bool kBF16Out, bool kGelu>
hipError_t launch_t(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, const float* bias,
                    int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, hipStream_t st) {
  const int64_t blocks = (N / kTileN) * ((M + kTileM - 1) / kTileM);
  hipLaunchKernelGGL((w4a4_gemm_kernel<kBF16Out, kGelu>), dim3((unsigned)blocks), dim3(kThreads), 0, st, Xq, xs,
                     Wq, ws, bias, M, N, K, Y, ldy);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                            const float* bias, int64_t M, int64_t N, int64_t K, bool gelu, void* Y, bool bf16_out,
                            int64_t ldy, hipStream_t st) {
  if (bf16_out) {
    return gelu ? launch_t<true, true>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st)
                : launch_t<true, false>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st);
  }
  return gelu ? launch_t<false, true>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st)
              : launch_t<false, false>(Xq, xs, Wq, ws, bias, M, N, K, Y, ldy, st);
}

}  // namespace qv
