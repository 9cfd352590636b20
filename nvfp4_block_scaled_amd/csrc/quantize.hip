// BF16 -> NVFP4 activation quantizer: a tensor-max pass and a block pass.
//
// Both passes are HBM-bound. Every floating-point step is a single IEEE
// binary32 operation with round-to-nearest-even (no contraction, no fast math),
// in the order stated in nvfp4.h, so the output is bit-identical to any other
// implementation of that order. The E4M3 scale is rounded with integer logic.
// The E2M1 codes come from v_cvt_scalef32_pk_fp4_f32 with scale operand 1.0:
// round-to-nearest-even on the E2M1 grid, saturating at 6, keeping the sign of
// zero -- checked equal to that rule on every finite BF16 value and two million
// random FP32 values -- at half a vector instruction per element.
#pragma clang fp contract(off)

#include "common.hpp"

namespace nvfp4 {

static constexpr int kAmaxBlocks = 1024;   // workgroups of the tensor-max pass
static constexpr int kThreads = 256;

size_t quantize_workspace_bytes(int64_t rows, int64_t K) {
  (void)rows;
  (void)K;
  return (size_t)kAmaxBlocks * sizeof(uint32_t);
}

// |x| of a BF16 value orders like its low 15 bits taken as an unsigned integer
// (finite inputs), so the maximum is taken on bit patterns.
__device__ __forceinline__ uint32_t absmax8(u32x4_t v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    m = max(m, v[i] & 0x7FFFu);
    m = max(m, (v[i] >> 16) & 0x7FFFu);
  }
  return m;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int w = 1; w < kThreads / 64; w++) m = max(m, red[w]);
    red[kThreads / 64] = m;
  }
  __syncthreads();
  return red[kThreads / 64];
}

// Pass 1: per-workgroup maximum of |x| bit patterns over a grid-strided range.
__global__ __launch_bounds__(kThreads) void amax_kernel(const u32x4_t *__restrict__ x, int64_t n16,
                                                        uint32_t *__restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (int64_t)gridDim.x * kThreads)
    m = max(m, absmax8(x[i]));
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// E4M3 byte of u >= 0 (or +inf): round to nearest even on the E4M3 grid,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float u) {
  if (!(u < 448.0f)) return 0x7Eu;                 // >= 448 or +inf
  if (u < 0.015625f) {                             // below 2^-6: grid step 2^-9
    return (uint32_t)__builtin_rintf(u * 512.0f);  // 0..8, and 8 encodes 2^-6
  }
  uint32_t b = __float_as_uint(u);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;   // keep 3 mantissa bits, RNE
  const uint32_t e = (b >> 23) - 127u + 7u;               // biased E4M3 exponent (1..15)
  return (e << 3) | ((b >> 20) & 7u);
}

// Value of a finite, non-negative E4M3 byte.
__device__ __forceinline__ float e4m3_value(uint32_t s) {
  const uint32_t e = s >> 3, m = s & 7u;
  if (e == 0) return (float)m * 0.001953125f;                      // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));          // 2^(e-7) * (1 + m/8)
}

// E2M1 magnitude code of v >= 0: the number of rounding thresholds v passes,
// with ties sent to the even code (0.25 -> 0, 0.75 -> 2, 1.25 -> 2, 1.75 -> 4,
// 2.5 -> 4, 3.5 -> 6, 5 -> 6); saturates at 7 (6.0); NaN gives 0.
// Pass 2: one thread per 16-element block, grid-striding. Every workgroup first
// reduces the pass-1 maxima (a few KB) to the tensor maximum and forms g.
//
// TILED: codes and scales go straight into the prepared tile layout of the
// activation (see nvfp4_tile_activation) at `codes`, for rows rounded up to 32
// (nblocks_out blocks; the blocks of the padding rows are written as zero).
template <bool TILED>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const u32x4_t *__restrict__ x, int64_t nblocks,
                                                            int64_t nblocks_out, int64_t K,
                                                            const uint32_t *__restrict__ partial, int npartial,
                                                            u32x2_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                            float *__restrict__ g_out, float *__restrict__ inv_g_out) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
  m = block_max_u32(m, red);
  const float amax_t = __uint_as_float(m << 16);
  const float g = (amax_t == 0.0f) ? 1.0f : 2688.0f / amax_t;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g_out[0] = g;
    if (inv_g_out) inv_g_out[0] = 1.0f / g;
  }
  for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks_out;
       blk += (int64_t)gridDim.x * kThreads) {
    const bool real = blk < nblocks;
    const u32x4_t v0 = real ? x[2 * blk] : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t v1 = real ? x[2 * blk + 1] : u32x4_t{0u, 0u, 0u, 0u};
    const uint32_t amax_bits = max(absmax8(v0), absmax8(v1));
    uint32_t sbyte = 0;
    if (amax_bits != 0) {
      const float amax_b = __uint_as_float(amax_bits << 16);
      const float t = amax_b / 6.0f;
      const float u = t * g;
      sbyte = e4m3_rne_sat(u);
    }
    u32x2_t out = {0u, 0u};
    if (sbyte != 0) {
      const float s = e4m3_value(sbyte);
      const float r = g / s;
      uint32_t words[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        words[i] = v0[i];
        words[4 + i] = v1[i];
      }
      // two BF16 elements per word, element 2i in the low half -> low nibble of byte i
#define NVFP4_CVT_BYTE(D, B)                                                                             \
  out[D] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[D], __uint_as_float(words[4 * D + B] << 16) * r,  \
                                                    __uint_as_float(words[4 * D + B] & 0xFFFF0000u) * r, \
                                                    1.0f, B)
      NVFP4_CVT_BYTE(0, 0); NVFP4_CVT_BYTE(0, 1); NVFP4_CVT_BYTE(0, 2); NVFP4_CVT_BYTE(0, 3);
      NVFP4_CVT_BYTE(1, 0); NVFP4_CVT_BYTE(1, 1); NVFP4_CVT_BYTE(1, 2); NVFP4_CVT_BYTE(1, 3);
#undef NVFP4_CVT_BYTE
    }
    if (TILED) {
      // block b of row `row` -> tile (row / 32, b / 4), unit 32 ((b % 4) / 2) + row % 32, half b % 2
      const int64_t nb = K / 16, kt = K / 64;
      const int64_t row = blk / nb, b = blk - row * nb;
      const int64_t tile = (row >> 5) * kt + (b >> 2);
      const int64_t rr = row & 31;
      uint8_t *base = reinterpret_cast<uint8_t *>(codes);
      *reinterpret_cast<u32x2_t *>(base + tile * 1024 + 16 * (32 * ((b & 3) >> 1) + rr) + 8 * (b & 1)) = out;
      base[nblocks_out * 8 + tile * 128 + rr * 4 + (b & 3)] = (uint8_t)sbyte;
    } else {
      codes[blk] = out;
      scales[blk] = (uint8_t)sbyte;
    }
  }
}

}  // namespace nvfp4

using namespace nvfp4;

namespace {

nvfp4_status quantize_common(const uint16_t *x, int64_t rows, int64_t K, bool tiled, void *codes, uint8_t *scales,
                             float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, hipStream_t s) {
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < quantize_workspace_bytes(rows, K)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(codes, tiled ? 16 : 8) || !aligned(ws, 4) || !aligned(g_dev, 4) ||
      (inv_g_dev && !aligned(inv_g_dev, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  const int64_t n16 = rows * K / 8;          // 16-byte chunks of x
  const int64_t nblocks = rows * K / 16;     // 16-element blocks
  const int64_t nblocks_out = tiled ? (rows + 31) / 32 * 32 * K / 16 : nblocks;
  hipLaunchKernelGGL(amax_kernel, dim3(kAmaxBlocks), dim3(kThreads), 0, s, (const u32x4_t *)x, n16,
                     (uint32_t *)ws);
  NVFP4_LAUNCH_CHECK();
  int64_t grid = (nblocks_out + kThreads - 1) / kThreads;
  if (grid > 8 * (int64_t)d.num_cus) grid = 8 * (int64_t)d.num_cus;   // the maxima are reduced once per workgroup
  if (grid < 1) grid = 1;
  if (tiled)
    hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, (const u32x4_t *)x, nblocks,
                       nblocks_out, K, (const uint32_t *)ws, kAmaxBlocks, (u32x2_t *)codes, nullptr, g_dev,
                       inv_g_dev);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, (const u32x4_t *)x,
                       nblocks, nblocks_out, K, (const uint32_t *)ws, kAmaxBlocks, (u32x2_t *)codes, scales, g_dev,
                       inv_g_dev);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // namespace

extern "C" nvfp4_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales,
                                       float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return NVFP4_ERR_NULL;
  return quantize_common(x, rows, K, false, codes, scales, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_quantize_tiled(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a_tiled,
                                             float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes,
                                             void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !a_tiled)) return NVFP4_ERR_NULL;
  return quantize_common(x, rows, K, true, a_tiled, nullptr, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}
