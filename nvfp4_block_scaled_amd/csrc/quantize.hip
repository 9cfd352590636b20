// BF16 -> NVFP4 activation quantizer: a tensor-max pass and a block pass (and,
// for the two-pass prefill, a residual pass per block inside the block pass).
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

#include <mutex>

#include "common.hpp"

namespace nvfp4 {

static constexpr int kAmaxBlocks = 1024;   // workgroups of the tensor-max pass
static constexpr int kThreads = 256;

size_t quantize_workspace_bytes(int64_t rows, int64_t K) {
  (void)rows;
  (void)K;
  return (size_t)kAmaxBlocks * sizeof(uint32_t);
}

// The quantizer's workspace for callers that cannot allocate: the tensor-max
// pass's per-workgroup maxima, kAmaxBlocks words (4 KiB) whatever the input
// size, in a device array of the library's own. Host code never passes
// `scratch` itself to a kernel (on the host it names a host-side stand-in):
// it passes the device address that hipGetSymbolAddress returns for it, looked
// up once per device with that device current.
static __device__ __align__(256) uint32_t scratch[kAmaxBlocks];
static void *g_scratch_ptr[kMaxDevices];
static nvfp4_status g_scratch_status[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

// Runs once per device, with `dev` the current device.
static void lookup_scratch(int dev) {
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  g_scratch_ptr[dev] = (e == hipSuccess) ? ptr : nullptr;
  g_scratch_status[dev] = (e == hipSuccess && ptr) ? NVFP4_OK : NVFP4_ERR_HIP;
}

// The scratch array's device address on the current device (looked up on the
// first use there unless nvfp4_init did it).
static nvfp4_status scratch_of_current(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], lookup_scratch, dev);
  *out = g_scratch_ptr[dev];
  return g_scratch_status[dev];
}

nvfp4_status device_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return NVFP4_ERR_VALUE;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return NVFP4_ERR_HIP;
  if (prev != device && hipSetDevice(device) != hipSuccess) return NVFP4_ERR_HIP;
  std::call_once(g_scratch_once[device], lookup_scratch, device);
  if (prev != device && hipSetDevice(prev) != hipSuccess) return NVFP4_ERR_HIP;
  return g_scratch_status[device];
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

// One 16-element block (two 16-byte chunks of BF16) under the global scale g:
// the scale byte (E4M3 of amax_b / 6 * g, 0 for an all-zero block) in *sbyte
// and the eight code bytes, element 2i in the low nibble of byte i.
__device__ __forceinline__ u32x2_t quantize_block(const u32x4_t v0, const u32x4_t v1, float g, uint32_t *sbyte) {
  const uint32_t amax_bits = max(absmax8(v0), absmax8(v1));
  uint32_t sb = 0;
  if (amax_bits != 0) {
    const float amax_b = __uint_as_float(amax_bits << 16);
    const float t = amax_b / 6.0f;
    const float u = t * g;
    sb = e4m3_rne_sat(u);
  }
  *sbyte = sb;
  u32x2_t out = {0u, 0u};
  if (sb != 0) {
    const float s = e4m3_value(sb);
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
  return out;
}

// quantize_block on sixteen FP32 values (the residual pass of the two-pass
// recipe): the same steps, with |v| maxima taken on floats (exact).
__device__ __forceinline__ u32x2_t quantize_block_f32(const float (&v)[16], float g, uint32_t *sbyte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t sb = 0;
  if (amax != 0.0f) {
    const float t = amax / 6.0f;
    const float u = t * g;
    sb = e4m3_rne_sat(u);
  }
  *sbyte = sb;
  u32x2_t out = {0u, 0u};
  if (sb != 0) {
    const float r = g / e4m3_value(sb);
#define NVFP4_CVT_F32(D, B) \
  out[D] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out[D], v[8 * D + 2 * B] * r, v[8 * D + 2 * B + 1] * r, 1.0f, B)
    NVFP4_CVT_F32(0, 0); NVFP4_CVT_F32(0, 1); NVFP4_CVT_F32(0, 2); NVFP4_CVT_F32(0, 3);
    NVFP4_CVT_F32(1, 0); NVFP4_CVT_F32(1, 1); NVFP4_CVT_F32(1, 2); NVFP4_CVT_F32(1, 3);
#undef NVFP4_CVT_F32
  }
  return out;
}

// The residual of a quantized block: r_i = x_i - fl32(code_i * scale / g) for
// the block's sixteen BF16 inputs (two 16-byte chunks), its codes and scale byte.
// code * scale is exact in FP32; the division and the subtraction round once each.
__device__ __forceinline__ void block_residual(const u32x4_t v0, const u32x4_t v1, u32x2_t codes, uint32_t sbyte,
                                               float g, float (&res)[16]) {
  const float s = sbyte ? e4m3_value(sbyte) : 0.0f;
  // byte B of code word D: elements 8 D + 2 B (low nibble) and 8 D + 2 B + 1, from word B of chunk D
#define NVFP4_RES(D, V, B)                                                                \
  {                                                                                       \
    const f32x2_t q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[D], 1.0f, B);        \
    res[8 * D + 2 * B] = __uint_as_float(V[B] << 16) - (q[0] * s) / g;                    \
    res[8 * D + 2 * B + 1] = __uint_as_float(V[B] & 0xFFFF0000u) - (q[1] * s) / g;        \
  }
  NVFP4_RES(0, v0, 0) NVFP4_RES(0, v0, 1) NVFP4_RES(0, v0, 2) NVFP4_RES(0, v0, 3)
  NVFP4_RES(1, v1, 0) NVFP4_RES(1, v1, 1) NVFP4_RES(1, v1, 2) NVFP4_RES(1, v1, 3)
#undef NVFP4_RES
}

// Every workgroup of pass 2 first reduces the pass-1 maxima (a few KB) to the
// tensor maximum and forms g (block 0 stores g and 1/g).
__device__ __forceinline__ float global_scale(const uint32_t *__restrict__ partial, int npartial, uint32_t *red,
                                              float *__restrict__ g_out, float *__restrict__ inv_g_out) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
  m = block_max_u32(m, red);
  const float amax_t = __uint_as_float(m << 16);
  const float g = (amax_t == 0.0f) ? 1.0f : 2688.0f / amax_t;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    g_out[0] = g;
    if (inv_g_out) inv_g_out[0] = 1.0f / g;
  }
  return g;
}

// Pass 2, row-major output: one thread per 16-element block, grid-striding.
__global__ __launch_bounds__(kThreads) void quantize_kernel(const u32x4_t *__restrict__ x, int64_t nblocks,
                                                            const uint32_t *__restrict__ partial, int npartial,
                                                            u32x2_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                            float *__restrict__ g_out, float *__restrict__ inv_g_out) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  const float g = global_scale(partial, npartial, red, g_out, inv_g_out);
  for (int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x; blk < nblocks;
       blk += (int64_t)gridDim.x * kThreads) {
    uint32_t sbyte;
    codes[blk] = quantize_block(x[2 * blk], x[2 * blk + 1], g, &sbyte);
    scales[blk] = (uint8_t)sbyte;
  }
}

// Pass 2, tile-layout output (the layout nvfp4_tile_activation writes): one
// wave per tile of 32 rows x 64 K, grid-striding over the tiles in their
// storage order. Lane 32 h + r quantizes blocks 2h and 2h+1 of the tile's row
// r; its 16 code bytes are unit 32 h + r of the tile's 1 KiB of codes and its
// two scale bytes sit at 4 r + 2h of the tile's 128 scale bytes, so a wave
// stores 1 KiB and 128 B contiguously. Rows from `rows` up to the next
// multiple of 32 read as zero and are written as zero.
__global__ __launch_bounds__(kThreads) void quantize_tiled_kernel(const u32x4_t *__restrict__ x, int64_t rows,
                                                                  int64_t K, int64_t ntiles,
                                                                  const uint32_t *__restrict__ partial, int npartial,
                                                                  uint8_t *__restrict__ out, float *__restrict__ g_out,
                                                                  float *__restrict__ inv_g_out) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  const float g = global_scale(partial, npartial, red, g_out, inv_g_out);
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int64_t kt = K / 64, x_row = K / 8;          // tiles along K; 16-byte chunks per row of x
  u32x4_t *const code_out = reinterpret_cast<u32x4_t *>(out);
  uint16_t *const scale_out = reinterpret_cast<uint16_t *>(out + ntiles * 1024);
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t tile = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); tile < ntiles; tile += wstride) {
    const int64_t rg = tile / kt, kk = tile - rg * kt;
    const int64_t row = rg * 32 + r;
    u32x4_t v[4] = {};
    if (row < rows) {
      const u32x4_t *src = x + row * x_row + kk * 8 + h * 4;
#pragma unroll
      for (int i = 0; i < 4; i++) v[i] = src[i];
    }
    uint32_t s0, s1;
    const u32x2_t c0 = quantize_block(v[0], v[1], g, &s0);
    const u32x2_t c1 = quantize_block(v[2], v[3], g, &s1);
    code_out[tile * 64 + lane] = u32x4_t{c0[0], c0[1], c1[0], c1[1]};
    scale_out[tile * 64 + 2 * r + h] = (uint16_t)(s0 | (s1 << 8));
  }
}

// Two-pass tile-layout output: the value pass into the K chunks [0, kt) of an
// activation of 2K columns and the residual pass, under the same g, into
// chunks [kt, 2 kt) of the same rows. Otherwise as quantize_tiled_kernel (one
// wave per 32 x 64 tile of x, lane 32 h + r on blocks 2h, 2h + 1 of row r).
__global__ __launch_bounds__(kThreads) void quantize_two_pass_tiled_kernel(
    const u32x4_t *__restrict__ x, int64_t rows, int64_t K, int64_t ntiles, const uint32_t *__restrict__ partial,
    int npartial, uint8_t *__restrict__ out, float *__restrict__ g_out, float *__restrict__ inv_g_out) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  const float g = global_scale(partial, npartial, red, g_out, inv_g_out);
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int64_t kt = K / 64, x_row = K / 8;
  u32x4_t *const code_out = reinterpret_cast<u32x4_t *>(out);
  uint16_t *const scale_out = reinterpret_cast<uint16_t *>(out + 2 * ntiles * 1024);   // 2 ntiles tiles of codes
  const int64_t wstride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t tile = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); tile < ntiles; tile += wstride) {
    const int64_t rg = tile / kt, kk = tile - rg * kt;
    const int64_t row = rg * 32 + r;
    u32x4_t v[4] = {};
    if (row < rows) {
      const u32x4_t *src = x + row * x_row + kk * 8 + h * 4;
#pragma unroll
      for (int i = 0; i < 4; i++) v[i] = src[i];
    }
    const int64_t t1 = rg * 2 * kt + kk, t2 = t1 + kt;       // value and residual tiles of the 2K layout
    uint32_t s0, s1;
    const u32x2_t c0 = quantize_block(v[0], v[1], g, &s0);
    const u32x2_t c1 = quantize_block(v[2], v[3], g, &s1);
    code_out[t1 * 64 + lane] = u32x4_t{c0[0], c0[1], c1[0], c1[1]};
    scale_out[t1 * 64 + 2 * r + h] = (uint16_t)(s0 | (s1 << 8));
    float res[16];
    block_residual(v[0], v[1], c0, s0, g, res);
    const u32x2_t e0 = quantize_block_f32(res, g, &s0);
    block_residual(v[2], v[3], c1, s1, g, res);
    const u32x2_t e1 = quantize_block_f32(res, g, &s1);
    code_out[t2 * 64 + lane] = u32x4_t{e0[0], e0[1], e1[0], e1[1]};
    scale_out[t2 * 64 + 2 * r + h] = (uint16_t)(s0 | (s1 << 8));
  }
}

}  // namespace nvfp4

using namespace nvfp4;

namespace {

nvfp4_status quantize_common(const uint16_t *x, int64_t rows, int64_t K, int mode, void *codes, uint8_t *scales,
                             float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, hipStream_t s) {
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < quantize_workspace_bytes(rows, K)) return NVFP4_ERR_WORKSPACE;
  const bool tiled = mode != 0;
  if (!aligned(x, 16) || !aligned(codes, tiled ? 16 : 8) || !aligned(ws, 4) || !aligned(g_dev, 4) ||
      (inv_g_dev && !aligned(inv_g_dev, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  const int64_t n16 = rows * K / 8;          // 16-byte chunks of x
  const int64_t nblocks = rows * K / 16;     // 16-element blocks
  hipLaunchKernelGGL(amax_kernel, dim3(kAmaxBlocks), dim3(kThreads), 0, s, (const u32x4_t *)x, n16,
                     (uint32_t *)ws);
  NVFP4_LAUNCH_CHECK();
  // every workgroup reduces the pass-1 maxima once, so the grid is capped
  const int64_t max_grid = 8 * (int64_t)d.num_cus;
  if (tiled) {
    const int64_t ntiles = (rows + 31) / 32 * (K / 64);
    const int64_t grid = std::max<int64_t>(1, std::min(max_grid, (ntiles + kThreads / 64 - 1) / (kThreads / 64)));
    if (mode == 2)
      hipLaunchKernelGGL(quantize_two_pass_tiled_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const u32x4_t *)x, rows, K, ntiles, (const uint32_t *)ws, kAmaxBlocks, (uint8_t *)codes,
                         g_dev, inv_g_dev);
    else
      hipLaunchKernelGGL(quantize_tiled_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, (const u32x4_t *)x, rows,
                         K, ntiles, (const uint32_t *)ws, kAmaxBlocks, (uint8_t *)codes, g_dev, inv_g_dev);
  } else {
    const int64_t grid = std::max<int64_t>(1, std::min(max_grid, (nblocks + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, (const u32x4_t *)x, nblocks,
                       (const uint32_t *)ws, kAmaxBlocks, (u32x2_t *)codes, scales, g_dev, inv_g_dev);
  }
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // namespace

extern "C" nvfp4_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales,
                                       float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return NVFP4_ERR_NULL;
  return quantize_common(x, rows, K, 0, codes, scales, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_quantize_tiled(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a_tiled,
                                             float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes,
                                             void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !a_tiled)) return NVFP4_ERR_NULL;
  return quantize_common(x, rows, K, 1, a_tiled, nullptr, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_quantize_two_pass_tiled(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a2_tiled,
                                                      float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes,
                                                      void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !a2_tiled)) return NVFP4_ERR_NULL;
  return quantize_common(x, rows, K, 2, a2_tiled, nullptr, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_quantize_tiled_noalloc(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a_tiled,
                                                     float *g_dev, float *inv_g_dev, void *stream) {
  if (!g_dev) return NVFP4_ERR_NULL;
  if (rows < 0 || K <= 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && (!x || !a_tiled)) return NVFP4_ERR_NULL;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  void *ws = nullptr;
  st = scratch_of_current(&ws);
  if (st != NVFP4_OK) return st;
  // the scratch holds exactly the workspace this quantizer needs, for any rows and K
  const size_t ws_bytes = sizeof(scratch);
  if (quantize_workspace_bytes(rows, K) > ws_bytes) return NVFP4_ERR_WORKSPACE;
  return quantize_common(x, rows, K, 1, a_tiled, nullptr, g_dev, inv_g_dev, ws, ws_bytes, (hipStream_t)stream);
}
