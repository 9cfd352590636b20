// BF16 -> NVFP4 activation quantizer (and, for the two-pass prefill, a
// residual pass per block). The global scale needs the maximum of |x| over the
// whole tensor before any block can be encoded. Two forms:
//  * one read of x (quantize_fused_kernel): when x fits in the vector registers
//    of a grid of one 1024-thread workgroup per CU (up to 5 tiles of 32 x 64 per
//    wave, 80 MiB of BF16 on 256 CUs), every workgroup loads its tiles once,
//    publishes its maximum, waits at a grid-wide barrier and encodes from the
//    registers;
//  * two reads (amax_kernel, then a block pass) for anything larger.
//
// Both forms are HBM-bound. Every floating-point step is a single IEEE
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
// The workspace: the tensor-max pass's per-workgroup maxima (kAmaxBlocks
// words), then the one-read form's barrier state: a generation word (16 bytes
// reserved) and one 64-bit slot per workgroup (at most kAmaxBlocks).
static constexpr size_t kFusedStateOff = (size_t)kAmaxBlocks * 4;
static constexpr size_t kFusedSlotsOff = kFusedStateOff + 16;
static constexpr size_t kQuantizeWsBytes = (kFusedSlotsOff + (size_t)kAmaxBlocks * 8 + 255) / 256 * 256;

size_t quantize_workspace_bytes(int64_t rows, int64_t K) {
  (void)rows;
  (void)K;
  return kQuantizeWsBytes;
}

// The quantizer's workspace for callers that cannot allocate (kQuantizeWsBytes,
// 12.25 KiB, whatever the input size), in a device array of the library's own.
// Host code never passes `scratch` itself to a kernel (on the host it names a
// host-side stand-in): it passes the device address that hipGetSymbolAddress
// returns for it, looked up once per device with that device current.
static __device__ __align__(256) uint32_t scratch[kQuantizeWsBytes / 4];
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

// Pass 1: per-workgroup maximum of |x| bit patterns over a grid-strided range,
// four independent 16-byte loads in flight per thread.
__global__ __launch_bounds__(kThreads) void amax_kernel(const u32x4_t *__restrict__ x, int64_t n16,
                                                        uint32_t *__restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64 + 1];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(x + i), b = __builtin_nontemporal_load(x + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(x + i + 2 * stride), d = __builtin_nontemporal_load(x + i + 3 * stride);
    m = max(m, max(max(absmax8(a), absmax8(b)), max(absmax8(c), absmax8(d))));
  }
  for (; i < n16; i += stride) m = max(m, absmax8(x[i]));
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

// ---------------------------------------------------------------- one read of x
//
// One workgroup of 1024 threads per CU. Workgroup w owns the run of myrun <= 80
// tiles (32 rows x 64 columns) w run .. w run + myrun - 1 in storage order, that
// is myrun * 256 16-byte chunks of x: cell (r, t) is row r of the run's tile t
// (128 contiguous bytes of x), and chunk c of the run is chunk c % 8 of cell
// e = c / 8, cells ordered tile-major (t = e / 32, r = e % 32). Thread tau holds
// chunks tau + 1024 i (i < kFusedChunks, 80 VGPRs), i.e. chunk q = tau % 8 of
// row r = (tau / 8) % 32 of tile t = tau / 256 + 4 i: one load instruction of a
// wave reads eight whole 128-byte rows of one tile, one code store of a wave
// writes two whole 128-byte lines of its tile's codes, and threads tau and
// tau ^ 1 hold the two halves of one 16-element block.
//
// While the loads arrive, each thread also forms every chunk's 16-element block
// maximum (its half and its partner's) divided by 6, and keeps it in LDS for
// the encode. Each workgroup stores the maximum of |x| bit patterns over its
// run in its slot of the workspace and waits until all gridDim.x slots are
// filled in this call. The workspace keeps a generation number: every workgroup reads it on
// entry and tags its slot with tag(gen) = gen ^ kTagMix in the high word of one
// 64-bit atomic store (the maximum in the low word), then waits until every
// slot carries that tag, then adds 1 to the generation. A workgroup passes the
// wait only after every workgroup has stored its slot, and each store uses the
// generation its workgroup read, so every read comes before every increment;
// the next call therefore reads gen + gridDim.x and its tag differs from this
// call's. Nothing needs resetting between calls and a workspace needs no
// initialisation: a slot of memory filled with any constant c cannot carry the
// tag of generation c, since c ^ kTagMix != c, and neither can the small
// maxima the two-read form leaves in the same bytes (their high words are 0).
// (A slot left untouched while the generation goes all the way round 2^32
// would match again; random bytes match with probability 2^-32 a slot.) Slot
// and generation accesses are agent-scope atomics (coherent across the XCDs).
// The host launches this form only when the whole grid fits on the device at
// once (the occupancy query), so every workgroup reaches its store; the wait
// is bounded all the same (kSpinLimit polls, about a second), and a workgroup
// whose wait runs out encodes its run with g = NaN.
//
// With g known, the workgroup tabulates g / scale for the 127 scale bytes
// (and, for the two-pass form, fl32(code * scale / g) for each scale byte and
// code) in LDS and encodes and stores its chunks one by one.
static constexpr int kFusedThreads = 1024;
static constexpr int kFusedWaves = kFusedThreads / 64;
static constexpr int kFusedChunks = 20;
static constexpr int kFusedRun = kFusedChunks * kFusedThreads / 256;   // 80 tiles per workgroup at most
static constexpr uint32_t kTagMix = 0x5EED5EEDu;
static constexpr uint32_t kNoMax = 0xFFFFFFFFu;     // the wait ran out (no BF16 magnitude reaches it)
static constexpr int kSpinLimit = 1 << 20;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// n / d for 0 <= n < 2^22 and 1 <= d < 2^22: an FP32 estimate, then one
// correction each way (the estimate is within one of the quotient).
__device__ __forceinline__ int div_small(int n, int d, float inv_d) {
  int q = (int)((float)n * inv_d);
  if (q * d > n) q--;
  if ((q + 1) * d <= n) q++;
  return q;
}

// E2M1 codes of eight elements (a 16-byte chunk of BF16, element 2i in the low
// half of word i) times r: four code bytes, element 2i in the low nibble of byte i.
__device__ __forceinline__ uint32_t codes8(const u32x4_t v, float r) {
  uint32_t out = 0u;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v[0] << 16) * r,
                                                 __uint_as_float(v[0] & 0xFFFF0000u) * r, 1.0f, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v[1] << 16) * r,
                                                 __uint_as_float(v[1] & 0xFFFF0000u) * r, 1.0f, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v[2] << 16) * r,
                                                 __uint_as_float(v[2] & 0xFFFF0000u) * r, 1.0f, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v[3] << 16) * r,
                                                 __uint_as_float(v[3] & 0xFFFF0000u) * r, 1.0f, 3);
  return out;
}

// Scale byte of a block from its |x| maximum under g: E4M3 of amax / 6 * g,
// 0 for an all-zero block.
__device__ __forceinline__ uint32_t block_scale_byte(float amax, float g) {
  if (amax == 0.0f) return 0u;
  const float t = amax / 6.0f;
  const float u = t * g;
  return e4m3_rne_sat(u);
}

// The value of the neighbouring lane of a pair (lane ^ 1), by a DPP quad
// permutation (no LDS round trip).
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
}

// The four scale bytes of a cell (blocks 0..3, held by its threads q = 0, 2, 4,
// 6) as one word, in the thread with q = 0 (DPP row shifts: lane + 2, + 4, + 6
// stay inside the 16-lane row).
__device__ __forceinline__ uint32_t cell_scales(uint32_t sb) {
  const uint32_t s1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x102, 0xF, 0xF, false);   // row_shl:2
  const uint32_t s2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x104, 0xF, 0xF, false);   // row_shl:4
  const uint32_t s3 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)sb, 0x106, 0xF, 0xF, false);   // row_shl:6
  return sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// e4m3_rne_sat without branches: both roundings formed, one selected.
__device__ __forceinline__ uint32_t e4m3_rne_sat_sel(float u) {
  const uint32_t b = __float_as_uint(u);
  const uint32_t bn = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;   // 3 mantissa bits, RNE
  const uint32_t norm = (((bn >> 23) - 120u) << 3) | ((bn >> 20) & 7u);
  const uint32_t sub = (uint32_t)__builtin_rintf(u * 512.0f);          // below 2^-6: step 2^-9
  const uint32_t r = (u < 0.015625f) ? sub : norm;
  return (u < 448.0f) ? r : 0x7Eu;                                       // >= 448, +inf or NaN
}

// fl32(a / 6) for a BF16 value a >= 0: a * fl32(1/6) corrected by one FMA step,
// which equals the IEEE division for every BF16 a >= 2^-120 (checked
// exhaustively); smaller a, whose quotient may be subnormal, divide.
__device__ __forceinline__ float bf16_div6(float a) {
  const float c = 1.0f / 6.0f;
  const float t0 = a * c;
  const float r = __builtin_fmaf(-t0, 6.0f, a);
  const float t = __builtin_fmaf(r, c, t0);
  return (a >= 0x1p-120f) ? t : a / 6.0f;
}

// MODE 0: row-major codes [rows][K/2] (out) and scales [rows][K/16] (scales_rm);
// MODE 1: the tile layout (out), as quantize_tiled_kernel;
// MODE 2: the two-pass tile layout (out), as quantize_two_pass_tiled_kernel.
// x and the outputs of this form are under 2^31 bytes (x fits in the
// registers), so 32-bit indices suffice.
template <int MODE>
__global__ __launch_bounds__(kFusedThreads) void quantize_fused_kernel(
    const u32x4_t *__restrict__ x, int rows, int K, int ntiles, int run, float inv_kt, uint8_t *state,
    uint8_t *__restrict__ out, uint8_t *__restrict__ scales_rm, float *__restrict__ g_out,
    float *__restrict__ inv_g_out) {
  __shared__ uint32_t red[kFusedWaves + 1];
  uint32_t *const gen = reinterpret_cast<uint32_t *>(state);
  uint64_t *const slots = reinterpret_cast<uint64_t *>(state + 16);
  // this call's tag, read before this workgroup's slot is stored
  const uint32_t tag = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ^ kTagMix;
  __shared__ float rtab[128];                                     // g / scale, per scale byte
  __shared__ float qtab[MODE == 2 ? 128 * 16 : 1];                // fl32(code * scale / g)
  __shared__ float dtab[kFusedChunks * kFusedThreads];            // amax_b / 6 of each thread's chunks
  const int tau = threadIdx.x, wave = tau >> 6, lane = tau & 63, q = tau & 7;
  const int kt = K / 64, x_row = K / 8;
  const int tile0 = (int)blockIdx.x * run;
  const int myrun = min(run, ntiles - tile0);            // the last run may be shorter
  const int r = (tau >> 3) & 31, t_base = tau >> 8;      // this thread's row and first tile

  u32x4_t v[kFusedChunks];
#pragma unroll
  for (int i = 0; i < kFusedChunks; i++) {
    const int tile = tile0 + t_base + 4 * i;
    const int rg = div_small(tile, kt, inv_kt), kk = tile - rg * kt;
    const int row = rg * 32 + r;
    v[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (t_base + 4 * i < myrun && row < rows) v[i] = __builtin_nontemporal_load(x + (row * x_row + kk * 8 + q));
  }
  // The tensor maximum, and each chunk's block maximum over the block's two
  // halves (threads tau and tau ^ 1) divided by 6, kept in LDS for the encode:
  // this work overlaps the loads still in flight, where after the wait it would
  // hold up the encode (the registers have no room for it: x fills them).
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kFusedChunks; i++) {
    const uint32_t mh = absmax8(v[i]);
    m = max(m, mh);
    const uint32_t mb = max(mh, pair_swap(mh));
    dtab[i * kFusedThreads + tau] = bf16_div6(__uint_as_float(mb << 16));
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (wave == 0) {
    const uint32_t bm = wave_max_u32(lane < kFusedWaves ? red[lane] : 0u);
    if (lane == 0)
      __hip_atomic_store(slots + blockIdx.x, ((uint64_t)tag << 32) | bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t tm = kNoMax;
    for (int it = 0; it < kSpinLimit; it++) {
      // the slots this lane polls (at most 1024 slots: 16 a lane), four loads at
      // a time (registers: x holds most of them)
      uint32_t mm = 0;
      int full = 1;
      for (int k0 = 0; k0 < 16 && 64 * k0 < (int)gridDim.x; k0 += 4) {
        uint64_t u[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
          u[k] = (lane + 64 * (k0 + k) < (int)gridDim.x)
                     ? __hip_atomic_load(slots + lane + 64 * (k0 + k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : ((uint64_t)tag << 32);
#pragma unroll
        for (int k = 0; k < 4; k++) {
          full &= ((uint32_t)(u[k] >> 32) == tag);
          mm = max(mm, (uint32_t)u[k]);
        }
      }
      if (__all(full)) {
        tm = wave_max_u32(mm);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) {
      red[kFusedWaves] = tm;
      // every workgroup has read this call's generation (its slot store used
      // it): advance it by one per workgroup, gridDim.x in all
      __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const uint32_t tmb = red[kFusedWaves];
  float g;
  if (tmb == kNoMax) {
    g = __builtin_nanf("");
  } else {
    const float amax_t = __uint_as_float(tmb << 16);
    g = (amax_t == 0.0f) ? 1.0f : 2688.0f / amax_t;
  }
  if (blockIdx.x == 0 && tau == 0) {
    g_out[0] = g;
    if (inv_g_out) inv_g_out[0] = 1.0f / g;
  }
  if (tau < 128) rtab[tau] = g / e4m3_value(tau);      // entry 0 is only read for zero blocks
  if (MODE == 2) {
    for (int k = tau; k < 128 * 16; k += kFusedThreads) {
      const float code = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((uint32_t)(k & 15), 1.0f, 0)[0];
      qtab[k] = (code * e4m3_value((uint32_t)(k >> 4))) / g;
    }
  }
  __syncthreads();

  // the indices are recomputed below from copies of tau and x the compiler
  // cannot see through, so it does not keep phase 1's 20 sets of them live
  // across the wait (they would not fit beside x in the registers)
  int tau2 = tau;
  asm volatile("" : "+v"(tau2));
#pragma unroll
  for (int i = 0; i < kFusedChunks; i++) asm volatile("" : "+v"(v[i]));
  const int t2_base = tau2 >> 8;
  const int code_off = (32 * (q >> 2) + r) * 16 + (q & 3) * 4;   // this thread's word in a tile's codes
  const int ntiles_out = (MODE == 2) ? 2 * ntiles : ntiles;
  uint8_t *const scale_base = out + (size_t)ntiles_out * 1024;
#pragma unroll
  for (int i = 0; i < kFusedChunks; i++) {
    const int t = t2_base + 4 * i;
    const bool have = t < myrun;                                  // the same for the whole wave
    const int tile = tile0 + t;
    // the block's maximum / 6, from phase 1 (this thread's own entry)
    const uint32_t sb = e4m3_rne_sat_sel(dtab[i * kFusedThreads + tau2] * g);   // 0 for a zero block
    uint32_t w = codes8(v[i], rtab[sb]);
    w = sb ? w : 0u;
    if (MODE == 0) {
      const int rg = div_small(tile, kt, inv_kt), kk = tile - rg * kt;
      const int row = rg * 32 + r;
      if (have && row < rows) {
        *reinterpret_cast<uint32_t *>(out + (row * (K / 2) + kk * 32 + q * 4)) = w;
        if ((q & 1) == 0) scales_rm[row * (K / 16) + kk * 4 + (q >> 1)] = (uint8_t)sb;
      }
    } else {
      int t1 = tile;
      if (MODE == 2) {
        const int rg = div_small(tile, kt, inv_kt), kk = tile - rg * kt;
        t1 = rg * 2 * kt + kk;
      }
      const uint32_t s4 = cell_scales(sb);
      if (have) {
        __builtin_nontemporal_store(w, reinterpret_cast<uint32_t *>(out + (t1 * 1024 + code_off)));
        if (q == 0) __builtin_nontemporal_store(s4, reinterpret_cast<uint32_t *>(scale_base + (t1 * 128 + 4 * r)));
      }
      if (MODE == 2) {
        // residual of the eight elements: x - fl32(code * scale / g)
        const float *qs = qtab + sb * 16;
        float res[8];
        float ra = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; b++) {
          res[2 * b] = __uint_as_float(v[i][b] << 16) - qs[(w >> (8 * b)) & 15u];
          res[2 * b + 1] = __uint_as_float(v[i][b] & 0xFFFF0000u) - qs[(w >> (8 * b + 4)) & 15u];
          ra = fmaxf(ra, fmaxf(fabsf(res[2 * b]), fabsf(res[2 * b + 1])));
        }
        const float rb = fmaxf(ra, __uint_as_float(pair_swap(__float_as_uint(ra))));
        const uint32_t sb2 = block_scale_byte(rb, g);
        uint32_t w2 = 0u;
        if (sb2) {
          const float rr = rtab[sb2];
          w2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w2, res[0] * rr, res[1] * rr, 1.0f, 0);
          w2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w2, res[2] * rr, res[3] * rr, 1.0f, 1);
          w2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w2, res[4] * rr, res[5] * rr, 1.0f, 2);
          w2 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w2, res[6] * rr, res[7] * rr, 1.0f, 3);
        }
        const uint32_t s4b = cell_scales(sb2);
        if (have) {
          const int t2 = t1 + kt;
          __builtin_nontemporal_store(w2, reinterpret_cast<uint32_t *>(out + (t2 * 1024 + code_off)));
          if (q == 0) __builtin_nontemporal_store(s4b, reinterpret_cast<uint32_t *>(scale_base + (t2 * 128 + 4 * r)));
        }
      }
    }
    // one chunk at a time: interleaving chunks would need registers x holds.
    // The tile-layout stores are non-temporal: each wave store fills whole
    // 128-byte lines that are written once, and streaming them past the cache
    // took [8192][5120] from 27.7 to 24.3 us (tiled) and from 43.4 to 38.5 us
    // (two-pass). The row-major form's 4-byte code and 1-byte scale stores
    // leave lines partly written, and as non-temporal stores they took it from
    // 30.3 to 58.7 us, so they stay ordinary stores.
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Whether each instantiation fits at least once on every CU (then a grid of up
// to num_cus workgroups is resident at once), per device.
static bool g_fused_fits[kMaxDevices][3];
static std::once_flag g_fused_once[kMaxDevices];

static void query_fused(int dev) {
  int nb = 0;
  g_fused_fits[dev][0] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, quantize_fused_kernel<0>,
                                                                      kFusedThreads, 0) == hipSuccess && nb >= 1;
  nb = 0;
  g_fused_fits[dev][1] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, quantize_fused_kernel<1>,
                                                                      kFusedThreads, 0) == hipSuccess && nb >= 1;
  nb = 0;
  g_fused_fits[dev][2] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, quantize_fused_kernel<2>,
                                                                      kFusedThreads, 0) == hipSuccess && nb >= 1;
}

// Tiles per workgroup (run) and grid of the one-read form for `ntiles` tiles
// on `cus` CUs; *grid = 0 when x does not fit.
static void fused_shape(int64_t ntiles, int cus, int *run, int64_t *grid) {
  *run = 0;
  *grid = 0;
  if (ntiles <= 0 || cus <= 0) return;
  const int64_t wgs = std::min<int64_t>(cus, kAmaxBlocks);
  const int64_t r = (ntiles + wgs - 1) / wgs;
  if (r > kFusedRun) return;
  *run = (int)r;
  *grid = (ntiles + r - 1) / r;
}

}  // namespace nvfp4

using namespace nvfp4;

namespace {

nvfp4_status quantize_common(const uint16_t *x, int64_t rows, int64_t K, int mode, void *codes, uint8_t *scales,
                             float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, hipStream_t s) {
  if (!ws) return NVFP4_ERR_WORKSPACE;
  if (ws_bytes < quantize_workspace_bytes(rows, K)) return NVFP4_ERR_WORKSPACE;
  const bool tiled = mode != 0;
  if (!aligned(x, 16) || !aligned(codes, tiled ? 16 : 8) || !aligned(ws, 16) || !aligned(g_dev, 4) ||
      (inv_g_dev && !aligned(inv_g_dev, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  std::call_once(g_fused_once[d.device], query_fused, d.device);
  // one read of x when it fits in the registers of one resident grid
  if (K % 64 == 0 && g_fused_fits[d.device][mode]) {
    const int64_t ntiles = (rows + 31) / 32 * (K / 64);
    int run = 0;
    int64_t grid = 0;
    fused_shape(ntiles, d.num_cus, &run, &grid);
    if (grid > 0) {
      const float inv_kt = 1.0f / (float)(K / 64);
#define NVFP4_FUSED(M)                                                                                              \
  hipLaunchKernelGGL(quantize_fused_kernel<M>, dim3((unsigned)grid), dim3(kFusedThreads), 0, s, (const u32x4_t *)x, \
                     (int)rows, (int)K, (int)ntiles, run, inv_kt, (uint8_t *)ws + kFusedStateOff, (uint8_t *)codes, scales,  \
                     g_dev, inv_g_dev)
      if (mode == 0)
        NVFP4_FUSED(0);
      else if (mode == 1)
        NVFP4_FUSED(1);
      else
        NVFP4_FUSED(2);
#undef NVFP4_FUSED
      NVFP4_LAUNCH_CHECK();
      return NVFP4_OK;
    }
  }
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
