// W4A16 NVFP4 GEMM for gfx950: y = alpha * x (W.SFW)^T, x/y BF16, FP32 accumulation.
//
// Kernels, chosen by M (and, for decode, by the number of 32-row groups):
//  * M <= 4 (decode): a weight-streaming kernel on the vector ALUs. A 1024-thread
//    workgroup owns 16 weight rows (half of a 32-row prepared tile group) over
//    the whole K; its 16 waves take interleaved pairs of 64-wide K tiles. Each
//    lane streams 16 packed bytes (32 codes of one row) per tile, converts code
//    pairs to exact unscaled BF16 (cvt_scalef32_pk_bf16_fp4), dots them with x
//    in FP32 (v_dot2_f32_bf16) and multiplies each 16-block's partial sum by
//    its scale once: about 1.1 vector instructions per weight at M = 1, so the
//    kernel is bound by HBM. The K-split is reduced inside the workgroup (lane
//    butterflies, then LDS over the waves in wave order), so no workgroup ever
//    waits on another and nothing crosses an XCD within the kernel. x is staged
//    once per workgroup in LDS and read by broadcast. With at least two 32-row
//    groups per CU, a wide variant is used instead: one 512-thread workgroup
//    per whole group, each wave keeping eight 1 KB tile loads in flight (two
//    batches of four); all its workgroups are resident at once. (A K split
//    across workgroups would need an agent-scope release per workgroup, an L2
//    write-back on this part, which measured several times slower.)
//  * M > 4: an LDS-tiled MFMA kernel (v_mfma_f32_32x32x16_bf16). BF16 x tiles
//    are staged through LDS (XOR-swizzled rows, conflict-free 16-byte reads);
//    weight codes and scales are staged as packed bytes in the prepared tile
//    format and dequantized exactly to BF16 in registers (E2M1 -> FP32, times
//    the E4M3 scale in FP32, exact; -> BF16, exact). When the output tiles alone
//    cannot fill the CUs, K is split across workgroups: each writes an FP32
//    partial tile to the workspace and a second kernel adds the partials in
//    split order 0, 1, 2, ... and applies the epilogue, so the result does not
//    depend on scheduling.
#include "common.hpp"

namespace nvfp4 {
namespace w4a16 {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- planning

struct Plan {
  int kind;          // 0 = vector decode kernel, 1 = MFMA tile kernel, 2 = wide vector decode kernel,
                     // 3 = skinny MFMA kernel
  int splits;        // K splits of the tile kernel (1 = none)
  int64_t grid_x;    // workgroups along the output
};

constexpr int kDecodeMaxM = 4;
constexpr int kSkinnyMaxM = 128;
constexpr int kDecodeThreads = 1024;      // 16 waves per 16-row group
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kDecodeLdsBytes = 64 * 1024;  // x staged in LDS: M * K * 2 bytes at most
constexpr int BM = 256, BN = 128;         // tile kernel

static int num_cus_or_default() {
  DeviceInfo d;
  if (device_info(&d) == NVFP4_OK && d.num_cus > 0) return d.num_cus;
  return 256;
}

static Plan make_plan(int64_t M, int64_t N, int64_t K) {
  Plan p{};
  const int cus = num_cus_or_default();
  const int64_t ktiles = K / 64;
  if (M <= kDecodeMaxM && M * K * 2 <= kDecodeLdsBytes) {
    // one 32-row group per workgroup once there are two groups per CU; below
    // that, 16-row workgroups with 16 waves keep more of the chip busy
    p.kind = N / 32 >= 2 * cus ? 2 : 0;
    p.splits = 1;
    p.grid_x = p.kind == 2 ? N / 32 : N / 16;
  } else if (M <= kSkinnyMaxM) {
    p.kind = 3;
    p.splits = 1;
    p.grid_x = N / 32;
  } else {
    p.kind = 1;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    p.grid_x = tiles;
    int64_t s = 1;
    while (tiles * s < cus && s * 2 <= ktiles / 4 && s < 16) s *= 2;
    p.splits = (int)s;
  }
  return p;
}

static size_t workspace_for(const Plan &p, int64_t M, int64_t N) {
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * (size_t)M * (size_t)N * 4;
}

// ---------------------------------------------------------------- decode kernel (M <= 4)

// Workgroup b owns weight rows [16 b, 16 b + 16): rows 16 (b & 1) .. of the
// 32-row prepared tile group b / 2. Lane (r = lane & 15, q = lane >> 4) of wave
// w handles row r, tile 2 p + (q >> 1) and K-half (q & 1) of that tile, for the
// tile pairs p = w, w + 16, w + 32, ...: one wave load reads two contiguous
// 512-byte half-tiles.
template <int M>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                                const uint8_t *__restrict__ wp, int64_t N,
                                                                int64_t K, float alpha, const float *alpha_dev,
                                                                uint16_t *__restrict__ y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];     // [M][K]
  __shared__ float red[kDecodeWaves][M][16];
  const int64_t T = K / 64;
  for (int64_t u = threadIdx.x; u < M * K / 8; u += kDecodeThreads) {
    const int64_t m = u / (K / 8), c = u - m * (K / 8);
    *reinterpret_cast<u32x4_t *>(xs + m * K + c * 8) = *reinterpret_cast<const u32x4_t *>(x + m * ldx + c * 8);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4, th = q >> 1, kh = q & 1;
  const int64_t ng = blockIdx.x >> 1;
  const int row = (blockIdx.x & 1) * 16 + r;                 // row inside the 32-row tile
  const uint8_t *codes = wp + ((ng * T) << 10) + 16 * (32 * kh + row);
  const uint8_t *scl = wp + N * K / 2 + ((ng * T) << 7) + row * 4;
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; m++) acc[m] = 0.0f;
  const int64_t pairs = (T + 1) / 2;
  constexpr int U = 2;  // tile pairs in flight per wave
  for (int64_t p0 = wave; p0 < pairs; p0 += (int64_t)kDecodeWaves * U) {
    u32x4_t cw[U];
    uint32_t sw[U];
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = 2 * (p0 + (int64_t)i * kDecodeWaves) + th;
      if (t < T) {
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(codes + (t << 10)));
        sw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(scl + (t << 7)));
      } else {
        cw[i] = u32x4_t{0u, 0u, 0u, 0u};
        sw[i] = 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = 2 * (p0 + (int64_t)i * kDecodeWaves) + th;
      if (t >= T) continue;
      const f32x2_t sc = e4m3x2_to_f32(sw[i] >> (16 * kh));
      const uint16_t *xk = xs + t * 64 + 32 * kh;
#pragma unroll
      for (int blk = 0; blk < 2; blk++) {
        float part[M];
#pragma unroll
        for (int m = 0; m < M; m++) part[m] = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; d++) {
          const int s = blk * 2 + d;
          bf16x2_t wv[4];
          codes8_to_bf16(cw[i][s], wv);
#pragma unroll
          for (int m = 0; m < M; m++) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xk + m * K + 8 * s);
#pragma unroll
            for (int e = 0; e < 4; e++)
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wv[e], as_bf16x2(xv[e]), part[m], false);
          }
        }
#pragma unroll
        for (int m = 0; m < M; m++) acc[m] = __builtin_fmaf(part[m], sc[blk], acc[m]);
      }
    }
  }
  // lanes r, r+16, r+32, r+48 hold the four (tile, half) streams of row r:
  // ((q0 + q1) + (q2 + q3)), the same bits in all four lanes
#pragma unroll
  for (int m = 0; m < M; m++) {
    acc[m] += __shfl_xor(acc[m], 16, 64);
    acc[m] += __shfl_xor(acc[m], 32, 64);
  }
  if (q == 0)
#pragma unroll
    for (int m = 0; m < M; m++) red[wave][m][r] = acc[m];
  __syncthreads();
  if (threadIdx.x < M * 16) {
    const int m = threadIdx.x >> 4, rr = threadIdx.x & 15;
    float v = red[0][m][rr];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; w++) v += red[w][m][rr];
    const float al = load_alpha(alpha, alpha_dev);
    y[m * ldy + blockIdx.x * 16 + rr] = f32_to_bf16_rne(al * v);
  }
}

// Wide decode (many row groups): workgroup g covers the 32-row prepared tile
// group g (rows 32g .. 32g+31) over the whole K with 8 waves; wave w takes the
// tiles w, w + 8, w + 16, ...; lane l is unit l of each tile (row r = l & 31,
// k in [32h, 32h + 32) with h = l >> 5), so one wave load is the tile's
// contiguous 1 KB. Loads run four tiles per wave ahead in a two-batch register
// ring (non-temporal: the weights are streamed once); the first batch is issued
// before x is staged. With at least two groups per CU every workgroup is
// resident at once, and a group is reduced inside its workgroup.
constexpr int kWideWaves = 8;
constexpr int kWideAhead = 4;

template <int M>
__global__ __launch_bounds__(kWideWaves * 64) void decode_wide_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                                    const uint8_t *__restrict__ wp, int64_t N,
                                                                    int64_t K, float alpha, const float *alpha_dev,
                                                                    uint16_t *__restrict__ y, int64_t ldy) {
  constexpr int W = kWideWaves, U = kWideAhead;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];     // [M][K]
  __shared__ float red[W][M][32];
  const int64_t T = K / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const int64_t g = blockIdx.x;
  const uint8_t *cb = wp + ((g * T) << 10) + lane * 16;
  const uint8_t *sb = wp + N * K / 2 + ((g * T) << 7) + r * 4;
  u32x4_t cw0[U], cw1[U];
  uint32_t sw0[U], sw1[U];
  auto issue = [&](u32x4_t (&cw)[U], uint32_t (&sw)[U], int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = t0 + (int64_t)i * W;
      if (t < T) {
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb + (t << 10)));
        sw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + (t << 7)));
      } else {
        cw[i] = u32x4_t{0u, 0u, 0u, 0u};
        sw[i] = 0u;
      }
    }
  };
  issue(cw0, sw0, wave);
  for (int64_t u = threadIdx.x; u < M * K / 8; u += W * 64) {
    const int64_t m = u / (K / 8), c = u - m * (K / 8);
    *reinterpret_cast<u32x4_t *>(xs + m * K + c * 8) = *reinterpret_cast<const u32x4_t *>(x + m * ldx + c * 8);
  }
  __syncthreads();

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; m++) acc[m] = 0.0f;
  auto compute = [&](const u32x4_t (&cw)[U], const uint32_t (&sw)[U], int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = t0 + (int64_t)i * W;
      if (t < T) {
        const f32x2_t sc = e4m3x2_to_f32(sw[i] >> (16 * h));
        const uint16_t *xk = xs + t * 64 + 32 * h;
#pragma unroll
        for (int blk = 0; blk < 2; blk++) {
          float part[M];
#pragma unroll
          for (int m = 0; m < M; m++) part[m] = 0.0f;
#pragma unroll
          for (int d = 0; d < 2; d++) {
            const int s = blk * 2 + d;
            bf16x2_t wv[4];
            codes8_to_bf16(cw[i][s], wv);
#pragma unroll
            for (int m = 0; m < M; m++) {
              const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xk + m * K + 8 * s);
#pragma unroll
              for (int e = 0; e < 4; e++)
                part[m] = __builtin_amdgcn_fdot2_f32_bf16(wv[e], as_bf16x2(xv[e]), part[m], false);
            }
          }
#pragma unroll
          for (int m = 0; m < M; m++) acc[m] = __builtin_fmaf(part[m], sc[blk], acc[m]);
        }
      }
    }
  };
  const int64_t step = (int64_t)W * U;
  for (int64_t t0 = wave; t0 < T; t0 += 2 * step) {
    issue(cw1, sw1, t0 + step);
    compute(cw0, sw0, t0);
    if (t0 + step >= T) break;
    issue(cw0, sw0, t0 + 2 * step);
    compute(cw1, sw1, t0 + step);
  }
  // lanes r and r + 32 hold the two K-halves of row r: the same sum in both
#pragma unroll
  for (int m = 0; m < M; m++) acc[m] += __shfl_xor(acc[m], 32, 64);
  if (h == 0)
#pragma unroll
    for (int m = 0; m < M; m++) red[wave][m][r] = acc[m];
  __syncthreads();
  if (threadIdx.x < M * 32) {
    const int m = threadIdx.x >> 5, rr = threadIdx.x & 31;
    float v = red[0][m][rr];
#pragma unroll
    for (int w = 1; w < W; w++) v += red[w][m][rr];
    const float al = load_alpha(alpha, alpha_dev);
    y[m * ldy + g * 32 + rr] = f32_to_bf16_rne(al * v);
  }
}

// ---------------------------------------------------------------- skinny MFMA kernel (4 < M <= 128)

// Workgroup g covers the 32-row prepared tile group g over the whole K with 8
// waves; wave w takes the tiles w, w + 8, ... as in the wide decode kernel. Per
// tile and MFMA step s (k = 32h + 8s + i, the same K order as the prepared
// weight units), lane l dequantizes its 8 codes of weight row 32g + (l & 31)
// exactly to BF16 (E2M1 -> FP32, times the E4M3 scale, -> BF16) as the B
// operand and loads the matching 8 BF16 of x rows 32 mt + (l & 31) as the A
// operand of v_mfma_f32_32x32x16_bf16 (MT 32-row x tiles; rows >= M read as
// zero through the buffer range check). Weights and x fragments are loaded a
// batch of tiles ahead. Each wave ends with a full 32 x 32 MT partial tile; the
// waves are added in a fixed tree (4+4, 2+2, 1+1) through LDS.
constexpr int kSkWaves = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc16(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  bf16x8_t b;
  __builtin_memcpy(&b, &v, 16);
  return b;
}

template <int MT>
__global__ __launch_bounds__(kSkWaves * 64) void skinny_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                             const uint8_t *__restrict__ wp, int64_t M, int64_t N,
                                                             int64_t K, float alpha, const float *alpha_dev,
                                                             uint16_t *__restrict__ y, int64_t ldy) {
  constexpr int W = kSkWaves;
  constexpr int U = MT == 1 ? 4 : (MT == 2 ? 2 : 1);     // tiles per wave per batch
  __shared__ f32x16_t red[4][MT][64];
  const int64_t T = K / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const int64_t g = blockIdx.x;
  const uint8_t *cb = wp + ((g * T) << 10) + lane * 16;
  const uint8_t *sb = wp + N * K / 2 + ((g * T) << 7) + r * 4;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc16(x, M * ldx * 2);
  uint32_t xo[MT];                                 // byte offset of this lane's x row, k = 32h
#pragma unroll
  for (int mt = 0; mt < MT; mt++) xo[mt] = (uint32_t)(((int64_t)(32 * mt + r) * ldx + 32 * h) * 2);

  struct Batch {
    u32x4_t cw[U];
    uint32_t sw[U];
    u32x4_t xv[U][MT][4];
  };
  auto issue = [&](Batch &b, int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = t0 + (int64_t)i * W;
      const bool in = t < T;
      const int64_t tc = in ? t : 0;
      b.cw[i] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb + (tc << 10)))
                   : u32x4_t{0u, 0u, 0u, 0u};
      b.sw[i] = in ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + (tc << 7))) : 0u;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int s = 0; s < 4; s++)
          b.xv[i][mt][s] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo[mt] + (uint32_t)(tc * 128 + 16 * s), 0, 0);
    }
  };
  f32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++) acc[mt] = f32x16_t{};
  auto compute = [&](const Batch &b, int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      if (t0 + (int64_t)i * W < T) {
        const f32x2_t sc = e4m3x2_to_f32(b.sw[i] >> (16 * h));
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const bf16x8_t bv = dequant8_bf16(b.cw[i][s], sc[s >> 1]);
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(b.xv[i][mt][s]), bv, acc[mt], 0, 0, 0);
        }
      }
    }
  };
  Batch b0, b1;
  issue(b0, wave);
  const int64_t step = (int64_t)W * U;
  for (int64_t t0 = wave; t0 < T; t0 += 2 * step) {
    issue(b1, t0 + step);
    compute(b0, t0);
    if (t0 + step >= T) break;
    issue(b0, t0 + 2 * step);
    compute(b1, t0 + step);
  }
  // fixed-order tree over the 8 waves' partial tiles
#pragma unroll
  for (int half = 4; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) red[wave - half][mt][lane] = acc[mt];
    __syncthreads();
    if (wave < half)
#pragma unroll
      for (int mt = 0; mt < MT; mt++) acc[mt] += red[wave][mt][lane];
    __syncthreads();
  }
  if (wave == 0) {
    const float al = load_alpha(alpha, alpha_dev);
    const int64_t n = g * 32 + r;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const int64_t m = 32 * mt + 8 * (j >> 2) + 4 * h + (j & 3);
        if (m < M) y[m * ldy + n] = f32_to_bf16_rne(al * acc[mt][j]);
      }
  }
}

// ---------------------------------------------------------------- MFMA tile kernel (M > 4)

// LDS stage (one 64-wide K chunk): x tile [256 rows][64 bf16] with the eight
// 16-byte units of each row XOR-swizzled by (row & 7); W codes [4 groups][1 KB]
// and W scales [4 groups][128 B] in the prepared format.
constexpr int X_BYTES = BM * 128;
constexpr int WC_OFF = X_BYTES;
constexpr int WS_OFF = WC_OFF + (BN / 32) * 1024;
constexpr int STAGE = WS_OFF + (BN / 32) * 128;   // 37376

struct TileParams {
  const uint16_t *x;
  int64_t ldx;
  const uint8_t *wp;
  int64_t M, N, K;
  float alpha;
  const float *alpha_dev;
  uint16_t *y;
  int64_t ldy;
  int tiles_n, splits;
  float *partial;
};

struct TileRegs {
  u32x4_t xv[8];   // x: 256 rows x 8 units / 256 threads
  u32x4_t wc;      // W codes: 4 KB / 256 threads
  uint32_t wsc;    // W scales: 512 B / 128 threads (as dwords)
};

__device__ __forceinline__ void tile_load(const TileParams &p, int64_t m0, int64_t n0, int64_t kt, TileRegs &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int q = t + kThreads * i;        // (row, unit)
    const int row = q >> 3, u = q & 7;
    const int64_t m = m0 + row;
    if (m < p.M)
      r.xv[i] = *reinterpret_cast<const u32x4_t *>(p.x + m * p.ldx + kt * 64 + u * 8);
    else
      r.xv[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  const int64_t T = p.K / 64;
  {
    const int g = t >> 6, u = t & 63;
    const int64_t ng = (n0 >> 5) + g;
    if (ng * 32 < p.N)
      r.wc = *reinterpret_cast<const u32x4_t *>(p.wp + ((ng * T + kt) << 10) + u * 16);
    else
      r.wc = u32x4_t{0u, 0u, 0u, 0u};
  }
  if (t < 128) {
    const int g = t >> 5, u = t & 31;
    const int64_t ng = (n0 >> 5) + g;
    if (ng * 32 < p.N)
      r.wsc = *reinterpret_cast<const uint32_t *>(p.wp + p.N * p.K / 2 + ((ng * T + kt) << 7) + u * 4);
    else
      r.wsc = 0u;
  }
}

__device__ __forceinline__ void tile_store(uint8_t *lds, const TileRegs &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int q = t + kThreads * i;
    const int row = q >> 3, u = q & 7;
    *reinterpret_cast<u32x4_t *>(lds + row * 128 + ((u ^ (row & 7)) << 4)) = r.xv[i];
  }
  *reinterpret_cast<u32x4_t *>(lds + WC_OFF + (t >> 6) * 1024 + (t & 63) * 16) = r.wc;
  if (t < 128) *reinterpret_cast<uint32_t *>(lds + WS_OFF + (t >> 5) * 128 + (t & 31) * 4) = r.wsc;
}

// Wave (wm, wn) owns rows [128 wm, 128 wm + 128) and columns [64 wn, 64 wn + 64)
// of the 256 x 128 tile: 4 x 2 MFMA tiles.
__device__ __forceinline__ void tile_compute(const uint8_t *lds, int wm, int wn, f32x16_t acc[4][2]) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  u32x4_t wf[2];
  f32x2_t sc[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int g = wn * 2 + j;
    wf[j] = *reinterpret_cast<const u32x4_t *>(lds + WC_OFF + g * 1024 + 16 * (32 * h + r));
    const uint32_t sw = *reinterpret_cast<const uint32_t *>(lds + WS_OFF + g * 128 + r * 4);
    sc[j] = e4m3x2_to_f32(sw >> (16 * h));
  }
#pragma unroll
  for (int s = 0; s < 4; s++) {
    bf16x8_t b[2], a[4];
#pragma unroll
    for (int j = 0; j < 2; j++) b[j] = dequant8_bf16(wf[j][s], sc[j][s >> 1]);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = wm * 128 + i * 32 + r;
      const int u = 4 * h + s;               // k = 32h + 8s .. +7
      a[i] = *reinterpret_cast<const bf16x8_t *>(lds + row * 128 + ((u ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void tile_kernel(TileParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t T = p.K / 64;
  const int64_t kt0 = split * T / p.splits, kt1 = (split + 1) * T / p.splits;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f32x16_t{};
  TileRegs regs;
  tile_load(p, m0, n0, kt0, regs);
  tile_store(smem, regs);
  __syncthreads();
  for (int64_t kt = kt0; kt < kt1; kt++) {
    const bool more = kt + 1 < kt1;
    if (more) tile_load(p, m0, n0, kt + 1, regs);
    tile_compute(smem + ((kt - kt0) & 1) * STAGE, wm, wn, acc);
    if (more) tile_store(smem + ((kt - kt0 + 1) & 1) * STAGE, regs);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const float al = load_alpha(p.alpha, p.alpha_dev);
  float *part = p.partial + (int64_t)split * p.M * p.N;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t n = n0 + wn * 64 + j * 32 + r;
      if (n >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m >= p.M) continue;
        if (p.splits == 1)
          p.y[m * p.ldy + n] = f32_to_bf16_rne(al * acc[i][j][e]);
        else
          part[m * p.N + n] = acc[i][j][e];
      }
    }
}

// Fixed-order sum of the split partials: y = alpha * (P_0 + P_1 + ... + P_{S-1}).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partial, int splits, int64_t M,
                                                            int64_t N, float alpha, const float *alpha_dev,
                                                            uint16_t *__restrict__ y, int64_t ldy) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N, n = idx - m * N;
  float v = partial[idx];
  for (int s = 1; s < splits; s++) v += partial[(int64_t)s * M * N + idx];
  y[m * ldy + n] = f32_to_bf16_rne(load_alpha(alpha, alpha_dev) * v);
}

}  // namespace w4a16

size_t w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0) return 0;
  w4a16::Plan p = w4a16::make_plan(M, N, K);
  return w4a16::workspace_for(p, M, N);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_gemm_w4a16(const uint16_t *x, int64_t ldx, const uint8_t *w_prep, int64_t M, int64_t N,
                                         int64_t K, float alpha, const float *alpha_dev, uint16_t *y, int64_t ldy,
                                         void *ws, size_t ws_bytes, void *stream) {
  if (M < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || ldx < K || ldy < N) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!x || !w_prep || !y) return NVFP4_ERR_NULL;
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return NVFP4_ERR_VALUE;
  if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(w_prep, 16) || !aligned(y, 2) ||
      (alpha_dev && !aligned(alpha_dev, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo di;
  nvfp4_status st = device_info(&di);
  if (st != NVFP4_OK) return st;
  const w4a16::Plan plan = w4a16::make_plan(M, N, K);
  const size_t need = w4a16::workspace_for(plan, M, N);
  if (need > 0 && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (plan.kind == 0 || plan.kind == 2) {
    if (plan.grid_x > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
    const size_t lds = (size_t)(M * K * 2);
#define NVFP4_DECODE_CASE(MM)                                                                                 \
  case MM:                                                                                                    \
    hipLaunchKernelGGL(w4a16::decode_kernel<MM>, dim3((unsigned)plan.grid_x), dim3(w4a16::kDecodeThreads), lds, \
                       s, x, ldx, w_prep, N, K, alpha, alpha_dev, y, ldy);                                    \
    break;
#define NVFP4_DECODE_WIDE_CASE(MM)                                                                            \
  case MM:                                                                                                    \
    hipLaunchKernelGGL(w4a16::decode_wide_kernel<MM>, dim3((unsigned)plan.grid_x),                            \
                       dim3(w4a16::kWideWaves * 64), lds, s, x, ldx, w_prep, N, K, alpha, alpha_dev, y, ldy); \
    break;
    if (plan.kind == 2) {
      switch ((int)M) {
        NVFP4_DECODE_WIDE_CASE(1)
        NVFP4_DECODE_WIDE_CASE(2)
        NVFP4_DECODE_WIDE_CASE(3)
        NVFP4_DECODE_WIDE_CASE(4)
        default: return NVFP4_ERR_SHAPE;
      }
    } else {
      switch ((int)M) {
        NVFP4_DECODE_CASE(1)
        NVFP4_DECODE_CASE(2)
        NVFP4_DECODE_CASE(3)
        NVFP4_DECODE_CASE(4)
        default: return NVFP4_ERR_SHAPE;
      }
    }
#undef NVFP4_DECODE_CASE
#undef NVFP4_DECODE_WIDE_CASE
  } else if (plan.kind == 3) {
    if (plan.grid_x > 0x7FFFFFFF || M * ldx * 2 > 0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
    const unsigned grid = (unsigned)plan.grid_x, threads = w4a16::kSkWaves * 64;
    if (M <= 32)
      hipLaunchKernelGGL(w4a16::skinny_kernel<1>, dim3(grid), dim3(threads), 0, s, x, ldx, w_prep, M, N, K, alpha,
                         alpha_dev, y, ldy);
    else if (M <= 64)
      hipLaunchKernelGGL(w4a16::skinny_kernel<2>, dim3(grid), dim3(threads), 0, s, x, ldx, w_prep, M, N, K, alpha,
                         alpha_dev, y, ldy);
    else
      hipLaunchKernelGGL(w4a16::skinny_kernel<4>, dim3(grid), dim3(threads), 0, s, x, ldx, w_prep, M, N, K, alpha,
                         alpha_dev, y, ldy);
  } else {
    const int64_t tiles_n = (N + w4a16::BN - 1) / w4a16::BN;
    if (plan.grid_x > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
    float *partial = need ? reinterpret_cast<float *>(ws) : nullptr;
    w4a16::TileParams p{x, ldx, w_prep, M, N, K, alpha, alpha_dev, y, ldy, (int)tiles_n, plan.splits, partial};
    hipLaunchKernelGGL(w4a16::tile_kernel, dim3((unsigned)plan.grid_x, (unsigned)plan.splits), dim3(w4a16::kThreads), 0,
                       s, p);
    NVFP4_LAUNCH_CHECK();
    if (plan.splits > 1) {
      const int64_t blocks = (M * N + 255) / 256;
      if (blocks > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
      hipLaunchKernelGGL(w4a16::splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, partial, plan.splits,
                         M, N, alpha, alpha_dev, y, ldy);
    }
  }
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}
