// W4A4 NVFP4 GEMM for gfx950: D = alpha * (A.SFA)(W.SFW)^T, FP32 accumulation.
//
// Design (MI355X / CDNA4):
//  * Contraction on the FP16 MFMA v_mfma_f32_32x32x16_f16. Every NVFP4 element
//    code * scale has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is an exact normal FP16 number: the dequantized operands are exact and
//    the only rounding is the FP32 accumulation (the scaled f8f6f4 MFMAs take a
//    power-of-two scale per 32 elements and cannot carry an E4M3 scale per 16).
//  * Workgroup tile 256 x 256, four waves in a 2 x 2 arrangement, each owning a
//    128 x 128 block of D as 4 x 4 MFMA tiles (256 FP32 accumulators per lane,
//    held in the accumulation registers).
//  * Each wave streams its own packed fragments from global memory straight
//    into registers: per 64-wide K chunk, 16 packed bytes (32 codes of one row)
//    and one scale word for each of its four A row groups and four W column
//    groups. Buffer loads with 32-bit lane offsets and the hardware range check
//    (ragged rows and columns read as zero). Chunks are loaded two ahead into a
//    three-deep register ring; no LDS and no barriers in the main loop. (On
//    this part, staging the packed bytes through LDS -- shared by the two waves
//    that use each fragment -- measured no faster: the unpack and the memory
//    instructions themselves, not L2 bandwidth, bound the loop.)
//  * The FP16 operands exist only in registers: cvt_scalef32_pk_f16_fp4 (code
//    pairs, scale operand 1.0) + v_pk_mul_f16 by the block scale, one vector
//    instruction per element, unpacked one MFMA step ahead and interleaved one
//    MFMA to four vector instructions.
//  * W is read in the prepared layout: 1 KB tiles of 64 16-byte units (unit
//    32h + r = row r, k in [32h, 32h+32)), so a wave's W fragment load is one
//    contiguous 1 KB; A is read in the standard packed layout (32 bytes of a
//    row per chunk).
//  * Persistent grid (one workgroup per CU) walking the tiles in an XCD-aware,
//    grouped order: workgroups that run on the same XCD (hardware ids congruent
//    mod 8) take consecutive tile indices, and consecutive indices cover a
//    kGroupM-tall band of tiles column by column, so a wave of tiles on one XCD
//    shares A rows and W columns in that XCD's L2.
//  * Epilogue: alpha * acc in FP32, converted (BF16 round-to-nearest-even or
//    FP32), staged through LDS and written as 16-byte row pieces.
//
// K-order inside a 64-wide chunk: lane half h (= lane / 32) holds k in
// [32h, 32h + 32) as four dwords; MFMA step s uses dword s of both halves, i.e.
// k = 32h + 8s + i. A and W use the same map, so the sum over steps covers the
// chunk exactly once, and each dword lies inside one 16-block (block 2h + s/2).
#include "common.hpp"

namespace nvfp4 {
namespace w4a4 {

constexpr int BM = 256, BN = 256;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;                 // tile-band height of the raster order
constexpr int LDS_BYTES = 65536;           // epilogue staging: 4 waves x 32 x 128 FP32

struct Params {
  const uint8_t *a_codes;   // [M][K/2]
  const uint8_t *a_scales;  // [M][K/16]
  const uint8_t *w_prep;    // prepared (N, K)
  void *d;
  int64_t M, N, K, ldd;
  float alpha;
  const float *alpha_dev;
  int tiles_m, tiles_n;
};

// Raw buffer resource over [base, base + bytes); loads at offsets >= bytes
// return 0 (the hardware range check), which zero-fills ragged rows/columns
// and makes loads past the last chunk harmless.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}

struct TileRsrc {
  const uint8_t *a, *as, *w, *ws;          // tile bases at chunk 0
  int64_t a_bytes, as_bytes, w_bytes, ws_bytes;
};

// Packed fragments of one chunk for this wave.
struct ChunkFrags {
  u32x4_t a[4], w[4];      // 32 codes of one row per lane (dword s feeds MFMA step s)
  half2_t as[4], ws[4];    // the lane's two block scales (blocks 2h, 2h+1) in FP16
};

// Exact FP16 operands of MFMA step s (k = 32h + 8s + 0..7) of a chunk.
__device__ __forceinline__ void unpack_step(const ChunkFrags &f, int s, half8_t a[4], half8_t b[4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) a[i] = dequant8_f16(f.a[i][s], f.as[i][s >> 1]);
#pragma unroll
  for (int j = 0; j < 4; j++) b[j] = dequant8_f16(f.w[j][s], f.ws[j][s >> 1]);
}

__device__ __forceinline__ void mfma_step(const half8_t a[4], const half8_t b[4], f32x16_t acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Per-lane constant byte offsets (relative to the tile) of this wave's loads:
// A rows wm*128 + 32i + r at half h, A scale words of those rows, and W tile
// units `lane` / W scale words of row r for column groups wn*4 + i.
struct WaveOff {
  uint32_t a[4], as[4], w[4], ws[4];
};

// Loads of chunk c: the rebased resources keep the range check on the row (A)
// or 32-row group (W); chunks at or past nch read as zeros (length 0).
__device__ __forceinline__ void load_frags(const TileRsrc &tr, const WaveOff &o, int64_t c, int64_t nch,
                                           ChunkFrags &f) {
  const int h = (threadIdx.x & 63) >> 5;
  const bool in = c < nch;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(tr.a, in ? tr.a_bytes : 0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(tr.w, in ? tr.w_bytes : 0);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(tr.as, in ? tr.as_bytes : 0);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(tr.ws, in ? tr.ws_bytes : 0);
  const int sa = (int)(c * 32), sw = (int)(c * 1024), ssa = (int)(c * 4), ssw = (int)(c * 128);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, o.a[i], sa, 0);
    f.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, o.w[i], sw, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t xa = __builtin_amdgcn_raw_buffer_load_b32(ras, o.as[i], ssa, 0);
    const uint32_t xw = __builtin_amdgcn_raw_buffer_load_b32(rws, o.ws[i], ssw, 0);
    f.as[i] = e4m3x2_to_f16(xa >> (16 * h));
    f.ws[i] = e4m3x2_to_f16(xw >> (16 * h));
  }
}

// One chunk of the main loop. f[P] holds chunk c, f[(P+1)%3] chunk c + 1 (in
// flight or arrived); chunk c + 2 is requested into f[(P+2)%3]. On entry (a, b)
// are chunk c's step-0 operands; on exit chunk c + 1's.
template <int P>
__device__ __forceinline__ void chunk_direct(const TileRsrc &tr, const WaveOff &o, int64_t c, int64_t nch,
                                             ChunkFrags f[3], half8_t a[4], half8_t b[4], f32x16_t acc[4][4]) {
  load_frags(tr, o, c + 2, nch, f[(P + 2) % 3]);
#pragma unroll
  for (int s = 0; s < 4; s++) {
    half8_t an[4], bn[4];
    if (s < 3) unpack_step(f[P], s + 1, an, bn);
    else unpack_step(f[(P + 1) % 3], 0, an, bn);
    mfma_step(a, b, acc);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a[i] = an[i];
      b[i] = bn[i];
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
#pragma unroll
  for (int k = 0; k < 64; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue through LDS: each wave writes a 32 x 128 block of alpha * acc to its
// own LDS region in row-major order, then writes it out as 16-byte row pieces.
template <bool OUT_BF16>
__device__ __forceinline__ void epilogue(uint8_t *smem, const Params &p, int64_t m0, int64_t n0, int wm, int wn,
                                         float alpha, f32x16_t acc[4][4]) {
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  constexpr int ROW_BYTES = 128 * ESZ;            // one wave's 128 columns
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  uint8_t *reg = smem + wave * (32 * 128 * 4);
  const int64_t col0 = n0 + wn * 128;
  const int64_t ncols = p.N - col0;               // columns of this wave still inside D
  const bool vec_ok = (p.ldd * ESZ) % 16 == 0 && ((uintptr_t)p.d & 15) == 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int row = 8 * (e >> 2) + 4 * h + (e & 3);
        const float v = alpha * acc[i][j][e];
        if (OUT_BF16)
          *reinterpret_cast<uint16_t *>(reg + row * ROW_BYTES + (j * 32 + r) * 2) = f32_to_bf16_rne(v);
        else
          *reinterpret_cast<float *>(reg + row * ROW_BYTES + (j * 32 + r) * 4) = v;
      }
    __syncthreads();
    constexpr int PIECES = ROW_BYTES / 16;        // 16-byte pieces per row
#pragma unroll
    for (int q = lane; q < 32 * PIECES; q += 64) {
      const int row = q / PIECES, pc = q % PIECES;
      const int64_t m = m0 + wm * 128 + i * 32 + row;
      const int64_t c = (int64_t)pc * (16 / ESZ);
      if (m < p.M && c < ncols) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(reg + row * ROW_BYTES + pc * 16);
        uint8_t *dst = reinterpret_cast<uint8_t *>(p.d) + (m * p.ldd + col0 + c) * ESZ;
        if (vec_ok) {
          *reinterpret_cast<u32x4_t *>(dst) = v;
        } else {
          // unaligned output rows: element stores
          const uint8_t *src = reinterpret_cast<const uint8_t *>(&v);
          for (int b = 0; b < 16; b += ESZ) {
            if (OUT_BF16) *reinterpret_cast<uint16_t *>(dst + b) = *reinterpret_cast<const uint16_t *>(src + b);
            else *reinterpret_cast<float *>(dst + b) = *reinterpret_cast<const float *>(src + b);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Tile index -> (tile_m, tile_n): bands of kGroupM tile rows, column-major inside a band.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_band = kGroupM * tiles_n;
  const int band = t / per_band;
  const int first = band * kGroupM;
  const int rows = min(kGroupM, tiles_m - first);
  const int w = t - band * per_band;
  tm = first + w % rows;
  tn = w / rows;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int total = p.tiles_m * p.tiles_n;
  const int G = gridDim.x;
  // XCD-aware logical id: hardware ids b, b+8, b+16, ... run on one XCD; give
  // them consecutive logical ids so they take neighbouring tiles.
  int pid = blockIdx.x;
  if ((G & 7) == 0) pid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const float alpha = load_alpha(p.alpha, p.alpha_dev);
  const int64_t nch = p.K / 64;
  const int64_t kb = p.K / 2, sb = p.K / 16, kt = p.K / 64;

  const int lane = t & 63, h = lane >> 5, r = lane & 31;
  WaveOff o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = wm * 128 + i * 32 + r;
    o.a[i] = (uint32_t)(row * kb + h * 16);
    o.as[i] = (uint32_t)(row * sb);
    o.w[i] = (uint32_t)(((wn * 4 + i) * kt) * 1024 + lane * 16);
    o.ws[i] = (uint32_t)(((wn * 4 + i) * kt) * 128 + r * 4);
  }

  for (int tile = pid; tile < total; tile += G) {
    int tm, tn;
    tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    TileRsrc tr;
    tr.a = p.a_codes + m0 * kb;
    tr.a_bytes = (p.M - m0) * kb;
    tr.as = p.a_scales + m0 * sb;
    tr.as_bytes = (p.M - m0) * sb;
    tr.w = p.w_prep + (n0 >> 5) * kt * 1024;
    tr.w_bytes = (p.N - n0) / 32 * kt * 1024;
    tr.ws = p.w_prep + p.N * p.K / 2 + (n0 >> 5) * kt * 128;
    tr.ws_bytes = (p.N - n0) / 32 * kt * 128;

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = f32x16_t{};
    ChunkFrags f[3];
    half8_t a[4], b[4];
    load_frags(tr, o, 0, nch, f[0]);
    load_frags(tr, o, 1, nch, f[1]);
    unpack_step(f[0], 0, a, b);
    for (int64_t c = 0; c < nch; c += 3) {
      chunk_direct<0>(tr, o, c, nch, f, a, b, acc);
      chunk_direct<1>(tr, o, c + 1, nch, f, a, b, acc);
      chunk_direct<2>(tr, o, c + 2, nch, f, a, b, acc);
    }
    __syncthreads();
    epilogue<OUT_BF16>(smem, p, m0, n0, wm, wn, alpha, acc);
  }
}

}  // namespace w4a4
}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_prep,
                                        int64_t M, int64_t N, int64_t K, float alpha, const float *alpha_dev,
                                        void *d, int out_dtype, int64_t ldd, void *ws, size_t ws_bytes,
                                        void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || ldd < N) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !w_prep || !d) return NVFP4_ERR_NULL;
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return NVFP4_ERR_VALUE;
  const size_t esz = out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
  if (!aligned(a_codes, 16) || !aligned(a_scales, 4) || !aligned(w_prep, 16) || !aligned(d, esz) ||
      (alpha_dev && !aligned(alpha_dev, 4)))
    return NVFP4_ERR_ALIGN;
  // 32-bit buffer offsets inside one 256-row tile of A and one 256-column tile of W
  if ((int64_t)w4a4::BM * (K / 2) > 0xFFFFFFFFll || (int64_t)(w4a4::BN / 32) * (K / 64) * 1024 > 0xFFFFFFFFll)
    return NVFP4_ERR_SHAPE;
  const int64_t tiles_m = (M + w4a4::BM - 1) / w4a4::BM;
  const int64_t tiles_n = (N + w4a4::BN - 1) / w4a4::BN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
  DeviceInfo di;
  nvfp4_status st = device_info(&di);
  if (st != NVFP4_OK) return st;
  w4a4::Params p{a_codes, a_scales, w_prep, d, M, N, K, ldd, alpha, alpha_dev, (int)tiles_m, (int)tiles_n};
  const int64_t total = tiles_m * tiles_n;
  const int grid = (int)(total < di.num_cus ? total : di.num_cus);
  if (out_dtype == NVFP4_OUT_BF16)
    hipLaunchKernelGGL(w4a4::gemm_kernel<true>, dim3(grid), dim3(w4a4::kThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(w4a4::gemm_kernel<false>, dim3(grid), dim3(w4a4::kThreads), 0, (hipStream_t)stream, p);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}
