// W4A4 NVFP4 GEMM for gfx950: D = alpha * (A.SFA)(W.SFW)^T, FP32 accumulation.
//
// Design (MI355X / CDNA4):
//  * Contraction on the FP16 MFMA v_mfma_f32_32x32x16_f16. Every NVFP4 element
//    code * scale has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is an exact normal FP16 number: the dequantized operands are exact and
//    the only rounding is the FP32 accumulation (the scaled f8f6f4 MFMAs take a
//    power-of-two scale per 32 elements and cannot carry an E4M3 scale per 16).
//  * Workgroup tile 256 x 256, four waves in a 2 x 2 arrangement, each owning a
//    128 x 128 block of D as 4 x 4 MFMA tiles (256 FP32 accumulators per lane).
//  * K advances 128 per stage (two 64-wide chunks). Packed codes and scale
//    bytes go global -> registers -> LDS (double buffered, one barrier per
//    stage); the FP16 operands never touch LDS: each lane reads 16 packed bytes
//    (32 codes of one row) and one scale word per chunk and unpacks them in
//    registers right before the MFMAs (cvt_scalef32_pk_f16_fp4 + v_pk_mul_f16).
//  * LDS holds both operands in the prepared-weight tile format: 1 KB code
//    tiles of 32 rows x 32 bytes and 128 B scale tiles of 32 rows x 4 bytes, so
//    a wave's fragment read is one contiguous, conflict-free 1 KB ds_read_b128.
//  * Persistent grid (one workgroup per CU) walking the tiles in an XCD-aware,
//    grouped order: workgroups that run on the same XCD (hardware ids congruent
//    mod 8) take consecutive tile indices, and consecutive indices cover a
//    kGroupM-tall band of tiles column by column, so a wave of tiles on one XCD
//    shares A rows and W columns in that XCD's L2.
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
constexpr int kChunksPerStage = 2;                 // 2 x 64 = 128 K per stage
constexpr int kGroups = 8;                         // 32-row groups per 256-row tile
constexpr int kGroupM = 8;                         // tile-band height of the raster order
// LDS stage layout (bytes)
constexpr int A_CODES = 0;                                   // [chunk][group][1024]
constexpr int W_CODES = A_CODES + kChunksPerStage * kGroups * 1024;
constexpr int A_SCALES = W_CODES + kChunksPerStage * kGroups * 1024;   // [chunk][group][128]
constexpr int W_SCALES = A_SCALES + kChunksPerStage * kGroups * 128;
constexpr int STAGE_BYTES = W_SCALES + kChunksPerStage * kGroups * 128;  // 36864

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
// return 0 (the hardware range check), which zero-fills ragged rows/columns.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}

// Per-thread constant parts of the global offsets of one stage (bytes).
struct LoadOffsets {
  uint32_t a[4];    // A codes: row (t/4 + 64 i) * K/2 + (t & 3) * 16
  uint32_t w[4];    // W codes: group (t/128 + 2 i), chunk (t/64) & 1, unit t & 63
  uint32_t as;      // A scales: row t
  uint32_t ws;      // W scales: group t/16, chunk (t/8) & 1, unit t & 7
};

// Registers holding one stage in flight from global memory.
struct StageRegs {
  u32x4_t a[4];      // A codes: 4 x 16 B per thread
  u32x4_t w[4];      // W codes
  uint32_t as[2];    // A scales: row t, chunks 0 and 1
  u32x4_t ws;        // W scales: threads 0..127, 16 B each
};

struct TileRsrc {
  const uint8_t *a, *as, *w, *ws;     // tile bases (chunk 0)
  int64_t a_bytes, as_bytes, w_bytes, ws_bytes;
};

__device__ __forceinline__ void load_stage(const TileRsrc &tr, const LoadOffsets &o, int64_t chunk0, StageRegs &r) {
  const int t = threadIdx.x;
  // Rebase each resource at this stage's first chunk; the remaining length keeps
  // the range check on the row (A) or 32-row group (W) index.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(tr.a + chunk0 * 32, tr.a_bytes - chunk0 * 32);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(tr.w + chunk0 * 1024, tr.w_bytes - chunk0 * 1024);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(tr.as + chunk0 * 4, tr.as_bytes - chunk0 * 4);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(tr.ws + chunk0 * 128, tr.ws_bytes - chunk0 * 128);
#pragma unroll
  for (int i = 0; i < 4; i++) r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, o.a[i], 0, 0);
#pragma unroll
  for (int i = 0; i < 4; i++) r.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, o.w[i], 0, 0);
  r.as[0] = __builtin_amdgcn_raw_buffer_load_b32(ras, o.as, 0, 0);
  r.as[1] = __builtin_amdgcn_raw_buffer_load_b32(ras, o.as + 4, 0, 0);
  if (t < 128) r.ws = __builtin_amdgcn_raw_buffer_load_b128(rws, o.ws, 0, 0);
}

__device__ __forceinline__ void store_stage(uint8_t *lds, const StageRegs &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // q = t + 256 i: row q/4 = t/4 + 64 i, part t & 3 (chunk part/2, half part&1)
    const int row = (t >> 2) + 64 * i, part = t & 3;
    *reinterpret_cast<u32x4_t *>(lds + A_CODES + (part >> 1) * 8192 + (row >> 5) * 1024 + (row & 31) * 32 +
                                 (part & 1) * 16) = r.a[i];
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int g = (t >> 7) + 2 * i, c = (t >> 6) & 1, u = t & 63;
    *reinterpret_cast<u32x4_t *>(lds + W_CODES + c * 8192 + g * 1024 + u * 16) = r.w[i];
  }
#pragma unroll
  for (int c = 0; c < 2; c++)
    *reinterpret_cast<uint32_t *>(lds + A_SCALES + c * 1024 + (t >> 5) * 128 + (t & 31) * 4) = r.as[c];
  if (t < 128) {
    const int g = t >> 4, c = (t >> 3) & 1, u = t & 7;
    *reinterpret_cast<u32x4_t *>(lds + W_SCALES + c * 1024 + g * 128 + u * 16) = r.ws;
  }
}

// Packed fragments of one 64-wide chunk for this wave, read from LDS.
struct ChunkFrags {
  u32x4_t a[4], w[4];      // 32 codes of one row per lane (dword s feeds MFMA step s)
  half2_t as[4], ws[4];    // the lane's two block scales (blocks 2h, 2h+1) in FP16
};

__device__ __forceinline__ void read_chunk(const uint8_t *lds, int c, int wm, int wn, ChunkFrags &f) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const uint8_t *ca = lds + A_CODES + c * 8192 + wm * 4096 + r * 32 + h * 16;
  const uint8_t *cw = lds + W_CODES + c * 8192 + wn * 4096 + r * 32 + h * 16;
  const uint8_t *sa = lds + A_SCALES + c * 1024 + wm * 512 + r * 4;
  const uint8_t *sw = lds + W_SCALES + c * 1024 + wn * 512 + r * 4;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f.a[i] = *reinterpret_cast<const u32x4_t *>(ca + i * 1024);
    f.as[i] = e4m3x2_to_f16(*reinterpret_cast<const uint32_t *>(sa + i * 128) >> (16 * h));
    f.w[i] = *reinterpret_cast<const u32x4_t *>(cw + i * 1024);
    f.ws[i] = e4m3x2_to_f16(*reinterpret_cast<const uint32_t *>(sw + i * 128) >> (16 * h));
  }
}

// Exact FP16 operands of MFMA step s (k = 32h + 8s + 0..7) of a chunk.
__device__ __forceinline__ void unpack_step(const ChunkFrags &f, int s, half8_t a[4], half8_t b[4]) {
#pragma unroll
  for (int i = 0; i < 4; i++) a[i] = dequant8_f16(f.a[i][s], f.as[i][s >> 1]);
#pragma unroll
  for (int j = 0; j < 4; j++) b[j] = dequant8_f16(f.w[j][s], f.ws[j][s >> 1]);
}

// One 64-wide chunk: 4 MFMA steps of 4 x 4 tiles. The operands of step s + 1
// are unpacked while the 16 MFMAs of step s run, and the schedule is pinned to
// one MFMA followed by four vector instructions, so that a single wave per SIMD
// keeps the matrix core fed (in-order issue would otherwise stall the unpack
// behind back-to-back MFMAs).
template <int C>
__device__ __forceinline__ void compute_chunk(const uint8_t *lds, int wm, int wn, f32x16_t acc[4][4]) {
  ChunkFrags f;
  read_chunk(lds, C, wm, wn, f);
  half8_t a[4], b[4];
  unpack_step(f, 0, a, b);
#pragma unroll
  for (int s = 0; s < 4; s++) {
    half8_t an[4], bn[4];
    if (s < 3) unpack_step(f, s + 1, an, bn);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (s < 3) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        a[i] = an[i];
        b[i] = bn[i];
      }
    }
  }
  // LDS reads, the scales and step 0's unpack, then {1 MFMA, 4 VALU} x 48, then 16 MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 80, 0);
#pragma unroll
  for (int k = 0; k < 48; k++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}

// One stage: prefetch the next stage into registers, compute this one from LDS
// buffer BUF, then store the prefetched registers into the other buffer.
template <int BUF>
__device__ __forceinline__ void do_stage(uint8_t *smem, const TileRsrc &tr, const LoadOffsets &o, int st,
                                         int nstages, int nchunks_total, int wm, int wn, StageRegs &regs,
                                         f32x16_t acc[4][4]) {
  const bool more = st + 1 < nstages;
  if (more) load_stage(tr, o, (int64_t)(st + 1) * kChunksPerStage, regs);
  const uint8_t *buf = smem + BUF * STAGE_BYTES;
  compute_chunk<0>(buf, wm, wn, acc);
  if (st * kChunksPerStage + 1 < nchunks_total) compute_chunk<1>(buf, wm, wn, acc);
  if (more) store_stage(smem + (1 - BUF) * STAGE_BYTES, regs);
  __syncthreads();
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
        if ((p.ldd * ESZ) % 16 == 0 && ((uintptr_t)p.d & 15) == 0) {
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
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];
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
  const int nchunks_total = (int)(p.K / 64);
  const int nstages = (nchunks_total + kChunksPerStage - 1) / kChunksPerStage;
  const int64_t kb = p.K / 2, sb = p.K / 16, kt = p.K / 64;

  LoadOffsets o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o.a[i] = (uint32_t)(((t >> 2) + 64 * i) * kb + (t & 3) * 16);
    o.w[i] = (uint32_t)((((t >> 7) + 2 * i) * kt + ((t >> 6) & 1)) * 1024 + (t & 63) * 16);
  }
  o.as = (uint32_t)(t * sb);
  o.ws = (uint32_t)((((t >> 4) & 7) * kt + ((t >> 3) & 1)) * 128 + (t & 7) * 16);

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

    StageRegs regs;
    load_stage(tr, o, 0, regs);
    store_stage(smem, regs);
    __syncthreads();
    for (int st = 0; st < nstages; st += 2) {
      do_stage<0>(smem, tr, o, st, nstages, nchunks_total, wm, wn, regs, acc);
      if (st + 1 < nstages) do_stage<1>(smem, tr, o, st + 1, nstages, nchunks_total, wm, wn, regs, acc);
    }
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
