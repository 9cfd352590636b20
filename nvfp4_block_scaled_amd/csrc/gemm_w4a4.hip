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
//  * A is first copied into the workspace in the prepared-weight tile layout
//    (32 rows x 64 k per 1 KB code tile, 128-byte scale tiles), one 16-byte
//    unit per thread; W is already in it. A wave's fragment of one 32-row group
//    for one K chunk is then one contiguous 1 KB load, for A as for W: reading
//    A in its row-major layout instead touches 32 cache lines per load
//    instruction, and measured about 14 % slower overall.
//  * Each wave streams its own packed fragments from global memory straight
//    into registers: per 64-wide K chunk, 16 packed bytes (32 codes of one row)
//    and one scale word for each of its four A row groups and four W column
//    groups. Buffer loads with 32-bit lane offsets and the hardware range check
//    (groups past the matrix read as zero). Chunks are loaded two ahead into a
//    three-deep register ring; no LDS and no barriers in the main loop. (On
//    this part, staging the packed bytes through LDS -- shared by the two waves
//    that use each fragment -- measured no faster.)
//  * The FP16 operands exist only in registers: cvt_scalef32_pk_f16_fp4 (code
//    pairs, scale operand 1.0) + v_pk_mul_f16 by the block scale, one vector
//    instruction per element, unpacked one MFMA step ahead and interleaved with
//    the current step's MFMAs (one scheduling region per step).
//  * Persistent grid (one workgroup per CU) walking the tiles in an XCD-aware,
//    grouped order: workgroups that run on the same XCD (hardware ids congruent
//    mod 8) take consecutive tile indices, and consecutive indices cover a
//    kGroupM-tall band of tiles column by column, so a wave of tiles on one XCD
//    shares A rows and W columns in that XCD's L2.
//  * Epilogue: alpha * acc in FP32 (alpha times the column's own scale when a
//    per-column scale is given), converted (BF16 round-to-nearest-even or
//    FP32), staged through LDS and written as 16-byte row pieces.
//  * A last round of 256 x 256 tiles that would use at most half the CUs runs
//    as a second launch over the tiles' 128 x 128 quadrants.
//  * Two-pass activations (value and residual passes of one activation under
//    one global scale) contract over 2K, both halves reading the same W chunks.
//
// K-order inside a 64-wide chunk: lane half h (= lane / 32) holds k in
// [32h, 32h + 32) as four dwords; MFMA step s uses dword s of both halves, i.e.
// k = 32h + 8s + i. A and W use the same map, so the sum over steps covers the
// chunk exactly once, and each dword lies inside one 16-block (block 2h + s/2).
#include "common.hpp"

namespace nvfp4 {
namespace w4a4 {

constexpr int kThreads = 256;
constexpr int kGroupM = 8;                 // tile-band height of the raster order

// Rows of A rounded up to whole 32-row groups, and the workspace that holds A
// in the tile layout.
__host__ __device__ inline int64_t padded_rows(int64_t M) { return (M + 31) / 32 * 32; }

// A [M][K/2] codes + [M][K/16] scales -> the tile layout of the prepared weight
// for padded_rows(M) rows (rows >= M are zero). A plain byte permutation: the
// GEMM applies each scale by a multiply, so signed, zero and NaN scales need no
// folding. Thread = one 16-byte code unit (tile t = g * K/64 + c, unit 32h + r:
// row 32g + r, chunk bytes [16h, 16h + 16)); the h = 0 thread also moves the
// row's scale word of the chunk. Writes are contiguous per wave.
__global__ __launch_bounds__(256) void tile_a_kernel(const uint8_t *__restrict__ a_codes,
                                                     const uint8_t *__restrict__ a_scales, int64_t M, int64_t K,
                                                     uint8_t *__restrict__ at) {
  const int64_t kt = K / 64;
  const int64_t Mp = padded_rows(M);
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tile = u >> 6;
  if (tile >= Mp / 32 * kt) return;
  const int unit = (int)(u & 63), h = unit >> 5, r = unit & 31;
  const int64_t g = tile / kt, c = tile - g * kt;
  const int64_t row = g * 32 + r;
  u32x4_t v = {0u, 0u, 0u, 0u};
  uint32_t sc = 0u;
  if (row < M) {
    v = *reinterpret_cast<const u32x4_t *>(a_codes + row * (K / 2) + c * 32 + h * 16);
    if (h == 0) sc = *reinterpret_cast<const uint32_t *>(a_scales + row * (K / 16) + c * 4);
  }
  *reinterpret_cast<u32x4_t *>(at + tile * 1024 + unit * 16) = v;
  if (h == 0) *reinterpret_cast<uint32_t *>(at + Mp * (K / 2) + tile * 128 + r * 4) = sc;
}

struct Params {
  const uint8_t *a_tiled;   // A in the tile layout, padded_rows(M) rows
  const uint8_t *w_prep;    // prepared (N, K)
  void *d;
  int64_t M, N, K, ldd;
  float alpha;
  const float *alpha_dev;
  const float *alpha_col;   // per-column scale [N] or null
  int tiles_m, tiles_n;     // tile grid of D (in workgroup tiles; in 256 x 256 tiles when quad)
  int count;                // tiles this launch computes
  int first;                // quad: first 256 x 256 tile (raster index) whose quadrants it computes
  int quad;                 // 1: 128 x 128 workgroups on the quadrants of 256 x 256 tiles first ..
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

// Packed fragments of one chunk for this wave: T A row groups and T W column
// groups (T = MFMA tiles per wave and dimension).
template <int T>
struct ChunkFrags {
  u32x4_t a[T], w[T];      // 32 codes of one row per lane (dword s feeds MFMA step s)
  uint32_t as[T], ws[T];   // the row's four block scales of the chunk (raw E4M3 bytes)
};

// The lane's two block scales of a chunk (blocks 2h, 2h+1) in FP16. Converted
// when the chunk's first step is unpacked, not when its loads are issued, so
// the wait for the scale loads comes a whole chunk after they were issued.
// Element 2i + b holds group i's scale of block 2h + b. Plain vectors, not
// arrays, so the values stay in registers.
struct ChunkScales {
  half8_t a, w;
};

template <int T>
__device__ __forceinline__ void convert_scales(const ChunkFrags<T> &f, ChunkScales &sc) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int i = 0; i < T; i++) {
    const half2_t xa = e4m3x2_to_f16(f.as[i] >> (16 * h));
    const half2_t xw = e4m3x2_to_f16(f.ws[i] >> (16 * h));
    sc.a[2 * i] = xa[0];
    sc.a[2 * i + 1] = xa[1];
    sc.w[2 * i] = xw[0];
    sc.w[2 * i + 1] = xw[1];
  }
}

// Exact FP16 operands of MFMA step s (k = 32h + 8s + 0..7) of a chunk.
template <int T>
__device__ __forceinline__ void unpack_step(const ChunkFrags<T> &f, const ChunkScales &sc, int s, half8_t a[T],
                                            half8_t b[T]) {
#pragma unroll
  for (int i = 0; i < T; i++) a[i] = dequant8_f16(f.a[i][s], sc.a[2 * i + (s >> 1)]);
#pragma unroll
  for (int j = 0; j < T; j++) b[j] = dequant8_f16(f.w[j][s], sc.w[2 * j + (s >> 1)]);
}

template <int T>
__device__ __forceinline__ void mfma_step(const half8_t a[T], const half8_t b[T], f32x16_t acc[T][T]) {
#pragma unroll
  for (int i = 0; i < T; i++)
#pragma unroll
    for (int j = 0; j < T; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Per-lane constant byte offsets (relative to the tile bases) of this wave's
// loads: tile unit `lane` and scale word of row r, for A row groups wm*T + i
// and W column groups wn*T + i.
template <int T>
struct WaveOff {
  uint32_t a[T], as[T], w[T], ws[T];
};

// Loads of chunk c: the rebased resources keep the range check on the row (A)
// or 32-row group (W); chunks at or past nch read as zeros (length 0).
// W's chunk for chunk c of the contraction: with TWO (the two-pass activation:
// value chunks 0 .. ktw - 1, then residual chunks ktw .. 2 ktw - 1) both halves
// read the same W chunks.
template <bool TWO>
__device__ __forceinline__ int64_t w_chunk(int64_t c, int64_t ktw) {
  return TWO && c >= ktw ? c - ktw : c;
}

template <int T, bool TWO>
__device__ __forceinline__ void load_frags(const TileRsrc &tr, const WaveOff<T> &o, int64_t c, int64_t nch,
                                           int64_t ktw, ChunkFrags<T> &f) {
  const bool in = c < nch;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(tr.a, in ? tr.a_bytes : 0);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(tr.w, in ? tr.w_bytes : 0);
  const __amdgpu_buffer_rsrc_t ras = make_rsrc(tr.as, in ? tr.as_bytes : 0);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(tr.ws, in ? tr.ws_bytes : 0);
  const int sw = (int)(c * 1024), ssw = (int)(c * 128);   // chunk c: next code tile, next scale tile
  const int64_t cw = w_chunk<TWO>(c, ktw);
  const int wsw = (int)(cw * 1024), wssw = (int)(cw * 128);
#pragma unroll
  for (int i = 0; i < T; i++) {
    f.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, o.a[i], sw, 0);
    f.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, o.w[i], wsw, 0);
  }
#pragma unroll
  for (int i = 0; i < T; i++) {
    f.as[i] = __builtin_amdgcn_raw_buffer_load_b32(ras, o.as[i], ssw, 0);
    f.ws[i] = __builtin_amdgcn_raw_buffer_load_b32(rws, o.ws[i], wssw, 0);
  }
}

// One chunk of the main loop. f[P] holds chunk c, f[(P+1)%3] chunk c + 1 (in
// flight or arrived); chunk c + 2 is requested into f[(P+2)%3]. On entry (a, b)
// are chunk c's step-0 operands and sc its scales; on exit chunk c + 1's.
//
// Each MFMA step is its own scheduling region (T*T MFMAs, each followed by its
// share of the next step's unpack: 16/T vector instructions, at most five for
// T = 4). Without the region boundaries the scheduler mixes MFMAs of
// consecutive steps and issues MFMAs on the same accumulator back to back,
// which stalls each for the previous one's full latency (measured 42 against
// 36 cycles per MFMA at T = 4). The chunk's sixteen loads are spread over the
// four steps (35.0 against 36.3 cycles per MFMA with all of them in step 0).
template <int P, int T, bool TWO>
__device__ __forceinline__ void chunk_direct(const TileRsrc &tr, const WaveOff<T> &o, int64_t c, int64_t nch,
                                             int64_t ktw, ChunkFrags<T> f[3], ChunkScales &sc, half8_t a[T], half8_t b[T],
                                             f32x16_t acc[T][T]) {
  constexpr int kValuPerMfma = 16 / T + (T == 4 ? 1 : 0);
  // chunk c + 2's loads, one kind per step: A codes, W codes, A scales, W scales
  const bool in2 = c + 2 < nch;
  const int sw2 = (int)((c + 2) * 1024), ssw2 = (int)((c + 2) * 128);
  const int64_t cw2 = w_chunk<TWO>(c + 2, ktw);
  const int wsw2 = (int)(cw2 * 1024), wssw2 = (int)(cw2 * 128);
  ChunkFrags<T> &f2 = f[(P + 2) % 3];
#pragma unroll
  for (int s = 0; s < 4; s++) {
    if (s == 0) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(tr.a, in2 ? tr.a_bytes : 0);
#pragma unroll
      for (int i = 0; i < T; i++) f2.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, o.a[i], sw2, 0);
    } else if (s == 1) {
      const __amdgpu_buffer_rsrc_t rw = make_rsrc(tr.w, in2 ? tr.w_bytes : 0);
#pragma unroll
      for (int i = 0; i < T; i++) f2.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, o.w[i], wsw2, 0);
    } else if (s == 2) {
      const __amdgpu_buffer_rsrc_t ras = make_rsrc(tr.as, in2 ? tr.as_bytes : 0);
#pragma unroll
      for (int i = 0; i < T; i++) f2.as[i] = __builtin_amdgcn_raw_buffer_load_b32(ras, o.as[i], ssw2, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rws = make_rsrc(tr.ws, in2 ? tr.ws_bytes : 0);
#pragma unroll
      for (int i = 0; i < T; i++) f2.ws[i] = __builtin_amdgcn_raw_buffer_load_b32(rws, o.ws[i], wssw2, 0);
    }
    half8_t an[T], bn[T];
    if (s < 3) {
      unpack_step<T>(f[P], sc, s + 1, an, bn);
    } else {
      convert_scales<T>(f[(P + 1) % 3], sc);
      unpack_step<T>(f[(P + 1) % 3], sc, 0, an, bn);
    }
    mfma_step<T>(a, b, acc);
#pragma unroll
    for (int i = 0; i < T; i++) {
      a[i] = an[i];
      b[i] = bn[i];
    }
    __builtin_amdgcn_sched_group_barrier(0x020, T, 0);   // this step's share of chunk c + 2's loads first
#pragma unroll
    for (int k = 0; k < T * T; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue through LDS: each wave writes a 32 x 32T block of alpha * acc to its
// own LDS region in row-major order, then writes it out as 16-byte row pieces.
template <bool OUT_BF16, int T, bool COLS>
__device__ __forceinline__ void epilogue(uint8_t *smem, const Params &p, int64_t m0, int64_t n0, int wm, int wn,
                                         float alpha, f32x16_t acc[T][T]) {
  constexpr int ESZ = OUT_BF16 ? 2 : 4;
  constexpr int ROW_BYTES = 32 * T * ESZ;         // one wave's 32T columns
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  uint8_t *reg = smem + wave * (32 * 32 * T * 4);
  const int64_t col0 = n0 + wn * 32 * T;
  const int64_t ncols = p.N - col0;               // columns of this wave still inside D
  const bool vec_ok = (p.ldd * ESZ) % 16 == 0 && ((uintptr_t)p.d & 15) == 0;
#pragma unroll
  for (int i = 0; i < T; i++) {
#pragma unroll
    for (int j = 0; j < T; j++) {
      // the alpha of this lane's column (columns past N are not stored)
      const float aj = COLS && j * 32 + r < ncols ? alpha * p.alpha_col[col0 + j * 32 + r] : alpha;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int row = 8 * (e >> 2) + 4 * h + (e & 3);
        const float v = aj * acc[i][j][e];
        if (OUT_BF16)
          *reinterpret_cast<uint16_t *>(reg + row * ROW_BYTES + (j * 32 + r) * 2) = f32_to_bf16_rne(v);
        else
          *reinterpret_cast<float *>(reg + row * ROW_BYTES + (j * 32 + r) * 4) = v;
      }
    }
    __syncthreads();
    constexpr int PIECES = ROW_BYTES / 16;        // 16-byte pieces per row
#pragma unroll
    for (int q = lane; q < 32 * PIECES; q += 64) {
      const int row = q / PIECES, pc = q % PIECES;
      const int64_t m = m0 + wm * 32 * T + i * 32 + row;
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

// Origin of launch tile `tile`. Plain launches walk their own BT x BT tiles in
// raster order; a quad launch (BT = 128) computes the four quadrants of the
// 256 x 256 tiles first, first + 1, ... (consecutive indices: one tile's
// quadrants, which then share A rows and W columns in one XCD's L2).
template <int BT>
__device__ __forceinline__ void tile_origin(const Params &p, int tile, int64_t &m0, int64_t &n0) {
  int tm, tn;
  if (BT == 128 && p.quad) {
    tile_coords(p.first + (tile >> 2), p.tiles_m, p.tiles_n, tm, tn);
    m0 = (int64_t)tm * 256 + ((tile >> 1) & 1) * 128;
    n0 = (int64_t)tn * 256 + (tile & 1) * 128;
  } else {
    tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
    m0 = (int64_t)tm * BT;
    n0 = (int64_t)tn * BT;
  }
}

// T = 4: 256 x 256 workgroup tiles, one workgroup per CU (all 512 registers of
// a lane in use). T = 2: 128 x 128 tiles, two workgroups per CU: for problems
// with fewer 256 x 256 tiles than CUs, and for the quadrants of the 256 x 256
// tiles of a last round that would leave at least half the CUs idle.
// COLS: p.alpha_col is set (a separate instantiation, so that the kernel
// without a per-column scale keeps its registers for the main loop).
// TWO: A is a two-pass activation of 2K columns (value, then residual, in the
// tile layout) against W of K columns: the contraction runs over 2K, and chunk
// c >= K/64 uses W's chunk c - K/64.
template <bool OUT_BF16, int T, bool COLS, bool TWO>
__global__ __launch_bounds__(kThreads, T == 4 ? 1 : 2) void gemm_kernel(Params p) {
  constexpr int BT = 64 * T;                      // workgroup tile edge
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * 32 * 32 * T * 4];
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int G = gridDim.x;
  // XCD-aware logical id: hardware ids b, b+8, b+16, ... run on one XCD; give
  // them consecutive logical ids so they take neighbouring tiles.
  int pid = blockIdx.x;
  if ((G & 7) == 0) pid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const float alpha = load_alpha(p.alpha, p.alpha_dev);
  const int64_t ktw = p.K / 64;                   // W's chunks
  const int64_t kt = TWO ? 2 * ktw : ktw;         // A's chunks, the contraction's length
  const int64_t nch = kt;

  const int lane = t & 63, r = lane & 31;
  WaveOff<T> o;
#pragma unroll
  for (int i = 0; i < T; i++) {
    o.a[i] = (uint32_t)(((wm * T + i) * kt) * 1024 + lane * 16);
    o.as[i] = (uint32_t)(((wm * T + i) * kt) * 128 + r * 4);
    o.w[i] = (uint32_t)(((wn * T + i) * ktw) * 1024 + lane * 16);
    o.ws[i] = (uint32_t)(((wn * T + i) * ktw) * 128 + r * 4);
  }

  for (int tile = pid; tile < p.count; tile += G) {
    int64_t m0, n0;
    tile_origin<BT>(p, tile, m0, n0);
    if (m0 >= p.M || n0 >= p.N) continue;   // a quadrant past the edge of D (uniform per workgroup)
    TileRsrc tr;
    const int64_t Mp = padded_rows(p.M);
    tr.a = p.a_tiled + (m0 >> 5) * kt * 1024;
    tr.a_bytes = (Mp - m0) / 32 * kt * 1024;
    tr.as = p.a_tiled + (TWO ? Mp * kt * 32 : Mp * p.K / 2) + (m0 >> 5) * kt * 128;
    tr.as_bytes = (Mp - m0) / 32 * kt * 128;
    tr.w = p.w_prep + (n0 >> 5) * ktw * 1024;
    tr.w_bytes = (p.N - n0) / 32 * ktw * 1024;
    tr.ws = p.w_prep + p.N * p.K / 2 + (n0 >> 5) * ktw * 128;
    tr.ws_bytes = (p.N - n0) / 32 * ktw * 128;

    f32x16_t acc[T][T];
#pragma unroll
    for (int i = 0; i < T; i++)
#pragma unroll
      for (int j = 0; j < T; j++) acc[i][j] = f32x16_t{};
    ChunkFrags<T> f[3];
    ChunkScales sc;
    half8_t a[T], b[T];
    load_frags<T, TWO>(tr, o, 0, nch, ktw, f[0]);
    load_frags<T, TWO>(tr, o, 1, nch, ktw, f[1]);
    convert_scales<T>(f[0], sc);
    unpack_step<T>(f[0], sc, 0, a, b);
    if constexpr (COLS) {
      // chunks in threes, the last ones padded with all-zero chunks: a tail as below
      // would push this instantiation's extra epilogue registers into more spills
      // (measured 7 % slower at 8192^3)
      for (int64_t c = 0; c < nch; c += 3) {
        chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
        chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
        chunk_direct<2, T, TWO>(tr, o, c + 2, nch, ktw, f, sc, a, b, acc);
      }
    } else {
      int64_t c = 0;
      for (; c + 3 <= nch; c += 3) {
        chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
        chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
        chunk_direct<2, T, TWO>(tr, o, c + 2, nch, ktw, f, sc, a, b, acc);
      }
      // the one or two chunks left when K/64 is not a multiple of 3 (ring position 0, then 1)
      if (c < nch) chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
      if (c + 1 < nch) chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
    }
    __syncthreads();
    epilogue<OUT_BF16, T, COLS>(smem, p, m0, n0, wm, wn, alpha, acc);
  }
}

}  // namespace w4a4
}  // namespace nvfp4

using namespace nvfp4;

size_t nvfp4::w4a4_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 64 != 0) return 0;
  return (size_t)(w4a4::padded_rows(M) * K / 2 + w4a4::padded_rows(M) * K / 16);
}

namespace {

nvfp4_status check_gemm_args(const uint8_t *w_prep, int64_t M, int64_t N, int64_t K, float alpha,
                             const float *alpha_dev, const float *alpha_col, void *d, int out_dtype, int64_t ldd) {
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_DTYPE;
  if (M < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || ldd < N) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!w_prep || !d) return NVFP4_ERR_NULL;
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return NVFP4_ERR_VALUE;
  const size_t esz = out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
  if (!aligned(w_prep, 16) || !aligned(d, esz) || (alpha_dev && !aligned(alpha_dev, 4)) ||
      (alpha_col && !aligned(alpha_col, 4)))
    return NVFP4_ERR_ALIGN;
  // 32-bit buffer offsets inside the code tiles of one 256-row (256-column) tile
  if ((int64_t)8 * (K / 64) * 1024 > 0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
  if ((M + 127) / 128 * ((N + 127) / 128) > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

template <int T, bool TWO>
void launch_tiles(const w4a4::Params &p, int grid, int out_dtype, hipStream_t s) {
  const dim3 g(grid), b(w4a4::kThreads);
  if (out_dtype == NVFP4_OUT_BF16) {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::gemm_kernel<true, T, true, TWO>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::gemm_kernel<true, T, false, TWO>), g, b, 0, s, p);
  } else {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::gemm_kernel<false, T, true, TWO>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::gemm_kernel<false, T, false, TWO>), g, b, 0, s, p);
  }
}

template <int T>
void launch_tiles(const w4a4::Params &p, int grid, int out_dtype, bool two, hipStream_t s) {
  if (two) launch_tiles<T, true>(p, grid, out_dtype, s);
  else launch_tiles<T, false>(p, grid, out_dtype, s);
}

// The GEMM kernel proper on A already in the tile layout (arguments checked).
//  * At least as many 256 x 256 tiles as CUs: the T = 4 kernel, one persistent
//    workgroup per CU. When the tiles do not make whole rounds and the last
//    round would use at most half the CUs, that round's tiles are left to a
//    second launch of the T = 2 kernel on their 128 x 128 quadrants (two
//    workgroups per CU, so the round takes about half as long). Each output
//    element sees the same sequence of MFMAs either way: the results are the
//    same bits as with T = 4 alone.
//  * Fewer: the T = 2 kernel on 128 x 128 tiles.
nvfp4_status launch_gemm(const uint8_t *a_tiled, const uint8_t *w_prep, int64_t M, int64_t N, int64_t K, float alpha,
                         const float *alpha_dev, const float *alpha_col, void *d, int out_dtype, int64_t ldd, bool two,
                         hipStream_t s) {
  DeviceInfo di;
  nvfp4_status st = device_info(&di);
  if (st != NVFP4_OK) return st;
  const int64_t cus = di.num_cus;
  const int64_t tm4 = (M + 255) / 256, tn4 = (N + 255) / 256, t4 = tm4 * tn4;
  if (t4 >= cus) {
    const int64_t rem = t4 % cus;
    const int64_t full = rem > 0 && 2 * rem <= cus ? t4 - rem : t4;
    w4a4::Params p{a_tiled, w_prep, d, M, N, K, ldd, alpha, alpha_dev, alpha_col, (int)tm4, (int)tn4, (int)full, 0, 0};
    launch_tiles<4>(p, (int)cus, out_dtype, two, s);
    NVFP4_LAUNCH_CHECK();
    if (full < t4) {
      p.count = (int)(4 * (t4 - full));   // <= 2 * cus: one workgroup per quadrant
      p.first = (int)full;
      p.quad = 1;
      launch_tiles<2>(p, p.count, out_dtype, two, s);
      NVFP4_LAUNCH_CHECK();
    }
    return NVFP4_OK;
  }
  const int64_t tm2 = (M + 127) / 128, tn2 = (N + 127) / 128, t2 = tm2 * tn2;
  w4a4::Params p{a_tiled, w_prep, d, M, N, K, ldd, alpha, alpha_dev, alpha_col, (int)tm2, (int)tn2, (int)t2, 0, 0};
  launch_tiles<2>(p, (int)(t2 < 2 * cus ? t2 : 2 * cus), out_dtype, two, s);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

void launch_tile_a(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K, uint8_t *at,
                   hipStream_t s) {
  const int64_t units = w4a4::padded_rows(M) / 32 * (K / 64) * 64;
  hipLaunchKernelGGL(w4a4::tile_a_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a_codes, a_scales,
                     M, K, at);
}

}  // namespace

extern "C" size_t nvfp4_tiled_activation_bytes(int64_t M, int64_t K) { return w4a4_workspace_bytes(M, K); }

extern "C" nvfp4_status nvfp4_tile_activation(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                              uint8_t *a_tiled, void *stream) {
  if (M < 0 || K <= 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_tiled) return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(a_scales, 4) || !aligned(a_tiled, 16)) return NVFP4_ERR_ALIGN;
  if (w4a4::padded_rows(M) / 32 * (K / 64) * 64 / 256 + 1 > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
  DeviceInfo di;
  nvfp4_status st = device_info(&di);
  if (st != NVFP4_OK) return st;
  launch_tile_a(a_codes, a_scales, M, K, a_tiled, (hipStream_t)stream);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

extern "C" nvfp4_status nvfp4_gemm_w4a4_tiled(const uint8_t *a_tiled, const uint8_t *w_prep, int64_t M, int64_t N,
                                              int64_t K, float alpha, const float *alpha_dev,
                                              const float *alpha_col, void *d, int out_dtype, int64_t ldd,
                                              void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a_tiled) return NVFP4_ERR_NULL;
  if (!aligned(a_tiled, 16)) return NVFP4_ERR_ALIGN;
  return launch_gemm(a_tiled, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, false,
                     (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_gemm_w4a4_two_pass_tiled(const uint8_t *a2_tiled, const uint8_t *w_prep, int64_t M,
                                                       int64_t N, int64_t K, float alpha, const float *alpha_dev,
                                                       const float *alpha_col, void *d, int out_dtype, int64_t ldd,
                                                       void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a2_tiled) return NVFP4_ERR_NULL;
  if (!aligned(a2_tiled, 16)) return NVFP4_ERR_ALIGN;
  // 32-bit buffer offsets inside one 256-row tile of the 2K-column activation
  if ((int64_t)8 * (2 * K / 64) * 1024 > 0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
  return launch_gemm(a2_tiled, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, true,
                     (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_prep,
                                        int64_t M, int64_t N, int64_t K, float alpha, const float *alpha_dev,
                                        const float *alpha_col, void *d, int out_dtype, int64_t ldd, void *ws,
                                        size_t ws_bytes, void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a_codes || !a_scales) return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(a_scales, 4)) return NVFP4_ERR_ALIGN;
  const size_t need = w4a4_workspace_bytes(M, K);
  if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  DeviceInfo di;
  st = device_info(&di);
  if (st != NVFP4_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *at = static_cast<uint8_t *>(ws);
  launch_tile_a(a_codes, a_scales, M, K, at, s);
  NVFP4_LAUNCH_CHECK();
  return launch_gemm(at, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, false, s);
}
