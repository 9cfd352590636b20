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
  int count;                // whole tiles this launch computes (raster indices 0 .. count - 1)
  int first;                // quad / split: first 256 x 256 tile (raster index) whose quadrants or
                            // K ranges it computes
  int quad;                 // 1: 128 x 128 workgroups on the quadrants of 256 x 256 tiles first ..
  int split;                // K ranges of each split tile (>= 2 when nsplit > 0)
  int nsplit;               // tiles first .. first + nsplit - 1 are split along K
  float *partials;          // FP32 partial tile of split work unit count + q at slot q
  uint32_t *sched;          // dynamic scheduling counters (null: static schedule)
};

// FP32 values of one 256 x 256 partial tile, in MFMA accumulator order:
// [wave][i][j][lane][16].
constexpr int64_t kPartialFloats = 4 * 4 * 4 * 64 * 16;
constexpr int kSchedCounters = 8;          // one work counter per XCD
constexpr size_t kSchedBytes = 256;        // their workspace region

// Work units of a launch: the whole tiles, then split * nsplit K ranges.
__host__ __device__ inline int work_units(const Params &p) { return p.count + p.nsplit * p.split; }

// Tile and K chunks [c0, c1) of work unit u (whole tiles: all nch chunks).
__device__ __forceinline__ void unit_chunks(const Params &p, int u, int64_t nch, int &tile, int64_t &c0,
                                            int64_t &c1) {
  if (u < p.count) {
    tile = u;
    c0 = 0;
    c1 = nch;
    return;
  }
  const int v = u - p.count, q = v % p.split;
  tile = p.first + v / p.split;
  c0 = nch * q / p.split;
  c1 = nch * (q + 1) / p.split;
}

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
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));   // written once: stream it
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

// The FP32 accumulators of a split work unit to its partial slot (T = 4 only):
// lane-contiguous 64 bytes per MFMA tile, so each wave writes 4 KB runs.
template <int T>
__device__ __forceinline__ void store_partial(const Params &p, int u, f32x16_t acc[T][T]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float *slot = p.partials + (int64_t)(u - p.count) * kPartialFloats;
#pragma unroll
  for (int i = 0; i < T; i++)
#pragma unroll
    for (int j = 0; j < T; j++) {
      f32x4_t *dst = reinterpret_cast<f32x4_t *>(slot + (((wave * T + i) * T + j) * 64 + lane) * 16);
#pragma unroll
      for (int q = 0; q < 4; q++)
        dst[q] = f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
}

// Dynamic schedule: the workgroups of hardware XCD x (ids congruent to x
// mod 8) take the work units of their own share of each round of G units from
// a counter of their own, sched[x], so an XCD's L2 sees the same tiles as
// under the static schedule while the order inside an XCD follows whichever
// workgroup is free first. The counters are zeroed by sched_reset_kernel,
// launched just before on the same stream. Every workgroup leaves the loop at
// its first fetch past the last unit, so the grid always drains.
__device__ __forceinline__ int fetch_unit(const Params &p, int G, int *s_unit) {
  const int nx = (G & 7) == 0 ? 8 : 1, per = G / nx, x = blockIdx.x % nx;
  __syncthreads();   // every wave has read the previous unit
  if (threadIdx.x == 0) {
    const int f = (int)atomicAdd(&p.sched[x], 1u);
    *s_unit = (f / per) * G + x * per + f % per;
  }
  __syncthreads();
  return *s_unit;
}

__global__ void sched_reset_kernel(uint32_t *sched) {
  if (threadIdx.x < kSchedCounters) sched[threadIdx.x] = 0u;
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
// XS (T = 4): the extended schedule, a separate instantiation so that the
// plain one keeps its registers: work units are the whole tiles, then the K
// ranges of split tiles, whose accumulators go to partial slots for
// split_fixup_kernel instead of D; with p.sched, workgroups fetch their units
// dynamically.
template <bool OUT_BF16, int T, bool COLS, bool TWO, bool XS>
__global__ __launch_bounds__(kThreads, T == 4 ? 1 : 2) void gemm_kernel(Params p) {
  constexpr int BT = 64 * T;                      // workgroup tile edge
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * 32 * 32 * T * 4];
  __shared__ int s_unit;
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
  const int units = XS ? work_units(p) : p.count;
  const bool dyn = XS && p.sched != nullptr;

  const int lane = t & 63, r = lane & 31;
  WaveOff<T> o;
#pragma unroll
  for (int i = 0; i < T; i++) {
    o.a[i] = (uint32_t)(((wm * T + i) * kt) * 1024 + lane * 16);
    o.as[i] = (uint32_t)(((wm * T + i) * kt) * 128 + r * 4);
    o.w[i] = (uint32_t)(((wn * T + i) * ktw) * 1024 + lane * 16);
    o.ws[i] = (uint32_t)(((wn * T + i) * ktw) * 128 + r * 4);
  }

  for (int u = dyn ? fetch_unit(p, G, &s_unit) : pid; u < units; u = dyn ? fetch_unit(p, G, &s_unit) : u + G) {
    int tile = u;
    int64_t c0 = 0, nch = kt;                      // chunks [c0, nch); loads at or past nch read zero
    if constexpr (XS) unit_chunks(p, u, kt, tile, c0, nch);
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
    load_frags<T, TWO>(tr, o, c0, nch, ktw, f[0]);
    load_frags<T, TWO>(tr, o, c0 + 1, nch, ktw, f[1]);
    convert_scales<T>(f[0], sc);
    unpack_step<T>(f[0], sc, 0, a, b);
    if constexpr (COLS) {
      // chunks in threes, the last ones padded with all-zero chunks: a tail as below
      // would push this instantiation's extra epilogue registers into more spills
      // (measured 7 % slower at 8192^3)
      for (int64_t c = c0; c < nch; c += 3) {
        chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
        chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
        chunk_direct<2, T, TWO>(tr, o, c + 2, nch, ktw, f, sc, a, b, acc);
      }
    } else {
      int64_t c = c0;
      for (; c + 3 <= nch; c += 3) {
        chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
        chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
        chunk_direct<2, T, TWO>(tr, o, c + 2, nch, ktw, f, sc, a, b, acc);
      }
      // the one or two chunks left when the range is not a multiple of 3 (ring position 0, then 1)
      if (c < nch) chunk_direct<0, T, TWO>(tr, o, c, nch, ktw, f, sc, a, b, acc);
      if (c + 1 < nch) chunk_direct<1, T, TWO>(tr, o, c + 1, nch, ktw, f, sc, a, b, acc);
    }
    if (XS && u >= p.count) {
      store_partial<T>(p, u, acc);
      continue;
    }
    __syncthreads();
    epilogue<OUT_BF16, T, COLS>(smem, p, m0, n0, wm, wn, alpha, acc);
  }
}

// Sums the partial tiles of each split 256 x 256 tile in range order (a fixed
// order, so the result does not depend on which workgroup ran which range)
// and applies the epilogue. Workgroup = (split tile, wave, MFMA row i) of the
// main kernel's layout; thread = (MFMA column j, lane): 16 values, four ranges'
// loads in flight at a time.
template <bool OUT_BF16, bool COLS>
__global__ __launch_bounds__(256) void split_fixup_kernel(Params p) {
  const int tl = blockIdx.x >> 4, wi = blockIdx.x & 15, wave = wi >> 2, i = wi & 3;
  const int j = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  int64_t m0, n0;
  tile_origin<256>(p, p.first + tl, m0, n0);
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t col = n0 + wn * 128 + j * 32 + r;
  const int64_t row0 = m0 + wm * 128 + i * 32 + 4 * h;
  const float *base =
      p.partials + (int64_t)tl * p.split * kPartialFloats + (((wave * 4 + i) * 4 + j) * 64 + lane) * 16;
  f32x16_t sum = f32x16_t{};
  for (int q0 = 0; q0 < p.split; q0 += 4) {
    f32x4_t v[4][4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const f32x4_t *src = reinterpret_cast<const f32x4_t *>(base + (int64_t)(q0 + b) * kPartialFloats);
#pragma unroll
      for (int q = 0; q < 4; q++) v[b][q] = q0 + b < p.split ? src[q] : f32x4_t{};
    }
#pragma unroll
    for (int b = 0; b < 4; b++)
      if (q0 + b < p.split)
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int e = 0; e < 4; e++) sum[4 * q + e] = sum[4 * q + e] + v[b][q][e];
  }
  if (col >= p.N) return;
  const float alpha = load_alpha(p.alpha, p.alpha_dev);
  const float aj = COLS ? alpha * p.alpha_col[col] : alpha;
#pragma unroll
  for (int e = 0; e < 16; e++) {
    const int64_t m = row0 + 8 * (e >> 2) + (e & 3);
    if (m < p.M) {
      const float v = aj * sum[e];
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(p.d)[m * p.ldd + col] = f32_to_bf16_rne(v);
      else
        reinterpret_cast<float *>(p.d)[m * p.ldd + col] = v;
    }
  }
}

}  // namespace w4a4
}  // namespace nvfp4

using namespace nvfp4;

size_t nvfp4::tiled_activation_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 64 != 0) return 0;
  return (size_t)(w4a4::padded_rows(M) * K / 2 + w4a4::padded_rows(M) * K / 16);
}

namespace {

// How a resolved config runs (M, N) with a contraction of nch chunks.
struct Plan {
  int T;               // MFMA tiles per wave and dimension (4: 256 x 256, 2: 128 x 128)
  int tiles_m, tiles_n;
  int grid;            // workgroups of the main launch
  int count;           // whole tiles of the main launch
  int split, nsplit;   // K ranges per split tile, split tiles
  int quad;            // tiles whose quadrants a second launch computes
  bool dynamic;
};

Plan make_plan(int64_t M, int64_t N, const nvfp4_config &c) {
  Plan p{};
  const int64_t cus = c.num_cus;
  p.dynamic = c.dynamic != 0;
  if (c.tile_m == 256) {
    p.T = 4;
    p.tiles_m = (int)((M + 255) / 256);
    p.tiles_n = (int)((N + 255) / 256);
    const int64_t t = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t rem = c.tail == NVFP4_TAIL_NONE ? 0 : t % cus;
    p.count = (int)(t - rem);
    if (c.tail == NVFP4_TAIL_QUADRANTS) p.quad = (int)rem;
    if (c.tail == NVFP4_TAIL_SPLIT && rem > 0) {
      p.split = c.split_k;
      p.nsplit = (int)rem;
    }
    const int64_t units = p.count + (int64_t)p.nsplit * p.split;
    p.grid = (int)(units < cus ? units : cus);
  } else {
    p.T = 2;
    p.tiles_m = (int)((M + 127) / 128);
    p.tiles_n = (int)((N + 127) / 128);
    const int64_t t = (int64_t)p.tiles_m * p.tiles_n;
    p.count = (int)t;
    p.grid = (int)(t < 2 * cus ? t : 2 * cus);
  }
  return p;
}

// Workspace of the tiled GEMM under a plan: the dynamic schedule's counters,
// then the split ranges' partial tiles.
size_t sched_bytes(const Plan &p) { return p.dynamic ? w4a4::kSchedBytes : 0; }
size_t partial_bytes(const Plan &p) { return (size_t)p.nsplit * p.split * w4a4::kPartialFloats * 4; }
size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

// The heuristic configuration for a contraction of length K:
//  * at least as many 256 x 256 tiles as CUs: those tiles, persistent. When
//    they do not make whole rounds and the last round would use at most half
//    the CUs, the leftover tiles run as 128 x 128 quadrants in a second launch,
//    or, for K >= kSplitMinK, split in two along K (the partials and their
//    fix-up cost about as much as 50 us of tile work, which only a long K
//    amortises: at K = 17408 the split took 8192 x 5120 from 989.5 to 971.4 us,
//    while at K = 5120 quadrants beat it, 992 against 1012.5 us on the prefill
//    shape);
//  * fewer: 128 x 128 tiles, two workgroups per CU.
constexpr int64_t kSplitMinK = 12288;

void nvfp4::w4a4_default_config(int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *c) {
  *c = nvfp4_config{};
  c->kernel = NVFP4_KERNEL_W4A4_TILES;
  c->num_cus = cus;
  const int64_t t4 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t4 >= cus) {
    c->tile_m = c->tile_n = 256;
    const int64_t rem = t4 % cus;
    if (rem > 0 && 2 * rem <= cus) {
      if (K >= kSplitMinK) {
        c->tail = NVFP4_TAIL_SPLIT;
        c->split_k = 2;
      } else {
        c->tail = NVFP4_TAIL_QUADRANTS;
      }
    }
  } else {
    c->tile_m = c->tile_n = 128;
  }
}

bool nvfp4::w4a4_config_valid(int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  (void)M;
  (void)N;
  if (c.kernel != NVFP4_KERNEL_W4A4_TILES || c.num_cus <= 0 || (c.dynamic != 0 && c.dynamic != 1)) return false;
  if (c.tile_m != c.tile_n || (c.tile_m != 256 && c.tile_m != 128)) return false;
  if (c.tail < NVFP4_TAIL_NONE || c.tail > NVFP4_TAIL_SPLIT) return false;
  if (c.tile_m == 128 && (c.tail != NVFP4_TAIL_NONE || c.dynamic != 0)) return false;
  if (c.tail == NVFP4_TAIL_SPLIT) return c.split_k >= 2 && c.split_k <= K / 64;
  return c.split_k == 0;
}

size_t nvfp4::w4a4_config_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  if (M <= 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || !w4a4_config_valid(M, N, K, c)) return 0;
  const Plan p = make_plan(M, N, c);
  const size_t tail = sched_bytes(p) + partial_bytes(p);
  if (op == NVFP4_OP_W4A4_TILED) return tail;
  return round256(tiled_activation_bytes(M, K)) + tail;
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

template <int T, bool TWO, bool XS>
void launch_tiles(const w4a4::Params &p, int grid, int out_dtype, hipStream_t s) {
  const dim3 g(grid), b(w4a4::kThreads);
  if (out_dtype == NVFP4_OUT_BF16) {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::gemm_kernel<true, T, true, TWO, XS>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::gemm_kernel<true, T, false, TWO, XS>), g, b, 0, s, p);
  } else {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::gemm_kernel<false, T, true, TWO, XS>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::gemm_kernel<false, T, false, TWO, XS>), g, b, 0, s, p);
  }
}

// The extended schedule (split ranges, dynamic fetch) exists for T = 4 only.
template <int T>
void launch_tiles(const w4a4::Params &p, int grid, int out_dtype, bool two, hipStream_t s) {
  const bool xs = T == 4 && (p.nsplit > 0 || p.sched != nullptr);
  if (two) {
    if (xs) launch_tiles<4, true, true>(p, grid, out_dtype, s);
    else launch_tiles<T, true, false>(p, grid, out_dtype, s);
  } else {
    if (xs) launch_tiles<4, false, true>(p, grid, out_dtype, s);
    else launch_tiles<T, false, false>(p, grid, out_dtype, s);
  }
}

void launch_fixup(const w4a4::Params &p, int out_dtype, hipStream_t s) {
  const dim3 g((unsigned)(p.nsplit * 16)), b(256);
  if (out_dtype == NVFP4_OUT_BF16) {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::split_fixup_kernel<true, true>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::split_fixup_kernel<true, false>), g, b, 0, s, p);
  } else {
    if (p.alpha_col) hipLaunchKernelGGL((w4a4::split_fixup_kernel<false, true>), g, b, 0, s, p);
    else hipLaunchKernelGGL((w4a4::split_fixup_kernel<false, false>), g, b, 0, s, p);
  }
}

// The GEMM proper on A in the tile layout under a resolved config (arguments
// checked; tail is the workspace region of the counters and partials, or null
// when the plan needs none). Launches, in stream order:
//  * static schedule: the persistent kernel over the whole tiles, then the
//    tail: the quadrant launch, or the split tiles' K ranges (the extended
//    instantiation, in a launch of their own so that the whole tiles keep the
//    plain one's registers) and the fix-up;
//  * dynamic schedule: the counters' reset, then one launch of the extended
//    instantiation over the whole tiles and the split ranges, then the fix-up.
// An output element sees the same MFMA sequence in a whole tile and in a
// quadrant, so those give the same bits; a split tile sums its ranges'
// partials instead.
nvfp4_status launch_gemm(const uint8_t *a_tiled, const uint8_t *w_prep, int64_t M, int64_t N, int64_t K, float alpha,
                         const float *alpha_dev, const float *alpha_col, void *d, int out_dtype, int64_t ldd, bool two,
                         const nvfp4_config &cfg, uint8_t *tail, hipStream_t s) {
  const Plan pl = make_plan(M, N, cfg);
  w4a4::Params p{};
  p.a_tiled = a_tiled;
  p.w_prep = w_prep;
  p.d = d;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ldd = ldd;
  p.alpha = alpha;
  p.alpha_dev = alpha_dev;
  p.alpha_col = alpha_col;
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.count = pl.count;
  p.first = pl.count;
  float *partials = pl.nsplit > 0 ? reinterpret_cast<float *>(tail + sched_bytes(pl)) : nullptr;
  const int64_t cus = cfg.num_cus;
  if (pl.dynamic) {
    p.sched = reinterpret_cast<uint32_t *>(tail);
    p.split = pl.split;
    p.nsplit = pl.nsplit;
    p.partials = partials;
    hipLaunchKernelGGL(w4a4::sched_reset_kernel, dim3(1), dim3(64), 0, s, p.sched);
    NVFP4_LAUNCH_CHECK();
    if (pl.grid > 0) {
      launch_tiles<4>(p, pl.grid, out_dtype, two, s);
      NVFP4_LAUNCH_CHECK();
    }
  } else {
    if (pl.count > 0) {
      const int grid = (int)(pl.T == 4 ? std::min<int64_t>(cus, pl.count) : pl.grid);
      if (pl.T == 4) launch_tiles<4>(p, grid, out_dtype, two, s);
      else launch_tiles<2>(p, grid, out_dtype, two, s);
      NVFP4_LAUNCH_CHECK();
    }
    if (pl.nsplit > 0) {
      w4a4::Params q = p;             // the split tiles' K ranges only
      q.count = 0;
      q.split = pl.split;
      q.nsplit = pl.nsplit;
      q.partials = partials;
      const int64_t units = (int64_t)pl.nsplit * pl.split;
      launch_tiles<4>(q, (int)std::min<int64_t>(cus, units), out_dtype, two, s);
      NVFP4_LAUNCH_CHECK();
    }
  }
  if (pl.nsplit > 0) {
    w4a4::Params q = p;
    q.count = pl.dynamic ? pl.count : 0;
    q.split = pl.split;
    q.nsplit = pl.nsplit;
    q.partials = partials;
    launch_fixup(q, out_dtype, s);
    NVFP4_LAUNCH_CHECK();
  }
  if (pl.quad > 0) {
    w4a4::Params q = p;
    q.count = 4 * pl.quad;   // one workgroup per quadrant
    q.first = pl.count;
    q.quad = 1;
    q.split = q.nsplit = 0;
    q.partials = nullptr;
    q.sched = nullptr;
    launch_tiles<2>(q, q.count, out_dtype, two, s);
    NVFP4_LAUNCH_CHECK();
  }
  return NVFP4_OK;
}

void launch_tile_a(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K, uint8_t *at,
                   hipStream_t s) {
  const int64_t units = w4a4::padded_rows(M) / 32 * (K / 64) * 64;
  hipLaunchKernelGGL(w4a4::tile_a_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a_codes, a_scales,
                     M, K, at);
}

// Resolves the config of a tiled-A call (contraction length Kc) and finds its
// workspace region. With no caller config and a workspace that cannot hold
// what the chosen config needs, the K-split tail becomes quadrants and the
// schedule static, which need none.
nvfp4_status tiled_config(int64_t M, int64_t N, int64_t Kc, const nvfp4_config *config, int cus, void *ws,
                          size_t ws_bytes, nvfp4_config *cfg, uint8_t **tail) {
  nvfp4_status st = resolve_config(NVFP4_OP_W4A4_TILED, M, N, Kc, config, cus, cfg);
  if (st != NVFP4_OK) return st;
  size_t need = w4a4_config_workspace_bytes(NVFP4_OP_W4A4_TILED, M, N, Kc, *cfg);
  if (need > 0 && (!ws || ws_bytes < need)) {
    if (config) return NVFP4_ERR_WORKSPACE;
    if (cfg->tail == NVFP4_TAIL_SPLIT) {
      cfg->tail = NVFP4_TAIL_QUADRANTS;
      cfg->split_k = 0;
    }
    cfg->dynamic = 0;
    need = 0;
  }
  if (need > 0 && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  *tail = need > 0 ? static_cast<uint8_t *>(ws) : nullptr;
  return NVFP4_OK;
}

}  // namespace

extern "C" size_t nvfp4_tiled_activation_bytes(int64_t M, int64_t K) { return tiled_activation_bytes(M, K); }

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
                                              const nvfp4_config *config, void *ws, size_t ws_bytes,
                                              void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a_tiled) return NVFP4_ERR_NULL;
  if (!aligned(a_tiled, 16)) return NVFP4_ERR_ALIGN;
  DeviceInfo di;
  st = device_info(&di);
  if (st != NVFP4_OK) return st;
  nvfp4_config cfg;
  uint8_t *tail = nullptr;
  st = tiled_config(M, N, K, config, di.num_cus, ws, ws_bytes, &cfg, &tail);
  if (st != NVFP4_OK) return st;
  return launch_gemm(a_tiled, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, false, cfg, tail,
                     (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_gemm_w4a4_two_pass_tiled(const uint8_t *a2_tiled, const uint8_t *w_prep, int64_t M,
                                                       int64_t N, int64_t K, float alpha, const float *alpha_dev,
                                                       const float *alpha_col, void *d, int out_dtype, int64_t ldd,
                                                       const nvfp4_config *config, void *ws, size_t ws_bytes,
                                                       void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a2_tiled) return NVFP4_ERR_NULL;
  if (!aligned(a2_tiled, 16)) return NVFP4_ERR_ALIGN;
  // 32-bit buffer offsets inside one 256-row tile of the 2K-column activation
  if ((int64_t)8 * (2 * K / 64) * 1024 > 0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
  DeviceInfo di;
  st = device_info(&di);
  if (st != NVFP4_OK) return st;
  nvfp4_config cfg;
  uint8_t *tail = nullptr;
  st = tiled_config(M, N, 2 * K, config, di.num_cus, ws, ws_bytes, &cfg, &tail);
  if (st != NVFP4_OK) return st;
  return launch_gemm(a2_tiled, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, true, cfg, tail,
                     (hipStream_t)stream);
}

extern "C" nvfp4_status nvfp4_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_prep,
                                        int64_t M, int64_t N, int64_t K, float alpha, const float *alpha_dev,
                                        const float *alpha_col, void *d, int out_dtype, int64_t ldd,
                                        const nvfp4_config *config, void *ws, size_t ws_bytes, void *stream) {
  nvfp4_status st = check_gemm_args(w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd);
  if (st != NVFP4_OK || M == 0) return st;
  if (!a_codes || !a_scales) return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(a_scales, 4)) return NVFP4_ERR_ALIGN;
  // the workspace holds at least A's tile copy (checked before any device query)
  if (!ws || ws_bytes < tiled_activation_bytes(M, K)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  DeviceInfo di;
  st = device_info(&di);
  if (st != NVFP4_OK) return st;
  nvfp4_config cfg;
  st = resolve_config(NVFP4_OP_W4A4, M, N, K, config, di.num_cus, &cfg);
  if (st != NVFP4_OK) return st;
  const size_t need = w4a4_config_workspace_bytes(NVFP4_OP_W4A4, M, N, K, cfg);
  if (ws_bytes < need) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *at = static_cast<uint8_t *>(ws);
  uint8_t *tail = at + round256(tiled_activation_bytes(M, K));
  if (need == round256(tiled_activation_bytes(M, K))) tail = nullptr;
  launch_tile_a(a_codes, a_scales, M, K, at, s);
  NVFP4_LAUNCH_CHECK();
  return launch_gemm(at, w_prep, M, N, K, alpha, alpha_dev, alpha_col, d, out_dtype, ldd, false, cfg, tail, s);
}
