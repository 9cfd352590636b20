// W4A16 NVFP4 GEMM for gfx950: y = alpha * x (W.SFW)^T, x/y BF16, FP32 accumulation.
//
// Kernels, chosen by M (and, for decode, by the number of 32-row groups):
//  * M <= 4 (decode): a weight-streaming kernel on the vector ALUs. A workgroup
//    owns one 32-row prepared tile group over the whole K (at M = 1, groups
//    left over after whole rounds of resident workgroups are cut into 8- or
//    16-row workgroups); its waves (12, or 8
//    once there are two groups per CU) take interleaved 64-wide K tiles, one
//    contiguous 1 KB tile per wave load. Each lane streams 16 packed bytes (32
//    codes of one row) per tile, converts code pairs to exact unscaled BF16
//    (cvt_scalef32_pk_bf16_fp4), dots them with x in FP32 (v_dot2_f32_bf16)
//    and multiplies each 16-block's partial sum by its scale once: about 1.3
//    vector instructions per weight at M = 1. The loads are range-checked
//    buffer loads issued unconditionally two batches ahead, so a wave waits
//    only for the batch it is about to use. The K-split is reduced inside the
//    workgroup (lane butterfly, then LDS over the waves in wave order), so no
//    workgroup ever waits on another and nothing crosses an XCD within the
//    kernel. x is staged once per workgroup in LDS and read by broadcast. (A K
//    split across workgroups would need an agent-scope release per workgroup,
//    an L2 write-back on this part, which measured several times slower.)
//  * 4 < M <= 64 (and M <= 4 when x does not fit in LDS): the skinny MFMA
//    kernel, the decode structure with v_mfma_f32_32x32x16_bf16 on one or two
//    32-row x tiles and one or two row groups per workgroup (below).
//  * M > 64: the big MFMA kernel, built like the W4A4 kernel (below), on
//    persistent workgroups over 256 x 256, 128 x 256 or 128 x 128 tiles. Output tiles that do not fill whole rounds of the
//    CUs, or are fewer than the CUs, are split along K: each split range writes
//    an FP32 partial tile to the workspace and a fix-up kernel adds the partials
//    in workgroup order and applies the epilogue, so the result does not depend
//    on scheduling.
#include "common.hpp"

#include <utility>

namespace nvfp4 {
namespace w4a16 {

constexpr int kThreads = 256;

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc16(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}
constexpr int kNonTemporal = 2;   // cache-policy bits of a streamed load

// ---------------------------------------------------------------- planning

struct Plan {
  int kind;          // 0 = vector decode kernel, 3 = skinny MFMA kernel, 4 = big MFMA kernel
  int dec;           // launch shape of the decode kernel (kDecodeShapes)
  int64_t grid_x;    // workgroups along the output
  int64_t nfull;     // decode: workgroups of R rows before the tail
  int tr;            // decode: rows per tail workgroup (0: no tail cut)
};

// Launch shapes of the vector decode kernel: R weight rows per workgroup, W
// waves, U tile loads per wave and ring batch.
struct DecodeShape {
  int R, W, U;
};
constexpr DecodeShape kDecodeShapes[] = {{32, 8, 2}, {32, 12, 2}};
constexpr int kDecodeWavesPerCu = 32;   // resident waves per CU at M = 1 (at most 64 registers)

constexpr int kDecodeMaxM = 4;          // the decode kernel's instantiations (explicit configs)
// The heuristic's decode range: from M = 3 the skinny row kernel is faster on
// the 27B-class layers (graph replays, M = 4: 34816 x 5120 31.6 -> 23.3 us,
// 6144 x 5120 8.7 -> 6.7 us; M = 2: decode 20.9 against 23.8 us).
constexpr int kDecodeDefaultMaxM = 2;
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnyDirectMaxM = 16;   // up to here the skinny kernel reads x rows directly
constexpr int kDecodeLdsBytes = 64 * 1024;  // x staged in LDS: M * K * 2 bytes at most

// Output tiles of the big kernel, as MFMA tiles per wave (TM x TN; the
// workgroup tile is 64 TM x 64 TN):
//  * 4 x 4 (256 x 256) when those fill the CUs, or when they are fewer but K
//    is long enough that splitting them over all CUs gives each at least
//    kBigSplitMinChunks 64-deep chunks and x's rows fill at least 7/8 of the
//    tile rows;
//  * else 128 x 256 when those fill the CUs or split that way, as 4 x 2 MFMA
//    tiles per wave with the 4 waves side by side along N (each wave
//    dequantizes W fragments for all four of its row tiles);
//  * else 128 x 128, as 4 x 1 MFMA tiles per wave with the 4 waves side by
//    side along N: each wave dequantizes one W fragment per step for four
//    MFMAs. (With 2 x 2 waves of 2 x 2 tiles, each W fragment was dequantized
//    by both waves of its column, nine vector instructions per MFMA against
//    five; the same bits, back to back on one box: M = 128 on 5120 x 5120
//    25.8 -> 24.4 us, 5120 x 17408 43.0 -> 39.0 us, M = 768 on 5120 x 5120
//    52.9 -> 46.2 us.)
// WGM is the number of waves along M (2 x 2 waves, or 1 x 4).
constexpr int64_t kBigSplitMinChunks = 32;
static void big_tile_shape(int64_t M, int64_t N, int64_t K, int cus, int &TM, int &TN, int &WGM) {
  const int64_t nch = K / 64;
  const int64_t tm4 = (M + 255) / 256, t44 = tm4 * ((N + 255) / 256);
  if (t44 >= cus || (t44 * nch >= kBigSplitMinChunks * cus && 8 * M >= 7 * 256 * tm4)) {
    TM = TN = 4;
    WGM = 2;
    return;
  }
  const int64_t t24 = ((M + 127) / 128) * ((N + 255) / 256);
  if (t24 >= cus || t24 * nch >= kBigSplitMinChunks * cus) {
    TM = 4;
    TN = 2;
    WGM = 1;
    return;
  }
  TM = 4;
  TN = 1;
  WGM = 1;
}

// One 32-row group per workgroup. Eight waves once there are two groups per
// CU; with fewer groups, twelve waves keep more loads in flight per CU (more
// waves or deeper rings, or 8- and 16-row workgroups over more CUs, measured
// slower on the 27B-class decode shapes).
static int decode_shape(int64_t N, int cus) { return N / 32 >= 2 * cus ? 0 : 1; }

// MFMA tiles per wave and waves along M of a TILES config's workgroup tile.
static void tiles_of(const nvfp4_config &c, int &TM, int &TN, int &WGM) {
  if (c.tile_m == 256) {
    TM = TN = 4;
    WGM = 2;
  } else if (c.tile_n == 256) {
    TM = 4;
    TN = 2;
    WGM = 1;
  } else {
    TM = 4;
    TN = 1;
    WGM = 1;
  }
}

static bool decode_fits(int64_t M, int64_t K) { return M <= kDecodeMaxM && M * K * 2 <= kDecodeLdsBytes; }

static Plan make_plan(int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  Plan p{};
  const int cus = c.num_cus;
  if (c.kernel == NVFP4_KERNEL_W4A16_DECODE) {
    p.kind = 0;
    p.dec = decode_shape(N, cus);
    const DecodeShape &sh = kDecodeShapes[p.dec];
    p.grid_x = p.nfull = N / sh.R;
    // Past at least one whole round of resident workgroups, the groups left
    // over are cut into 8- or 16-row workgroups when those still get a CU
    // each (M = 1 only: more rows take more registers and fewer workgroups
    // stay resident). Larger leftovers run faster uncut.
    if (p.dec == 0 && M == 1) {
      const int64_t round = (int64_t)cus * (kDecodeWavesPerCu / sh.W);
      const int64_t full = p.nfull / round * round, rem = p.nfull - full;
      const int tr = rem * 4 <= cus ? 8 : rem * 2 <= cus ? 16 : 0;
      if (full > 0 && rem > 0 && tr > 0) {
        p.tr = tr;
        p.grid_x = full + rem * (32 / tr);
        p.nfull = full;
      }
    }
  } else if (c.kernel == NVFP4_KERNEL_W4A16_SKINNY) {
    p.kind = 3;
    p.grid_x = N / 32;
  } else {
    p.kind = 4;
  }
  return p;
}

// The skinny kernel reads x from the workspace in MFMA fragment order:
// roundup32(M) rows x K BF16.
static size_t skinny_x_bytes(int64_t M, int64_t K) { return (size_t)((M + 31) / 32 * 32) * (size_t)K * 2; }

// Launch shape of the skinny kernels: W waves, NG row groups per workgroup,
// and RP > 0 (x rows padded to RP = 8, 16, 32 or 64) for the row kernel, which
// stages x rows through LDS, or RP = 0 for the fragment kernel, which reads a
// fragment-order copy of x from the workspace (or, for M <= 16, x directly).
// The row kernel needs no workspace: rows >= M read zero, or whatever bytes of
// x their 32-bit offsets wrap to (the buffer range ends with x's last
// element), and only feed output rows that are not stored; rows < M stay below
// the M ldx 2 bytes the dispatch bounds.
// Measured on the 27B-class layer shapes (graph replays, one box), fragment
// kernel with its copy -> row kernel:
//   M = 8:  6144 x 5120 9.6 -> 6.5 us, 5120 x 17408 22.7 -> 15.5 us, 34816 x 5120 31.2 -> 23.3 us;
//   M = 17: 13.0 -> 9.1 us, 30.5 -> 21.6 us, 36.1 -> 29.5 us;
//   M = 33: 17.7 -> 13.0 us, 44.2 -> 33.0 us, 50.9 -> 46.9 us.
// With two row groups per workgroup the RP = 64 kernel holds 190 registers
// (one workgroup per CU) and loses at M = 64 on 34816 x 5120 (55.4 against
// 52.0 us), so weights with at least as many row groups as CUs keep the
// fragment kernel above M = 48.
struct SkinnyShape {
  int W, NG, RP;
};
static SkinnyShape skinny_shape(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t groups = N / 32;
  int RP = M <= 8 ? 8 : M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 0;
  if (RP == 64 && groups >= cus && M > 48) RP = 0;
  if (K / 64 * 1024 > 0x7FFFFFFFll) RP = 0;   // the row kernel's 32-bit weight offsets
  if (groups < cus) return {RP == 64 ? 8 : 16, 1, RP};
  return {8, groups % 2 == 0 ? 2 : 1, RP};
}

// Schedule of the big kernel (tile shapes: big_tile_shape).
//  * 256 x 256 tiles (one workgroup per CU): G = CUs persistent workgroups
//    each run full / G whole tiles; the rem = total - full tiles left over are
//    split along K over all G workgroups. With fewer tiles than CUs, full = 0
//    and every tile is split that way (with x staged through LDS, this took
//    5120 x 17408 at M = 1024 from 311 us with 128 x 128 tiles to 262 us; with
//    x read straight into registers, a threshold of 32 rather than 48 chunks
//    per workgroup took 5120 x 17408 at M = 512 from 155 to 131 us, while 24
//    made 6144 x 5120 at M = 1024, 30 chunks each, slower: 113 against 100 us;
//    at M = 384, a quarter of the 256-row tiles empty, it was slower too).
//  * 128 x 256 tiles (one workgroup per CU; x read directly, or through LDS
//    when every tile is split into short ranges) follow the same rules. With
//    2 x 2 waves of 2 x 4 MFMA tiles, 34816 x 5120 at M = 128 took
//    84.5 us against 92.6 with 128 x 128 tiles, but both waves of a column
//    dequantized the same W fragments: nine vector instructions per MFMA, and
//    the counters showed the MFMA and vector work barely overlapping.
//  * 128 x 128 tiles (two workgroups per CU), at least as many as CUs: one
//    workgroup per tile up to two per CU, then whole rounds; a CU running two
//    workgroups loses little against one that runs one, and splitting these
//    tiles measured slower.
//  * Fewer 128 x 128 tiles than CUs: every tile is split along K into S equal
//    ranges, G = S x tiles workgroups. S = CUs / tiles (one workgroup per CU),
//    or 2 CUs / tiles when that is below 3; at most 8 and K / 1024 (short
//    ranges lose their prologue and fix-up to the split); no split below 3.
//    On the 27B-class layers a CU running two short ranges finished well after
//    the CUs running one, so the split keeps to one per CU where it can.
// Split ranges write FP32 partials (two slots per workgroup) that a fix-up
// kernel adds in workgroup order.
constexpr int kMaxKSplit = 8;
// 1024-element accumulator parts per fix-up workgroup: 2 for 128 x 128 tiles
// (twice the workgroups of 4 parts: M = 128 on 6144 x 5120 28.1 -> 27.0 us,
// 5120 x 17408 46.6 -> 45.3 us; 1 part was no better), else 4.
constexpr int fixup_parts(int TM, int TN) { return TM * TN == 4 ? 2 : 4; }
// How a tile kernel's x reaches the MFMAs (XP): a fragment-order copy of x
// that every wave reads into its own registers (kXDirect), or 128 rows staged
// once per workgroup through LDS and shared by its four waves (kXLds; kXLdsDeep
// with the deeper register rings of one workgroup per CU).
constexpr int kXDirect = 0, kXLds = 1, kXLdsDeep = 2;
// The 128 x 256 tiles' longest K range (chunks per workgroup) on the LDS path.
// Measured by graph replay on the 27B-class layers, all tiles split:
// 34816 x 5120 at M = 128 (42 chunks) 79.9 -> 72.7 us, 5120 x 17408 at M = 256
// (42) 80.5 -> 71.8 us, 5120 x 5120 at M = 1024 (50) 80.3 -> 78.0 us; with
// longer ranges or whole tiles the direct path's loop was faster than the copy
// it needs: 6144 x 5120 at M = 1024 (60) 89.3 against 89.9 us, 5120 x 17408 at
// M = 1024 (170) 187.8 against 192.3 us, 34816 x 5120 at M = 512 (whole tiles)
// 173 against 196 us.
constexpr int64_t kLdsMaxRange = 50;

struct BigSched {
  int TM, TN, WGM;   // MFMA tiles per wave; waves along M
  int64_t tiles_m, tiles_n, total, G, full, rem;
  int64_t tile_rows() const { return 32 * TM * WGM; }
  int64_t tile_cols() const { return 32 * TN * (4 / WGM); }
};

static BigSched big_sched(int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  BigSched b{};
  const int cus = c.num_cus;
  tiles_of(c, b.TM, b.TN, b.WGM);
  b.tiles_m = (M + b.tile_rows() - 1) / b.tile_rows();
  b.tiles_n = (N + b.tile_cols() - 1) / b.tile_cols();
  b.total = b.tiles_m * b.tiles_n;
  const bool direct = b.TM * b.TN >= 8;       // one workgroup per CU
  const int64_t slots = (int64_t)cus * (direct ? 1 : 2);
  if (direct) {
    b.G = slots;
    b.full = b.total / b.G * b.G;             // 0 when the tiles are fewer than the CUs
  } else if (b.total >= cus) {
    b.G = b.total < slots ? b.total : slots;
    b.full = b.total;
  } else {
    int64_t S = cus / b.total;                // one workgroup per CU ...
    if (S < 3) S = slots / b.total;            // ... else two
    if (S > kMaxKSplit) S = kMaxKSplit;
    if (S > K / 1024) S = K / 1024;            // at least 16 chunks per range
    if (S < 3) S = 1;                          // a two-way split measured slower than none
    b.G = S * b.total;
    b.full = S == 1 ? b.total : 0;
  }
  b.rem = b.total - b.full;
  return b;
}

// 4 waves x TM x TN MFMA tiles x 64 lanes x 16 FP32
static size_t big_partial_bytes(const BigSched &b) { return (size_t)b.TM * b.TN * 16384; }

// The big kernel's workspace: the split ranges' partial tiles (2 per
// workgroup, when tiles are split), then, for the tiles that read x directly,
// x in fragment order over whole output tiles of rows (xmt 32-row tiles).
static size_t big_partials_span(const BigSched &b) {
  return b.rem > 0 ? ((size_t)b.G * 2 * big_partial_bytes(b) + 255) / 256 * 256 : 0;
}
// The x path of a schedule: 128 x 128 tiles always stage x through LDS (deep
// rings when the grid holds one workgroup per CU); 128 x 256 tiles do when
// every tile is split and the ranges are short; 256 x 256 tiles never.
// (256 x 256 tiles on the LDS path, with 256 rows of x per chunk, measured
// slower on whole tiles: 34816 x 5120 at M = 1024 325 -> 384 us.)
static int big_xpath(const BigSched &b, int64_t K, int cus) {
  if (b.TM * b.TN < 8) return b.G <= cus ? kXLdsDeep : kXLds;
  if (b.TM * b.TN == 8 && b.full == 0 && b.rem * (K / 64) <= kLdsMaxRange * b.G) return kXLdsDeep;
  return kXDirect;
}
static int64_t big_xmt(const BigSched &b, int64_t K, int cus) {
  return big_xpath(b, K, cus) == kXDirect ? b.tiles_m * b.tile_rows() / 32 : 0;
}
static size_t big_xf_bytes(const BigSched &b, int64_t K, int cus) {
  return (size_t)big_xmt(b, K, cus) * 32 * (size_t)K * 2;
}

static size_t workspace_for(const Plan &p, const nvfp4_config &c, int64_t M, int64_t N, int64_t K) {
  if (p.kind == 3)
    return M > kSkinnyDirectMaxM && skinny_shape(M, N, K, c.num_cus).RP == 0 ? skinny_x_bytes(M, K) : 0;
  if (p.kind == 4) {
    const BigSched b = big_sched(M, N, K, c);
    return big_partials_span(b) + big_xf_bytes(b, K, c.num_cus);
  }
  return 0;
}

// ---------------------------------------------------------------- decode kernel (M <= 4)

// Workgroup b owns the R weight rows R (b % (32/R)) + [0, R) of the 32-row
// prepared tile group b / (32/R), over the whole K, with W waves. A wave load
// covers 32/R consecutive tiles: lane l takes tile l / 2R of them, K-half
// h = (l / R) & 1 and row r = l % R, i.e. unit 32 h + row of the tile, so the
// load reads 2 (32/R) contiguous runs of 16 R bytes (one 1 KB run for R = 32).
// Wave w takes the tile groups w, w + W, w + 2W, ...; the loads run U groups
// per wave ahead in a two-batch register ring (non-temporal: the weights are
// streamed once), and the first batch is issued between x's first loads and
// their stores into LDS. Per 16-element
// block the BF16 products go through fdot2 into an FP32 partial that is scaled
// once; the row's lanes are added by a butterfly (the same bits in every lane)
// and the waves in wave order through LDS.
template <int M, int R, int W, int U>
__device__ __forceinline__ void decode_rows(int64_t b, uint16_t *xs, const uint16_t *__restrict__ x, int64_t ldx,
                                            const uint8_t *__restrict__ wp, int64_t N, int64_t K, float alpha,
                                            const float *alpha_dev, const float *alpha_col, uint16_t *__restrict__ y, int64_t ldy) {
  constexpr int TPL = 32 / R;                       // tiles per wave load
  __shared__ float red[W][M][R];
  const int64_t T = K / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tl = lane / (2 * R), h = (lane / R) & 1, r = lane % R;
  const int64_t g = b / TPL;
  const int row0 = (int)(b % TPL) * R;               // first row of the workgroup inside the group
  // Every load is unconditional: the resource of tile group j0 + i W starts at
  // its first tile and ends at the last tile of the row group, so the lanes
  // past it read zeros, and the waits before a compute step can leave the
  // next batch in flight.
  const uint8_t *cbase = wp + ((g * T) << 10);
  const uint8_t *sbase = wp + N * K / 2 + ((g * T) << 7);
  const uint32_t oc = 16u * (32 * h + row0 + r) + ((uint32_t)tl << 10), os = 4u * (row0 + r) + ((uint32_t)tl << 7);
  const int64_t groups = (T + TPL - 1) / TPL;
  u32x4_t cw0[U], cw1[U];
  uint32_t sw0[U], sw1[U];
  auto issue = [&](u32x4_t (&cw)[U], uint32_t (&sw)[U], int64_t j0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t tu = (j0 + (int64_t)i * W) * TPL, rem = T - tu;
      const __amdgpu_buffer_rsrc_t rc = make_rsrc16(cbase + (tu << 10), rem > 0 ? rem << 10 : 0);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc16(sbase + (tu << 7), rem > 0 ? rem << 7 : 0);
      cw[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, kNonTemporal);
      sw[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, kNonTemporal);
    }
  };
  // x: the first kXEarly 16-byte units per thread are requested before the first
  // weight batch (unconditionally: threads past the end read x's first unit and
  // drop it), so staging them waits for x alone; any rest after it.
  constexpr int kXEarly = 2;
  const int64_t nx = (int64_t)M * K / 8;
  u32x4_t xe[kXEarly];
#pragma unroll
  for (int i = 0; i < kXEarly; i++) {
    const int64_t u = threadIdx.x + (int64_t)i * W * 64;
    const int64_t m = u / (K / 8), c = u - m * (K / 8);
    xe[i] = *reinterpret_cast<const u32x4_t *>(u < nx ? x + m * ldx + c * 8 : x);
  }
  issue(cw0, sw0, wave);
#pragma unroll
  for (int i = 0; i < kXEarly; i++) {
    const int64_t u = threadIdx.x + (int64_t)i * W * 64;
    const int64_t m = u / (K / 8), c = u - m * (K / 8);
    if (u < nx) *reinterpret_cast<u32x4_t *>(xs + m * K + c * 8) = xe[i];
  }
  for (int64_t u = threadIdx.x + (int64_t)kXEarly * W * 64; u < nx; u += W * 64) {
    const int64_t m = u / (K / 8), c = u - m * (K / 8);
    *reinterpret_cast<u32x4_t *>(xs + m * K + c * 8) = *reinterpret_cast<const u32x4_t *>(x + m * ldx + c * 8);
  }
  __syncthreads();

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; m++) acc[m] = 0.0f;
  auto compute = [&](const u32x4_t (&cw)[U], const uint32_t (&sw)[U], int64_t j0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = (j0 + (int64_t)i * W) * TPL + tl;
      if (t >= T) continue;
      const f32x2_t sc = e4m3x2_to_f32(sw[i] >> (16 * h));
      const uint16_t *xk = xs + t * 64 + 32 * h;
#pragma unroll
      for (int blk = 0; blk < 2; blk++) {
        float part[M];
#pragma unroll
        for (int m = 0; m < M; m++) part[m] = 0.0f;
#pragma unroll
        for (int d = 0; d < 2; d++) {
          const int st = blk * 2 + d;
          bf16x2_t wv[4];
          codes8_to_bf16(cw[i][st], wv);
#pragma unroll
          for (int m = 0; m < M; m++) {
            const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xk + m * K + 8 * st);
#pragma unroll
            for (int e = 0; e < 4; e++)
              part[m] = __builtin_amdgcn_fdot2_f32_bf16(wv[e], as_bf16x2(xv[e]), part[m], false);
          }
        }
#pragma unroll
        for (int m = 0; m < M; m++) acc[m] = __builtin_fmaf(part[m], sc[blk], acc[m]);
      }
    }
  };
  const int64_t step = (int64_t)W * U;
  for (int64_t j0 = wave; j0 < groups; j0 += 2 * step) {
    issue(cw1, sw1, j0 + step);
    compute(cw0, sw0, j0);
    if (j0 + step >= groups) break;
    issue(cw0, sw0, j0 + 2 * step);
    compute(cw1, sw1, j0 + step);
  }
  // lanes r + R j (j < 64 / R) hold the (tile, half) streams of row r
#pragma unroll
  for (int m = 0; m < M; m++)
#pragma unroll
    for (int off = R; off < 64; off <<= 1) acc[m] += __shfl_xor(acc[m], off, 64);
  if (lane < R)
#pragma unroll
    for (int m = 0; m < M; m++) red[wave][m][r] = acc[m];
  __syncthreads();
  if (threadIdx.x < M * R) {
    const int m = threadIdx.x / R, rr = threadIdx.x % R;
    float v = red[0][m][rr];
#pragma unroll
    for (int w = 1; w < W; w++) v += red[w][m][rr];
    const float al = load_alpha(alpha, alpha_dev);
    const int64_t n = g * 32 + row0 + rr;
    y[m * ldy + n] = f32_to_bf16_rne(col_alpha(al, alpha_col, n) * v);
  }
}

// The decode launch: workgroups below nfull own R rows each (decode_rows
// above). With TR > 0 the row groups past nfull are cut into TR-row
// workgroups: nfull covers whole rounds of resident workgroups, and the groups
// left over would otherwise run alone at the end, one workgroup each on a
// fraction of the CUs, at the rate one workgroup's loads in flight allow.
// Cut finer, they spread over more CUs and finish sooner (34816 x 5120 at
// M = 1, 1088 groups for 1024 resident workgroups: 19.5 against 18.5 us).
template <int M, int R, int W, int U, int TR>
__global__ __launch_bounds__(W * 64) void decode_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                        const uint8_t *__restrict__ wp, int64_t N, int64_t K,
                                                        float alpha, const float *alpha_dev, const float *alpha_col,
                                                        uint16_t *__restrict__ y, int64_t ldy, int64_t nfull) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];     // [M][K]
  const int64_t b = blockIdx.x;
  if constexpr (TR == 0) {
    decode_rows<M, R, W, U>(b, xs, x, ldx, wp, N, K, alpha, alpha_dev, alpha_col, y, ldy);
  } else {
    if (b < nfull)
      decode_rows<M, R, W, U>(b, xs, x, ldx, wp, N, K, alpha, alpha_dev, alpha_col, y, ldy);
    else
      decode_rows<M, TR, W, U>(nfull * (R / TR) + (b - nfull), xs, x, ldx, wp, N, K, alpha, alpha_dev, alpha_col, y, ldy);
  }
}

// ---------------------------------------------------------------- skinny MFMA kernel (4 < M <= 64)

// Workgroup b covers the NG 32-row prepared tile groups NG b .. NG b + NG - 1
// over the whole K with W waves; wave w takes the tiles w, w + W, ... as in the
// decode kernel. Per tile, group g and MFMA step s (k = 32h + 8s + i, the same
// K order as the prepared weight units), lane l dequantizes its 8 codes of
// weight row 32g + (l & 31)
// exactly to BF16 (E2M1 -> FP32, times the E4M3 scale, -> BF16) as the B
// operand and loads the matching 8 BF16 of x rows 32 mt + (l & 31) as the A
// operand of v_mfma_f32_32x32x16_bf16 (MT 32-row x tiles). For M > 16 (XF) x is
// first copied into the workspace in fragment order (tile t, step s, x tile mt:
// 64 lanes x 16 bytes, rows >= M zero), so each fragment load is one contiguous
// 1 KB instead of 32 scattered rows; for M <= 16 the scattered direct reads
// cost less than the copy (rows >= M read as zero through the buffer range
// check). Weights and x fragments are loaded one tile per wave ahead (a
// two-tile register ring): the x fragments cost 16 MT registers per tile, and
// deeper rings lowered the occupancy enough to measure slower. Each wave ends
// with NG full 32 x 32 MT partial tiles; they are added in wave order through
// LDS, one output tile at a time (a fixed tree of 4 levels with 8 barriers
// cost ~1 us more per call). W = 8 waves, or 16 when there are fewer row
// groups than CUs (more loads in flight on each busy CU; measured 17 % faster
// at M = 8 on 5120 x 17408, slower on 34816 x 5120). This fragment kernel
// serves 48 < M <= 64 on weights with at least as many row groups as CUs, and
// otherwise only K beyond the row kernel's 32-bit weight offsets.
constexpr int kSkAhead = 1;   // tiles per wave and ring batch

// Register-ring stages of the row kernel (deeper rings measured slower).
constexpr int kSkinnyRowsDepth = 2;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  bf16x8_t b;
  __builtin_memcpy(&b, &v, 16);
  return b;
}

// x [M][ldx] BF16 -> fragment order: unit u = ((t * 4 + s) * MT + mt) * 64 + lane
// holds x[32 mt + (lane & 31)][64 t + 32 (lane >> 5) + 8 s .. +8] (zero past M).
// Workgroup (t, mt) moves the 32 rows x 64 k block: thread q reads 16 bytes
// of row q / 8 (eight threads per 128-byte row piece) and writes them to
// their unit.
__global__ __launch_bounds__(256) void tile_x_kernel(const uint16_t *__restrict__ x, int64_t ldx, int64_t M,
                                                     int64_t K, int MT, u32x4_t *__restrict__ xf) {
  const int64_t t = blockIdx.x / MT;
  const int mt = (int)(blockIdx.x - t * MT);
  const int q = threadIdx.x, r = q >> 3, piece = q & 7;    // piece = 4 h + s
  const int64_t row = 32 * (int64_t)mt + r;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < M) v = *reinterpret_cast<const u32x4_t *>(x + row * ldx + t * 64 + piece * 8);
  const int h = piece >> 2, s = piece & 3;
  xf[((t * 4 + s) * MT + mt) * 64 + 32 * h + r] = v;
}

template <int MT, bool XF, int W, int NG>
__global__ __launch_bounds__(W * 64) void skinny_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                             const uint8_t *__restrict__ wp, int64_t M, int64_t N,
                                                             int64_t K, float alpha, const float *alpha_dev, const float *alpha_col,
                                                             uint16_t *__restrict__ y, int64_t ldy,
                                                             const uint8_t *__restrict__ xf) {
  constexpr int U = kSkAhead;                          // tiles per wave per batch
  __shared__ float red[W * 16 * 64];                   // one output tile of every wave
  const int64_t T = K / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const int64_t g0 = (int64_t)blockIdx.x * NG;         // the workgroup's first row group
  const uint8_t *cb = wp + ((g0 * T) << 10) + lane * 16;
  const uint8_t *sb = wp + N * K / 2 + ((g0 * T) << 7) + r * 4;
  const uint8_t *xl = XF ? xf + lane * 16 : nullptr;   // this lane's unit of every x fragment
  // x's buffer ends with row M - 1's last element, so an offset of a row >= M
  // that wraps in 32 bits reads x's own bytes or zero, never past the allocation
  const __amdgpu_buffer_rsrc_t rx = make_rsrc16(x, XF ? 0 : ((M - 1) * ldx + K) * 2);
  uint32_t xo[MT];                                 // direct reads: byte offset of this lane's x row, k = 32h
#pragma unroll
  for (int mt = 0; mt < MT; mt++) xo[mt] = (uint32_t)(((int64_t)(32 * mt + r) * ldx + 32 * h) * 2);

  struct Batch {
    u32x4_t cw[U][NG];
    uint32_t sw[U][NG];
    u32x4_t xv[U][MT][4];
  };
  auto issue = [&](Batch &b, int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      const int64_t t = t0 + (int64_t)i * W;
      const bool in = t < T;
      const int64_t tc = in ? t : 0;
#pragma unroll
      for (int q = 0; q < NG; q++) {
        b.cw[i][q] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(cb + ((q * T + tc) << 10)))
                        : u32x4_t{0u, 0u, 0u, 0u};
        b.sw[i][q] =
            in ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + ((q * T + tc) << 7))) : 0u;
      }
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int s = 0; s < 4; s++)
          b.xv[i][mt][s] = XF ? *reinterpret_cast<const u32x4_t *>(xl + (((tc * 4 + s) * MT + mt) << 10))
                              : __builtin_amdgcn_raw_buffer_load_b128(rx, xo[mt] + (uint32_t)(tc * 128 + 16 * s), 0, 0);
    }
  };
  f32x16_t acc[NG][MT];
#pragma unroll
  for (int q = 0; q < NG; q++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[q][mt] = f32x16_t{};
  auto compute = [&](const Batch &b, int64_t t0) {
#pragma unroll
    for (int i = 0; i < U; i++) {
      if (t0 + (int64_t)i * W < T) {
#pragma unroll
        for (int q = 0; q < NG; q++) {
          const f32x2_t sc = e4m3x2_to_f32(b.sw[i][q] >> (16 * h));
#pragma unroll
          for (int s = 0; s < 4; s++) {
            const bf16x8_t bv = dequant8_bf16(b.cw[i][q][s], sc[s >> 1]);
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
              acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(b.xv[i][mt][s]), bv, acc[q][mt], 0, 0, 0);
          }
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
  // per output tile: every wave's partial tile to LDS (element j of lane l at
  // (wave * 16 + j) * 64 + l, so each store and load of a wave is one
  // contiguous 256 bytes), then every thread adds its elements over the waves
  // in wave order
  const float al = load_alpha(alpha, alpha_dev);
#pragma unroll
  for (int q = 0; q < NG; q++) {
    const int64_t n = (g0 + q) * 32 + r;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 16; j++) red[(wave * 16 + j) * 64 + lane] = acc[q][mt][j];
      __syncthreads();
#pragma unroll
      for (int e = wave; e < 16; e += W) {   // e: the accumulator element this wave adds up
        const int64_t m = 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < W; w++) v += red[(w * 16 + e) * 64 + lane];
        if (m < M) y[m * ldy + n] = f32_to_bf16_rne(col_alpha(al, alpha_col, n) * v);
      }
    }
  }
}

// The skinny contraction for M <= RP <= 64 without barriers in the main loop:
// wave w takes the tiles w, w + W, ... through a D-deep register ring, as the
// direct skinny kernel does, and stages each tile's x (RP rows x 64 columns,
// RP / 8 coalesced 16-byte loads per lane) through a private LDS slot: the
// wave writes the tile into its slot in fragment order and reads its
// fragments back (LDS operations of one wave complete in order, so no barrier
// is needed, and the next tile's write cannot pass the reads). The texture
// path then moves the RP real rows of x (1 KB per tile for RP = 8) instead of
// 32 rows of fragments, and no copy of x is made. The slot's 16-byte units
// are XOR-swizzled within each run of 8 rows, so the stores of one row's
// 128 bytes and the loads of a fragment each hit 8 distinct bank groups.
// Dequantization, RP <= 16: one MFMA per 16-element scale block (a lane-half
// swap of the code dwords gives every lane block b's 8 codes for its half),
// with the power of two of the block scale folded into the conversion (exact)
// and its mantissa (frexp, in [0.5, 1)) applied to that block's MFMA result in
// the rows < RP; the factor 2 is applied at the end. RP = 32 and 64: the
// codes are dequantized exactly to BF16 (E2M1 -> FP32, times the scale) and
// the MFMAs of the RP / 32 x tiles accumulate, as in the fragment kernel (16
// per-block multiplies for 32 rows outweigh the saved conversions).
template <int W, int NG, int RP, int D>
__global__ __launch_bounds__(W * 64) void skinny_rows_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                                  const uint8_t *__restrict__ wp, int64_t M, int64_t N,
                                                                  int64_t K, float alpha, const float *alpha_dev,
                                                                  const float *alpha_col, uint16_t *__restrict__ y,
                                                                  int64_t ldy) {
  constexpr bool FULL = RP >= 32;             // full dequantization, MFMAs accumulate
  constexpr int MTR = FULL ? RP / 32 : 1;     // 32-row x tiles
  constexpr int JR = FULL ? 16 : RP / 2;      // accumulator registers per x tile holding rows < RP
  constexpr int SLOT = RP * 128;              // a tile's x fragments: 4 blocks x 2 halves x RP rows x 16 B
  constexpr int PPL = RP / 8;                 // 16-byte x pieces per lane and tile
  constexpr int LDS_F = W * SLOT / 4;         // the x slots, then one row group's partial tiles (JR * 64 floats per wave)
  __shared__ __attribute__((aligned(16))) float lds[LDS_F];
  const int64_t T = K / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  const int64_t g0 = (int64_t)blockIdx.x * NG;
  const uint8_t *cb = wp + ((g0 * T) << 10);
  const uint8_t *sb = wp + N * K / 2 + ((g0 * T) << 7);
  const uint32_t oc = (uint32_t)lane * 16u, os = (uint32_t)r * 4u;
  // one resource per row group and kind, ending at the group's last tile: the
  // offsets of tiles past it fall outside the range and read zero
  __amdgpu_buffer_rsrc_t rc[NG], rs[NG];
#pragma unroll
  for (int q = 0; q < NG; q++) {
    rc[q] = make_rsrc16(cb + ((q * T) << 10), T << 10);
    rs[q] = make_rsrc16(sb + ((q * T) << 7), T << 7);
  }
  // rows >= M read zero, or (an offset wrapped in 32 bits) some of x's own
  // bytes: the buffer ends with row M - 1's last element
  const __amdgpu_buffer_rsrc_t rx = make_rsrc16(x, ((M - 1) * ldx + K) * 2);
  uint8_t *slot = reinterpret_cast<uint8_t *>(lds) + wave * SLOT;
  // Lane piece: row m, 8 columns 8 pc of the tile, pc = 2 b + hh for 16-block b
  // and k-half hh; in fragment order it is unit (b, hh, m). Within each group
  // of 8 units (8 rows of one b, hh) the unit index is XORed with pc, so the 8
  // lanes that write one row's 128 bytes, and the 8 lanes that read a fragment,
  // hit 8 distinct 16-byte bank groups (unswizzled, the writes conflicted ~10
  // cycles per LDS instruction).
  uint32_t xgo[PPL], xlo[PPL];
#pragma unroll
  for (int i = 0; i < PPL; i++) {
    const int m = 8 * i + (lane >> 3), pc = lane & 7;   // row, 8-column piece of the tile
    xgo[i] = (uint32_t)(((int64_t)m * ldx + 8 * pc) * 2);
    xlo[i] = (uint32_t)((pc >> 1) * (2 * RP * 16) + ((pc & 1) * RP + (m ^ pc)) * 16);
  }
  uint32_t frag[MTR][4];
#pragma unroll
  for (int mt = 0; mt < MTR; mt++)
#pragma unroll
    for (int b = 0; b < 4; b++) {
      if constexpr (FULL) {   // step s = b: k = 32 h + 8 s, unit (2 h + s / 2, s % 2, 32 mt + r)
        frag[mt][b] =
            (uint32_t)(((2 * h + (b >> 1)) * 2 * RP + (b & 1) * RP + ((32 * mt + r) ^ (4 * h + b))) * 16);
      } else {
        frag[mt][b] = (uint32_t)((b * 2 * RP + h * RP + ((r & (RP - 1)) ^ (2 * b + h))) * 16);
      }
    }
  struct Stage {
    u32x4_t cw[NG];
    uint32_t sw[NG];
    u32x4_t xg[PPL];
  };
  auto issue = [&](Stage &st, int64_t t) {
    const uint32_t tc = t < T ? (uint32_t)t : (uint32_t)T;   // T: the first offset past the range
#pragma unroll
    for (int q = 0; q < NG; q++) {
      st.cw[q] = __builtin_amdgcn_raw_buffer_load_b128(rc[q], oc + (tc << 10), 0, kNonTemporal);
      st.sw[q] = __builtin_amdgcn_raw_buffer_load_b32(rs[q], os + (tc << 7), 0, kNonTemporal);
    }
    const uint32_t xt = (uint32_t)((t < T ? t : T - 1) * 128);
#pragma unroll
    for (int i = 0; i < PPL; i++) st.xg[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, xgo[i] + xt, 0, 0);
  };
  f32x16_t acc[NG][MTR];
#pragma unroll
  for (int q = 0; q < NG; q++)
#pragma unroll
    for (int mt = 0; mt < MTR; mt++) acc[q][mt] = f32x16_t{};
  auto compute = [&](const Stage &st) {
#pragma unroll
    for (int i = 0; i < PPL; i++) *reinterpret_cast<u32x4_t *>(slot + xlo[i]) = st.xg[i];
    u32x4_t xv[MTR][4];
#pragma unroll
    for (int mt = 0; mt < MTR; mt++)
#pragma unroll
      for (int b = 0; b < 4; b++) xv[mt][b] = *reinterpret_cast<const u32x4_t *>(slot + frag[mt][b]);
    if constexpr (FULL) {
#pragma unroll
      for (int q = 0; q < NG; q++) {
        const f32x2_t sc = e4m3x2_to_f32(st.sw[q] >> (16 * h));
#pragma unroll
        for (int s = 0; s < 4; s++) {
          const bf16x8_t bv = dequant8_bf16(st.cw[q][s], sc[s >> 1]);
#pragma unroll
          for (int mt = 0; mt < MTR; mt++)
            acc[q][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xv[mt][s]), bv, acc[q][mt], 0, 0, 0);
        }
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < NG; q++) {
      const f32x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st.sw[q], 1.0f, false);
      const f32x2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(st.sw[q], 1.0f, true);
      const float sc[4] = {s01[0], s01[1], s23[0], s23[1]};
      const auto p02 = __builtin_amdgcn_permlane32_swap(st.cw[q][0], st.cw[q][1], false, false);
      const auto p13 = __builtin_amdgcn_permlane32_swap(st.cw[q][2], st.cw[q][3], false, false);
      const uint32_t bw[4] = {p02[0], p13[0], p02[1], p13[1]};
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const bf16x2_t w2[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[b], sc[b], 0),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[b], sc[b], 1),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[b], sc[b], 2),
                                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(bw[b], sc[b], 3)};
        bf16x8_t bv;
        __builtin_memcpy(&bv, w2, 16);
        const f32x16_t rb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xv[0][b]), bv, f32x16_t{}, 0, 0, 0);
        const float mb = __builtin_amdgcn_frexp_mantf(sc[b]);
#pragma unroll
        for (int jj = 0; jj < JR; jj++) acc[q][0][jj] = __builtin_fmaf(mb, rb[jj], acc[q][0][jj]);
      }
    }
  };
  Stage stg[D];
#pragma unroll
  for (int d = 0; d < D; d++) issue(stg[d], wave + (int64_t)d * W);
  const int64_t nt = wave < T ? (T - wave + W - 1) / W : 0;   // this wave's tiles
  int64_t i = 0;
  for (; i + D <= nt; i += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      compute(stg[d]);
      __builtin_amdgcn_sched_barrier(0);
      issue(stg[d], wave + (i + d + D) * W);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D - 1; d++)
    if (i + d < nt) compute(stg[d]);
  // per row group and x tile: the waves' partial tiles (rows < RP) to LDS,
  // then every thread adds its elements over the waves in order
  const float al = load_alpha(alpha, alpha_dev);
#pragma unroll
  for (int q = 0; q < NG; q++)
#pragma unroll
    for (int mt = 0; mt < MTR; mt++) {
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < JR; jj++) lds[(wave * JR + jj) * 64 + lane] = acc[q][mt][jj];
      __syncthreads();
      for (int e = threadIdx.x; e < JR * 64; e += W * 64) {
        const int jj = e / 64, l = e % 64;
        const int64_t m = 32 * mt + 8 * (jj >> 2) + 4 * (l >> 5) + (jj & 3);
        if (m >= M) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < W; w++) v += lds[(w * JR + jj) * 64 + l];
        const int64_t n = (g0 + q) * 32 + (l & 31);
        // 2: the frexp mantissas lie in [0.5, 1)
        y[m * ldy + n] = f32_to_bf16_rne(col_alpha(al, alpha_col, n) * (FULL ? v : 2.0f * v));
      }
    }
}

// ---------------------------------------------------------------- big MFMA kernel (M > 64)

// The W4A4 kernel's structure with x in BF16. Persistent workgroups of 4 waves
// over 32 TM WGM x 32 TN (4 / WGM) output tiles, each wave owning TM x TN
// v_mfma_f32_32x32x16_bf16 tiles: 256 x 256 (TM = TN = 4, 2 x 2 waves) and
// 128 x 256 (TM = 4, TN = 2, 1 x 4 waves), one workgroup per CU, read x in
// fragment order straight into registers (tile_mainloop_d); 128 x 128 (4 x 1
// tiles, 1 x 4 waves, up to two workgroups per CU) stages x through LDS
// (tile_mainloop), and so do 128 x 256 tiles that are all split into short K
// ranges (big_xpath).
//  * W: each wave loads its TN column groups' fragments of a 64-wide K chunk
//    straight into registers (one contiguous 1 KB each plus a scale word), two
//    chunks ahead in a three-deep ring, and dequantizes them exactly to BF16
//    (E2M1 -> FP32, times the E4M3 scale, -> BF16) one MFMA step ahead.
//  * x through LDS: the tile's 128 rows x 64 k BF16 (16 KB) are loaded one chunk (or kDeepX chunks) ahead with
//    coalesced 16-byte loads (rows past M read as zero through the buffer range
//    check), written into one of two LDS buffers and read back as MFMA
//    fragments. The 16-byte units of a row are XOR-swizzled by row / 2: an LDS
//    cycle serves 16 lanes of a 16-byte read (16 consecutive rows of one unit),
//    and with 128-byte rows on 64 four-byte banks a swizzle by row alone put
//    rows r and r + 8 on the same banks (the bank-conflict counter read as many
//    cycles as the LDS instructions took; now zero). One LDS-only barrier per
//    chunk; the x loads are issued before the W loads (kept in that order by a
//    scheduling barrier: loads complete in order, so waiting for x before its
//    LDS store leaves the W prefetch in flight).
//  * One scheduling region per MFMA step, as in the W4A4 kernel.
namespace big {

constexpr int kThreads = 256;
constexpr int kGroupM = 8;
// Ring depths of the 128 x 128 LDS path when the grid holds one workgroup per
// CU: W loaded kDeepW - 1 chunks ahead, x kDeepX chunks ahead (3 and 1 with
// two workgroups per CU, whose registers must fit twice). Measured at M = 128
// (graph replays, one box): 6144 x 5120 28.6 -> 28.0 us, 5120 x 17408
// 46.3 -> 45.4 us, and 6144 x 5120 at M = 512 55.3 -> 53.4 us; (6, 3), (4, 2)
// and (8, 3) were no better.
constexpr int kDeepW = 6;
constexpr int kDeepX = 2;

struct Params {
  const uint16_t *x;
  int64_t ldx;
  const uint8_t *wp;
  uint16_t *y;
  int64_t ldy, M, N, K;
  float alpha;
  const float *alpha_dev;
  const float *alpha_col;  // per-column scale [N] or null
  int tiles_m, tiles_n;
  int full;          // tiles [0, full) run whole, persistent over gridDim.x workgroups
  int rem;           // tiles [full, full + rem) are split along K over all workgroups
  float *partials;   // 2 slots per workgroup of partial tiles (rem > 0)
  const uint8_t *xf; // x in MFMA fragment order (tile_x_kernel with xmt row tiles)
  int xmt;           // 32-row tiles of xf: M rounded up to whole output tiles
};

// One partial tile: 4 waves x TM x TN MFMA tiles x 64 lanes x 16 FP32, in the
// accumulator layout.
template <int TM, int TN>
constexpr int64_t partial_floats() {
  return (int64_t)4 * TM * TN * 64 * 16;
}

// Chunk range [s, e) of workgroup `pid` in the split part: the rem x nch
// (tile, chunk) units cut into G contiguous, nearly equal ranges. As rem < G,
// a range is shorter than one tile and touches at most two.
__device__ __forceinline__ void split_range(int64_t pid, int64_t G, int64_t units, int64_t &s, int64_t &e) {
  s = pid * units / G;
  e = (pid + 1) * units / G;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)n, 0x00020000);
}

template <int T>
struct WFrags {
  u32x4_t w[T];
  uint32_t ws[T];
};

template <int T>
struct XRegs {
  u32x4_t v[2 * T];
};

struct TileBase {
  const uint8_t *x, *w, *ws;
  int64_t x_bytes, w_bytes, ws_bytes;
};

template <int T>
__device__ __forceinline__ void load_w(const TileBase &tb, const uint32_t (&ow)[T], const uint32_t (&ows)[T],
                                       int64_t c, int64_t nch, WFrags<T> &f) {
  const bool in = c < nch;
  const __amdgpu_buffer_rsrc_t rw = rsrc(tb.w, in ? tb.w_bytes : 0);
  const __amdgpu_buffer_rsrc_t rs = rsrc(tb.ws, in ? tb.ws_bytes : 0);
#pragma unroll
  for (int j = 0; j < T; j++) f.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, ow[j], (int)(c * 1024), 0);
#pragma unroll
  for (int j = 0; j < T; j++) f.ws[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, ows[j], (int)(c * 128), 0);
}

// x chunk c of the tile: thread t loads units q = t + 256 i (row q >> 3, unit q & 7).
template <int T>
__device__ __forceinline__ void load_x(const TileBase &tb, int64_t ldx, int64_t c, int64_t nch, XRegs<T> &xr) {
  const __amdgpu_buffer_rsrc_t rx = rsrc(tb.x, c < nch ? tb.x_bytes : 0);
#pragma unroll
  for (int i = 0; i < 2 * T; i++) {
    const int q = (int)threadIdx.x + kThreads * i;
    const uint32_t off = (uint32_t)(((int64_t)(q >> 3) * ldx + c * 64 + (q & 7) * 8) * 2);
    xr.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
  }
}

template <int T>
__device__ __forceinline__ void store_x(uint8_t *buf, const XRegs<T> &xr) {
#pragma unroll
  for (int i = 0; i < 2 * T; i++) {
    const int q = (int)threadIdx.x + kThreads * i;
    const int row = q >> 3, u = q & 7;
    *reinterpret_cast<u32x4_t *>(buf + row * 128 + ((u ^ ((row >> 1) & 7)) << 4)) = xr.v[i];
  }
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// x fragments of MFMA step s from LDS: k = 32h + 8s .. +7 of row wm*32T + 32i + r.
template <int T>
__device__ __forceinline__ void read_x(const uint8_t *buf, int s, int wm, bf16x8_t (&a)[T]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int u = 4 * h + s;
#pragma unroll
  for (int i = 0; i < T; i++) {
    const int row = wm * 32 * T + 32 * i + r;
    a[i] = *reinterpret_cast<const bf16x8_t *>(buf + row * 128 + ((u ^ ((row >> 1) & 7)) << 4));
  }
}

// W fragments of MFMA step s, dequantized from dword s.
template <int T>
__device__ __forceinline__ void deq_w(const WFrags<T> &f, const f32x2_t (&sc)[T], int s, bf16x8_t (&b)[T]) {
#pragma unroll
  for (int j = 0; j < T; j++) b[j] = dequant8_bf16(f.w[j][s], sc[j][s >> 1]);
}

template <int T>
__device__ __forceinline__ void scales_of(const WFrags<T> &f, f32x2_t (&sc)[T]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int j = 0; j < T; j++) sc[j] = e4m3x2_to_f32(f.ws[j] >> (16 * h));
}

// One chunk c, at phase P of the rings: W goes through a DW-chunk register
// ring (f[c % DW] holds chunk c's fragments, loaded DW - 1 chunks ahead) and x
// through an XA-chunk register ring (xr[c % XA] receives chunk c + XA, loaded
// XA chunks ahead) into LDS buffer c & 1 at the end of chunk c - 1. On entry
// (a, b) are step 0's operands and sc chunk c's scales; on exit, chunk
// c + 1's.
template <int P, int TM, int TN, int XT, int DW, int XA>
__device__ __forceinline__ void chunk(const TileBase &tb, int64_t ldx, const uint32_t (&ow)[TN],
                                      const uint32_t (&ows)[TN], int64_t c, int64_t nch, WFrags<TN> (&f)[DW],
                                      XRegs<XT> (&xr)[XA], f32x2_t (&sc)[TN], uint8_t *smem, int wm,
                                      bf16x8_t (&a)[TM], bf16x8_t (&b)[TN], f32x16_t (&acc)[TM][TN]) {
  constexpr int kValu = 16 / TM + 1;                // dequant instructions per MFMA, rounded up
  constexpr int FW = P % DW, FN = (P + 1) % DW;
  constexpr int XBUF = 64 * XT * 128;               // one chunk of x in LDS
  load_x<XT>(tb, ldx, c + XA, nch, xr[P % XA]);     // its previous chunk went into LDS at the end of chunk c - 1
  __builtin_amdgcn_sched_barrier(0);   // x first (see above)
  load_w<TN>(tb, ow, ows, c + DW - 1, nch, f[(P + DW - 1) % DW]);
  uint8_t *cur = smem + (c & 1) * XBUF;
  uint8_t *nxt = smem + ((c + 1) & 1) * XBUF;
#pragma unroll
  for (int s = 0; s < 4; s++) {
    bf16x8_t an[TM], bn[TN];
    if (s < 3) {
      read_x<TM>(cur, s + 1, wm, an);
      deq_w<TN>(f[FW], sc, s + 1, bn);
    } else {
      scales_of<TN>(f[FN], sc);
      deq_w<TN>(f[FN], sc, 0, bn);
    }
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < TM; i++)
      if (s < 3) a[i] = an[i];
#pragma unroll
    for (int j = 0; j < TN; j++) b[j] = bn[j];
    if (s == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2 * XT, 0);
#pragma unroll
    for (int k = 0; k < TM * TN; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
      if (s < 3 && k < TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  store_x<XT>(nxt, xr[(P + 1) % XA]);
  lds_barrier();
  read_x<TM>(nxt, 0, wm, a);   // the next chunk's step-0 x, now that it is in LDS
}

// Chunks c + Q, Q in Qs, while below n (the conditions are uniform over the
// workgroup, so every wave meets the same barriers).
template <int TM, int TN, int XT, int DW, int XA, int... Qs>
__device__ __forceinline__ void chunk_run(std::integer_sequence<int, Qs...>, bool all, const TileBase &tb,
                                          int64_t ldx, const uint32_t (&ow)[TN], const uint32_t (&ows)[TN], int64_t c,
                                          int64_t n, WFrags<TN> (&f)[DW], XRegs<XT> (&xr)[XA], f32x2_t (&sc)[TN],
                                          uint8_t *smem, int wm, bf16x8_t (&a)[TM], bf16x8_t (&b)[TN],
                                          f32x16_t (&acc)[TM][TN]) {
  ((all || c + Qs < n ? chunk<Qs, TM, TN, XT, DW, XA>(tb, ldx, ow, ows, c + Qs, n, f, xr, sc, smem, wm, a, b, acc)
                      : void()),
   ...);
}

constexpr int ring_period(int a, int b) {
  int p = a;
  while (p % b != 0) p += a;
  return p;
}

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_band = kGroupM * tiles_n;
  const int band = t / per_band;
  const int first = band * kGroupM;
  const int rows = min(kGroupM, tiles_m - first);
  const int w = t - band * per_band;
  tm = first + w % rows;
  tn = w / rows;
}

// Chunks [c0, c0 + n) of tile `tile` into acc (zeroed first). The tile bases
// are moved to chunk c0, so chunk c of the loop is chunk c0 + c of the tile and
// the loads past the range are empty.
template <int TM, int TN, int WGM, int DW, int XA>
__device__ __forceinline__ void tile_mainloop(const Params &p, int tile, int64_t c0, int64_t n, uint8_t *smem,
                                              const uint32_t (&ow)[TN], const uint32_t (&ows)[TN], int wm,
                                              f32x16_t (&acc)[TM][TN], int64_t &m0, int64_t &n0) {
  constexpr int XT = TM * WGM / 2;   // x rows staged per chunk: 64 XT (the tile's rows)
  const int64_t kt = p.K / 64;
  int tm, tn;
  tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
  m0 = (int64_t)tm * 32 * TM * WGM;
  n0 = (int64_t)tn * 32 * TN * (4 / WGM);
  TileBase tb;
  tb.x = reinterpret_cast<const uint8_t *>(p.x + m0 * p.ldx + c0 * 64);
  tb.x_bytes = (p.M - m0) * p.ldx * 2 - c0 * 128;
  tb.w = p.wp + ((n0 >> 5) * kt + c0) * 1024;
  tb.w_bytes = (p.N - n0) / 32 * kt * 1024 - c0 * 1024;
  tb.ws = p.wp + p.N * p.K / 2 + ((n0 >> 5) * kt + c0) * 128;
  tb.ws_bytes = (p.N - n0) / 32 * kt * 128 - c0 * 128;

#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = f32x16_t{};
  WFrags<TN> f[DW];
  XRegs<XT> xr[XA];
  f32x2_t sc[TN];
  bf16x8_t a[TM], b[TN];
  __syncthreads();   // the previous tile's waves are done with the LDS buffers
  load_x<XT>(tb, p.ldx, 0, n, xr[0]);
#pragma unroll
  for (int q = 1; q < XA; q++) load_x<XT>(tb, p.ldx, q, n, xr[q]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < DW - 1; q++) load_w<TN>(tb, ow, ows, q, n, f[q]);
  store_x<XT>(smem, xr[0]);
  lds_barrier();
  scales_of<TN>(f[0], sc);
  read_x<TM>(smem, 0, wm, a);
  deq_w<TN>(f[0], sc, 0, b);
  // chunks in whole periods of the two rings, then the ones left (padding the
  // range to whole periods ran all-zero chunks: a 16-chunk K range took 18
  // with the three-chunk period)
  constexpr int PER = ring_period(DW, XA);
  using Period = std::make_integer_sequence<int, PER>;
  int64_t c = 0;
  for (; c + PER <= n; c += PER)
    chunk_run<TM, TN, XT, DW, XA>(Period{}, true, tb, p.ldx, ow, ows, c, n, f, xr, sc, smem, wm, a, b, acc);
  chunk_run<TM, TN, XT, DW, XA>(std::make_integer_sequence<int, PER - 1>{}, false, tb, p.ldx, ow, ows, c, n, f, xr,
                                sc, smem, wm, a, b, acc);
}

// The main loop with x read straight into registers from its fragment-order
// copy (xf), like the A operand of the W4A4 kernel: chunk c, step s of row tile
// rt is the 1 KB at ((c * 4 + s) * xmt + rt) * 1024, one 16-byte unit per lane.
// x fragments go through a six-slot register ring indexed by the global step
// (the loop body is three chunks, twelve steps), each loaded five steps before
// its MFMAs into the slot the previous step freed; W keeps its three-chunk ring.
// No LDS and no barriers.
template <int T>
struct XRing {
  u32x4_t v[6][T];
};

// x's fragment-order range of a split: chunks [c0, c0 + n) of the tile's row
// tiles, one chunk = 4 steps x xmt row tiles x 1 KB.
struct XRange {
  const uint8_t *base;
  int64_t bytes;
};

// Step s of chunk c (relative to the range) into v. The chunk and step go in
// the scalar offset, which the buffer range check does not cover, so a chunk
// at or past the end of the range gets a zero-length resource: its loads read
// zero instead of whatever lies past the range.
template <int T>
__device__ __forceinline__ void load_xf(const XRange &xr, const uint32_t (&ox)[T], int64_t c, int64_t n, int s,
                                        int xmt, u32x4_t (&v)[T]) {
  const __amdgpu_buffer_rsrc_t rx = rsrc(xr.base, c < n ? xr.bytes : 0);
  const int so = c < n ? (int)((c * 4 + s) * xmt * 1024) : 0;
#pragma unroll
  for (int i = 0; i < T; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, ox[i], so, 0);
}

template <int P, int TM, int TN>
__device__ __forceinline__ void chunk_d(const TileBase &tb, const XRange &rx, const uint32_t (&ox)[TM],
                                        int xmt, const uint32_t (&ow)[TN], const uint32_t (&ows)[TN], int64_t c,
                                        int64_t nch, WFrags<TN> (&f)[3], f32x2_t (&sc)[TN], XRing<TM> &xr,
                                        bf16x8_t (&b)[TN], f32x16_t (&acc)[TM][TN]) {
  constexpr int kValu = 16 / TM + 1;              // dequant instructions per MFMA, rounded up
  const bool in2 = c + 2 < nch;
  WFrags<TN> &f2 = f[(P + 2) % 3];
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const int g = 4 * P + s;                      // step in the three-chunk body
    // x of step g + 5 into the slot step g - 1 used
    load_xf<TM>(rx, ox, c + (s + 5) / 4, nch, (s + 5) % 4, xmt, xr.v[(g + 5) % 6]);
    if (s == 0) {
      const __amdgpu_buffer_rsrc_t rw = rsrc(tb.w, in2 ? tb.w_bytes : 0);
#pragma unroll
      for (int j = 0; j < TN; j++) f2.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, ow[j], (int)((c + 2) * 1024), 0);
    } else if (s == 1) {
      const __amdgpu_buffer_rsrc_t rs = rsrc(tb.ws, in2 ? tb.ws_bytes : 0);
#pragma unroll
      for (int j = 0; j < TN; j++) f2.ws[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, ows[j], (int)((c + 2) * 128), 0);
    }
    bf16x8_t bn[TN];
    if (s < 3) {
      deq_w<TN>(f[P], sc, s + 1, bn);
    } else {
      scales_of<TN>(f[(P + 1) % 3], sc);
      deq_w<TN>(f[(P + 1) % 3], sc, 0, bn);
    }
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int j = 0; j < TN; j++)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xr.v[g % 6][i]), b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < TN; j++) b[j] = bn[j];
    if (s < 2)   // this step's loads first
      __builtin_amdgcn_sched_group_barrier(0x020, TM + TN, 0);
    else
      __builtin_amdgcn_sched_group_barrier(0x020, TM, 0);
#pragma unroll
    for (int k = 0; k < TM * TN; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int TM, int TN, int WGM>
__device__ __forceinline__ void tile_mainloop_d(const Params &p, int tile, int64_t c0, int64_t n,
                                                const uint32_t (&ow)[TN], const uint32_t (&ows)[TN], int wm,
                                                f32x16_t (&acc)[TM][TN], int64_t &m0, int64_t &n0) {
  const int64_t kt = p.K / 64;
  int tm, tn;
  tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
  m0 = (int64_t)tm * 32 * TM * WGM;
  n0 = (int64_t)tn * 32 * TN * (4 / WGM);
  TileBase tb;
  tb.w = p.wp + ((n0 >> 5) * kt + c0) * 1024;
  tb.w_bytes = (p.N - n0) / 32 * kt * 1024 - c0 * 1024;
  tb.ws = p.wp + p.N * p.K / 2 + ((n0 >> 5) * kt + c0) * 128;
  tb.ws_bytes = (p.N - n0) / 32 * kt * 128 - c0 * 128;
  // x: chunks [c0, c0 + n) of the tile's row tiles; loads past the range read zero
  const int64_t xchunk = (int64_t)4 * p.xmt * 1024;
  const XRange rx{p.xf + c0 * xchunk, n * xchunk};
  const int lane = threadIdx.x & 63;
  uint32_t ox[TM];
#pragma unroll
  for (int i = 0; i < TM; i++) ox[i] = (uint32_t)(((m0 >> 5) + wm * TM + i) * 1024 + lane * 16);

#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++) acc[i][j] = f32x16_t{};
  WFrags<TN> f[3];
  f32x2_t sc[TN];
  bf16x8_t b[TN];
  XRing<TM> xr;
#pragma unroll
  for (int s = 0; s < 5; s++) load_xf<TM>(rx, ox, s / 4, n, s % 4, p.xmt, xr.v[s]);
  load_w<TN>(tb, ow, ows, 0, n, f[0]);
  load_w<TN>(tb, ow, ows, 1, n, f[1]);
  scales_of<TN>(f[0], sc);
  deq_w<TN>(f[0], sc, 0, b);
  int64_t c = 0;   // chunks in threes, then the one or two left (as in tile_mainloop)
  for (; c + 3 <= n; c += 3) {
    chunk_d<0, TM, TN>(tb, rx, ox, p.xmt, ow, ows, c, n, f, sc, xr, b, acc);
    chunk_d<1, TM, TN>(tb, rx, ox, p.xmt, ow, ows, c + 1, n, f, sc, xr, b, acc);
    chunk_d<2, TM, TN>(tb, rx, ox, p.xmt, ow, ows, c + 2, n, f, sc, xr, b, acc);
  }
  if (c < n) chunk_d<0, TM, TN>(tb, rx, ox, p.xmt, ow, ows, c, n, f, sc, xr, b, acc);
  if (c + 1 < n) chunk_d<1, TM, TN>(tb, rx, ox, p.xmt, ow, ows, c + 1, n, f, sc, xr, b, acc);
}

// Epilogue of a whole tile: per wave 32 x 32TN staging of BF16 in LDS (after
// every wave is done with x), then 16-byte row pieces.
template <int TM, int TN, bool COLS>
__device__ __forceinline__ void tile_epilogue(const Params &p, uint8_t *smem, float alpha, int64_t m0, int64_t n0,
                                              int wave, int wm, int wn, f32x16_t (&acc)[TM][TN]) {
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  __syncthreads();
  constexpr int ROW_BYTES = 32 * TN * 2;
  uint8_t *reg = smem + wave * (32 * ROW_BYTES);
  const int64_t col0 = n0 + wn * 32 * TN;
  const int64_t ncols = p.N - col0;
  const bool vec_ok = (p.ldy * 2) % 16 == 0 && ((uintptr_t)p.y & 15) == 0;
#pragma unroll
  for (int i = 0; i < TM; i++) {
#pragma unroll
    for (int j = 0; j < TN; j++) {
      // the alpha of this lane's column (columns past N are not stored)
      const float aj = COLS && j * 32 + r < ncols ? alpha * p.alpha_col[col0 + j * 32 + r] : alpha;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int row = 8 * (e >> 2) + 4 * h + (e & 3);
        *reinterpret_cast<uint16_t *>(reg + row * ROW_BYTES + (j * 32 + r) * 2) = f32_to_bf16_rne(aj * acc[i][j][e]);
      }
    }
    __syncthreads();
    constexpr int PIECES = ROW_BYTES / 16;
    for (int q = lane; q < 32 * PIECES; q += 64) {
      const int row = q / PIECES, pc = q % PIECES;
      const int64_t m = m0 + wm * 32 * TM + i * 32 + row;
      const int64_t cc = (int64_t)pc * 8;
      if (m < p.M && cc < ncols) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(reg + row * ROW_BYTES + pc * 16);
        uint16_t *dst = p.y + m * p.ldy + col0 + cc;
        if (vec_ok) {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));   // written once: stream it
        } else {
          const uint16_t *src = reinterpret_cast<const uint16_t *>(&v);
          for (int e2 = 0; e2 < 8; e2++) dst[e2] = src[e2];
        }
      }
    }
    __syncthreads();
  }
}

// TM x TN MFMA tiles per wave, the 4 waves WGM x (4 / WGM) over the tile; XP
// is the x path (big_xpath): the fragment-order copy read straight into
// registers (tile_mainloop_d), or x staged through LDS (tile_mainloop), with
// the deeper register rings when the grid holds one workgroup per CU.
// COLS: p.alpha_col is set (a separate instantiation, so that the kernel
// without a per-column scale keeps its registers for the main loop).
template <int TM, int TN, int WGM, bool COLS, int XP>
__global__ __launch_bounds__(kThreads, TM * TN >= 8 || XP == kXLdsDeep ? 1 : 2) void big_kernel(Params p) {
  constexpr bool kLds = XP != kXDirect;
  constexpr bool DEEP = XP == kXLdsDeep;
  constexpr int WGN = 4 / WGM;
  // LDS path: two x chunks; direct paths: the epilogue's BF16 staging
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds ? 2 * (32 * TM * WGM) * 128 : 4 * 32 * 32 * TN * 2];
  const int t = threadIdx.x, wave = t >> 6, wm = wave / WGN, wn = wave % WGN;
  const int lane = t & 63, r = lane & 31;
  const int G = gridDim.x;
  int pid = blockIdx.x;
  if ((G & 7) == 0) pid = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const float alpha = load_alpha(p.alpha, p.alpha_dev);
  const int64_t nch = p.K / 64, kt = p.K / 64;
  uint32_t ow[TN], ows[TN];
#pragma unroll
  for (int j = 0; j < TN; j++) {
    ow[j] = (uint32_t)(((wn * TN + j) * kt) * 1024 + lane * 16);
    ows[j] = (uint32_t)(((wn * TN + j) * kt) * 128 + r * 4);
  }
  f32x16_t acc[TM][TN];
  int64_t m0, n0;
  for (int tile = pid; tile < p.full; tile += G) {
    if constexpr (kLds)
      tile_mainloop<TM, TN, WGM, DEEP ? kDeepW : 3, DEEP ? kDeepX : 1>(p, tile, 0, nch, smem, ow, ows, wm, acc, m0,
                                                                      n0);
    else
      tile_mainloop_d<TM, TN, WGM>(p, tile, 0, nch, ow, ows, wm, acc, m0, n0);
    tile_epilogue<TM, TN, COLS>(p, smem, alpha, m0, n0, wave, wm, wn, acc);
  }
  if (p.rem > 0) {
    int64_t s, e;
    split_range(pid, G, (int64_t)p.rem * nch, s, e);
    for (int seg = 0; s < e; seg++) {
      const int64_t rho = s / nch, c0 = s - rho * nch, c1 = min(nch, c0 + (e - s));
      if constexpr (kLds)
        tile_mainloop<TM, TN, WGM, DEEP ? kDeepW : 3, DEEP ? kDeepX : 1>(p, p.full + (int)rho, c0, c1 - c0, smem, ow,
                                                                        ows, wm, acc, m0, n0);
      else
        tile_mainloop_d<TM, TN, WGM>(p, p.full + (int)rho, c0, c1 - c0, ow, ows, wm, acc, m0, n0);
      float *dst = p.partials + ((int64_t)pid * 2 + seg) * partial_floats<TM, TN>() +
                   (int64_t)wave * TM * TN * 1024 + lane * 16;
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int q = 0; q < 4; q++)
            *reinterpret_cast<f32x4_t *>(dst + (i * TN + j) * 1024 + 4 * q) =
                f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      s += c1 - c0;
    }
  }
}

// Split tiles: workgroup (rho, g) takes 4 x 1024 of tile full + rho's
// accumulator elements, the four wave-tiles `part` = 4 g .. 4 g + 3 (thread t:
// lane t % 64, elements 4 (t / 64) .. + 3 of that lane in each), adds them over
// every workgroup whose range touches the tile, in workgroup order, then
// applies alpha and the BF16 conversion. TM TN workgroups per tile; with four
// parts per thread, sixteen loads are in flight together (a workgroup per
// part left the kernel bound by load latency: 17.6 us after the 128 x 256 tile
// kernel at M = 128 on 34816 x 5120).
template <int TM, int TN, int WGM>
__global__ __launch_bounds__(kThreads) void big_fixup_kernel(Params p, int G) {
  constexpr int WGN = 4 / WGM;
  constexpr int PP = fixup_parts(TM, TN);           // 1024-element parts per workgroup
  constexpr int WPT = 4 * TM * TN / PP;             // workgroups per tile
  const int rho = blockIdx.x / WPT, pg = blockIdx.x % WPT;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6, h = lane >> 5, r = lane & 31;
  const int64_t nch = p.K / 64, units = (int64_t)p.rem * nch;
  const int64_t lo = (int64_t)rho * nch, hi = lo + nch;   // the tile's units
  int tm, tn;
  tile_coords(p.full + rho, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 32 * TM * WGM, n0 = (int64_t)tn * 32 * TN * WGN;
  // first workgroup whose range ends past lo
  int64_t first = lo * G / units;
  if (first > 0) first--;
  for (;;) {
    int64_t s, e;
    split_range(first, G, units, s, e);
    if (e > lo || first == G - 1) break;
    first++;
  }
  // the contributing workgroups are first .. last (ranges are contiguous)
  int64_t last = first;
  for (;;) {
    int64_t s, e;
    if (last + 1 >= G) break;
    split_range(last + 1, G, units, s, e);
    if (s >= hi) break;
    last++;
  }
  // Their partials are loaded four workgroups at a time; a slot with no
  // partial (past last, or an empty range) reads zero through the buffer range
  // check, and adding +0 to a sum that started at +0 changes nothing, so each
  // sum is the same as one over the contributors in order.
  const int64_t pbytes = (int64_t)G * 2 * partial_floats<TM, TN>() * 4;
  const __amdgpu_buffer_rsrc_t rp = rsrc(p.partials, pbytes);
  const int64_t off = (int64_t)(PP * pg) * 1024 + lane * 16 + 4 * q;
  f32x4_t v[PP];
#pragma unroll
  for (int u = 0; u < PP; u++) v[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t w0 = first; w0 <= last; w0 += 4) {
    f32x4_t t[4][PP];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int64_t w = w0 + k;
      int64_t s, e;
      split_range(w, G, units, s, e);
      const bool ok = w <= last && e > lo && s < e;
      const int seg = s >= lo ? 0 : 1;
      const int64_t base = ((w * 2 + seg) * partial_floats<TM, TN>() + off) * 4;
#pragma unroll
      for (int u = 0; u < PP; u++) {
        const uint32_t o = ok ? (uint32_t)(base + u * 4096) : (uint32_t)pbytes;
        t[k][u] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, o, 0, 0));
      }
    }
#pragma unroll
    for (int k = 0; k < 4; k++)
#pragma unroll
      for (int u = 0; u < PP; u++) v[u] += t[k][u];
  }
  const float alpha = load_alpha(p.alpha, p.alpha_dev);
#pragma unroll
  for (int u = 0; u < PP; u++) {
    const int part = PP * pg + u;   // (wave, i, j)
    const int wave = part / (TM * TN), i = (part / TN) % TM, j = part % TN;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t col = n0 + wn * 32 * TN + 32 * j + r;
    const float ac = col < p.N ? col_alpha(alpha, p.alpha_col, col) : alpha;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int e = 4 * q + k;
      const int64_t m = m0 + wm * 32 * TM + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m < p.M && col < p.N) p.y[m * p.ldy + col] = f32_to_bf16_rne(ac * v[u][k]);
    }
  }
}

// The tile kernel's instantiations: per-column alpha or not, and the x path
// (big_xpath): 128 x 128 tiles on LDS (deep rings with one workgroup per CU),
// 128 x 256 tiles direct or on LDS, 256 x 256 tiles direct.
template <int TM, int TN, int WGM, int XP>
static void launch_big_x(bool cols, unsigned grid, hipStream_t s, const Params &bp) {
  if (cols)
    hipLaunchKernelGGL((big_kernel<TM, TN, WGM, true, XP>), dim3(grid), dim3(kThreads), 0, s, bp);
  else
    hipLaunchKernelGGL((big_kernel<TM, TN, WGM, false, XP>), dim3(grid), dim3(kThreads), 0, s, bp);
}
template <int TM, int TN, int WGM>
static void launch_big(int xpath, bool cols, unsigned grid, hipStream_t s, const Params &bp) {
  if constexpr (TM * TN < 8) {
    if (xpath == kXLdsDeep)
      launch_big_x<TM, TN, WGM, kXLdsDeep>(cols, grid, s, bp);
    else
      launch_big_x<TM, TN, WGM, kXLds>(cols, grid, s, bp);
  } else if constexpr (TM * TN == 8) {
    if (xpath == kXLdsDeep)
      launch_big_x<TM, TN, WGM, kXLdsDeep>(cols, grid, s, bp);
    else
      launch_big_x<TM, TN, WGM, kXDirect>(cols, grid, s, bp);
  } else {
    launch_big_x<TM, TN, WGM, kXDirect>(cols, grid, s, bp);
  }
}

}  // namespace big

}  // namespace w4a16

// The heuristic configuration: the decode kernel while x fits in its LDS
// (M <= 4), the skinny kernel up to M = 64, else the tile kernel with
// big_tile_shape's tiles.
void w4a16_default_config(int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *c) {
  *c = nvfp4_config{};
  c->num_cus = cus;
  if (w4a16::decode_fits(M, K) && M <= w4a16::kDecodeDefaultMaxM) {
    c->kernel = NVFP4_KERNEL_W4A16_DECODE;
  } else if (M <= w4a16::kSkinnyMaxM) {
    c->kernel = NVFP4_KERNEL_W4A16_SKINNY;
  } else {
    int TM, TN, WGM;
    w4a16::big_tile_shape(M, N, K, cus, TM, TN, WGM);
    c->kernel = NVFP4_KERNEL_W4A16_TILES;
    c->tile_m = 32 * TM * WGM;
    c->tile_n = 32 * TN * (4 / WGM);
  }
}

bool w4a16_config_valid(int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  (void)N;
  if (c.num_cus <= 0 || c.tail != NVFP4_TAIL_NONE || c.split_k != 0 || c.dynamic != 0) return false;
  switch (c.kernel) {
    case NVFP4_KERNEL_W4A16_DECODE: return w4a16::decode_fits(M, K);
    case NVFP4_KERNEL_W4A16_SKINNY: return M <= w4a16::kSkinnyMaxM;
    case NVFP4_KERNEL_W4A16_TILES:
      return (c.tile_m == 256 && c.tile_n == 256) || (c.tile_m == 128 && c.tile_n == 256) ||
             (c.tile_m == 128 && c.tile_n == 128);
    default: return false;
  }
}

size_t w4a16_config_workspace_bytes(int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  if (M <= 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || !w4a16_config_valid(M, N, K, c)) return 0;
  const w4a16::Plan p = w4a16::make_plan(M, N, K, c);
  return w4a16::workspace_for(p, c, M, N, K);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_gemm_w4a16(const uint16_t *x, int64_t ldx, const uint8_t *w_prep, int64_t M, int64_t N,
                                         int64_t K, float alpha, const float *alpha_dev, const float *alpha_col,
                                         uint16_t *y, int64_t ldy, const nvfp4_config *config, void *ws,
                                         size_t ws_bytes, void *stream) {
  if (M < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0 || ldx < K || ldy < N) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  if (!x || !w_prep || !y) return NVFP4_ERR_NULL;
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return NVFP4_ERR_VALUE;
  if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(w_prep, 16) || !aligned(y, 2) ||
      (alpha_dev && !aligned(alpha_dev, 4)) || (alpha_col && !aligned(alpha_col, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo di;
  nvfp4_status st = device_info(&di);
  if (st != NVFP4_OK) return st;
  nvfp4_config cfg;
  st = resolve_config(NVFP4_OP_W4A16, M, N, K, config, di.num_cus, &cfg);
  if (st != NVFP4_OK) return st;
  const w4a16::Plan plan = w4a16::make_plan(M, N, K, cfg);
  const size_t need = w4a16::workspace_for(plan, cfg, M, N, K);
  if (need > 0 && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
  if (need > 0 && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (plan.kind == 0) {
    if (plan.grid_x > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
    const size_t lds = (size_t)(M * K * 2);
    const int key = plan.dec * 8 + (int)M;
#define NVFP4_DECODE_CASE(D, MM)                                                                               \
  case D * 8 + MM: {                                                                                           \
    constexpr w4a16::DecodeShape sh = w4a16::kDecodeShapes[D];                                                 \
    hipLaunchKernelGGL((w4a16::decode_kernel<MM, sh.R, sh.W, sh.U, 0>), dim3((unsigned)plan.grid_x),        \
                       dim3(sh.W * 64), lds, s, x, ldx, w_prep, N, K, alpha, alpha_dev, alpha_col, y, ldy, plan.nfull);   \
    break;                                                                                                     \
  }
#define NVFP4_DECODE_SHAPE(D) \
  NVFP4_DECODE_CASE(D, 1) NVFP4_DECODE_CASE(D, 2) NVFP4_DECODE_CASE(D, 3) NVFP4_DECODE_CASE(D, 4)
    constexpr w4a16::DecodeShape s0 = w4a16::kDecodeShapes[0];
    if (plan.tr == 8)
      hipLaunchKernelGGL((w4a16::decode_kernel<1, s0.R, s0.W, s0.U, 8>), dim3((unsigned)plan.grid_x),
                         dim3(s0.W * 64), lds, s, x, ldx, w_prep, N, K, alpha, alpha_dev, alpha_col, y, ldy, plan.nfull);
    else if (plan.tr == 16)
      hipLaunchKernelGGL((w4a16::decode_kernel<1, s0.R, s0.W, s0.U, 16>), dim3((unsigned)plan.grid_x),
                         dim3(s0.W * 64), lds, s, x, ldx, w_prep, N, K, alpha, alpha_dev, alpha_col, y, ldy, plan.nfull);
    else
      switch (key) {
        NVFP4_DECODE_SHAPE(0)
        NVFP4_DECODE_SHAPE(1)
        default: return NVFP4_ERR_SHAPE;
      }
#undef NVFP4_DECODE_SHAPE
#undef NVFP4_DECODE_CASE
  } else if (plan.kind == 4) {
    const w4a16::BigSched b = w4a16::big_sched(M, N, K, cfg);
    // fragment-order x: 32-bit offsets inside it
    const int xpath = w4a16::big_xpath(b, K, cfg.num_cus);
    if (b.total > 0x7FFFFFFF || w4a16::big_xf_bytes(b, K, cfg.num_cus) > 0x7FFFFFFFull) return NVFP4_ERR_SHAPE;
    if (xpath != w4a16::kXDirect && b.tile_rows() * ldx * 2 > 0xFFFFFFFFll)
      return NVFP4_ERR_SHAPE;   // LDS path: 32-bit x offsets
    const int64_t xmt = w4a16::big_xmt(b, K, cfg.num_cus);
    uint8_t *xf = xmt > 0 ? static_cast<uint8_t *>(ws) + w4a16::big_partials_span(b) : nullptr;
    if (xmt > 0) {
      hipLaunchKernelGGL(w4a16::tile_x_kernel, dim3((unsigned)(K / 64 * xmt)), dim3(256), 0, s, x, ldx, M, K,
                         (int)xmt, reinterpret_cast<u32x4_t *>(xf));
      NVFP4_LAUNCH_CHECK();
    }
    w4a16::big::Params bp{x,     ldx,           w_prep,        y,           ldy,          M,
                          N,     K,             alpha,         alpha_dev,   alpha_col,   (int)b.tiles_m, (int)b.tiles_n,
                          (int)b.full, (int)b.rem, static_cast<float *>(ws), xf, (int)xmt};
    const unsigned grid = (unsigned)b.G,
                   fix_grid = (unsigned)(b.rem * 4 * b.TM * b.TN / w4a16::fixup_parts(b.TM, b.TN));
#define NVFP4_BIG(TMV, TNV, WGMV)                                                                                \
  w4a16::big::launch_big<TMV, TNV, WGMV>(xpath, alpha_col != nullptr, grid, s, bp);                 \
  if (b.rem > 0) {                                                                                               \
    NVFP4_LAUNCH_CHECK();                                                                                        \
    hipLaunchKernelGGL((w4a16::big::big_fixup_kernel<TMV, TNV, WGMV>), dim3(fix_grid), dim3(w4a16::big::kThreads), \
                       0, s, bp, (int)b.G);                                                                      \
  }
    if (b.TN == 4) {
      NVFP4_BIG(4, 4, 2)
    } else if (b.TN == 2) {
      NVFP4_BIG(4, 2, 1)
    } else {
      NVFP4_BIG(4, 1, 1)
    }
#undef NVFP4_BIG
  } else if (plan.kind == 3) {
    if (plan.grid_x > 0x7FFFFFFF || M * ldx * 2 > 0xFFFFFFFFll) return NVFP4_ERR_SHAPE;
    const int MT = M <= 32 ? 1 : 2;
    const w4a16::SkinnyShape sh = w4a16::skinny_shape(M, N, K, cfg.num_cus);
    const bool xf_path = sh.RP == 0 && M > w4a16::kSkinnyDirectMaxM;
    if (xf_path && (int64_t)MT * 64 * K > 0x7FFFFFFFll) return NVFP4_ERR_SHAPE;   // 32-bit fragment offsets
    uint8_t *xf = static_cast<uint8_t *>(ws);
    if (xf_path) {
      hipLaunchKernelGGL(w4a16::tile_x_kernel, dim3((unsigned)(K / 64 * MT)), dim3(256), 0, s, x, ldx, M, K, MT,
                         reinterpret_cast<u32x4_t *>(xf));
      NVFP4_LAUNCH_CHECK();
    }
    const unsigned grid = (unsigned)(plan.grid_x / sh.NG);
    if (sh.RP > 0) {
#define NVFP4_SKINNY_ROWS(WV, NGV, RPV)                                                                          \
  if (sh.W == WV && sh.NG == NGV && sh.RP == RPV) {                                                              \
    hipLaunchKernelGGL((w4a16::skinny_rows_kernel<WV, NGV, RPV, w4a16::kSkinnyRowsDepth>), dim3(grid),           \
                       dim3(WV * 64), 0, s, x, ldx, w_prep, M, N, K, alpha, alpha_dev, alpha_col, y, ldy);      \
  } else
      NVFP4_SKINNY_ROWS(16, 1, 8)
      NVFP4_SKINNY_ROWS(16, 1, 16)
      NVFP4_SKINNY_ROWS(8, 2, 8)
      NVFP4_SKINNY_ROWS(8, 2, 16)
      NVFP4_SKINNY_ROWS(8, 1, 8)
      NVFP4_SKINNY_ROWS(8, 1, 16)
      NVFP4_SKINNY_ROWS(16, 1, 32)
      NVFP4_SKINNY_ROWS(8, 2, 32)
      NVFP4_SKINNY_ROWS(8, 1, 32)
      NVFP4_SKINNY_ROWS(8, 2, 64)
      NVFP4_SKINNY_ROWS(8, 1, 64)
      return NVFP4_ERR_SHAPE;
#undef NVFP4_SKINNY_ROWS
      NVFP4_LAUNCH_CHECK();
      return NVFP4_OK;
    }
#define NVFP4_SKINNY_X(WV, NGV, MTV, XFV)                                                                      \
  hipLaunchKernelGGL((w4a16::skinny_kernel<MTV, XFV, WV, NGV>), dim3(grid), dim3(WV * 64), 0, s, x, ldx,           \
                     w_prep, M, N, K, alpha, alpha_dev, alpha_col, y, ldy, xf)
#define NVFP4_SKINNY(WV, NGV)                                                                                  \
  if (sh.W == WV && sh.NG == NGV) {                                                                            \
    if (!xf_path) NVFP4_SKINNY_X(WV, NGV, 1, false);                                                          \
    else if (MT == 1) NVFP4_SKINNY_X(WV, NGV, 1, true);                                                       \
    else NVFP4_SKINNY_X(WV, NGV, 2, true);                                                                    \
  } else
    NVFP4_SKINNY(16, 1)
    NVFP4_SKINNY(8, 2)
    NVFP4_SKINNY(8, 1)
    return NVFP4_ERR_SHAPE;
#undef NVFP4_SKINNY
#undef NVFP4_SKINNY_X
  }
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}
