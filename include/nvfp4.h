/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled GEMM library.
 *
 * The operation (Colfax Research, "Optimizing an NVFP4 Blockscaled GEMM on RTX
 * PRO 6000 Blackwell GPU (SM120)", introduction and "Version 2"; TileLang PR
 * #3290, "Summary"):
 *
 *   W4A4:  D[m][n] = alpha * sum_k (A[m][k] * SFA[m][k/16]) * (B[n][k] * SFB[n][k/16])
 *   W4A16: y[m][n] = alpha * sum_k  x[m][k] * (W[n][k] * SFW[n][k/16])
 *
 * A, B, W hold 4-bit E2M1 codes packed two per byte along K (element 2j in the
 * low nibble of byte j); SFA, SFB, SFW hold one E4M3 (or UE4M3) scale byte per
 * 16 consecutive K-elements of a row; x and y are BF16; alpha is FP32 and is
 * applied to the FP32 accumulator before the output conversion (Colfax
 * article, "Version 3").
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev or described as device memory are device pointers
 *    owned by the caller. The library never allocates, frees or retains a
 *    pointer beyond the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously; the call returns after the enqueue.
 *  - Argument checks run on the host before anything is enqueued; a non-OK
 *    status means nothing was launched.
 *  - Results are deterministic: the same inputs give bit-identical outputs on
 *    every call, in or out of hipGraph capture.
 *  - Sizes are int64_t; all device offsets are 64-bit.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* a size is negative/zero where not allowed, or K % 64, N % 32, ld checks fail */
  NVFP4_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks the stated alignment */
  NVFP4_ERR_DTYPE = 4,       /* an enum argument (scale kind, output dtype, op) is out of range */
  NVFP4_ERR_VALUE = 5,       /* a host scalar is not finite */
  NVFP4_ERR_WORKSPACE = 6,   /* workspace missing or smaller than nvfp4_workspace_bytes() */
  NVFP4_ERR_UNSUPPORTED = 7, /* the current device is not gfx950 */
  NVFP4_ERR_HIP = 8          /* a HIP runtime call or launch failed */
} nvfp4_status;

typedef enum { NVFP4_SCALE_UE4M3 = 0, NVFP4_SCALE_E4M3 = 1 } nvfp4_scale_kind;
typedef enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 } nvfp4_out_dtype;
typedef enum {
  NVFP4_OP_W4A4 = 0,        /* nvfp4_gemm_w4a4 (A row-major: the call tiles it into the workspace) */
  NVFP4_OP_W4A16 = 1,       /* nvfp4_gemm_w4a16 */
  NVFP4_OP_QUANTIZE = 2,    /* nvfp4_quantize and its tiled forms */
  NVFP4_OP_W4A4_TILED = 3   /* nvfp4_gemm_w4a4_tiled and nvfp4_gemm_w4a4_two_pass_tiled */
} nvfp4_op;

/* Launch configuration of a GEMM (TileLang PR #3290, "Summary" and "Tests": a
 * heuristic get_config, explicit configs that a caller or a test passes, and
 * per-GPU tuned tables keyed by SM count that are not applied on another SM
 * count; Colfax article, "Version 7: Autotuning"). Every field is an int32. */
typedef enum {
  NVFP4_KERNEL_AUTO = 0,          /* in a request: let the library choose */
  NVFP4_KERNEL_W4A4_TILES = 1,    /* W4A4: persistent MFMA kernel over 256 x 256 or 128 x 128 tiles */
  NVFP4_KERNEL_W4A16_DECODE = 2,  /* W4A16, M <= 4 and M * K * 2 <= 64 KiB: vector-ALU weight streaming */
  NVFP4_KERNEL_W4A16_SKINNY = 3,  /* W4A16, M <= 64: MFMA over 32-row weight groups, whole K per workgroup */
  NVFP4_KERNEL_W4A16_TILES = 4    /* W4A16: persistent MFMA kernel over 256 x 256, 128 x 256 or 128 x 128 tiles */
} nvfp4_kernel;
typedef enum {
  NVFP4_TAIL_NONE = 0,       /* tiles past the last whole round of the CUs run as one more round */
  NVFP4_TAIL_QUADRANTS = 1,  /* ... as 128 x 128 quadrants, two workgroups per CU, in a second launch */
  NVFP4_TAIL_SPLIT = 2       /* ... split along K over the CUs; a fix-up kernel adds the FP32 partials */
} nvfp4_tail;
typedef enum { NVFP4_CONFIG_HEURISTIC = 0, NVFP4_CONFIG_TUNED = 1, NVFP4_CONFIG_EXPLICIT = 2 } nvfp4_config_source;
typedef struct {
  int32_t kernel;    /* nvfp4_kernel */
  int32_t tile_m;    /* rows of D per workgroup tile (W4A4 and W4A16 tiles; 0 otherwise) */
  int32_t tile_n;    /* columns of D per workgroup tile */
  int32_t tail;      /* nvfp4_tail (W4A4 on 256 x 256 tiles; NONE otherwise) */
  int32_t split_k;   /* K ranges per tail tile with NVFP4_TAIL_SPLIT (>= 2), else 0 */
  int32_t dynamic;   /* W4A4: 1 = workgroups take their tiles from atomic counters in the workspace */
  int32_t num_cus;   /* CU count the launch is sized for (0 in a request: the current device's) */
  int32_t source;    /* nvfp4_config_source (set by nvfp4_get_config; ignored in a request) */
} nvfp4_config;

/* Per-device set-up, done outside any graph capture (TileLang PR #3290,
 * "Changes": the per-device state is created up front, never lazily inside a
 * capture). Checks that HIP device `device` is gfx950 and records its CU
 * count, which selects the launch configurations. Calling it is optional: the
 * first call of any entry point on a device does the same, so only a caller
 * whose first call would be inside a capture needs it. Thread-safe; repeated
 * calls are cheap. The calling thread's current device is left unchanged.
 * Returns NVFP4_ERR_VALUE for a device index out of range,
 * NVFP4_ERR_UNSUPPORTED for a device that is not gfx950. */
nvfp4_status nvfp4_init(int device);

/* Human-readable name of a status code (static string, never NULL). */
const char *nvfp4_status_str(int status);

/* Size in bytes of a prepared weight: N*K/2 + N*K/16, the same as the packed
 * codes plus the scales (TileLang PR #3290, "Design: Weight layout").
 * Returns 0 for N % 32 != 0, K % 64 != 0 or non-positive sizes. */
size_t nvfp4_prepared_weight_bytes(int64_t N, int64_t K);

/* Workspace bytes an op needs for (M, N, K); 0 means no workspace is used.
 * The workspace is caller-owned device memory, sized by this query before any
 * graph capture and passed to every call, so no call allocates (TileLang PR
 * #3290, "Changes": the workspace of split-K partials exists before a capture
 * and is never created inside one; one workspace per stream that runs
 * concurrently).
 * The workspace holds A in the prepared tile layout (W4A4: (M rounded up to
 * 32) * K * 9/16 bytes); for W4A16, x in MFMA fragment order (16 < M <= 64:
 * (M rounded up to 32) * K * 2 bytes; M > 64 on 256 x 256 or 128 x 256
 * output tiles: M rounded up to the tile rows, * K * 2 bytes) after the FP32
 * partial tiles of output tiles split along K (M > 64 when the tiles do not
 * fill whole rounds of the CUs; the tile shape and this size depend on the
 * device's CU count); or, for the quantizer (12.25 KiB), per-workgroup maxima
 * and the one-read form's barrier slots with the generation number that tags
 * them. Every call overwrites what it reads, or (the quantizer's slots) tags
 * it with a generation it advances, so no workspace needs initialising. */
size_t nvfp4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* The configuration a GEMM call with config == NULL uses for (op, M, N, K) on
 * a device with num_cus CUs (num_cus == 0: the current device's): a tuned
 * table entry when the table for that CU count has one for the shape, else the
 * heuristic. num_cus < 0 returns the heuristic for -num_cus CUs without looking
 * at the table (what a tuning run compares against). Host-only (no device
 * work when num_cus != 0). op: NVFP4_OP_W4A4, NVFP4_OP_W4A4_TILED (two-pass
 * calls: K is the contraction length 2K), or NVFP4_OP_W4A16. */
nvfp4_status nvfp4_get_config(int op, int64_t M, int64_t N, int64_t K, int num_cus, nvfp4_config *out);

/* Workspace bytes of a call that uses `config` (NULL: nvfp4_workspace_bytes).
 * Returns 0 when the config is not valid for the shape. */
size_t nvfp4_config_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config *config);

/* Zeroes a workspace on `stream` with a fill kernel (no hipMemset, so it may be
 * captured; TileLang PR #3290, "Changes", on the workspace). No kernel of this
 * library needs a zeroed workspace: every call writes what it later reads. The
 * call lets a caller clear one without hipMemset. ws: 16-byte aligned device
 * memory, ws_bytes % 4 == 0 (NVFP4_ERR_ALIGN otherwise). */
nvfp4_status nvfp4_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Prepare a weight once (TileLang PR #3290, "Design: Weight layout").
 *  w_codes  [N][K/2] bytes, device, packed E2M1, 16-byte aligned.
 *  w_scales [N][K/16] bytes, device, E4M3 (kind = NVFP4_SCALE_E4M3) or UE4M3.
 *  N % 32 == 0, K % 64 == 0.
 *  w_prep   nvfp4_prepared_weight_bytes(N, K) bytes, device, 16-byte aligned.
 * The prepared layout: 32 (n) x 64 (k) tiles in n-major, k-minor order; the
 * first N*K/2 bytes hold 1024-byte code tiles of 64 16-byte units, unit
 * 32h + r holding the standard-packed codes of row r for k in [32h, 32h+32)
 * of the tile; the rest are 128-byte scale tiles in the same order (row r,
 * block b at byte 4r+b). Blocks with a zero scale get zero codes and scale 0;
 * blocks with a negative scale get their code signs flipped and the scale magnitude;
 * NaN scale bytes (and, for UE4M3, bytes with bit 7 set) keep their codes, get
 * scale byte 0x7F (NaN) and are counted.
 *  bad_count_dev  device int32 or NULL; when given it is overwritten with the
 *  number of invalid scale bytes (read it after the stream completes).
 * NaN scales are an input error (TileLang PR #3290, "Changes", input
 * validation). They sit in device memory, so this call counts them instead of
 * reading them back: the Python binding synchronises once after the call and
 * raises ValueError when the count is not zero (preparation is one-time work,
 * off the hot path). Weights prepared from such bytes give NaN in the output
 * columns they touch. */
nvfp4_status nvfp4_prepare_weight(const uint8_t *w_codes, const uint8_t *w_scales, int scale_kind,
                                  int64_t N, int64_t K, uint8_t *w_prep, int32_t *bad_count_dev,
                                  void *stream);

/* W4A4 GEMM: D = alpha_eff * (A.SFA)(W.SFW)^T with FP32 accumulation, where
 * alpha_eff = alpha * (*alpha_dev) in FP32 (alpha alone when alpha_dev is NULL).
 *  alpha_col  NULL, or a per-column scale: FP32 [N], device, 4-byte aligned
 *           (a weight with a global or a per-column scale: TileLang PR #3290,
 *           "Summary"). Column n of the output is then scaled by
 *           fl32(alpha_eff * alpha_col[n]) instead of alpha_eff, the product
 *           formed in FP32 before the accumulator is multiplied by it.
 *  a_codes  [M][K/2] bytes, device, 16-byte aligned (rows are K/2 bytes apart).
 *  a_scales [M][K/16] bytes, device, E4M3 or UE4M3 bytes read as E4M3, 4-byte
 *           aligned. A NaN scale (0x7F/0xFF) propagates NaN into its output row.
 *  w_prep   prepared weight of shape (N, K).
 *  d        [M][ldd] elements of out_dtype (FP32 or BF16 with round-to-nearest-
 *           even), device, element-aligned; ldd >= N.
 *  M >= 0 (M == 0 is a no-op), N % 32 == 0, K % 64 == 0.
 *  config  NULL (nvfp4_get_config's choice), or an explicit launch
 *      configuration: kernel NVFP4_KERNEL_W4A4_TILES (or AUTO), tile_m ==
 *      tile_n == 256 or 128, tail NONE / QUADRANTS / SPLIT with split_k in
 *      [2, K/64] (256 x 256 tiles only), dynamic 0 or 1, num_cus >= 0. An
 *      invalid config returns NVFP4_ERR_VALUE.
 *  ws  workspace of nvfp4_config_workspace_bytes(NVFP4_OP_W4A4, M, N, K, config)
 *      bytes (nvfp4_workspace_bytes for config == NULL), device, 16-byte
 *      aligned, no initialisation needed: the call first copies A into it in
 *      the prepared tile layout (nvfp4_tile_activation), then runs the GEMM
 *      from there (nvfp4_gemm_w4a4_tiled), with the K-split partials and the
 *      dynamic scheduler's counters (reset by a kernel on every call) in the
 *      rest. Calls that share a workspace must not run concurrently.
 * The K split of the tail (row "split-K partials + fixed-order reduce": TileLang
 * PR #3290, "Design": FP32 partials of split tiles summed in a fixed order)
 * sums each tile's ranges in range order, so results are bit-identical from
 * call to call; they differ in the last bits from an unsplit launch, whose
 * FP32 sum runs in another order. */
nvfp4_status nvfp4_gemm_w4a4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *w_prep,
                             int64_t M, int64_t N, int64_t K, float alpha, const float *alpha_dev,
                             const float *alpha_col, void *d, int out_dtype, int64_t ldd,
                             const nvfp4_config *config, void *ws, size_t ws_bytes, void *stream);

/* Bytes of an activation in the tile layout: nvfp4_prepared_weight_bytes for M
 * rounded up to 32 rows (0 for M <= 0 or K % 64 != 0). */
size_t nvfp4_tiled_activation_bytes(int64_t M, int64_t K);

/* Copies A ([M][K/2] codes, [M][K/16] scale bytes; 16- and 4-byte aligned) into
 * the tile layout of a prepared weight (see nvfp4_prepare_weight) at a_tiled
 * (nvfp4_tiled_activation_bytes(M, K) bytes, 16-byte aligned, device), rows
 * M .. rounded-up-to-32 zero. A plain byte permutation, without the weight's
 * sign/zero folding (the GEMM multiplies by every scale, so none is needed).
 * For an activation that feeds several GEMMs: tile it once, then call
 * nvfp4_gemm_w4a4_tiled. M >= 0 (0 is a no-op), K % 64 == 0. */
nvfp4_status nvfp4_tile_activation(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                   uint8_t *a_tiled, void *stream);

/* nvfp4_gemm_w4a4 on an A that nvfp4_tile_activation has already tiled; the
 * other arguments as there. The workspace (nvfp4_config_workspace_bytes with
 * NVFP4_OP_W4A4_TILED) holds only the K-split partials and the scheduler's
 * counters. With config == NULL, ws may be NULL: the call then runs the
 * chosen configuration without them (a K-split tail as quadrants, a dynamic
 * schedule as the static one), so it needs no workspace at all. */
nvfp4_status nvfp4_gemm_w4a4_tiled(const uint8_t *a_tiled, const uint8_t *w_prep, int64_t M, int64_t N, int64_t K,
                                   float alpha, const float *alpha_dev, const float *alpha_col, void *d,
                                   int out_dtype, int64_t ldd, const nvfp4_config *config, void *ws,
                                   size_t ws_bytes, void *stream);

/* Two-pass W4A4 GEMM: D = alpha_eff * (A1 + A2)(W.SFW)^T, A1 and A2 the two
 * passes of nvfp4_quantize_two_pass_tiled (a2_tiled, rows M, K columns per
 * pass) against a prepared weight of shape (N, K): one contraction over 2K in
 * which the residual half reads the same W chunks as the value half (TileLang
 * PR #3290, "Follow-ups"). alpha_eff as for nvfp4_gemm_w4a4 (the passes share
 * g, so alpha is the one-pass prefill's 1/(gA gW)); other arguments, the
 * config (sized for a contraction of length 2K) and the workspace
 * (NVFP4_OP_W4A4_TILED with K = 2K) as for nvfp4_gemm_w4a4_tiled. */
nvfp4_status nvfp4_gemm_w4a4_two_pass_tiled(const uint8_t *a2_tiled, const uint8_t *w_prep, int64_t M, int64_t N,
                                            int64_t K, float alpha, const float *alpha_dev, const float *alpha_col,
                                            void *d, int out_dtype, int64_t ldd, const nvfp4_config *config,
                                            void *ws, size_t ws_bytes, void *stream);

/* W4A16 GEMM: y = alpha_eff * x (W.SFW)^T, x and y BF16, FP32 accumulation
 * (TileLang PR #3290, "Summary": BF16 activations against NVFP4 weights with
 * E4M3 block scales, for M = 1 .. 1024 rows). alpha, alpha_dev and alpha_col
 * (NULL or FP32 [N]: column n scaled by fl32(alpha_eff * alpha_col[n])) as for
 * nvfp4_gemm_w4a4.
 *  x  [M][ldx] BF16 (uint16 bit patterns), device, 16-byte aligned, ldx % 8 == 0, ldx >= K.
 *  y  [M][ldy] BF16, device, 2-byte aligned, ldy >= N.
 *  M >= 0, N % 32 == 0, K % 64 == 0.
 *  config  NULL (nvfp4_get_config's choice) or an explicit kernel
 *      (TileLang PR #3290, "Tests": explicit configs): DECODE (M <= 4 and
 *      M * K * 2 <= 64 KiB), SKINNY (M <= 64) or TILES with (tile_m, tile_n)
 *      = (256, 256), (128, 256) or (128, 128); tail, split_k and dynamic 0.
 *      An invalid config returns NVFP4_ERR_VALUE.
 *  ws  workspace of nvfp4_config_workspace_bytes(NVFP4_OP_W4A16, M, N, K,
 *      config) bytes (may be NULL when that is 0). Calls that share a
 *      workspace must not run concurrently (use one workspace per stream). */
nvfp4_status nvfp4_gemm_w4a16(const uint16_t *x, int64_t ldx, const uint8_t *w_prep, int64_t M,
                              int64_t N, int64_t K, float alpha, const float *alpha_dev,
                              const float *alpha_col, uint16_t *y, int64_t ldy, const nvfp4_config *config,
                              void *ws, size_t ws_bytes, void *stream);

/* BF16 -> NVFP4 quantizer for activations fed to W4A4 (the format as the pages
 * use it: packed E2M1 codes, E4M3 block scales, a per-tensor global scale;
 * TileLang PR #3290, "Summary". The pages do not print the recipe; this library
 * uses: per-tensor g = 2688 / max|x| (1 if the tensor is zero); per 16-block
 * scale = E4M3_RNE_sat((amax_b / 6) * g); codes = E2M1_RNE_sat(x * (g / scale))
 * with x's sign, all in IEEE FP32; zero-scale blocks get zero codes).
 *  x       [rows][K] BF16, device, 16-byte aligned, K % 16 == 0 and K % 8 == 0.
 *  codes   [rows][K/2] bytes out, 8-byte aligned.  scales [rows][K/16] UE4M3 bytes out.
 *  g_dev   device float out: g.  inv_g_dev  device float out (may be NULL): 1/g in FP32.
 *  ws      nvfp4_workspace_bytes(NVFP4_OP_QUANTIZE, rows, 0, K) bytes (no init needed).
 * Inputs must be finite. rows == 0 writes g = 1.
 * When K % 64 == 0 and x fits in the vector registers of one grid that is
 * resident all at once (up to 80 tiles of 32 x 64 per workgroup, one
 * workgroup per CU: 80 MiB of BF16 on 256 CUs), x is read once: the
 * workgroups exchange their maxima through the workspace and wait for each
 * other there once. The wait is bounded (about a second): if kernels on other
 * streams keep some of its workgroups off the CUs for longer than that, the
 * workgroups whose wait ran out encode their rows with g = NaN, which leaves
 * those rows' scales and codes meaningless (and g_dev NaN when workgroup 0 is
 * among them). Larger inputs, and other K, read x twice with no wait. */
nvfp4_status nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales,
                            float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes, void *stream);

/* nvfp4_quantize writing its codes and scales straight into the activation tile
 * layout of nvfp4_tile_activation (a_tiled: nvfp4_tiled_activation_bytes(rows,
 * K) bytes, 16-byte aligned; rows rounded up to 32, the padding rows zero), so
 * a quantized activation feeds nvfp4_gemm_w4a4_tiled with no copy. The same
 * bytes as nvfp4_tile_activation applied to nvfp4_quantize's output.
 * K % 64 == 0; other arguments as for nvfp4_quantize. */
nvfp4_status nvfp4_quantize_tiled(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a_tiled, float *g_dev,
                                  float *inv_g_dev, void *ws, size_t ws_bytes, void *stream);

/* Two-pass activation quantization (TileLang PR #3290, "Follow-ups": the W4A4
 * prefill whose activations are quantized in two NVFP4 passes, value then
 * residual; the pages give no recipe beyond that, this library uses): pass 1
 * is nvfp4_quantize's recipe with the tensor's global scale g; the residual
 * r = x - fl32(code * scale / g) (code * scale exact, then one division and
 * one subtraction in IEEE FP32) is quantized by the same steps (block maximum
 * of |r|, scale, codes) under the same g, so both passes share one alpha.
 *  a2_tiled  nvfp4_tiled_activation_bytes(rows, 2 K) bytes, 16-byte aligned:
 *            the tile layout of a [rows][2K] activation whose K chunks
 *            0 .. K/64 - 1 hold pass 1 and K/64 .. K/32 - 1 pass 2.
 * Other arguments as for nvfp4_quantize_tiled (K % 64 == 0). */
nvfp4_status nvfp4_quantize_two_pass_tiled(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a2_tiled,
                                           float *g_dev, float *inv_g_dev, void *ws, size_t ws_bytes,
                                           void *stream);

/* nvfp4_quantize_tiled for callers that cannot allocate device memory: code
 * under graph capture, tight serving loops, and harnesses that forbid
 * allocation. It takes no workspace and allocates nothing (no hipMalloc, no
 * hipFree): the 12.25 KiB the quantizer needs (the tensor-max pass's
 * per-workgroup maxima, or the one-read form's barrier slots and generation
 * number) live in a static device array of the library, one per GPU, held
 * until the process ends. That size does not depend on rows or K, so no input
 * is too large for it, and nothing needs clearing between calls (each call
 * writes what it reads, or tags it with a generation number it advances). Calls that overlap on one GPU (on
 * different streams) share that array and race: serialise them. The first
 * call on a device looks up the array's address there; nvfp4_init(device)
 * does it up front. Arguments, outputs and errors as for nvfp4_quantize_tiled. */
nvfp4_status nvfp4_quantize_tiled_noalloc(const uint16_t *x, int64_t rows, int64_t K, uint8_t *a_tiled,
                                          float *g_dev, float *inv_g_dev, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
