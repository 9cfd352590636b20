// Launch configurations of the GEMMs: the choice for a call without one (a
// tuned table for the device's CU count when it has the shape, else the
// heuristic of each GEMM), the check of a caller's explicit config, and the
// workspace sizes that follow from a config. Host code only.
//
// TileLang PR #3290 ("Summary", "Changes", "Tests") describes the same three
// parts for its W4A16 GEMM: a shape-independent heuristic get_config, explicit
// configs that callers and tests pass, and per-GPU tuned tables keyed by SM
// count that are not applied on a GPU with another SM count. The Colfax
// article ("Version 7: Autotuning") tunes its W4A4 launch parameters the same
// way, per problem size.
#include "common.hpp"

namespace nvfp4 {

namespace {

// One tuned entry: for a device with `cus` CUs, op, an (N, K) weight shape and
// M in [m_lo, m_hi], the config measured fastest among the valid ones.
struct TunedEntry {
  int cus, op;
  int64_t N, K, m_lo, m_hi;
  nvfp4_config cfg;
};

// Tuned on MI355X (256 CUs), with the benchmark's inputs: every valid config
// of the shape timed back to back on one device, the fastest kept. A shape
// that is not here, or a device with another CU count, takes the heuristic.
constexpr TunedEntry kTuned[] = {
#include "tuned_table.inc"
};

bool is_w4a4(int op) { return op == NVFP4_OP_W4A4 || op == NVFP4_OP_W4A4_TILED; }

}  // namespace

int device_cus_or_default() {
  DeviceInfo d;
  if (device_info(&d) == NVFP4_OK && d.num_cus > 0) return d.num_cus;
  return 256;
}

// The config of a call without one: the tuned entry for (cus, op, N, K, M),
// else the heuristic. W4A4 and its tiled form share entries (the tiled form's
// K is the contraction length).
static bool tuned_config(int op, int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *out) {
  const int key = is_w4a4(op) ? NVFP4_OP_W4A4 : op;
  for (const TunedEntry &e : kTuned) {
    if (e.cus == cus && e.op == key && e.N == N && e.K == K && M >= e.m_lo && M <= e.m_hi) {
      *out = e.cfg;
      out->num_cus = cus;
      out->source = NVFP4_CONFIG_TUNED;
      return true;
    }
  }
  return false;
}

static nvfp4_status default_config(int op, int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *out) {
  if (tuned_config(op, M, N, K, cus, out)) return NVFP4_OK;
  if (is_w4a4(op)) w4a4_default_config(M, N, K, cus, out);
  else if (op == NVFP4_OP_W4A16) w4a16_default_config(M, N, K, cus, out);
  else return NVFP4_ERR_DTYPE;
  out->source = NVFP4_CONFIG_HEURISTIC;
  return NVFP4_OK;
}

static bool config_valid(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  return is_w4a4(op) ? w4a4_config_valid(M, N, K, c) : w4a16_config_valid(M, N, K, c);
}

nvfp4_status resolve_config(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config *req, int device_cus,
                            nvfp4_config *out) {
  if (!req) return default_config(op, M, N, K, device_cus, out);
  nvfp4_config c = *req;
  if (c.num_cus == 0) c.num_cus = device_cus;
  if (is_w4a4(op) && c.kernel == NVFP4_KERNEL_AUTO) c.kernel = NVFP4_KERNEL_W4A4_TILES;
  c.source = NVFP4_CONFIG_EXPLICIT;
  if (!config_valid(op, M, N, K, c)) return NVFP4_ERR_VALUE;
  *out = c;
  return NVFP4_OK;
}

static size_t config_workspace(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config &c) {
  if (is_w4a4(op)) return w4a4_config_workspace_bytes(op, M, N, K, c);
  if (op == NVFP4_OP_W4A16) return w4a16_config_workspace_bytes(M, N, K, c);
  return 0;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_get_config(int op, int64_t M, int64_t N, int64_t K, int num_cus, nvfp4_config *out) {
  if (!out) return NVFP4_ERR_NULL;
  if (!is_w4a4(op) && op != NVFP4_OP_W4A16) return NVFP4_ERR_DTYPE;
  if (M <= 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (num_cus < 0) {   // the heuristic alone, for -num_cus CUs (what tuning compares against)
    if (is_w4a4(op)) w4a4_default_config(M, N, K, -num_cus, out);
    else w4a16_default_config(M, N, K, -num_cus, out);
    out->source = NVFP4_CONFIG_HEURISTIC;
    return NVFP4_OK;
  }
  const int cus = num_cus > 0 ? num_cus : device_cus_or_default();
  return default_config(op, M, N, K, cus, out);
}

extern "C" size_t nvfp4_config_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config *config) {
  if (op == NVFP4_OP_QUANTIZE) return quantize_workspace_bytes(M, K);
  if (!is_w4a4(op) && op != NVFP4_OP_W4A16) return 0;
  if (M <= 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0) return 0;
  nvfp4_config c;
  if (resolve_config(op, M, N, K, config, device_cus_or_default(), &c) != NVFP4_OK) return 0;
  return config_workspace(op, M, N, K, c);
}

extern "C" size_t nvfp4_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
  return nvfp4_config_workspace_bytes(op, M, N, K, nullptr);
}
