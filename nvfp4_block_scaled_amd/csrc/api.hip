// C ABI entry points that are not GEMMs: device init, status strings, sizes,
// workspace init, and the one-time weight preparation kernel.
#include <math.h>
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace nvfp4 {

// One entry per device, filled exactly once (std::call_once), so host threads
// that make their first call at the same time all see a complete entry.
static DeviceInfo g_info[kMaxDevices];
static nvfp4_status g_info_status[kMaxDevices];
static std::once_flag g_info_once[kMaxDevices];

static void fill_device_info(int dev) {
  DeviceInfo &d = g_info[dev];
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
    g_info_status[dev] = NVFP4_ERR_HIP;
    return;
  }
  d.num_cus = p.multiProcessorCount;
  d.gfx950 = (strncmp(p.gcnArchName, "gfx950", 6) == 0);
  d.device = dev;
  g_info_status[dev] = d.gfx950 ? NVFP4_OK : NVFP4_ERR_UNSUPPORTED;
}

nvfp4_status device_info_of(int dev, DeviceInfo *out) {
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
  std::call_once(g_info_once[dev], fill_device_info, dev);
  if (out) *out = g_info[dev];
  return g_info_status[dev];
}

nvfp4_status device_info(DeviceInfo *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  return device_info_of(dev, out);
}

// ---------------------------------------------------------------- kernels

__global__ void fill_zero_kernel(uint32_t *p, size_t nwords) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < nwords; i += stride) p[i] = 0u;
}

// One thread per (row n, 16-block b): fold the block's scale into its codes and
// scatter codes and scale into the 32x64 tile layout described in nvfp4.h.
__global__ __launch_bounds__(256) void prepare_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, int kind,
                                                      int64_t N, int64_t K, uint8_t *__restrict__ prep,
                                                      int32_t *bad_count) {
  const int64_t nblk = K / 16;
  const int64_t total = N * nblk;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t n = idx / nblk;
  const int64_t b = idx - n * nblk;
  u32x2_t c = *reinterpret_cast<const u32x2_t *>(codes + n * (K / 2) + b * 8);
  const uint32_t s = scales[idx];
  const uint32_t mag = s & 0x7Fu;
  uint32_t out_s;
  bool bad, neg, zero;
  if (kind == NVFP4_SCALE_E4M3) {
    bad = (mag == 0x7Fu);
    zero = (mag == 0u);
    neg = ((s & 0x80u) != 0u) && !zero && !bad;
  } else {
    bad = ((s & 0x80u) != 0u) || (s == 0x7Fu);
    zero = (s == 0u);
    neg = false;
  }
  if (bad) {
    out_s = 0x7Fu;
    if (bad_count) atomicAdd(bad_count, 1);
  } else if (zero) {
    out_s = 0u;
    c = u32x2_t{0u, 0u};
  } else {
    out_s = mag;
    if (neg) c ^= u32x2_t{0x88888888u, 0x88888888u};
  }
  const int64_t tile = (n / 32) * (K / 64) + b / 4;
  const int64_t r = n % 32;
  const int64_t bb = b % 4;
  // chunk byte 8 bb of row r: 16-byte unit 32 (bb / 2) + r, byte 8 (bb % 2)
  *reinterpret_cast<u32x2_t *>(prep + tile * 1024 + 16 * (32 * (bb >> 1) + r) + 8 * (bb & 1)) = c;
  prep[N * K / 2 + tile * 128 + r * 4 + bb] = (uint8_t)out_s;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

nvfp4_status nvfp4_init(int device) {
  if (device < 0 || device >= kMaxDevices) return NVFP4_ERR_VALUE;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess) return NVFP4_ERR_HIP;
  if (device >= count) return NVFP4_ERR_VALUE;
  nvfp4_status st = device_info_of(device, nullptr);
  if (st != NVFP4_OK) return st;
  return device_setup(device);
}

const char *nvfp4_status_str(int s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "bad shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_DTYPE: return "bad enum argument";
    case NVFP4_ERR_VALUE: return "non-finite host scalar";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_UNSUPPORTED: return "device is not gfx950";
    case NVFP4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t nvfp4_prepared_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0) return 0;
  return (size_t)(N * K / 2 + N * K / 16);
}

nvfp4_status nvfp4_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (ws_bytes == 0) return NVFP4_OK;
  if (!ws) return NVFP4_ERR_NULL;
  if (!aligned(ws, 16) || ws_bytes % 4 != 0) return NVFP4_ERR_ALIGN;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  size_t nwords = ws_bytes / 4;
  unsigned grid = (unsigned)((nwords + 255) / 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (uint32_t *)ws, nwords);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_prepare_weight(const uint8_t *w_codes, const uint8_t *w_scales, int scale_kind, int64_t N,
                                  int64_t K, uint8_t *w_prep, int32_t *bad_count_dev, void *stream) {
  if (!w_codes || !w_scales || !w_prep) return NVFP4_ERR_NULL;
  if (scale_kind != NVFP4_SCALE_UE4M3 && scale_kind != NVFP4_SCALE_E4M3) return NVFP4_ERR_DTYPE;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 64 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(w_codes, 16) || !aligned(w_prep, 16) || (bad_count_dev && !aligned(bad_count_dev, 4)))
    return NVFP4_ERR_ALIGN;
  DeviceInfo d;
  nvfp4_status st = device_info(&d);
  if (st != NVFP4_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (bad_count_dev) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(64), 0, s, (uint32_t *)bad_count_dev, (size_t)1);
    NVFP4_LAUNCH_CHECK();
  }
  const int64_t total = N * (K / 16);
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7FFFFFFF) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)grid), dim3(256), 0, s, w_codes, w_scales, scale_kind, N, K,
                     w_prep, bad_count_dev);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
