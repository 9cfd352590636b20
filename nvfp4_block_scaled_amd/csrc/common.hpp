// Shared device helpers for the gfx950 NVFP4 kernels: vector types, the exact
// E2M1/E4M3 -> FP16/BF16 unpack, and host-side launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- unpack
//
// An NVFP4 element is code * scale with a 2-significant-bit E2M1 code and a
// 4-significant-bit E4M3 scale, so the product has at most 6 significant bits
// and lies in [2^-10, 2688]: FP16 holds every such product exactly as a normal
// number, and so does BF16. The gfx950 conversions below apply only the
// exponent of their FP32 scale operand, so they are used with scale 1.0 (an
// exact E2M1 -> FP16/BF16 or E4M3 -> FP16/F32 conversion) and the E4M3 scale
// is multiplied in afterwards.

// Two scale bytes (bits 0..15 of w) -> their exact FP16 values.
__device__ __forceinline__ half2_t e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// Two scale bytes (bits 0..15 of w) -> their exact FP32 values.
__device__ __forceinline__ f32x2_t e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}

// 8 packed E2M1 codes (k, k+1, ..., k+7 from the low nibble up) times one FP16
// scale -> 8 exact FP16 products in k order. Four conversions and four packed
// multiplies; every product is exact, so the multiply does not round.
__device__ __forceinline__ half8_t dequant8_f16(uint32_t w, _Float16 s) {
  half2_t sc = {s, s};
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  half8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// 8 packed E2M1 codes times one FP32 scale -> 8 exact BF16 products in k order.
// The codes convert exactly to FP32, the FP32 product is exact (6 significant
// bits), and the round-to-nearest-even conversion to BF16 is then exact too.
__device__ __forceinline__ bf16x8_t dequant8_bf16(uint32_t w, float s) {
  f32x2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  bf16x8_t r = {(__bf16)(q0[0] * s), (__bf16)(q0[1] * s), (__bf16)(q1[0] * s), (__bf16)(q1[1] * s),
                (__bf16)(q2[0] * s), (__bf16)(q2[1] * s), (__bf16)(q3[0] * s), (__bf16)(q3[1] * s)};
  return r;
}

// 8 packed E2M1 codes -> 8 exact unscaled BF16 values in k order (as 4 pairs).
__device__ __forceinline__ void codes8_to_bf16(uint32_t w, bf16x2_t out[4]) {
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
}

// A dword as two BF16 values (low half first). Goes through a scalar copy:
// clang 22 mis-lowers __builtin_bit_cast applied directly to an element of an
// ext_vector (it reads element 0 whatever the index).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
  bf16x2_t b;
  __builtin_memcpy(&b, &u, 4);
  return b;
}

// FP32 -> BF16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  __bf16 b = (__bf16)v;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float load_alpha(float alpha, const float *alpha_dev) {
  return alpha_dev ? alpha * __builtin_nontemporal_load(alpha_dev) : alpha;
}

// The alpha of output column n: alpha_eff times the column's own scale
// alpha_col[n] (one FP32 product), or alpha_eff when there is no per-column scale.
__device__ __forceinline__ float col_alpha(float al, const float *alpha_col, int64_t n) {
  return alpha_col ? al * alpha_col[n] : al;
}

// ---------------------------------------------------------------- host side

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
  bool gfx950 = false;
};

constexpr int kMaxDevices = 64;

// Per-device properties of the current device (device_info) or of a given one,
// filled once per device by nvfp4_init or by the first call that needs them.
nvfp4_status device_info(DeviceInfo *out);
nvfp4_status device_info_of(int dev, DeviceInfo *out);

// Per-device set-up done by nvfp4_init beyond device_info (it makes `device`
// current for the duration of the call and restores the caller's device).
nvfp4_status device_setup(int device);

// Workspace of the quantizer (0 = none), and A in the tile layout.
size_t quantize_workspace_bytes(int64_t rows, int64_t K);
size_t tiled_activation_bytes(int64_t M, int64_t K);

// Launch configurations (config.hip): the heuristic of each GEMM, the check of
// an explicit config, and the workspace a config needs (0 for an invalid one).
// A resolved config has its kernel and num_cus set.
void w4a4_default_config(int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *c);
bool w4a4_config_valid(int64_t M, int64_t N, int64_t K, const nvfp4_config &c);
size_t w4a4_config_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config &c);
void w4a16_default_config(int64_t M, int64_t N, int64_t K, int cus, nvfp4_config *c);
bool w4a16_config_valid(int64_t M, int64_t N, int64_t K, const nvfp4_config &c);
size_t w4a16_config_workspace_bytes(int64_t M, int64_t N, int64_t K, const nvfp4_config &c);

// The config a call runs: the caller's (checked: NVFP4_ERR_VALUE if invalid;
// num_cus 0 becomes device_cus) or, for NULL, the tuned table's / heuristic's
// for device_cus CUs.
nvfp4_status resolve_config(int op, int64_t M, int64_t N, int64_t K, const nvfp4_config *req, int device_cus,
                            nvfp4_config *out);

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace nvfp4

#define NVFP4_LAUNCH_CHECK()                                  \
  do {                                                        \
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP; \
  } while (0)
