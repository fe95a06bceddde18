// Internal declarations of the gfx950 Float8 linear library: device helpers
// shared by the kernels and the host-side launchers called by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8_linear.h"

namespace fp8l {

// ------------------------------------------------------------ device math --

// bf16 bit pattern -> fp32 (exact: bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// Saturating round-to-nearest-even E4M3 ("fn") codes of four fp32 values,
// packed little-endian into one dword (a in byte 0 ... d in byte 3).
// Magnitudes >= 448 clamp to 448 before the hardware conversion (which
// rounds to nearest even); NaN bypasses the clamp so it stays NaN.
__device__ __forceinline__ float sat448(float v) {
  float c = __builtin_amdgcn_fmed3f(v, -FP8L_E4M3_MAX, FP8L_E4M3_MAX);
  return (v != v) ? v : c;
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

// Saturating round-to-nearest-even E5M2 codes (gradients): magnitudes
// >= 57344 clamp to 57344 (so +-inf too) before the hardware conversion;
// NaN bypasses the clamp.
__device__ __forceinline__ float sat57344(float v) {
  float c = __builtin_amdgcn_fmed3f(v, -FP8L_E5M2_MAX, FP8L_E5M2_MAX);
  return (v != v) ? v : c;
}

__device__ __forceinline__ uint32_t e5m2x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(sat57344(a), sat57344(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(sat57344(c), sat57344(d), w, true);
  return (uint32_t)w;
}

// Code format of a quantized operand: 0 = E4M3, 1 = E5M2.
template <int FMT>
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  return FMT ? e5m2x4(a, b, c, d) : e4m3x4(a, b, c, d);
}

// Scale from an amax: s = fmax / max(a, 1e-12) as one IEEE fp32 division
// (HIP's default fp32 divide is correctly rounded), fmax = 448 (E4M3) or
// 57344 (E5M2).  A NaN amax compares false and yields NaN.
template <int FMT = 0>
__device__ __forceinline__ float scale_from_amax(float a) {
  float d = (a < FP8L_AMAX_EPS) ? FP8L_AMAX_EPS : a;
  return (FMT ? FP8L_E5M2_MAX : FP8L_E4M3_MAX) / d;
}

// ---------------------------------------------------------- host launchers --

// Quantize (amax partials -> scales -> cast + transpose), all enqueued on
// `stream`.  Arguments were validated by the C ABI.
size_t quantize_workspace_bytes(int64_t rows, int64_t cols, int scaling);
hipError_t quantize_launch(const void *x, int64_t rows, int64_t cols,
                           int scaling, void *q, void *qt, float *scale,
                           float *scale_t, float *amax_out, void *workspace,
                           hipStream_t stream);
hipError_t encode_launch(const float *in, uint8_t *out, int64_t n, int fmt,
                         hipStream_t stream);
// Tensorwise amax of x into amax_out[0] (workspace: the tensorwise quantize
// workspace of the same shape).
hipError_t amax_launch(const void *x, int64_t rows, int64_t cols, float *amax_out,
                       void *workspace, hipStream_t stream);
// Cast with a given tensorwise multiplier scale[0]: q and its transpose qt.
hipError_t quantize_scaled_launch(const void *x, int64_t rows, int64_t cols,
                                  const float *scale, void *q, void *qt, hipStream_t stream);

// C[M,N] (bf16) = (A[M,K] . B[N,K]^T) * (1/sa) * (1/sb); with rowwise, sa
// has M entries and sb N entries, else one each.
// fmt_a: code format of A (0 = E4M3, 1 = E5M2); B is E4M3.
hipError_t gemm_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                       const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                       int64_t K, uint16_t *C, hipStream_t stream);
// The same GEMM with fp32 output: C32[M,N] = fl32(fl32(acc / sa) / sb).
hipError_t gemm_f32_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                           const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                           int64_t K, float *C, hipStream_t stream);

}  // namespace fp8l
