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

// ------------------------------------------------- amax partial maxima --
//
// The amax is taken on |bf16| bit patterns with integer max (for
// non-negative values the bit order is the value order; NaN patterns sort
// above +inf).  A producer kernel that writes a bf16 tensor can take its
// partial maxima on the way, in one of the two layouts the quantize's
// second half reads:
//  - tensorwise: u32 part[nb], one maximum per workgroup, nb <= TW_MAX_BLOCKS
//  - rowwise: tiles of AM_TR rows x AM_TC columns; u16 rowpart[tiles_c][rows]
//    (row maxima over one tile's columns) and colpart[tiles_r][cols]
//    (column maxima over one tile's rows), where quantize_rowwise_partials
//    places them in the workspace.
constexpr int AM_TR = 64;
constexpr int AM_TC = 256;
constexpr int AM_THREADS = 256;
constexpr int TW_MAX_BLOCKS = 2048;

// per-half maxima of two u16 pairs
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  uint32_t lo = max(a & 0xFFFFu, b & 0xFFFFu);
  uint32_t hi = max(a >> 16, b >> 16);
  return lo | (hi << 16);
}

// max over the two u16 halves of a dword
__device__ __forceinline__ uint32_t hmax16(uint32_t a) {
  return max(a & 0xFFFFu, a >> 16);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// max over the 32 lanes of each half-wave
__device__ __forceinline__ uint32_t half_wave_max(uint32_t v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 load16(const void *p) {
  uint4 v = *reinterpret_cast<const uint4 *>(p);
  return {v.x, v.y, v.z, v.w};
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
// The second half of quantize_launch for an x whose partial maxima a
// producer kernel has already written into `workspace` (layouts above):
// rowwise, the row / column scales, then the cast; tensorwise, the cast,
// whose workgroups reduce the nparts block maxima (nparts = 0: x is empty).
hipError_t quantize_finish_launch(const void *x, int64_t rows, int64_t cols, int scaling,
                                  int nparts, void *q, void *qt, float *scale,
                                  float *scale_t, float *amax_out, void *workspace,
                                  hipStream_t stream);
// Where the rowwise partial maxima of a [rows, cols] x sit in a quantize
// workspace.
void quantize_rowwise_partials(void *workspace, int64_t rows, int64_t cols,
                               uint16_t **rowpart, uint16_t **colpart);
// Tensorwise amax of x into amax_out[0] (workspace: the tensorwise quantize
// workspace of the same shape).
hipError_t amax_launch(const void *x, int64_t rows, int64_t cols, float *amax_out,
                       void *workspace, hipStream_t stream);
// Cast with a given tensorwise multiplier scale[0]: q and its transpose qt.
hipError_t quantize_scaled_launch(const void *x, int64_t rows, int64_t cols,
                                  const float *scale, void *q, void *qt, hipStream_t stream);

// The fp8 copies and scales of one quantized tensor.
struct Fp8Out {
  void *q, *qt;
  float *scale, *scale_t, *amax;
};

// SwiGLU producers (swiglu.hip): the elementwise pass writes its bf16
// outputs with their amax partial maxima, then each output's quantize
// finishes with quantize_finish_launch.  The workspace holds two shares,
// one per output.
size_t swiglu_workspace_bytes(int64_t rows, int64_t hidden, int scaling);
hipError_t swiglu_fwd_launch(const void *a, const void *b, int64_t rows, int64_t hidden,
                             int scaling, void *h, void *hq, void *hqt, float *scale,
                             float *scale_t, float *amax_out, void *workspace,
                             hipStream_t stream);
hipError_t swiglu_bwd_launch(const void *dh, const void *a, const void *b, int64_t rows,
                             int64_t hidden, int scaling, void *da, void *db,
                             const Fp8Out &qa, const Fp8Out &qb, void *workspace,
                             hipStream_t stream);

// C[M,N] (bf16) = (A[M,K] . B[N,K]^T) * (1/sa) * (1/sb); with rowwise, sa
// has M entries and sb N entries, else one each.
// fmt_a: code format of A (0 = E4M3, 1 = E5M2); B is E4M3.
hipError_t gemm_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                       const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                       int64_t K, uint16_t *C, hipStream_t stream);
// Several such GEMMs (bf16 outputs, same scaling and format of A) in one
// launch; count 1..4.
struct GemmDesc {
  const uint8_t *A;
  const float *sa;
  const uint8_t *B;
  const float *sb;
  void *C;
  int64_t M, N, K;
};
hipError_t gemm_group_launch(const GemmDesc *d, int count, int rowwise, int fmt_a,
                             hipStream_t stream);
// The same GEMM added into C: C = bf16(fl32(C) + fl32(bf16 GEMM result)).
hipError_t gemm_acc_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                           const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                           int64_t K, uint16_t *C, hipStream_t stream);
// The same GEMM with fp32 output: C32[M,N] = fl32(fl32(acc / sa) / sb).
hipError_t gemm_f32_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                           const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                           int64_t K, float *C, hipStream_t stream);

}  // namespace fp8l
