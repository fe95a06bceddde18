// MFMA-only throughput probe (measurement support, not a step of the
// method): how fast the chip runs the fp8 matrix instruction that the GEMM
// is built from, v_mfma_f32_16x16x128_f8f6f4 with E4M3 operands, when
// nothing else runs: no memory traffic, no LDS, no epilogue.  Its rate on
// given operand bytes is the ceiling that the GEMM's main loop can reach on
// such data, under the same board power limit.
//
// Each wave loads 16 fragments (16 rows x 128 B each; 8 play the A role,
// 8 the B role) from a 32 KB slice of the caller's code buffer, then runs
// iters x 512 MFMAs on them into 8 x 8 blocks of fp32 accumulators, the
// GEMM's register layout: per pass, for each B fragment j, the A fragments
// in a snake order (7..0 under even j, 0..7 under odd j), and the pass
// index r rotates which A fragment meets which accumulator block
// ((i + r) mod 8), so successive passes pair the operands differently.
// The accumulators' sum is stored so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int FRAG = 16 * 128;            // bytes of one fragment
constexpr int SET = 16 * FRAG;            // one wave's 16 fragments: 32 KB

__global__ __launch_bounds__(THREADS) void k_mfma_loop(const uint8_t *__restrict__ codes,
                                                       int64_t nsets, int iters,
                                                       float *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6);
  const uint8_t *base = codes + (w % nsets) * SET + lane * 32;
  v8i fa[8], fb[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    fa[f] = *reinterpret_cast<const v8i *>(base + f * FRAG);
    fb[f] = *reinterpret_cast<const v8i *>(base + (8 + f) * FRAG);
  }
  v4f acc[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int i = (j & 1) ? s : 7 - s;
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              fb[j], fa[(i + r) & 7], acc[j][i], 0, 0, 0, 0, 0, 0);
        }
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) t += acc[j][i][0] + acc[j][i][1] + acc[j][i][2] + acc[j][i][3];
  sink[(int64_t)blockIdx.x * THREADS + threadIdx.x] = t;
}

// One instruction per wave on caller-given operands: the accumulation
// behaviour of v_mfma_f32_16x16x128_f8f6f4 itself (how it sums the 128
// products of one k-step and adds them to the accumulator), observed on
// crafted codes.  Case w: P [16][128] and Q [16][128] codes (row-major),
// C and D [16][16] fp32 (row-major), D[i][j] = C[i][j] + sum_k P[i][k] Q[j][k]
// as the instruction forms it.  Operand lanes as in the GEMM: lane l holds
// row l % 16 and bytes 32 (l / 16) .. 32 (l / 16) + 31 of that row; output
// register r of lane l is row i = 4 (l / 16) + r of P, column j = l % 16.
// F0 / F1: code format of P / Q (0 = E4M3, 1 = E5M2).
template <int F0, int F1>
__global__ __launch_bounds__(THREADS) void k_mfma_single(const uint8_t *__restrict__ P,
                                                         const uint8_t *__restrict__ Q,
                                                         const float *__restrict__ C,
                                                         float *__restrict__ D, int64_t ncases) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6);
  if (w >= ncases) return;                 // whole waves only
  const int64_t off = w * FRAG + (lane & 15) * 128 + (lane >> 4) * 32;
  const v8i a = *reinterpret_cast<const v8i *>(P + off);
  const v8i b = *reinterpret_cast<const v8i *>(Q + off);
  v4f c;
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = C[w * 256 + (4 * (lane >> 4) + r) * 16 + (lane & 15)];
  const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F0, F1, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) D[w * 256 + (4 * (lane >> 4) + r) * 16 + (lane & 15)] = d[r];
}

}  // namespace

// P, Q: device buffers of ncases * 2048 code bytes (32-byte aligned); C, D:
// device float[ncases * 256] (C read, D written); fmt_p, fmt_q: 0 = E4M3,
// 1 = E5M2 (pairs (0,0), (0,1), (1,0), (1,1)).  Workgroups of 4 waves, one
// case per wave.  Returns 0, 1 for a bad argument (nothing launched), 5 for
// a launch failure.
extern "C" __attribute__((visibility("default"))) int fp8_probe_mfma_single(
    const void *P, const void *Q, const float *C, float *D, int64_t ncases, int fmt_p,
    int fmt_q, void *stream) {
  if (!P || !Q || !C || !D || ncases < 1 || ncases > (int64_t)1 << 24) return 1;
  if ((fmt_p & ~1) || (fmt_q & ~1)) return 1;
  if ((reinterpret_cast<uintptr_t>(P) & 31) || (reinterpret_cast<uintptr_t>(Q) & 31) ||
      (reinterpret_cast<uintptr_t>(C) & 3) || (reinterpret_cast<uintptr_t>(D) & 3))
    return 1;
  auto k = fmt_p ? (fmt_q ? k_mfma_single<1, 1> : k_mfma_single<1, 0>)
                 : (fmt_q ? k_mfma_single<0, 1> : k_mfma_single<0, 0>);
  const unsigned blocks = (unsigned)((ncases + 3) / 4);
  hipLaunchKernelGGL(k, dim3(blocks), dim3(THREADS), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t *>(P), static_cast<const uint8_t *>(Q), C, D,
                     ncases);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// codes: device buffer of ncodes E4M3 bytes (at least 32768; each wave
// reads one 32 KB slice, wave w slice w mod (ncodes / 32768)); workgroups
// of 256 threads; iters passes of 512 MFMAs per wave (each 2*16*16*128
// flops); sink: device float[workgroups * 256], written.  Returns 0, 1 for
// a bad argument (nothing launched), 5 for a launch failure.
extern "C" __attribute__((visibility("default"))) int fp8_probe_mfma_loop(
    const void *codes, int64_t ncodes, int workgroups, int iters, float *sink, void *stream) {
  if (!codes || !sink || workgroups < 1 || iters < 1 || ncodes < SET) return 1;
  if ((reinterpret_cast<uintptr_t>(codes) & 31) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return 1;
  hipLaunchKernelGGL(k_mfma_loop, dim3((unsigned)workgroups), dim3(THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t *>(codes),
                     ncodes / SET, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
