// Scaled fp8 (E4M3) GEMM for gfx950 with a bf16 epilogue:
//
//   C[m][n] = bf16( fp32( fp32(acc * (1/sa[m])) * (1/sb[n]) ) ),
//   acc     = sum_k value(A[m][k]) * value(B[n][k])      (fp32 accumulate)
//
// Both operands are contiguous along k ("TN"), which is what the forward
// GEMM and both backward GEMMs of a Float8 linear see once quantize has
// written the transposed copies.  The fp8 GEMMs are the reason the method
// exists (the forum index "torchtitan", topic "Enabling Float8 All-Gather in
// FSDP2": fp8 speeds up large GEMMs; "Torchtitan: A PyTorch Library for
// Parallelism Techniques explained", section 3, "Float8 Training").
//
// Design (CDNA4):
//  - 256 x 256 output tile per 512-thread workgroup (8 wave64s in a 2 x 4
//    grid, 128 x 64 outputs per wave = 4 x 2 MFMA tiles of 32 x 32).
//  - K step of 128 bytes; per step each wave issues 2 x 8 MFMAs of
//    v_mfma_f32_32x32x64_f8f6f4 (format 0 = E4M3 for both operands, no
//    block scales), accumulating in 128 fp32 registers.
//  - A and B K-slabs are staged in LDS (2 x 32 KB per stage, two stages =
//    128 KB of gfx950's 160 KB) with one barrier per K step: the global
//    loads of step k+1 are issued before the MFMAs of step k and written to
//    the other stage after them.
//  - LDS rows are 128 bytes; the eight 16-byte chunks of row r are stored
//    XOR-swizzled by (r % 8), so the eight consecutive rows that a group of
//    lanes reads for one MFMA operand hit eight different chunk positions
//    (no bank conflicts for ds_read_b128), and the global->LDS writes stay
//    conflict-free too.
//  - Workgroups are remapped so that consecutive tiles of the grouped
//    (GROUP_M tile-rows at a time) order land on the same XCD and share its
//    L2.
//  - Tails: rows beyond M / N and 16-byte K chunks beyond K are loaded as
//    zeros, outputs beyond M / N are not stored (M, N, K multiples of 16).
#include "fp8l_internal.h"

namespace fp8l {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;          // bytes = fp8 elements along K per stage
constexpr int THREADS = 512;
constexpr int WAVES_M = 2;
constexpr int WAVES_N = 4;
constexpr int WM = BM / WAVES_M; // 128 rows per wave
constexpr int WN = BN / WAVES_N; // 64 cols per wave
constexpr int TM = WM / 32;      // 4 MFMA tiles along M per wave
constexpr int TN = WN / 32;      // 2 MFMA tiles along N per wave
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;
constexpr int LOADS_A = BM * BK / 16 / THREADS;  // 16-byte loads per thread
constexpr int LOADS_B = BN * BK / 16 / THREADS;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// blockIdx -> (tile_m, tile_n): blocks are dealt to the XCDs round-robin, so
// block b runs on XCD b % 8.  Renumber so that each XCD receives one
// contiguous range of the grouped tile order.
__device__ __forceinline__ void tile_of_block(int b, int nblocks, int tiles_m,
                                              int tiles_n, int &tm, int &tn) {
  const int xcd = b % NUM_XCD;
  const int local = b / NUM_XCD;
  int base = 0;
  for (int x = 0; x < xcd; ++x) base += (nblocks - x + NUM_XCD - 1) / NUM_XCD;
  const int p = base + local;
  const int group = GROUP_M * tiles_n;
  const int first_m = (p / group) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = p % group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

__global__ __launch_bounds__(THREADS) void k_gemm_fp8_tn(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, int a_vec,
    const uint8_t *__restrict__ B, const float *__restrict__ sb, int b_vec,
    int M, int N, int K, uint16_t *__restrict__ C, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  // global -> register staging of one K step
  uint4 ra[LOADS_A], rb[LOADS_B];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LOADS_A; ++i) {
      const int id = tid + i * THREADS;
      const int row = id >> 3, ck = id & 7;
      const int gm = m0 + row, gk = k0 + ck * 16;
      ra[i] = (gm < M && gk < K)
                  ? *reinterpret_cast<const uint4 *>(A + (size_t)gm * K + gk)
                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < LOADS_B; ++i) {
      const int id = tid + i * THREADS;
      const int row = id >> 3, ck = id & 7;
      const int gn = n0 + row, gk = k0 + ck * 16;
      rb[i] = (gn < N && gk < K)
                  ? *reinterpret_cast<const uint4 *>(B + (size_t)gn * K + gk)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int stage) {
    uint8_t *sA = smem[stage];
    uint8_t *sB = smem[stage] + BM * BK;
#pragma unroll
    for (int i = 0; i < LOADS_A; ++i) {
      const int id = tid + i * THREADS;
      *reinterpret_cast<uint4 *>(sA + swz(id >> 3, id & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LOADS_B; ++i) {
      const int id = tid + i * THREADS;
      *reinterpret_cast<uint4 *>(sB + swz(id >> 3, id & 7)) = rb[i];
    }
  };

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  const int lrow = lane & 31;         // operand row within a 32-row tile
  const int khalf = lane >> 5;        // which 32-byte half of a 64-byte K slice

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const uint8_t *sA = smem[stage];
    const uint8_t *sB = smem[stage] + BM * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 64; ++kk) {
      const int ck = kk * 4 + khalf * 2;   // first of the two 16-byte chunks
      v8i a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + lrow;
        const uint4 lo = *reinterpret_cast<const uint4 *>(sA + swz(row, ck));
        const uint4 hi = *reinterpret_cast<const uint4 *>(sA + swz(row, ck + 1));
        a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 32 + lrow;
        const uint4 lo = *reinterpret_cast<const uint4 *>(sB + swz(row, ck));
        const uint4 hi = *reinterpret_cast<const uint4 *>(sB + swz(row, ck + 1));
        b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[i], b[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(stage ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column n = lane % 32 of each 32x32 tile and rows
  // (r / 4) * 8 + (lane / 32) * 4 + r % 4 for its 16 accumulators r.
  const float inv_a0 = a_vec ? 0.f : 1.0f / sa[0];
  const float inv_b0 = b_vec ? 0.f : 1.0f / sb[0];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * WN + j * 32 + lrow;
    if (n >= N) continue;
    const float inv_b = b_vec ? 1.0f / sb[n] : inv_b0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * WM + i * 32 + (r >> 2) * 8 + khalf * 4 + (r & 3);
        if (m < M) {
          const float inv_a = a_vec ? 1.0f / sa[m] : inv_a0;
          float v = acc[i][j][r] * inv_a;
          v = v * inv_b;
          C[(size_t)m * N + n] = (uint16_t)bf16_rne(v);
        }
      }
    }
  }
}

}  // namespace

hipError_t gemm_launch(const uint8_t *A, const float *sa, int a_vec,
                       const uint8_t *B, const float *sb, int b_vec, int64_t M,
                       int64_t N, int64_t K, uint16_t *C, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(k_gemm_fp8_tn, dim3((unsigned)(tiles_m * tiles_n)), dim3(THREADS), 0,
                     stream, A, sa, a_vec, B, sb, b_vec, (int)M, (int)N, (int)K, C,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8l
