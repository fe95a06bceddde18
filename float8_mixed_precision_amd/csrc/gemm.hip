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
// Design (CDNA4; one 256-thread workgroup per CU, 1 wave per SIMD):
//  - Output tile 256 x 256; 4 wave64s in a 2 x 2 grid own 128 x 128 each =
//    4 x 4 tiles of v_mfma_f32_32x32x64_f8f6f4 (format 0 = E4M3 for both
//    operands, no block scales).  A wave's 256 fp32 accumulators live in
//    AGPRs; its operand fragments are double-buffered in VGPRs.
//  - K advances 128 bytes per stage, so every LDS row is one full 128-byte
//    cache line of a global row: loads of whole lines run at about twice
//    the per-CU rate of half lines.  Two 64 KB stages (A slab 256 x 128 B,
//    B slab 256 x 128 B) are filled by buffer_load_dwordx4 ... lds (global
//    to LDS without VGPRs); each wave-instruction moves 8 rows x 128 B.
//  - A stage is two MFMA k-steps of 64 bytes.  Per k-tile t:
//      half-step 0: 16 MFMAs on k-step (t,0), interleaved with the reads of
//                   (t,1)'s fragments from stage t%2;
//      wait for this wave's DMA of k-tile t+1, one barrier (everyone's DMA
//      landed, everyone finished reading stage t%2);
//      half-step 1: 16 MFMAs on (t,1), interleaved with the reads of
//                   (t+1,0)'s fragments from the other stage and with the
//                   16 DMA transfers of k-tile t+2 into stage t%2.
//    A DMA thus has two half-steps to land, and the only wait is vmcnt(0).
//  - Chunk c (16 B) of LDS row r sits at c ^ h(r), h(r) = (r & 7) ^
//    ((r >> 3) & 1): conflict-free for the 32-row fragment reads whether a
//    ds_read_b128 phase serves 8 lanes / 128 B or 16 lanes / 256 B.  The
//    swizzle is applied on the global side of the DMA (which writes each
//    instruction's 64 x 16 B to consecutive LDS addresses).
//  - M, N and K tails: rows past M / N and 16-byte chunks past K are read
//    through buffer offsets past the buffer size, which return zeros.
//  - The MFMA's first operand is the B (n) fragment, the second the A (m)
//    fragment, so a lane holds 4 consecutive n of one m.  The epilogue
//    scales, rounds to bf16 (v_cvt_pk_bf16_f32, round to nearest even) and
//    stages the 128 x 128 tile in LDS to write whole 256-byte rows with
//    16-byte buffer stores (out-of-range stores are dropped by the buffer
//    bounds check).
//  - Workgroups are renumbered so that each XCD receives one contiguous
//    range of a grouped tile order (GROUP_M tile-rows at a time), for L2
//    reuse.
//
// Accumulation precision of the instruction (measured on gfx950): products
// are exact; the products of each group of 8 consecutive k are summed in a
// fixed-point window of about 13-14 bits below the group's largest product,
// and the group sums are then added to the accumulator at fp32 precision.
#include "fp8l_internal.h"

namespace fp8l {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                  // fp8 elements (bytes) of K per stage
constexpr int THREADS = 256;
constexpr int WM = 128;                  // rows per wave
constexpr int WN = 128;                  // cols per wave
constexpr int TM = WM / 32;              // MFMA tiles along M per wave
constexpr int TN = WN / 32;              // MFMA tiles along N per wave
constexpr int SLAB = BM * BK;            // 32 KB
constexpr int STAGE_BYTES = 2 * SLAB;    // 64 KB: A slab, then B slab
constexpr int EP_STRIDE = 272;           // staged output row: 256 B + 16 B pad
constexpr int EP_WAVE = WM * EP_STRIDE;  // staged output of one wave
constexpr int LDS_BYTES = 2 * STAGE_BYTES > 4 * EP_WAVE ? 2 * STAGE_BYTES : 4 * EP_WAVE;
constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = 0x80000000u;    // operand offset that reads as zero
constexpr uint32_t OOB_C = 0xFFFFFF00u;  // output offset that is dropped

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// s_waitcnt with only one counter constrained (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// One 16-byte global -> LDS transfer per lane: lane i's bytes land at LDS
// address m0 + 16 i.  Inline asm, so that the compiler neither moves LDS
// reads across it nor inserts waits of its own; completion is tracked with
// explicit vmcnt waits.  m0 is named as clobbered (nothing else in this
// kernel uses it); clang warns that it does not track reserved registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr,
                                      uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

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

template <bool KFULL>   // K % 128 == 0: no K tail, no per-chunk K check
__global__ __launch_bounds__(THREADS) void k_gemm_fp8_tn(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, int a_vec,
    const uint8_t *__restrict__ B, const float *__restrict__ sb, int b_vec,
    int M, int N, int K, uint16_t *__restrict__ C, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int kh = lane >> 5;            // which 32-byte half of a 64-byte k-step

  int tmi, tni;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * BM;
  const int n0 = tni * BN;

  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, M * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, N * K, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsC =
      __builtin_amdgcn_make_buffer_rsrc((void *)C, (short)0, M * N * 2, 0x00020000);

  // ---- DMA: wave w, instruction q (0..15; 0..7 A, 8..15 B) fills slab
  // rows w*64 + (q&7)*8 + lane/8.  Row r keeps logical chunk c at physical
  // chunk c ^ h(r) with h(r) = lane/8 ^ (q & 1) here, so lane i loads
  // logical chunk (i % 8) ^ (i / 8) ^ (q & 1).  The per-lane row offsets are
  // fixed for the whole loop; k0 travels in the scalar offset.
  const int lr = lane >> 3;
  const int c_even = (lane & 7) ^ lr;
  const int c_odd = c_even ^ 1;
  const int klim_e = K - c_even * 16;          // chunk valid while k0 < klim
  const int klim_o = K - c_odd * 16;
  uint32_t voff[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = (q >= 8 ? n0 : m0) + wave * 64 + (q & 7) * 8 + lr;
    const int lim = q >= 8 ? N : M;
    const int c = (q & 1) ? c_odd : c_even;
    voff[q] = row < lim ? (uint32_t)(row * K + c * 16) : OOB;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
  const uint32_t wave_dst = lds_base + (uint32_t)(wave * 64 * BK);

#define FP8L_DMA1(STAGE, KT, Q)                                                   \
  do {                                                                            \
    const uint32_t k0_ = (uint32_t)((KT) * BK);                                   \
    const bool kok_ = KFULL || (int)k0_ < (((Q) & 1) ? klim_o : klim_e);          \
    const uint32_t dst_ = wave_dst + (uint32_t)((STAGE) * STAGE_BYTES +           \
                          ((Q) >= 8 ? SLAB : 0) + ((Q) & 7) * 1024);              \
    dma16((Q) >= 8 ? rsB : rsA, dst_, kok_ ? voff[Q] : OOB, k0_);                 \
  } while (0)
#define FP8L_DMAALL(ST, KT)                                                       \
  FP8L_DMA1(ST, KT, 0); FP8L_DMA1(ST, KT, 1); FP8L_DMA1(ST, KT, 2);               \
  FP8L_DMA1(ST, KT, 3); FP8L_DMA1(ST, KT, 4); FP8L_DMA1(ST, KT, 5);               \
  FP8L_DMA1(ST, KT, 6); FP8L_DMA1(ST, KT, 7); FP8L_DMA1(ST, KT, 8);               \
  FP8L_DMA1(ST, KT, 9); FP8L_DMA1(ST, KT, 10); FP8L_DMA1(ST, KT, 11);             \
  FP8L_DMA1(ST, KT, 12); FP8L_DMA1(ST, KT, 13); FP8L_DMA1(ST, KT, 14);            \
  FP8L_DMA1(ST, KT, 15);

  // ---- fragment reads: row = wm*128 + i*32 + lane%32 (h(row) depends only
  // on lane%16); k-step kk reads logical chunks kk*4 + kh*2 + {0, 1}
  const int hr = (lane & 7) ^ ((lane >> 3) & 1);
  const int fArow = (wm * WM + (lane & 31)) * BK;
  const int fBrow = SLAB + (wn * WN + (lane & 31)) * BK;
  const int fc00 = (((0 * 4 + kh * 2 + 0) ^ hr) << 4);
  const int fc01 = (((0 * 4 + kh * 2 + 1) ^ hr) << 4);
  const int fc10 = (((1 * 4 + kh * 2 + 0) ^ hr) << 4);
  const int fc11 = (((1 * 4 + kh * 2 + 1) ^ hr) << 4);

  v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
  v16f acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // 16-byte piece Q (0..15) of a fragment set, in the order the MFMAs
  // consume them: B0, A0, A1, A2, A3, B1, B2, B3 (low, high halves)
#define FP8L_READ1(STAGE, KK, Q, NA, NB)                                          \
  do {                                                                            \
    constexpr int p_ = (Q) / 2, h_ = (Q) % 2;                                     \
    constexpr bool isb_ = p_ == 0 || p_ >= 5;                                     \
    constexpr int f_ = p_ == 0 ? 0 : (p_ <= 4 ? p_ - 1 : p_ - 4);                 \
    const int co_ = (KK) == 0 ? (h_ ? fc01 : fc00) : (h_ ? fc11 : fc10);          \
    const uint8_t *src_ = lds + (STAGE) * STAGE_BYTES + (isb_ ? fBrow : fArow) +  \
                          f_ * 32 * BK + co_;                                     \
    const v4u v_ = *reinterpret_cast<const v4u *>(src_);                          \
    if (isb_) { NB[f_][4 * h_] = (int)v_.x; NB[f_][4 * h_ + 1] = (int)v_.y;       \
                NB[f_][4 * h_ + 2] = (int)v_.z; NB[f_][4 * h_ + 3] = (int)v_.w; } \
    else      { NA[f_][4 * h_] = (int)v_.x; NA[f_][4 * h_ + 1] = (int)v_.y;       \
                NA[f_][4 * h_ + 2] = (int)v_.z; NA[f_][4 * h_ + 3] = (int)v_.w; } \
  } while (0)
#define FP8L_MFMA1(Q, CA, CB)                                                     \
  do {                                                                            \
    constexpr int j_ = (Q) / 4, i_ = (Q) % 4;                                     \
    acc[j_][i_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                \
        CB[j_], CA[i_], acc[j_][i_], 0, 0, 0, 0, 0, 0);                           \
  } while (0)
  // slot Q of half-step 0 / 1; sched_barrier keeps the interleaving
#define FP8L_SLOT0(Q, ST)                                                         \
  FP8L_MFMA1(Q, fa0, fb0); FP8L_READ1(ST, 1, Q, fa1, fb1);                        \
  __builtin_amdgcn_sched_barrier(0);
#define FP8L_SLOT1(Q, ST, STN, KT)                                                \
  FP8L_MFMA1(Q, fa1, fb1); FP8L_READ1(STN, 0, Q, fa0, fb0); FP8L_DMA1(ST, KT, Q); \
  __builtin_amdgcn_sched_barrier(0);
#define FP8L_READ0(Q) FP8L_READ1(0, 0, Q, fa0, fb0);

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    FP8L_DMAALL(0, 0)
    FP8L_DMAALL(1, 1)
    wait_vmcnt0();
    __builtin_amdgcn_s_barrier();
    FP8L_READ0(0) FP8L_READ0(1) FP8L_READ0(2) FP8L_READ0(3)
    FP8L_READ0(4) FP8L_READ0(5) FP8L_READ0(6) FP8L_READ0(7)
    FP8L_READ0(8) FP8L_READ0(9) FP8L_READ0(10) FP8L_READ0(11)
    FP8L_READ0(12) FP8L_READ0(13) FP8L_READ0(14) FP8L_READ0(15)
    for (int t = 0; t < nk; ++t) {
      const int st = t & 1;
      FP8L_SLOT0(0, st) FP8L_SLOT0(1, st) FP8L_SLOT0(2, st) FP8L_SLOT0(3, st)
      FP8L_SLOT0(4, st) FP8L_SLOT0(5, st) FP8L_SLOT0(6, st) FP8L_SLOT0(7, st)
      FP8L_SLOT0(8, st) FP8L_SLOT0(9, st) FP8L_SLOT0(10, st) FP8L_SLOT0(11, st)
      FP8L_SLOT0(12, st) FP8L_SLOT0(13, st) FP8L_SLOT0(14, st) FP8L_SLOT0(15, st)
      // this wave's DMA of k-tile t+1 landed and its reads of stage st are
      // complete; after the barrier that holds for every wave: stage st^1 is
      // readable and stage st can be refilled (past the end: with zeros, in
      // a stage no later step reads)
      wait_vmcnt0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      const int stn = st ^ 1;
      const int kt2 = t + 2;
      FP8L_SLOT1(0, st, stn, kt2) FP8L_SLOT1(1, st, stn, kt2)
      FP8L_SLOT1(2, st, stn, kt2) FP8L_SLOT1(3, st, stn, kt2)
      FP8L_SLOT1(4, st, stn, kt2) FP8L_SLOT1(5, st, stn, kt2)
      FP8L_SLOT1(6, st, stn, kt2) FP8L_SLOT1(7, st, stn, kt2)
      FP8L_SLOT1(8, st, stn, kt2) FP8L_SLOT1(9, st, stn, kt2)
      FP8L_SLOT1(10, st, stn, kt2) FP8L_SLOT1(11, st, stn, kt2)
      FP8L_SLOT1(12, st, stn, kt2) FP8L_SLOT1(13, st, stn, kt2)
      FP8L_SLOT1(14, st, stn, kt2) FP8L_SLOT1(15, st, stn, kt2)
    }
    wait_vmcnt0();   // no DMA may still target this workgroup's LDS
  }
#undef FP8L_READ0
#undef FP8L_SLOT1
#undef FP8L_SLOT0
#undef FP8L_MFMA1
#undef FP8L_READ1
#undef FP8L_DMAALL
#undef FP8L_DMA1

  // ---- epilogue, staged through LDS: after one barrier every wave is done
  // with the operand stages; each wave writes its scaled bf16 128 x 128 tile
  // to its own region (rows padded to 272 bytes), then stores whole rows
  // with 16-byte chunks (16 lanes per 256-byte row).
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint8_t *ep = lds + wave * EP_WAVE;
  const float inv_a0 = a_vec ? 0.f : 1.0f / sa[0];
  const float inv_b0 = b_vec ? 0.f : 1.0f / sb[0];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int ml = i * 32 + (lane & 31);               // row within the wave tile
    const int m = m0 + wm * WM + ml;
    const float inv_a = a_vec ? (m < M ? 1.0f / sa[m] : 0.f) : inv_a0;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = j * 32 + g * 8 + kh * 4;         // col within the wave tile
        const int n = n0 + wn * WN + nl;
        float inv_b[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          inv_b[e] = b_vec ? (n + e < N ? 1.0f / sb[n + e] : 0.f) : inv_b0;
        f32x2 v01 = {(acc[j][i][g * 4 + 0] * inv_a) * inv_b[0],
                     (acc[j][i][g * 4 + 1] * inv_a) * inv_b[1]};
        f32x2 v23 = {(acc[j][i][g * 4 + 2] * inv_a) * inv_b[2],
                     (acc[j][i][g * 4 + 3] * inv_a) * inv_b[3]};
        const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
        const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
        *reinterpret_cast<uint2 *>(ep + ml * EP_STRIDE + nl * 2) = make_uint2(p01, p23);
      }
    }
  }
  const int nbase = n0 + wn * WN;
  const int mrow0 = m0 + wm * WM;
#pragma unroll
  for (int it0 = 0; it0 < WM * WN * 2 / 16 / 64; it0 += 8) {
    v4u v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = (it0 + u) * 64 + lane;
      v[u] = *reinterpret_cast<const v4u *>(ep + (id >> 4) * EP_STRIDE + (id & 15) * 16);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int id = (it0 + u) * 64 + lane;
      const int m = mrow0 + (id >> 4);
      const int n = nbase + (id & 15) * 8;
      const uint32_t off = (m < M && n < N) ? (uint32_t)((m * N + n) * 2) : OOB_C;
      __builtin_amdgcn_raw_buffer_store_b128(v[u], rsC, off, 0, 0);
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
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if (K % BK == 0)
    hipLaunchKernelGGL(k_gemm_fp8_tn<true>, grid, dim3(THREADS), 0, stream, A, sa, a_vec, B,
                       sb, b_vec, (int)M, (int)N, (int)K, C, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL(k_gemm_fp8_tn<false>, grid, dim3(THREADS), 0, stream, A, sa, a_vec, B,
                       sb, b_vec, (int)M, (int)N, (int)K, C, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace fp8l
