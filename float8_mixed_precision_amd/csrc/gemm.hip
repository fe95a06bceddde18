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
//    8 x 8 blocks of v_mfma_f32_16x16x128_f8f6f4 (format 0 = E4M3 for both
//    operands, no block scales).  Under a power-limited clock this shape
//    sustains about 16% more throughput than the 32x32x64 form on the same
//    data (measured: 1.97 vs 1.70 GHz with normal-distributed operands).
//    A wave's 256 fp32 accumulators live in AGPRs.
//  - K advances 128 bytes per stage, which is one MFMA k-step and one full
//    128-byte cache line of every global row: whole lines load at about
//    twice the per-CU rate of half lines.  Two 64 KB stages (A slab
//    256 x 128 B, B slab 256 x 128 B) are filled by buffer_load_dwordx4 ...
//    lds (global to LDS without VGPRs); each instruction moves 8 rows x 128 B.
//  - Fragments: 8 A and 8 B per k-tile (16 rows x 128 B each, 8 VGPRs per
//    lane), 128 VGPRs in all, each refilled as soon as it falls free.  The
//    64 MFMAs of k-tile t run in two halves ordered by B fragment:
//      first half:  A0-3 x B0..B7; reads A7..A4(t) and B7(t)
//      -- wait for this wave's DMA of k-tile t+1 and its reads; barrier --
//      second half: A4-7 x B0..B7; reads A3..A0(t+1) and each B_j(t+1) right
//                   after the last use of B_j(t), and issues the 16 DMA
//                   instructions of k-tile t+2 into t's stage, one every
//                   other MFMA
//    Within a half the A fragment runs in a snake, 3 2 1 0 under B_0,
//    0 1 2 3 under B_1, and so on, so every MFMA after the first changes
//    exactly one of its two operands.  The chip runs this loop at its board
//    power limit, and fewer operand changes cost less switching energy:
//    measured 0.5-0.8% faster than restarting the A order under each B.
//    Every fragment read is issued about 28-32 MFMAs (~1000 cycles) before
//    its first use: with one wave per SIMD, LDS reads are latency-bound
//    (measured ~110 B/clk/CU at 4 waves, ~210 at 8), and a shorter lead
//    stalls the MFMAs.  DMA instructions are spread out because the
//    global->LDS path sustains ~54-64 B/clk/CU, so a burst of them blocks
//    issue.  There is one barrier per k-tile.
//  - Chunk c (16 B) of LDS row r sits at c ^ h(r), h(r) = (r & 7) ^
//    ((r >> 3) & 1): conflict-free for the 16-row fragment reads whether a
//    ds_read_b128 phase serves 8 lanes / 128 B or 16 lanes / 256 B.  The
//    swizzle is applied on the global side of the DMA (which writes each
//    instruction's 64 x 16 B to consecutive LDS addresses).
//  - Operand lanes: lane l holds row l % 16 of a fragment and 32 bytes of
//    its k-range, chunks 2 (l / 16) and 2 (l / 16) + 1 (any assignment of k
//    to lanes works that is the same for both operands).
//  - M, N and K tails: rows past M / N and 16-byte chunks past K are read
//    through buffer offsets past the buffer size, which return zeros.
//  - The MFMA's first operand is the B (n) fragment, the second the A (m)
//    fragment: output register r of lane l is n = 4 (l / 16) + r, m = l % 16
//    of its 16 x 16 block, so a lane holds 4 consecutive n of one m.  The
//    epilogue scales, rounds to bf16 (v_cvt_pk_bf16_f32, round to nearest
//    even) and stages the 128 x 128 tile in LDS, 32 rows at a time, to write
//    whole 256-byte rows with 16-byte buffer stores (out-of-range stores are
//    dropped by the buffer bounds check).
//  - Persistent: one workgroup per compute unit walks a fixed list of tiles,
//    with the operand loads of the next tile overlapping the end of the
//    current one (k_gemm_fp8_pers below).  Each XCD works through its own
//    contiguous share of a grouped tile order (GROUP_M = 4 tile-rows at a
//    time): the 32 tiles an XCD runs at once form a 4 x 8 block, and at the
//    8B FFN shapes an XCD's whole share stays within one 4-row group, so its
//    A panels are reused from L2 across successive rounds of tiles
//    (measured ~3% faster than 8 x 4 blocks, ~3% faster than 2 x 16).  A
//    grouped launch of problems with different K follows a balanced
//    schedule computed on the host (gemm_schedule.h).
//
// Accumulation.  The instruction's products are exact, but one k-step of
// 128 products is not an fp32 sum in some order: probes of the bare
// instruction show each group of 8 consecutive k aligned to 2^(E - 13), E
// the group's largest exponent sum, with the bits below truncated toward
// zero, and the 16 group sums and the accumulator then combined at fp32-like
// precision.  The result therefore differs from a sequential fp32 sum by
// more than rounding order where a group holds products 14 or more binades
// apart; the parity tests bound that difference per element.
#include "fp8l_internal.h"
#include "gemm_schedule.h"

namespace fp8l {
#ifdef FP8L_PHASE_TIMING
// Measurement build only (a separate library compiled with
// -DFP8L_PHASE_TIMING): per tile, the shader-clock counter (s_memtime) and
// the 100 MHz real-time counter (s_memrealtime) at the tile's top, after its
// first k-tile, after its last k-tile and after its last store is issued,
// written by one lane of the workgroup that ran it; record tile * G + b for
// workgroup b's tile-th tile (G workgroups), the first PHASE_MAX_BLOCKS
// records of the latest launch.  Read with fp8_gemm_phase_read.
constexpr int PHASE_MAX_BLOCKS = 8192;
__device__ unsigned long long g_phase[PHASE_MAX_BLOCKS * 8];
#endif
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;                  // fp8 elements (bytes) of K per stage
constexpr int THREADS = 256;
constexpr int WM = 128;                  // rows per wave
constexpr int WN = 128;                  // cols per wave
constexpr int FR = 16;                   // rows per fragment
constexpr int NF = WM / FR;              // fragments per operand per wave (8)
constexpr int SLAB = BM * BK;            // 32 KB
constexpr int STAGE_BYTES = 2 * SLAB;    // 64 KB: A slab, then B slab
constexpr int SCALE_BYTES = (BM + BN) * 4;  // rowwise: sa of the tile's rows, then sb of its cols
constexpr int GROUP_M = 4;
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = 0x80000000u;    // operand offset that reads as zero
constexpr uint32_t OOB_C = 0xFFFFFF00u;  // output offset that is dropped
// Cache policy of the output stores: non-temporal ("nt").  The output is not
// read again by the GEMM, and streaming it out keeps it from evicting the
// operand panels from L2 and from leaving dirty lines in the Infinity Cache
// that the next kernel would have to write back (measured: the GEMMs of the
// FFN step 3% faster, the amax passes after them faster too).
constexpr int C_STORE_AUX = 2;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// s_waitcnt with only one counter constrained (gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier that is also a compiler barrier for memory accesses, so
// no LDS read or write is moved across it (the barrier intrinsic alone does
// not order plain loads and stores).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 16-byte global -> LDS transfer per lane: lane i's bytes land at LDS
// address m0 + 16 i.  Inline asm, so that the compiler neither moves LDS
// reads across it nor inserts waits of its own; completion is tracked with
// explicit vmcnt waits.  m0 is named as clobbered (nothing else in this
// kernel uses it); clang warns that it does not track reserved registers.
// The LDS address is wave-uniform; readfirstlane keeps it in a scalar
// register where the compiler has placed it in a vector one (it folds away
// where the value is already scalar).  The compiler keeps the 32 addresses
// of a k-tile's transfers (16 per stage) in scalar registers across the
// loop; adding a constant inside the asm instead saved those registers but
// cost the loop an instruction per transfer (~20 cycles per k-tile).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr,
                                      uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Up to MAX_GROUP GEMMs of one variant in one launch (the kernel's only
// argument).  A problem whose last round of tiles would leave compute units
// idle (896 tiles on 256) shares that round with the others.
constexpr int MAX_GROUP = 4;
struct GemmGroup {
  const uint8_t *A[MAX_GROUP];
  const float *sa[MAX_GROUP];
  const uint8_t *B[MAX_GROUP];
  const float *sb[MAX_GROUP];
  void *C[MAX_GROUP];
  int M[MAX_GROUP], N[MAX_GROUP], K[MAX_GROUP];
  int tiles_m[MAX_GROUP], tiles_n[MAX_GROUP];
  int count;
  int total;   // tiles of all problems
  // nonzero when the two arrays below hold a balanced
  // schedule (gemm_schedule.h): the entry of workgroup l of XCD x for
  // problem p in half l % 2 of sched[x][p][l / 2], the smallest count of XCD
  // x's workgroups for problem p in byte p of sched_min[x] (whole words, so
  // that the kernel reads them with scalar loads)
  int balanced;
  uint32_t sched_min[NUM_XCD];
  uint32_t sched[NUM_XCD][MAX_GROUP][16];
};
static_assert(NUM_XCD == sched::XCDS && MAX_GROUP == sched::MAX_PROBLEMS &&
              sched::MAX_WG == 32, "schedule layout");
static_assert(sizeof(GemmGroup) <= 4096, "kernel arguments");

// element i of a kernel-argument array for a wave-uniform i (selects, so the
// array is never copied to private memory)
template <class T>
__device__ __forceinline__ T pick(const T (&v)[MAX_GROUP], int i) {
  T r = v[0];
#pragma unroll
  for (int k = 1; k < MAX_GROUP; ++k)
    if (i == k) r = v[k];
  return r;
}

// ---------------------------------------------------------------------------
// Persistent form.  One workgroup per compute unit (gridDim.x = G =
// min(tiles, compute units)); each workgroup walks a fixed list of tiles
// (decode_tile), so the per-tile launch cost and the pipeline fill are paid
// once per workgroup instead of once per tile.  One DMA stream runs two
// k-tiles ahead of the MFMAs across tile boundaries: the next tile's first
// two k-tiles load during the current tile's last two, and its first
// fragments are read at the top of the tile, so a tile starts without a
// prologue.  The epilogue stages through its own 32 KB LDS region (4 passes
// of 32 rows per wave, 16-byte chunks XOR-swizzled by row instead of
// padding), so it never touches the operand stages that are filling for the
// next tile; it leaves its stores in flight while the next tile's first
// k-tile starts.  No tile clears its accumulators: the MFMAs of each tile's
// first k-tile take a zero accumulator input.
// Nothing is shared between workgroups: correctness does not depend on how
// many are resident at once.
constexpr int EPI_OFF = 2 * STAGE_BYTES;        // 128 KB
constexpr int EPI_WAVE_BYTES = 8 * 1024;        // per wave: 32 rows x 256 B
constexpr int EPI_BYTES = 4 * EPI_WAVE_BYTES;   // 32 KB (rowwise: each wave's scales first)
// epilogue stores left in flight when the next tile's first k-tile waits for
// its operands (bf16: 4 passes x 8 stores per lane)
constexpr int EPI_STORES = 32;
// Rowwise scales.  Each wave keeps two scale tables at the start of its
// staging (tiles of even and odd index) and stages its rowwise epilogues in
// the second half.  A tile's scales are transferred two tiles ahead, after
// the stores of an epilogue (SCALE_DMAS transfers, always issued), and
// become reciprocals between the MFMAs of the last k-tile of the tile
// before it.
constexpr int SCALE_DMAS = 2;
constexpr int RW_STAGE_OFF = EPI_WAVE_BYTES / 2;
static_assert(2 * SCALE_BYTES <= RW_STAGE_OFF, "two scale tables below the rowwise staging");
static_assert(EPI_WAVE_BYTES == 64 * BK, "a wave's staging is at its operand offset + EPI_OFF");

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A wave-uniform float read through the scalar cache (s_load): its wait
// counts on lgkmcnt.  A vector load's wait would count on vmcnt, which
// completes in issue order, and so also wait for the operand transfers in
// flight before it.
__device__ __forceinline__ float scalar_load(const float *p) {
  return *(const __attribute__((address_space(4))) float *)p;
}

// This lane's index in its wave (0..63), read from the hardware at the
// point of use (v_mbcnt over a full mask).  Volatile, so the compiler
// neither keeps an earlier copy live across the loops (nor spills one) to
// reuse here: it recomputes it in two instructions.
__device__ __forceinline__ int hw_lane() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// Four reciprocals (IEEE division, as 1/s is computed everywhere else).
__device__ __forceinline__ v4f recip4(v4f s) {
  return (v4f){1.0f / s.x, 1.0f / s.y, 1.0f / s.z, 1.0f / s.w};
}

// The 16-byte slot of a scale table (row scales, then column scales) whose
// 4 scales lane l of wave (wm, wn) turns into reciprocals: lanes 0-31 the
// wave's 128 rows, lanes 32-63 its 128 columns.
__device__ __forceinline__ int rcp_slot(int l, int wm, int wn) {
  // (l >> 5) selects the column part without a select between two
  // wave-uniform values, which the compiler held (and spilled) in vector
  // registers
  const int row0 = wm * (WM / 4), col0 = (BM + wn * WN) / 4 - 32;
  return l + row0 + (l >> 5) * (col0 - row0);
}

// Tile i (i = 0, 1, ...) of persistent workgroup b.  Workgroups are dealt
// to the XCDs round-robin (b on XCD x = b % 8, the l-th of its nx, l =
// b / 8), and each XCD works through its own contiguous share of every
// problem's grouped tile order, problem after problem, as the XCD's blocks
// would with one workgroup per tile dealt round-robin.  Without a schedule the
// XCD's workgroups take positions l, l + nx, l + 2 nx, ... of that sequence;
// with one (g.balanced) workgroup l runs the count of tiles of problem p
// that its entry gives, at the positions sched::position assigns.  Either
// way the tiles an
// XCD runs at one time are neighbours in the grouped order and share operand
// panels in its L2.
struct TileCoord {
  int pi, m0, n0;
  bool valid;
};
__device__ __forceinline__ TileCoord decode_tile(const GemmGroup &g, int b, int i, int G) {
  const int x = b % NUM_XCD;
  const int l = b / NUM_XCD;
  const int nx = (G - x + NUM_XCD - 1) / NUM_XCD;   // workgroups on XCD x
  int s = l + i * nx;                                // round-robin position
  for (int pi = 0; pi < g.count; ++pi) {
    const int tiles_m = pick(g.tiles_m, pi), tiles_n = pick(g.tiles_n, pi);
    const int T = tiles_m * tiles_n;
    int pos;                                         // position in XCD x's share
    if (g.balanced) {
      const uint32_t e = g.sched[x][pi][l >> 1] >> (16 * (l & 1));
      const int n = (int)(e & 255);
      if (i >= n) {
        i -= n;
        continue;
      }
      pos = sched::position(i, l, nx, (int)((g.sched_min[x] >> (8 * pi)) & 255),
                            (int)((e >> 8) & 255));
    } else {
      const int cnt = (T - x + NUM_XCD - 1) / NUM_XCD;  // XCD x's share of problem pi
      if (s >= cnt) {
        s -= cnt;
        continue;
      }
      pos = s;
    }
    int base = 0;
    for (int xx = 0; xx < x; ++xx) base += (T - xx + NUM_XCD - 1) / NUM_XCD;
    const int q = base + pos;                          // grouped order index
    const int group = GROUP_M * tiles_n;
    const int first_m = (q / group) * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int in_group = q % group;
    return {pi, (first_m + in_group % gm) * BM, (in_group / gm) * BN, true};
  }
  return {0, 0, 0, false};
}

// KFULL: K % 128 == 0 (no K tail, no per-chunk K check).  RW: rowwise
// scales (sa[M], sb[N]) instead of one scale per operand.  F32: fp32 output
// (the scaled value before bf16 rounding) instead of bf16.  FA: code format
// of A (0 = E4M3, 1 = E5M2 gradients); B is E4M3.  The instruction's
// format selectors apply to its first and second source operand, here the
// B and the A fragment.  ACC (bf16 output only): C holds a bf16 matrix on
// entry and receives bf16(fl32(C) + fl32(bf16 result)), the sum of two
// gradient contributions as bf16 tensors add.
template <bool KFULL, bool RW, bool F32, int FA, bool ACC>
__global__ __launch_bounds__(THREADS) void k_gemm_fp8_pers(GemmGroup g) {
  static_assert(!(F32 && ACC), "accumulation is into a bf16 output");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[EPI_OFF + EPI_BYTES];
  const int G = gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds;
  const uint32_t wave_dst = lds_base + (uint32_t)(wave * 64 * BK);

  // ---- DMA cursor: the unit (tile, k-tile) whose operands load next.  Wave
  // w, instruction q (0..7 A, 8..15 B) fills slab rows w*64 + (q&7)*8 +
  // lane/8, 16-byte chunk (lane%8) ^ (lane/8) ^ (q&1): row r keeps logical
  // chunk c at physical chunk c ^ h(r), h(r) = (r & 7) ^ ((r >> 3) & 1), so
  // lane i loads logical chunk (i % 8) ^ (i / 8) ^ (q & 1).  The
  // tile's first row is in the buffer resource (base A + m0 K, M - m0 rows),
  // so the per-lane offsets depend only on K, and rows past the matrix fail
  // the bounds check on the vector offset alone (they read as zero).
  const int lr = lane >> 3;
  const int c_even = (lane & 7) ^ lr;
  const int c_odd = c_even ^ 1;
  int d_tile = 0, d_kt = 0, d_nk = 0, d_K = -1;     // d_tile: this workgroup's tile index
  bool d_valid = true;
  // Tile coordinates, decoded once per tile at its top instead of inside the
  // main loop: a_*, b_*, c_* are this workgroup's tiles cur, cur + 1 and
  // cur + 2 (problem, first row and column, and whether the tile exists).
  // The cursor runs at most two units ahead of the MFMAs, so while tile i
  // computes (cur = i + 1 once its top has passed) it reaches at most tile
  // i + 2; before the first tile it reaches at most tile 2.
  int a_pi, a_m0, a_n0, b_pi, b_m0, b_n0, c_pi, c_m0, c_n0;
  bool a_ok, b_ok, c_ok;
  {
    const TileCoord t0 = decode_tile(g, blockIdx.x, 0, G);
    const TileCoord t1 = decode_tile(g, blockIdx.x, 1, G);
    const TileCoord t2 = decode_tile(g, blockIdx.x, 2, G);
    a_pi = t0.pi; a_m0 = t0.m0; a_n0 = t0.n0; a_ok = t0.valid;
    b_pi = t1.pi; b_m0 = t1.m0; b_n0 = t1.n0; b_ok = t1.valid;
    c_pi = t2.pi; c_m0 = t2.m0; c_n0 = t2.n0; c_ok = t2.valid;
  }
  int cur = 0;
  __amdgpu_buffer_rsrc_t d_rsA, d_rsB;
  uint32_t voff[16];
  // The cursor's steps are macros rather than lambdas: a lambda reaches the
  // kernel's variables through its captured references, and once inlined a
  // choice between two of them can turn into a load through a chosen
  // pointer, which pins the variables (and a copy of the kernel arguments)
  // in private memory.
  //
  // FP8P_SETVOFF: per-lane offsets for the cursor's K, from the lane index
  // read afresh (recomputed where needed rather than kept live or spilled).
#define FP8P_SETVOFF()                                                          \
  do {                                                                          \
    const int lane_v = hw_lane();                                               \
    const int lr_v = lane_v >> 3;                                               \
    const int ce_v = (lane_v & 7) ^ lr_v;                                       \
    _Pragma("unroll") for (int q = 0; q < 16; ++q) {                            \
      const int row = wave * 64 + (q & 7) * 8 + lr_v;                           \
      voff[q] = (uint32_t)(row * d_K + ((q & 1) ? ce_v ^ 1 : ce_v) * 16);       \
    }                                                                           \
  } while (0)
  // FP8P_DSETUP: the cursor enters tile d_tile.  The host launches no
  // problem with K = 0 (k_gemm_k0 writes those), so every tile has at least
  // one k-tile.  Past the last tile decode_tile gives problem 0's origin,
  // which serves the empty buffers an exhausted cursor still issues its
  // (zero-filling) transfers from, into the stage no one reads any more.
#define FP8P_DSETUP()                                                           \
  do {                                                                          \
    const bool sa_ = d_tile == cur, sb_ = d_tile == cur + 1;                    \
    const int pi_ = sa_ ? a_pi : (sb_ ? b_pi : c_pi);                           \
    const int m0_ = sa_ ? a_m0 : (sb_ ? b_m0 : c_m0);                           \
    const int n0_ = sa_ ? a_n0 : (sb_ ? b_n0 : c_n0);                           \
    const bool ok_ = sa_ ? a_ok : (sb_ ? b_ok : c_ok);                          \
    const int M_ = pick(g.M, pi_), N_ = pick(g.N, pi_), K_ = pick(g.K, pi_);    \
    d_nk = (K_ + BK - 1) / BK;                                                  \
    d_valid = ok_ && d_nk > 0;                                                  \
    d_rsA = __builtin_amdgcn_make_buffer_rsrc(                                  \
        (void *)(pick(g.A, pi_) + (size_t)m0_ * K_), (short)0,                  \
        d_valid ? (M_ - m0_) * K_ : 0, 0x00020000);                             \
    d_rsB = __builtin_amdgcn_make_buffer_rsrc(                                  \
        (void *)(pick(g.B, pi_) + (size_t)n0_ * K_), (short)0,                  \
        d_valid ? (N_ - n0_) * K_ : 0, 0x00020000);                             \
    if (K_ != d_K) {                                                            \
      d_K = K_;                                                                 \
      FP8P_SETVOFF();                                                           \
    }                                                                           \
  } while (0)
  // FP8P_DADV: the cursor moves to the next unit
#define FP8P_DADV()                                                             \
  do {                                                                          \
    if (d_valid && ++d_kt == d_nk) {                                            \
      d_kt = 0;                                                                 \
      ++d_tile;                                                                 \
      FP8P_DSETUP();                                                            \
    }                                                                           \
  } while (0)
  FP8P_DSETUP();

#define FP8P_DMA1(STAGE, Q)                                                       \
  do {                                                                            \
    const uint32_t k0_ = (uint32_t)(d_kt * BK);                                   \
    const bool kok_ = KFULL || (int)k0_ + (((Q) & 1) ? c_odd : c_even) * 16 < d_K; \
    const uint32_t dst_ = wave_dst + (uint32_t)((STAGE) * STAGE_BYTES +           \
                          ((Q) >= 8 ? SLAB : 0) + ((Q) & 7) * 1024);              \
    dma16((Q) >= 8 ? d_rsB : d_rsA, dst_, kok_ ? voff[Q] : OOB, k0_);             \
  } while (0)
  // FP8P_SCALES: rowwise: the 256 row and 256 column scales of the tile at
  // (PI, M0, N0), as stored, by DMA into this wave's scale table BUF (a wave
  // writes and reads only its own).  Rows and columns past the matrix read
  // as zero (dimensions are multiples of 16, so a lane's 4 scales are all
  // inside or all outside); OK false reads nothing and writes zeros, so the
  // count of transfers stays fixed.
#define FP8P_SCALES(OK, PI, M0, N0, BUF)                                          \
  do {                                                                            \
    const uint32_t base_ = wave_dst + (uint32_t)(EPI_OFF + (BUF) * SCALE_BYTES);  \
    const uint32_t lo_ = (uint32_t)hw_lane() * 16;                                \
    dma16(__builtin_amdgcn_make_buffer_rsrc(                                      \
              (void *)(pick(g.sa, PI) + (M0)), (short)0,                          \
              (OK) ? (pick(g.M, PI) - (M0)) * 4 : 0, 0x00020000),                 \
          base_, lo_, 0);                                                         \
    dma16(__builtin_amdgcn_make_buffer_rsrc(                                      \
              (void *)(pick(g.sb, PI) + (N0)), (short)0,                          \
              (OK) ? (pick(g.N, PI) - (N0)) * 4 : 0, 0x00020000),                 \
          base_ + BM * 4, lo_, 0);                                                \
  } while (0)

  // ---- fragment reads: fragment f of A is rows wm*128 + f*16 + lane%16,
  // lane l reads logical chunks 2(l/16) and 2(l/16)+1 of its row (h(row)
  // depends only on lane%16); the per-lane offsets are set at the top of
  // each tile
  int fArow, fBrow, fc0, fc1;
  v8i fa[NF], fb[NF];
  v4f acc[NF][NF];   // [j: n block][i: m block]

#define FP8P_RD(STAGE, X, F, H)                                                   \
  do {                                                                            \
    const uint8_t *src_ = lds + (STAGE) * STAGE_BYTES +                           \
                          ((X) ? fBrow : fArow) + (F) * FR * BK + ((H) ? fc1 : fc0); \
    const v4u v_ = *reinterpret_cast<const v4u *>(src_);                          \
    if (X) { fb[F][4 * (H)] = (int)v_.x; fb[F][4 * (H) + 1] = (int)v_.y;          \
             fb[F][4 * (H) + 2] = (int)v_.z; fb[F][4 * (H) + 3] = (int)v_.w; }    \
    else   { fa[F][4 * (H)] = (int)v_.x; fa[F][4 * (H) + 1] = (int)v_.y;          \
             fa[F][4 * (H) + 2] = (int)v_.z; fa[F][4 * (H) + 3] = (int)v_.w; }    \
  } while (0)
  // MFMA of block (J, I)
#define FP8P_MF(J, I)                                                             \
  acc[J][I] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                   \
      fb[J], fa[I], acc[J][I], 0, FA, 0, 0, 0, 0)
// the same with a zero accumulator input (a tile's first k-tile)
#define FP8P_MFZ(J, I)                                                            \
  acc[J][I] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                   \
      fb[J], fa[I], (v4f){0.f, 0.f, 0.f, 0.f}, 0, FA, 0, 0, 0, 0)
// step S of a half k-tile with MF (FP8P_MF or FP8P_MFZ)
#define FP8P_MX(MF, S, I0) MF((S) / 4, (I0) + ((((S) / 4) & 1) ? (S) % 4 : 3 - (S) % 4));
#define FP8P_E() __builtin_amdgcn_sched_barrier(0);
#define FP8P_H1(ST, MF) \
  FP8P_MX(MF, 0, 0) FP8P_RD(ST, 0, 7, 0); FP8P_E() \
  FP8P_MX(MF, 1, 0) FP8P_RD(ST, 0, 7, 1); FP8P_E() \
  FP8P_MX(MF, 2, 0) FP8P_RD(ST, 0, 6, 0); FP8P_E() \
  FP8P_MX(MF, 3, 0) FP8P_RD(ST, 0, 6, 1); FP8P_E() \
  FP8P_MX(MF, 4, 0) FP8P_RD(ST, 0, 5, 0); FP8P_E() \
  FP8P_MX(MF, 5, 0) FP8P_RD(ST, 0, 5, 1); FP8P_E() \
  FP8P_MX(MF, 6, 0) FP8P_RD(ST, 0, 4, 0); FP8P_E() \
  FP8P_MX(MF, 7, 0) FP8P_RD(ST, 0, 4, 1); FP8P_E() \
  FP8P_MX(MF, 8, 0) FP8P_RD(ST, 1, 7, 0); FP8P_E() \
  FP8P_MX(MF, 9, 0) FP8P_RD(ST, 1, 7, 1); FP8P_E() \
  FP8P_MX(MF, 10, 0) FP8P_E() FP8P_MX(MF, 11, 0) FP8P_E() FP8P_MX(MF, 12, 0) FP8P_E() \
  FP8P_MX(MF, 13, 0) FP8P_E() FP8P_MX(MF, 14, 0) FP8P_E() FP8P_MX(MF, 15, 0) FP8P_E() \
  FP8P_MX(MF, 16, 0) FP8P_E() FP8P_MX(MF, 17, 0) FP8P_E() FP8P_MX(MF, 18, 0) FP8P_E() \
  FP8P_MX(MF, 19, 0) FP8P_E() FP8P_MX(MF, 20, 0) FP8P_E() FP8P_MX(MF, 21, 0) FP8P_E() \
  FP8P_MX(MF, 22, 0) FP8P_E() FP8P_MX(MF, 23, 0) FP8P_E() FP8P_MX(MF, 24, 0) FP8P_E() \
  FP8P_MX(MF, 25, 0) FP8P_E() FP8P_MX(MF, 26, 0) FP8P_E() FP8P_MX(MF, 27, 0) FP8P_E() \
  FP8P_MX(MF, 28, 0) FP8P_E() FP8P_MX(MF, 29, 0) FP8P_E() FP8P_MX(MF, 30, 0) FP8P_E() \
  FP8P_MX(MF, 31, 0) FP8P_E()
#define FP8P_H2(STN, DST, MF) \
  FP8P_MX(MF, 0, 4) FP8P_RD(STN, 0, 3, 0); FP8P_E() \
  FP8P_MX(MF, 1, 4) FP8P_DMA1(DST, 0); FP8P_E() \
  FP8P_MX(MF, 2, 4) FP8P_RD(STN, 0, 3, 1); FP8P_E() \
  FP8P_MX(MF, 3, 4) FP8P_DMA1(DST, 1); FP8P_E() \
  FP8P_MX(MF, 4, 4) FP8P_RD(STN, 0, 2, 0); FP8P_RD(STN, 1, 0, 0); FP8P_E() \
  FP8P_MX(MF, 5, 4) FP8P_RD(STN, 1, 0, 1); FP8P_DMA1(DST, 2); FP8P_E() \
  FP8P_MX(MF, 6, 4) FP8P_RD(STN, 0, 2, 1); FP8P_E() \
  FP8P_MX(MF, 7, 4) FP8P_DMA1(DST, 3); FP8P_E() \
  FP8P_MX(MF, 8, 4) FP8P_RD(STN, 0, 1, 0); FP8P_RD(STN, 1, 1, 0); FP8P_E() \
  FP8P_MX(MF, 9, 4) FP8P_RD(STN, 1, 1, 1); FP8P_DMA1(DST, 4); FP8P_E() \
  FP8P_MX(MF, 10, 4) FP8P_RD(STN, 0, 1, 1); FP8P_E() \
  FP8P_MX(MF, 11, 4) FP8P_DMA1(DST, 5); FP8P_E() \
  FP8P_MX(MF, 12, 4) FP8P_RD(STN, 0, 0, 0); FP8P_RD(STN, 1, 2, 0); FP8P_E() \
  FP8P_MX(MF, 13, 4) FP8P_RD(STN, 1, 2, 1); FP8P_DMA1(DST, 6); FP8P_E() \
  FP8P_MX(MF, 14, 4) FP8P_RD(STN, 0, 0, 1); FP8P_E() \
  FP8P_MX(MF, 15, 4) FP8P_DMA1(DST, 7); FP8P_E() \
  FP8P_MX(MF, 16, 4) FP8P_RD(STN, 1, 3, 0); FP8P_E() \
  FP8P_MX(MF, 17, 4) FP8P_RD(STN, 1, 3, 1); FP8P_DMA1(DST, 8); FP8P_E() \
  FP8P_MX(MF, 18, 4) FP8P_E() \
  FP8P_MX(MF, 19, 4) FP8P_DMA1(DST, 9); FP8P_E() \
  FP8P_MX(MF, 20, 4) FP8P_RD(STN, 1, 4, 0); FP8P_E() \
  FP8P_MX(MF, 21, 4) FP8P_RD(STN, 1, 4, 1); FP8P_DMA1(DST, 10); FP8P_E() \
  FP8P_MX(MF, 22, 4) FP8P_E() \
  FP8P_MX(MF, 23, 4) FP8P_DMA1(DST, 11); FP8P_E() \
  FP8P_MX(MF, 24, 4) FP8P_RD(STN, 1, 5, 0); FP8P_E() \
  FP8P_MX(MF, 25, 4) FP8P_RD(STN, 1, 5, 1); FP8P_DMA1(DST, 12); FP8P_E() \
  FP8P_MX(MF, 26, 4) FP8P_E() \
  FP8P_MX(MF, 27, 4) FP8P_DMA1(DST, 13); FP8P_E() \
  FP8P_MX(MF, 28, 4) FP8P_RD(STN, 1, 6, 0); FP8P_E() \
  FP8P_MX(MF, 29, 4) FP8P_RD(STN, 1, 6, 1); FP8P_DMA1(DST, 14); FP8P_E() \
  FP8P_MX(MF, 30, 4) FP8P_E() \
  FP8P_MX(MF, 31, 4) FP8P_DMA1(DST, 15); FP8P_E()

// last k-tile of a tile: the DMAs only (the next tile's first fragments are
// read after the epilogue, which keeps them out of its registers), and two
// hooks for vector work issued between its matrix instructions
#define FP8P_H2D(DST, MF, HK1, HK2) \
  FP8P_MX(MF, 0, 4) FP8P_E() FP8P_MX(MF, 1, 4) FP8P_DMA1(DST, 0); FP8P_E() \
  FP8P_MX(MF, 2, 4) FP8P_E() FP8P_MX(MF, 3, 4) FP8P_DMA1(DST, 1); FP8P_E() \
  FP8P_MX(MF, 4, 4) HK1; FP8P_E() FP8P_MX(MF, 5, 4) FP8P_DMA1(DST, 2); FP8P_E() \
  FP8P_MX(MF, 6, 4) FP8P_E() FP8P_MX(MF, 7, 4) FP8P_DMA1(DST, 3); FP8P_E() \
  FP8P_MX(MF, 8, 4) FP8P_E() FP8P_MX(MF, 9, 4) FP8P_DMA1(DST, 4); FP8P_E() \
  FP8P_MX(MF, 10, 4) FP8P_E() FP8P_MX(MF, 11, 4) FP8P_DMA1(DST, 5); FP8P_E() \
  FP8P_MX(MF, 12, 4) HK2; FP8P_E() FP8P_MX(MF, 13, 4) FP8P_DMA1(DST, 6); FP8P_E() \
  FP8P_MX(MF, 14, 4) FP8P_E() FP8P_MX(MF, 15, 4) FP8P_DMA1(DST, 7); FP8P_E() \
  FP8P_MX(MF, 16, 4) FP8P_E() FP8P_MX(MF, 17, 4) FP8P_DMA1(DST, 8); FP8P_E() \
  FP8P_MX(MF, 18, 4) FP8P_E() FP8P_MX(MF, 19, 4) FP8P_DMA1(DST, 9); FP8P_E() \
  FP8P_MX(MF, 20, 4) FP8P_E() FP8P_MX(MF, 21, 4) FP8P_DMA1(DST, 10); FP8P_E() \
  FP8P_MX(MF, 22, 4) FP8P_E() FP8P_MX(MF, 23, 4) FP8P_DMA1(DST, 11); FP8P_E() \
  FP8P_MX(MF, 24, 4) FP8P_E() FP8P_MX(MF, 25, 4) FP8P_DMA1(DST, 12); FP8P_E() \
  FP8P_MX(MF, 26, 4) FP8P_E() FP8P_MX(MF, 27, 4) FP8P_DMA1(DST, 13); FP8P_E() \
  FP8P_MX(MF, 28, 4) FP8P_E() FP8P_MX(MF, 29, 4) FP8P_DMA1(DST, 14); FP8P_E() \
  FP8P_MX(MF, 30, 4) FP8P_E() FP8P_MX(MF, 31, 4) FP8P_DMA1(DST, 15); FP8P_E()

  // ---- the first two units' operands (the fragments are read at the top
  // of each tile)
  if (d_valid) {
#pragma unroll
    for (int q = 0; q < 16; ++q) FP8P_DMA1(0, q);
    FP8P_DADV();
#pragma unroll
    for (int q = 0; q < 16; ++q) FP8P_DMA1(1, q);
    FP8P_DADV();
  }
  // rowwise: the first two tiles' scales
  if (RW) {
    FP8P_SCALES(a_ok, a_pi, a_m0, a_n0, 0);
    FP8P_SCALES(b_ok, b_pi, b_m0, b_n0, 1);
  }
  wait_vmcnt0();
  barrier_lds();

  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  uint8_t *epi = lds + EPI_OFF + wave * EPI_WAVE_BYTES;
  // rowwise: the entry of table BUF that this lane turns into reciprocals:
  // 4 of the wave's 128 row scales (lanes 0-31) or 128 column scales (lanes
  // 32-63).  One wave's LDS accesses run in order, so its later reads see
  // what it wrote.
#define FP8P_RCP_AT(BUF)                                                          \
  (reinterpret_cast<v4f *>(epi + (BUF) * SCALE_BYTES) + rcp_slot(hw_lane(), wm, wn))
  if (RW) {                                       // tile 0's scales
    v4f *r_ = FP8P_RCP_AT(0);
    *r_ = recip4(*r_);
  }
  int st = 0;          // stage of the current unit
  for (int tile = 0;; ++tile) {
    const TileCoord tc = {a_pi, a_m0, a_n0, a_ok};
    if (!tc.valid) break;
    const int pi = tc.pi, m0 = tc.m0, n0 = tc.n0;
    // the decoded tiles move on, before the fragment reads below: the
    // decode's scalar loads share the LDS reads' wait counter, and waiting
    // for them here waits for nothing else
    a_pi = b_pi; a_m0 = b_m0; a_n0 = b_n0; a_ok = b_ok;
    b_pi = c_pi; b_m0 = c_m0; b_n0 = c_n0; b_ok = c_ok;
    {
      const TileCoord t3 = decode_tile(g, blockIdx.x, tile + 3, G);
      c_pi = t3.pi; c_m0 = t3.m0; c_n0 = t3.n0; c_ok = t3.valid;
    }
    ++cur;
    const int M = pick(g.M, pi), N = pick(g.N, pi), K = pick(g.K, pi);
    const int nk = (K + BK - 1) / BK;
    const float *__restrict__ sa = pick(g.sa, pi);
    const float *__restrict__ sb = pick(g.sb, pi);
#ifdef FP8L_PHASE_TIMING
    const unsigned long long ph_t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long ph_r0 = __builtin_amdgcn_s_memrealtime();
    unsigned long long ph_ta = ph_t0, ph_ra = ph_r0;
#endif
    // the cursor's per-lane offsets and the fragment offsets, recomputed
    // here from the lane index instead of being kept (or spilled) across the
    // epilogue
    FP8P_SETVOFF();
    {
      const int lane_v = hw_lane();
      // fragment f of A: rows wm*128 + f*16 + lane%16; lane reads logical
      // chunks 2(lane/16) and 2(lane/16)+1, swizzled by h(row)
      const int hr = (lane_v & 7) ^ ((lane_v >> 3) & 1);
      const int g4 = lane_v >> 4;
      fArow = (wm * WM + (lane_v & 15)) * BK;
      fBrow = SLAB + (wn * WN + (lane_v & 15)) * BK;
      fc0 = ((2 * g4) ^ hr) << 4;
      fc1 = ((2 * g4 + 1) ^ hr) << 4;
    }
    {
      // A0-3 and B0-6 of the tile's first k-tile (complete in stage st: this
      // wave waited for its part and passed a barrier since)
#pragma unroll
      for (int f = 0; f < 4; ++f) { FP8P_RD(st, 0, f, 0); FP8P_RD(st, 0, f, 1); }
#pragma unroll
      for (int f = 0; f < 7; ++f) { FP8P_RD(st, 1, f, 0); FP8P_RD(st, 1, f, 1); }
    }
    // the last k-tile (MF: FP8P_MF, or FP8P_MFZ when it is also the first).
    // It waits for everything but, where it follows the previous epilogue
    // directly (K <= 128, bf16 tensorwise), that epilogue's stores.
    // Rowwise, the next tile's scales (issued after those stores, so this
    // wait counts them) become reciprocals between its matrix
    // instructions.
#define FP8P_LAST(MF)                                                             \
  do {                                                                            \
    FP8P_H1(st, MF)                                                               \
    if (nk == 1 && !F32 && !RW)                                                   \
      wait_vmcnt<EPI_STORES>();                                                   \
    else                                                                          \
      wait_vmcnt0();                                                              \
    wait_lgkm0();                                                                 \
    barrier_lds();                                                                \
    v4f *rn_ = nullptr;                                                           \
    v4f sn_ = {};                                                                 \
    if (RW) {                                                                     \
      rn_ = FP8P_RCP_AT((tile + 1) & 1);                                          \
      sn_ = *rn_;                                                                 \
    }                                                                             \
    FP8P_H2D(st, MF, if (RW) sn_ = recip4(sn_), if (RW) *rn_ = sn_)               \
    FP8P_DADV();                                                                  \
    st ^= 1;                                                                      \
  } while (0)
    if (nk > 1) {
      // the first k-tile, peeled: its matrix instructions start from a zero
      // accumulator input, so no tile clears its 256 accumulator registers
      // first.  It waits for its successor's operands, issued before the
      // previous tile's epilogue, whose stores (and, for rowwise scales,
      // the scale transfers after them) may still be in flight behind them
      // (vmcnt counts in issue order): all but those.
      FP8P_H1(st, FP8P_MFZ)
      if (!F32)
        wait_vmcnt<EPI_STORES + (RW ? SCALE_DMAS : 0)>();
      else
        wait_vmcnt0();
      wait_lgkm0();
      barrier_lds();
      FP8P_H2(st ^ 1, st, FP8P_MFZ)
      FP8P_DADV();
      st ^= 1;
#ifdef FP8L_PHASE_TIMING
      ph_ta = __builtin_amdgcn_s_memtime();
      ph_ra = __builtin_amdgcn_s_memrealtime();
#endif
      // every further k-tile but the last reads the next one's first
      // fragments and loads the one after; each waits for everything
      for (int t = 1; t < nk - 1; ++t) {
        FP8P_H1(st, FP8P_MF)
        wait_vmcnt0();
        wait_lgkm0();
        barrier_lds();
        FP8P_H2(st ^ 1, st, FP8P_MF)
        FP8P_DADV();
        st ^= 1;
      }
      FP8P_LAST(FP8P_MF);
    } else {
      FP8P_LAST(FP8P_MFZ);                        // one k-tile (K <= 128)
    }
#undef FP8P_LAST
#ifdef FP8L_PHASE_TIMING
    const unsigned long long ph_t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long ph_r1 = __builtin_amdgcn_s_memrealtime();
#endif

    // ---- epilogue: scale, round, stage 32 rows of the wave's 128 x 128 tile
    // at a time in the wave's 8 KB (row r's 16-byte chunk c at c ^ (r % 16),
    // its 8-byte halves swapped where r % 16 >= 8), write whole rows
    const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(
        pick(g.C, pi), (short)0, M * N * (F32 ? 4 : 2), 0x00020000);
    const int lane_e = hw_lane();
    const int ml16 = lane_e & 15;                 // row within a 16-row block
    const int nq = (lane_e >> 4) * 4;             // first of the lane's 4 columns in a block
    const float inv_a0 = RW ? 0.f : 1.0f / scalar_load(sa);
    const float inv_b0 = RW ? 0.f : 1.0f / scalar_load(sb);
    // tensorwise: one reciprocal per operand
    float inv_ar[NF];
    v4f inv_br[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      inv_ar[f] = inv_a0;
      inv_br[f] = (v4f){inv_b0, inv_b0, inv_b0, inv_b0};
    }
    // rowwise: the tile's reciprocal scales
    const float *tab = reinterpret_cast<const float *>(epi + (tile & 1) * SCALE_BYTES);
    uint8_t *stg = epi + RW_STAGE_OFF;            // rowwise staging
    if (RW && F32) {
      // rowwise fp32: the tile's columns in two halves of 64, one 16-row
      // block per pass: 16 rows x 256 B (row r's 16-byte chunk c at
      // c ^ (r % 16)); the reciprocals are read from the table where they
      // are used
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int col = n0 + wn * WN + jh * 64 + (lane_e & 15) * 4;
        const bool col_ok = col < N;
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          const float ia = tab[wm * WM + i * FR + ml16];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = jh * 4 + jj;
            const v4f ib = *reinterpret_cast<const v4f *>(tab + BM + wn * WN + j * FR + nq);
            const v4f v = {(acc[j][i][0] * ia) * ib[0], (acc[j][i][1] * ia) * ib[1],
                           (acc[j][i][2] * ia) * ib[2], (acc[j][i][3] * ia) * ib[3]};
            const int ch = (jj * 4 + (lane_e >> 4)) ^ ml16;
            *reinterpret_cast<v4f *>(stg + ml16 * 256 + ch * 16) = v;
          }
          const int row0 = m0 + wm * WM + i * FR;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = u * 4 + (lane_e >> 4);
            const v4u v = *reinterpret_cast<const v4u *>(
                stg + r * 256 + (((lane_e & 15) ^ r) * 16));
            const uint32_t off = (col_ok && row0 + r < M) ? (uint32_t)(((row0 + r) * N + col) * 4)
                                                          : OOB_C;
            __builtin_amdgcn_raw_buffer_store_b128(v, rsC, off, 0, C_STORE_AUX);
          }
        }
      }
    } else if (F32) {
      // one 16-row block per pass: 16 rows x 512 B (32 chunks per row)
#pragma unroll
      for (int i = 0; i < NF; ++i) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          const v4f ib = inv_br[j];
          const v4f v = {(acc[j][i][0] * inv_ar[i]) * ib[0], (acc[j][i][1] * inv_ar[i]) * ib[1],
                         (acc[j][i][2] * inv_ar[i]) * ib[2], (acc[j][i][3] * inv_ar[i]) * ib[3]};
          const int ch = (j * 4 + (lane_e >> 4)) ^ ml16;
          *reinterpret_cast<v4f *>(epi + ml16 * 512 + ch * 16) = v;
        }
        const int row0 = m0 + wm * WM + i * FR;
        const int col = n0 + wn * WN + (lane_e & 31) * 4;
        const bool col_ok = col < N;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = u * 2 + (lane_e >> 5);
          const v4u v = *reinterpret_cast<const v4u *>(
              epi + r * 512 + (((lane_e & 31) ^ (r & 15)) * 16));
          const uint32_t off = (col_ok && row0 + r < M) ? (uint32_t)(((row0 + r) * N + col) * 4)
                                                        : OOB_C;
          __builtin_amdgcn_raw_buffer_store_b128(v, rsC, off, 0, C_STORE_AUX);
        }
      }
    } else if (RW) {
      // rowwise bf16: the tile's columns in two halves of 64, 32 rows x
      // 128 B per pass (row r's 16-byte chunk c at c ^ (r % 8), its 8-byte
      // halves swapped where r % 16 >= 8); the reciprocals are read from the
      // table where they are used (2 row and 4 column values at a time), so
      // that they add few registers to the epilogue's
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const int scol = n0 + wn * WN + jh * 64 + (lane_e & 7) * 8;
        const bool col_ok = scol < N;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float ia0 = tab[wm * WM + 2 * p * FR + ml16];
          const float ia1 = tab[wm * WM + (2 * p + 1) * FR + ml16];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int j = jh * 4 + jj;
            const v4f ib = *reinterpret_cast<const v4f *>(tab + BM + wn * WN + j * FR + nq);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
              const int i = 2 * p + ii;
              const int ml = ii * FR + ml16;      // row within the pass
              const float ia = ii ? ia1 : ia0;
              f32x2 v01 = {(acc[j][i][0] * ia) * ib[0], (acc[j][i][1] * ia) * ib[1]};
              f32x2 v23 = {(acc[j][i][2] * ia) * ib[2], (acc[j][i][3] * ia) * ib[3]};
              const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
              const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
              // byte column (jj*16 + nq)*2 of the half: chunk 2jj + nq/8
              const int ch = (2 * jj + (nq >> 3)) ^ (ml16 & 7);
              *reinterpret_cast<uint2 *>(stg + ml * 128 + ch * 16 +
                                         (((nq & 7) * 2) ^ ((ml16 >> 3) << 3))) =
                  make_uint2(p01, p23);
            }
          }
          // 4 instructions: rows u*8 + lane/8 of the pass, 8 columns each
          const int srow = m0 + wm * WM + p * 32 + (lane_e >> 3);
          v4u v[4];
          uint32_t off[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = u * 8 + (lane_e >> 3);
            v[u] = *reinterpret_cast<const v4u *>(stg + r * 128 + (((lane_e & 7) ^ (r & 7)) * 16));
            // rows with r % 16 >= 8 (u odd) hold their halves swapped
            if (u & 1) v[u] = (v4u){v[u].z, v[u].w, v[u].x, v[u].y};
            const bool ok = col_ok && srow + u * 8 < M;
            off[u] = ok ? (uint32_t)(((srow + u * 8) * N + scol) * 2) : OOB_C;
          }
          if (ACC) {
            v4u cin[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) cin[u] = __builtin_amdgcn_raw_buffer_load_b128(rsC, off[u], 0, 0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const uint32_t x = v[u][d], y = cin[u][d];
                const f32x2 sum = {__uint_as_float(x << 16) + __uint_as_float(y << 16),
                                   __uint_as_float(x & 0xFFFF0000u) + __uint_as_float(y & 0xFFFF0000u)};
                v[u][d] = __builtin_bit_cast(uint32_t, __builtin_convertvector(sum, bf16x2));
              }
            }
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(v[u], rsC, off[u], 0, C_STORE_AUX);
        }
      }
    } else {
      const int scol = n0 + wn * WN + (lane_e & 15) * 8;
      const bool col_ok = scol < N;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * p + ii;
          const int ml = ii * FR + ml16;          // row within the pass
#pragma unroll
          for (int j = 0; j < NF; ++j) {
            const v4f ib = inv_br[j];
            const float ia = inv_ar[i];
            f32x2 v01 = {(acc[j][i][0] * ia) * ib[0], (acc[j][i][1] * ia) * ib[1]};
            f32x2 v23 = {(acc[j][i][2] * ia) * ib[2], (acc[j][i][3] * ia) * ib[3]};
            const uint32_t p01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, bf16x2));
            const uint32_t p23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, bf16x2));
            // byte column (j*16 + nq)*2: chunk 2j + nq/8, 8 bytes in at
            // (nq%8)*2, the two halves of the chunk swapped in rows 8..15 of
            // a block (16 lanes of one write then cover all 32 banks)
            const int ch = (2 * j + (nq >> 3)) ^ ml16;
            *reinterpret_cast<uint2 *>(epi + ml * 256 + ch * 16 +
                                       (((nq & 7) * 2) ^ ((ml16 >> 3) << 3))) =
                make_uint2(p01, p23);
          }
        }
        // 8 instructions: rows u*4 + lane/16 of the pass, 8 columns each
        const int srow = m0 + wm * WM + p * 32 + (lane_e >> 4);
        v4u v[8];
        uint32_t off[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int r = u * 4 + (lane_e >> 4);
          v[u] = *reinterpret_cast<const v4u *>(epi + r * 256 + (((lane_e & 15) ^ (r & 15)) * 16));
          // rows with r % 16 >= 8 (u = 2, 3, 6, 7) hold their halves swapped
          if (u & 2) v[u] = (v4u){v[u].z, v[u].w, v[u].x, v[u].y};
          const bool ok = col_ok && srow + u * 4 < M;
          off[u] = ok ? (uint32_t)(((srow + u * 4) * N + scol) * 2) : OOB_C;
        }
        if (ACC) {
          v4u cin[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) cin[u] = __builtin_amdgcn_raw_buffer_load_b128(rsC, off[u], 0, 0);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t x = v[u][d], y = cin[u][d];
              const f32x2 sum = {__uint_as_float(x << 16) + __uint_as_float(y << 16),
                                 __uint_as_float(x & 0xFFFF0000u) + __uint_as_float(y & 0xFFFF0000u)};
              v[u][d] = __builtin_bit_cast(uint32_t, __builtin_convertvector(sum, bf16x2));
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) __builtin_amdgcn_raw_buffer_store_b128(v[u], rsC, off[u], 0, C_STORE_AUX);
      }
    }
#ifdef FP8L_PHASE_TIMING
    const int slot = tile * G + (int)blockIdx.x;    // round-major record index
    if (wave == 0 && hw_lane() == 0 && slot < PHASE_MAX_BLOCKS) {
      const unsigned long long ph_t2 = __builtin_amdgcn_s_memtime();
      const unsigned long long ph_r2 = __builtin_amdgcn_s_memrealtime();
      unsigned long long *d = g_phase + (size_t)slot * 8;
      d[0] = ph_t0; d[1] = ph_r0; d[2] = ph_ta; d[3] = ph_ra;
      d[4] = ph_t1; d[5] = ph_r1; d[6] = ph_t2; d[7] = ph_r2;
    }
#endif
    // rowwise: the scales of the tile after next go into the table this
    // tile is done with, after the stores (the next tile's first wait lets
    // both run on).  A wave stages and keeps its scales only in its own part
    // of the epilogue region, and the next tile's operands were made visible
    // by the barrier of this tile's last k-tile: no barrier here.
    if (RW) FP8P_SCALES(b_ok, b_pi, b_m0, b_n0, tile & 1);
  }
#undef FP8P_H2D
#undef FP8P_H2
#undef FP8P_H1
#undef FP8P_E
#undef FP8P_MX
#undef FP8P_MFZ
#undef FP8P_MF
#undef FP8P_RD
#undef FP8P_SCALES
#undef FP8P_RCP_AT
#undef FP8P_DMA1
#undef FP8P_DADV
#undef FP8P_DSETUP
#undef FP8P_SETVOFF
}

}  // namespace

namespace {

// K = 0: the product over an empty contraction is zero.  Such problems are
// not given to the GEMM kernel (each of its tiles has at least one k-tile,
// which lets every tile start its accumulators from a zero input instead of
// clearing them); this kernel writes their outputs instead: zeros, or with
// ACC the bf16 sum of C and a zero product, fl32(C) + 0 rounded (which
// turns -0 into +0 and keeps everything else).  n16: 16-byte chunks of C.
template <bool F32, bool ACC>
__global__ __launch_bounds__(256) void k_gemm_k0(void *C, int n16) {
  v4u *c = reinterpret_cast<v4u *>(C);
  for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < n16; i += (int)(gridDim.x * 256)) {
    v4u v = {0u, 0u, 0u, 0u};
    if (ACC) {
      v = c[i];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t x = v[d];
        const float lo = __uint_as_float(x << 16) + 0.f;
        const float hi = __uint_as_float(x & 0xFFFF0000u) + 0.f;
        v[d] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
      }
    }
    c[i] = v;
  }
}

// One launch over the problems of d (count <= MAX_GROUP, bf16 or fp32
// outputs per F32, accumulating per ACC); empty problems get no workgroups,
// and problems with K = 0 a launch of k_gemm_k0 each.
template <bool F32, int FA, bool ACC = false>
hipError_t launch_group(const GemmDesc *d, int count, int rowwise, hipStream_t stream) {
  GemmGroup g = {};
  int blocks = 0;
  bool kfull = true;
  // the problems in launch order: longest K first (stable), so that a
  // balanced schedule places the long tiles first
  int order[MAX_GROUP], n_order = 0;
  for (int i = 0; i < count; ++i) {
    if (d[i].M == 0 || d[i].N == 0) continue;
    if (d[i].K == 0) {
      const int n16 = (int)(d[i].M * d[i].N * (F32 ? 4 : 2) / 16);
      const int nb = n16 < 256 * 1024 ? (n16 + 255) / 256 : 1024;
      hipLaunchKernelGGL((k_gemm_k0<F32, ACC>), dim3((unsigned)nb), dim3(256), 0, stream,
                         d[i].C, n16);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      continue;
    }
    order[n_order++] = i;
  }
  for (int a = 1; a < n_order; ++a)
    for (int b = a; b > 0 && d[order[b]].K > d[order[b - 1]].K; --b) {
      const int t = order[b];
      order[b] = order[b - 1];
      order[b - 1] = t;
    }
  for (int o = 0; o < n_order; ++o) {
    const int i = order[o];
    const int c = g.count++;
    g.A[c] = d[i].A;
    g.sa[c] = d[i].sa;
    g.B[c] = d[i].B;
    g.sb[c] = d[i].sb;
    g.C[c] = d[i].C;
    g.M[c] = (int)d[i].M;
    g.N[c] = (int)d[i].N;
    g.K[c] = (int)d[i].K;
    g.tiles_m[c] = (int)((d[i].M + BM - 1) / BM);
    g.tiles_n[c] = (int)((d[i].N + BN - 1) / BN);
    blocks += g.tiles_m[c] * g.tiles_n[c];
    kfull = kfull && d[i].K % BK == 0;
  }
  if (blocks == 0) return hipSuccess;
  g.total = blocks;
  // one workgroup per compute unit (256 on gfx950), each walking its tiles
  constexpr int kComputeUnits = 256;
  auto kern = rowwise ? (kfull ? k_gemm_fp8_pers<true, true, F32, FA, ACC>
                               : k_gemm_fp8_pers<false, true, F32, FA, ACC>)
                      : (kfull ? k_gemm_fp8_pers<true, false, F32, FA, ACC>
                               : k_gemm_fp8_pers<false, false, F32, FA, ACC>);
  const int grid = blocks < kComputeUnits ? blocks : kComputeUnits;
  // equal K: round-robin dealing is already the balanced schedule
  bool mixed = false;
  for (int c = 1; c < g.count; ++c) mixed = mixed || g.K[c] != g.K[0];
  if (mixed) {
    int tiles[MAX_GROUP], ktiles[MAX_GROUP];
    for (int c = 0; c < g.count; ++c) {
      tiles[c] = g.tiles_m[c] * g.tiles_n[c];
      ktiles[c] = (g.K[c] + BK - 1) / BK;
    }
    sched::Packed pk;
    if (sched::balance(grid, g.count, tiles, ktiles, pk)) {
      g.balanced = 1;
      for (int x = 0; x < NUM_XCD; ++x)
        for (int c = 0; c < MAX_GROUP; ++c) {
          g.sched_min[x] |= (uint32_t)pk.min_count[x][c] << (8 * c);
          for (int l = 0; l < 32; ++l)
            g.sched[x][c][l >> 1] |= (uint32_t)pk.entry[x][c][l] << (16 * (l & 1));
        }
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(THREADS), 0, stream, g);
  return hipGetLastError();
}

template <bool F32, int FA, bool ACC = false>
hipError_t launch_variant(const uint8_t *A, const float *sa, const uint8_t *B,
                          const float *sb, int rowwise, int64_t M, int64_t N, int64_t K,
                          void *C, hipStream_t stream) {
  const GemmDesc d = {A, sa, B, sb, C, M, N, K};
  return launch_group<F32, FA, ACC>(&d, 1, rowwise, stream);
}

}  // namespace

hipError_t gemm_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                       const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                       int64_t K, uint16_t *C, hipStream_t stream) {
  return fmt_a ? launch_variant<false, 1>(A, sa, B, sb, rowwise, M, N, K, C, stream)
               : launch_variant<false, 0>(A, sa, B, sb, rowwise, M, N, K, C, stream);
}

hipError_t gemm_acc_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                           const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                           int64_t K, uint16_t *C, hipStream_t stream) {
  return fmt_a ? launch_variant<false, 1, true>(A, sa, B, sb, rowwise, M, N, K, C, stream)
               : launch_variant<false, 0, true>(A, sa, B, sb, rowwise, M, N, K, C, stream);
}

hipError_t gemm_group_launch(const GemmDesc *d, int count, int rowwise, int fmt_a,
                             hipStream_t stream) {
  if (count < 1 || count > MAX_GROUP) return hipErrorInvalidValue;
  return fmt_a ? launch_group<false, 1>(d, count, rowwise, stream)
               : launch_group<false, 0>(d, count, rowwise, stream);
}

hipError_t gemm_f32_launch(const uint8_t *A, const float *sa, const uint8_t *B,
                           const float *sb, int rowwise, int fmt_a, int64_t M, int64_t N,
                           int64_t K, float *C, hipStream_t stream) {
  return fmt_a ? launch_variant<true, 1>(A, sa, B, sb, rowwise, M, N, K, C, stream)
               : launch_variant<true, 0>(A, sa, B, sb, rowwise, M, N, K, C, stream);
}

}  // namespace fp8l

#ifdef FP8L_PHASE_TIMING
// Copies the first `bytes` of the timestamp array (8 u64 per workgroup:
// memtime, realtime at start, after the prologue, after the main loop, at
// the end) to host memory; synchronous.  Returns 0, or 5 on a HIP error.
extern "C" __attribute__((visibility("default"))) int fp8_gemm_phase_read(void *host,
                                                                          size_t bytes) {
  if (bytes > sizeof(fp8l::g_phase)) bytes = sizeof(fp8l::g_phase);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(fp8l::g_phase), bytes, 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 5;
}
#endif
