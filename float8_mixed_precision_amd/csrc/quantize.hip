// Dynamic-scaling quantization of a bf16 matrix to E4M3 on gfx950:
//   tensorwise:
//   1. k_amax_tw       : one read pass, grid-stride; per-block maxima of |x|
//   2. (in k_cast_transpose) every block reduces the partial maxima itself,
//                        s = 448 / max(amax, 1e-12); block 0 stores s
//                        (k_finalize_tw_empty does that alone for an empty x)
//   rowwise:
//   1. k_amax_partial  : one read pass; per-tile row / column maxima
//   2. k_finalize_rowwise: reduce the partials, one scale per row / column
//   both:
//   3. k_cast_transpose: second read pass; writes q (row-major) directly and
//                        qt (the transpose) through an LDS tile
// The method is Float8 training of linear layers ("Torchtitan: A PyTorch
// Library for Parallelism Techniques explained", section 3, "Float8
// Training"); the 8-bit format is E4M3, named on the "torchtitan" tutorial
// page, Part XI, item 9.  The scaling recipe (dynamic amax, per tensor or per
// row / column) is the reading stated in include/fp8_linear.h.
//
// The amax is taken on |bf16| bit patterns with integer max: for
// non-negative values the bit order is the value order, and NaN patterns
// (exponent all ones, mantissa non-zero) sort above +inf, so a NaN anywhere
// makes the amax NaN without a floating-point compare.
#include "fp8l_internal.h"

namespace fp8l {
namespace {

// tensorwise amax: chunks of 256 threads x 8 loads of 16 bytes (32 KB),
// at most TW_MAX_BLOCKS workgroups in a grid-stride loop.  Workspace: one
// u32 partial maximum per block.  (The rowwise tile AM_TR x AM_TC and
// TW_MAX_BLOCKS are in fp8l_internal.h: producer kernels elsewhere write
// partials in the same layouts.)
constexpr int TW_UNROLL = 8;
constexpr int TW_CHUNK = AM_THREADS * TW_UNROLL;   // 16-byte vectors per chunk

// cast tile: 128 rows x 128 columns per 512-thread workgroup, one 4-row
// group per thread (a single pass: no thread's loads wait behind its own
// earlier stores, which complete in issue order).
constexpr int CT_T = 128;
constexpr int CT_THREADS = 512;
constexpr int CT_PASSES = CT_T / (CT_THREADS / 16 * 4);
static_assert(CT_PASSES >= 1 && CT_T % (CT_THREADS / 16 * 4) == 0, "cast rows per pass");
// Tile order of the cast: groups of CT_GROUP row tiles, the row tile
// fastest within a group, so the workgroups running at one time write
// neighbouring 128-byte segments of each qt row.  q and qt are written with
// non-temporal stores when CT_NT.  (Both are set from measurements of the
// whole step; see the notes at k_cast_transpose.)
#ifndef FP8L_CAST_GROUP
#define FP8L_CAST_GROUP 2
#endif
#ifndef FP8L_CAST_NT
#define FP8L_CAST_NT 0
#endif
constexpr int CT_GROUP = FP8L_CAST_GROUP;
constexpr bool CT_NT = FP8L_CAST_NT != 0;
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- amax --
//
// Tensorwise.  Every load is issued unconditionally (index clamped into the
// tensor, the value masked afterwards), so a thread's 8 loads are in flight
// together.  Each block writes its maximum to part[block].
__global__ __launch_bounds__(AM_THREADS) void k_amax_tw(
    const uint4 *__restrict__ x, int64_t n16, uint32_t *__restrict__ part) {
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  const int64_t nchunks = (n16 + TW_CHUNK - 1) / TW_CHUNK;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const int64_t base = ch * TW_CHUNK + tid;
    uint4 v[TW_UNROLL];
#pragma unroll
    for (int u = 0; u < TW_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * AM_THREADS;
      v[u] = x[i < n16 ? i : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < TW_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * AM_THREADS;
      const uint32_t keep = i < n16 ? 0x7FFF7FFFu : 0u;
      acc = max_u16x2(acc, max_u16x2(max_u16x2(v[u].x & keep, v[u].y & keep),
                                     max_u16x2(v[u].z & keep, v[u].w & keep)));
    }
  }
  __shared__ uint32_t red[AM_THREADS / 64];
  uint32_t m = wave_max(hmax16(acc));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = red[0];
#pragma unroll
    for (int w = 1; w < AM_THREADS / 64; ++w) t = max(t, red[w]);
    part[blockIdx.x] = t;
  }
}

// The tensor's amax from the nb partial maxima, by a whole NTHR-thread block
// (all loads in flight together, index clamped and value masked); nb = 0 is
// an empty tensor: amax 0.  Returns the u16 bits of |amax| to every thread.
template <int NTHR>
__device__ __forceinline__ uint32_t tw_amax_bits(const uint32_t *__restrict__ part, int nb,
                                                 uint32_t *red) {
  static_assert(TW_MAX_BLOCKS % NTHR == 0 && NTHR % 64 == 0, "whole waves, equal shares");
  const int tid = threadIdx.x;
  uint32_t t = 0;
  if (nb > 0) {
    uint32_t pv[TW_MAX_BLOCKS / NTHR];
#pragma unroll
    for (int k = 0; k < TW_MAX_BLOCKS / NTHR; ++k) {
      const int i = tid + k * NTHR;
      pv[k] = part[i < nb ? i : nb - 1];
    }
#pragma unroll
    for (int k = 0; k < TW_MAX_BLOCKS / NTHR; ++k) t = max(t, pv[k]);
  }
  t = wave_max(t);
  if ((tid & 63) == 0) red[tid >> 6] = t;
  __syncthreads();
  uint32_t mm = red[0];
#pragma unroll
  for (int w = 1; w < NTHR / 64; ++w) mm = max(mm, red[w]);
  return mm;
}

// Shard amax only: one block reduces the partials and stores |amax|.
__global__ __launch_bounds__(AM_THREADS) void k_amax_finish(
    const uint32_t *__restrict__ part, int nb, float *amax_out) {
  __shared__ uint32_t red[AM_THREADS / 64];
  const uint32_t am = tw_amax_bits<AM_THREADS>(part, nb, red);
  if (threadIdx.x == 0) amax_out[0] = bf16_to_f32(am);
}

// Empty tensor: the scale of amax 0.
template <int FMT>
__global__ __launch_bounds__(64) void k_finalize_tw_empty(float *scale, float *scale_t,
                                                          float *amax_out) {
  if (threadIdx.x == 0) {
    const float sc = scale_from_amax<FMT>(0.f);
    scale[0] = sc;
    scale_t[0] = sc;
    if (amax_out) amax_out[0] = 0.f;
  }
}

// Rowwise: rowpart[tile_c][r] = max over the tile's columns of row r,
//          colpart[tile_r][c] = max over the tile's rows of column c.
// Loads are unconditional (row clamped into the tensor, column chunk to 0)
// and masked afterwards, so the 8 loads of a thread are in flight together.
__global__ __launch_bounds__(AM_THREADS) void k_amax_partial(
    const uint16_t *__restrict__ x, int rows, int cols, int tiles_c,
    uint16_t *__restrict__ rowpart, uint16_t *__restrict__ colpart) {
  const int tid = threadIdx.x;
  const int tile_c = blockIdx.x % tiles_c;
  const int tile_r = blockIdx.x / tiles_c;
  const int cx = tid & 31;        // 8-column chunk within the tile
  const int ry = tid >> 5;        // 0..7, row phase
  const int r0 = tile_r * AM_TR;
  const int c = tile_c * AM_TC + cx * 8;
  const bool col_ok = c < cols;
  const int cl = col_ok ? c : 0;

  U4 v[AM_TR / 8];
#pragma unroll
  for (int i = 0; i < AM_TR / 8; ++i) {
    const int r = r0 + ry + 8 * i;
    v[i] = load16(x + (size_t)min(r, rows - 1) * cols + cl);
  }
  uint32_t cm[4] = {0, 0, 0, 0};  // column maxima, 2 per dword
#pragma unroll
  for (int i = 0; i < AM_TR / 8; ++i) {
    const int r = r0 + ry + 8 * i;
    const uint32_t keep = (col_ok && r < rows) ? 0x7FFF7FFFu : 0u;
    const uint32_t x0 = v[i].x & keep, x1 = v[i].y & keep;
    const uint32_t x2 = v[i].z & keep, x3 = v[i].w & keep;
    cm[0] = max_u16x2(cm[0], x0);
    cm[1] = max_u16x2(cm[1], x1);
    cm[2] = max_u16x2(cm[2], x2);
    cm[3] = max_u16x2(cm[3], x3);
    uint32_t rm = hmax16(max_u16x2(max_u16x2(x0, x1), max_u16x2(x2, x3)));
    rm = half_wave_max(rm);        // the 32 lanes of a half-wave share row r
    if (cx == 0 && r < rows) rowpart[(size_t)tile_c * rows + r] = (uint16_t)rm;
  }

  // reduce the column maxima over the 8 row phases through LDS
  __shared__ uint32_t cred[8][AM_TC / 2];
#pragma unroll
  for (int j = 0; j < 4; ++j) cred[ry][cx * 4 + j] = cm[j];
  __syncthreads();
  if (tid < AM_TC / 2) {
    uint32_t t = cred[0][tid];
#pragma unroll
    for (int p = 1; p < 8; ++p) t = max_u16x2(t, cred[p][tid]);
    const int cc = tile_c * AM_TC + tid * 2;
    if (cc < cols) {
      uint16_t *dst = colpart + (size_t)tile_r * cols + cc;
      dst[0] = (uint16_t)(t & 0xFFFFu);
      dst[1] = (uint16_t)(t >> 16);
    }
  }
}

// ------------------------------------------------------------- finalize --

// One scale per row and per column from the partial maxima.  Workgroups
// [0, nbr) cover 64 rows each (max over tiles_c row partials), the rest 64
// columns each (max over tiles_r column partials).  Thread (o, sl), o =
// tid % 64, sl = tid / 64, reduces partials sl, sl + 4, ... of output o with
// eight loads in flight at a time (index clamped into the array, value
// masked), and the four slices meet in LDS.  (One thread per output walking
// its partials serially took as long as the amax pass itself.)
constexpr int FR_OUT = 64;
constexpr int FR_SLICES = 4;
constexpr int FR_UNROLL = 8;
static_assert(FR_OUT * FR_SLICES == 256, "one finalize workgroup is 256 threads");
template <int FMT>
__global__ __launch_bounds__(256) void k_finalize_rowwise(
    const uint16_t *__restrict__ rowpart, const uint16_t *__restrict__ colpart,
    int rows, int cols, int tiles_c, int tiles_r, int nbr, float *scale, float *scale_t,
    float *amax_out) {
  const int o = threadIdx.x % FR_OUT;
  const int sl = threadIdx.x / FR_OUT;
  const bool is_row = (int)blockIdx.x < nbr;
  const int n = is_row ? rows : cols;                 // >= 1 for any launched block
  const int T = is_row ? tiles_c : tiles_r;
  const uint16_t *__restrict__ part = is_row ? rowpart : colpart;
  const int i = (is_row ? (int)blockIdx.x : (int)blockIdx.x - nbr) * FR_OUT + o;
  const int ic = i < n ? i : n - 1;
  uint32_t m = 0;
  for (int t0 = sl; t0 < T; t0 += FR_SLICES * FR_UNROLL) {
    uint32_t v[FR_UNROLL];
#pragma unroll
    for (int u = 0; u < FR_UNROLL; ++u) {
      const int t = t0 + FR_SLICES * u;
      v[u] = part[(size_t)(t < T ? t : T - 1) * n + ic];
    }
#pragma unroll
    for (int u = 0; u < FR_UNROLL; ++u)
      if (t0 + FR_SLICES * u < T) m = max(m, v[u]);
  }
  __shared__ uint32_t red[FR_SLICES][FR_OUT];
  red[sl][o] = m;
  __syncthreads();
  if (sl == 0 && i < n) {
#pragma unroll
    for (int k = 1; k < FR_SLICES; ++k) m = max(m, red[k][o]);
    const float a = bf16_to_f32(m);
    if (is_row) {
      scale[i] = scale_from_amax<FMT>(a);
      if (amax_out) amax_out[i] = a;
    } else {
      scale_t[i] = scale_from_amax<FMT>(a);
      if (amax_out) amax_out[rows + i] = a;
    }
  }
}

// -------------------------------------------------------- cast+transpose --
//
// Tile of 128 rows x 128 columns.  Thread (c8, rg): c8 = tid % 16 selects an
// 8-column chunk, rg = tid / 16 a group of 4 consecutive rows, rows
// rg*4 + {0..3} (one pass with 512 threads).
//
// Phase A: 16-byte coalesced loads of bf16 (a wave reads 4 rows x 256 B per
// instruction), scale, convert, 8-byte stores of q (4 rows x 128 B per
// wave).  The 4 x 8 block of qt codes is transposed in registers into eight
// dwords (4 consecutive rows of one column each) and written to the LDS tile
// lds[col][row] (128 B per column).  The 16-byte row chunk of a column is
// XOR-swizzled with the column's chunk index (col / 8) so that the 16 column
// chunks of a wave spread over the banks.
//
// Phase B: each thread reads 16-byte chunks (16 rows of one column) from LDS
// and stores them to qt: eight threads write one 128-byte qt row segment.
//
// MODE_TW: the block first reduces the amax pass's partial maxima to the
// tensor's scale; block 0 also stores it (scale, scale_t, amax_out).
// MODE_RW: scale / scale_t are inputs (from k_finalize_rowwise).
// MODE_GIVEN: scale[0] is a tensorwise multiplier given by the caller.
// FMT: 0 = E4M3 codes, 1 = E5M2 codes (scale onto 57344).
constexpr int MODE_TW = 0, MODE_RW = 1, MODE_GIVEN = 2;
template <int MODE, int FMT>
__global__ __launch_bounds__(CT_THREADS) void k_cast_transpose(
    const uint16_t *__restrict__ x, int rows, int cols, int tiles_c,
    float *__restrict__ scale, float *__restrict__ scale_t,
    const uint32_t *__restrict__ part, int nparts, float *__restrict__ amax_out,
    uint8_t *__restrict__ q, uint8_t *__restrict__ qt) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[CT_T * CT_T];
  const int tid = threadIdx.x;
  // block -> (tile_r, tile_c): groups of CT_GROUP row tiles (the last one
  // possibly shorter), row tile fastest within a group
  const int tiles_r = (rows + CT_T - 1) / CT_T;
  const int per_group = CT_GROUP * tiles_c;
  const int first_r = ((int)blockIdx.x / per_group) * CT_GROUP;
  const int gm = min(tiles_r - first_r, CT_GROUP);
  const int in_group = (int)blockIdx.x % per_group;
  const int tile_r = first_r + in_group % gm;
  const int tile_c = in_group / gm;
  const int r0 = tile_r * CT_T;
  const int c0 = tile_c * CT_T;
  const int c8 = tid & 15;
  const int rg = tid >> 4;
  const int c = c0 + c8 * 8;
  const bool col_ok = c < cols;
  constexpr bool ROWWISE = MODE == MODE_RW;

  // rowwise scale vectors 16-byte aligned (the interface promises 4): read
  // them as float4, else one float at a time
  const bool vec_scales =
      ROWWISE && ((reinterpret_cast<uintptr_t>(scale) | reinterpret_cast<uintptr_t>(scale_t)) &
                  15u) == 0;
  float sc[8];                    // column scales (rowwise) of the 8 columns
  float s_t = 0.f;                // tensor scale
  if (ROWWISE) {
    if (col_ok && vec_scales) {
      const float4 a = *reinterpret_cast<const float4 *>(scale_t + c);
      const float4 b = *reinterpret_cast<const float4 *>(scale_t + c + 4);
      sc[0] = a.x; sc[1] = a.y; sc[2] = a.z; sc[3] = a.w;
      sc[4] = b.x; sc[5] = b.y; sc[6] = b.z; sc[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[j] = col_ok ? scale_t[c + j] : 0.f;
    }
  } else if (MODE == MODE_GIVEN) {
    s_t = scale[0];
  } else {
    __shared__ uint32_t red[CT_THREADS / 64];
    const uint32_t am = tw_amax_bits<CT_THREADS>(part, nparts, red);
    const float a = bf16_to_f32(am);
    s_t = scale_from_amax<FMT>(a);
    if (blockIdx.x == 0 && tid == 0) {
      scale[0] = s_t;
      scale_t[0] = s_t;
      if (amax_out) amax_out[0] = a;
    }
  }

#pragma unroll
  for (int pass = 0; pass < CT_PASSES; ++pass) {
    const int rl = pass * (CT_THREADS / 4) + rg * 4;   // local row of the 4-row group
    const int r = r0 + rl;
    // rows is a multiple of 16, so the 4 rows are all in or all out
    const bool ok = col_ok && r < rows;
    uint32_t lo[4], hi[4];               // qt codes: cols 0-3 / 4-7 of each row
    if (ok) {
      // the 4 rows' scales (rowwise; r is a multiple of 4)
      float srs[4] = {s_t, s_t, s_t, s_t};
      if (ROWWISE) {
        if (vec_scales) {
          const float4 v = *reinterpret_cast<const float4 *>(scale + r);
          srs[0] = v.x; srs[1] = v.y; srs[2] = v.z; srs[3] = v.w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) srs[j] = scale[r + j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const U4 v = load16(x + (size_t)(r + j) * cols + c);
        float f[8];
        f[0] = bf16_to_f32(v.x & 0xFFFFu); f[1] = bf16_to_f32(v.x >> 16);
        f[2] = bf16_to_f32(v.y & 0xFFFFu); f[3] = bf16_to_f32(v.y >> 16);
        f[4] = bf16_to_f32(v.z & 0xFFFFu); f[5] = bf16_to_f32(v.z >> 16);
        f[6] = bf16_to_f32(v.w & 0xFFFFu); f[7] = bf16_to_f32(v.w >> 16);
        const float s = srs[j];
        const uint32_t q0 = fp8x4<FMT>(f[0] * s, f[1] * s, f[2] * s, f[3] * s);
        const uint32_t q1 = fp8x4<FMT>(f[4] * s, f[5] * s, f[6] * s, f[7] * s);
        v2u_t *qdst = reinterpret_cast<v2u_t *>(q + (size_t)(r + j) * cols + c);
        if (CT_NT)
          __builtin_nontemporal_store((v2u_t){q0, q1}, qdst);
        else
          *qdst = (v2u_t){q0, q1};
        if (ROWWISE) {
          lo[j] = fp8x4<FMT>(f[0] * sc[0], f[1] * sc[1], f[2] * sc[2], f[3] * sc[3]);
          hi[j] = fp8x4<FMT>(f[4] * sc[4], f[5] * sc[5], f[6] * sc[6], f[7] * sc[7]);
        } else {
          lo[j] = q0;
          hi[j] = q1;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) lo[j] = hi[j] = 0;
    }
    // 4x4 byte transposes: column k of the block = byte k of each row dword
    uint32_t t[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sh = 8 * k;
      t[k] = ((lo[0] >> sh) & 0xFFu) | (((lo[1] >> sh) & 0xFFu) << 8) |
             (((lo[2] >> sh) & 0xFFu) << 16) | (((lo[3] >> sh) & 0xFFu) << 24);
      t[4 + k] = ((hi[0] >> sh) & 0xFFu) | (((hi[1] >> sh) & 0xFFu) << 8) |
                 (((hi[2] >> sh) & 0xFFu) << 16) | (((hi[3] >> sh) & 0xFFu) << 24);
    }
    // Column col's 128 codes sit in one 128-byte LDS row: 16-row chunk
    // ch at ch ^ (col / 8 % 8), and within it the 4-row dword s at
    // s ^ 2 (col / 64).  A half-wave's writes (c8 = 0..15, two row groups)
    // then hit 32 distinct banks: the chunk swizzle separates c8 % 8, the
    // dword swap c8 and c8 + 8.
    const int chunk = rl >> 4;                // 16-row chunk of the column
    const int pchunk = chunk ^ (c8 & 7);
    const int slot = ((rl >> 2) & 3) ^ ((c8 >> 3) << 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int col = c8 * 8 + k;
      *reinterpret_cast<uint32_t *>(lds + col * CT_T + pchunk * 16 + slot * 4) = t[k];
    }
  }
  __syncthreads();

#pragma unroll
  for (int p = 0; p < (CT_T * CT_T / 16) / CT_THREADS; ++p) {
    const int id = tid + p * CT_THREADS;
    const int col = id >> 3;
    const int rc = id & 7;
    const int gc = c0 + col;
    const int gr = r0 + rc * 16;
    if (gc < cols && gr < rows) {
      const int pc = rc ^ ((col >> 3) & 7);
      v4u_t v = *reinterpret_cast<const v4u_t *>(lds + col * CT_T + pc * 16);
      if (col & 64) v = (v4u_t){v.z, v.w, v.x, v.y};   // undo the dword swap
      v4u_t *tdst = reinterpret_cast<v4u_t *>(qt + (size_t)gc * rows + gr);
      if (CT_NT)
        __builtin_nontemporal_store(v, tdst);
      else
        *tdst = v;
    }
  }
}

// --------------------------------------------------------------- encode --

template <int FMT>
__global__ __launch_bounds__(256) void k_encode(const float *__restrict__ in,
                                                uint8_t *__restrict__ out,
                                                int64_t n) {
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = reinterpret_cast<const float4 *>(in)[i];
    reinterpret_cast<uint32_t *>(out)[i] = fp8x4<FMT>(v.x, v.y, v.z, v.w);
  }
  // tail (n not a multiple of 4)
  const int64_t t = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n && t < n4 * 4 + 4) out[t] = (uint8_t)(fp8x4<FMT>(in[t], 0.f, 0.f, 0.f) & 0xFFu);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct AmaxGeom {
  int64_t tiles_r, tiles_c;
};

AmaxGeom amax_geom(int64_t rows, int64_t cols) {
  return {cdiv(rows, AM_TR), cdiv(cols, AM_TC)};
}

// As many workgroups as keep every one at the same number of chunks (the
// grid-stride loop then ends in one round), at most TW_MAX_BLOCKS.
int64_t tw_blocks(int64_t rows, int64_t cols) {
  const int64_t nchunks = cdiv(rows * cols / 8, TW_CHUNK);
  if (nchunks <= TW_MAX_BLOCKS) return nchunks;
  return cdiv(nchunks, cdiv(nchunks, TW_MAX_BLOCKS));
}

}  // namespace

size_t quantize_workspace_bytes(int64_t rows, int64_t cols, int scaling) {
  const AmaxGeom g = amax_geom(rows, cols);
  size_t bytes;
  if (!(scaling & FP8L_ROWWISE)) {
    bytes = (size_t)tw_blocks(rows, cols) * sizeof(uint32_t);
  } else {
    bytes = (size_t)(g.tiles_c * rows + g.tiles_r * cols) * sizeof(uint16_t) + 256;
  }
  return (bytes + 255) & ~(size_t)255;
}

namespace {

template <int FMT>
hipError_t finish_fmt(const void *x, int64_t rows, int64_t cols, bool rowwise, int nparts,
                      void *q, void *qt, float *scale, float *scale_t, float *amax_out,
                      void *workspace, hipStream_t stream) {
  const uint16_t *xb = static_cast<const uint16_t *>(x);
  const int R = (int)rows, C = (int)cols;
  if (rowwise) {
    const AmaxGeom g = amax_geom(rows, cols);
    uint16_t *rowpart, *colpart;
    quantize_rowwise_partials(workspace, rows, cols, &rowpart, &colpart);
    const int64_t nbr = cdiv(rows, FR_OUT), nbc = cdiv(cols, FR_OUT);
    if (nbr + nbc > 0)
      hipLaunchKernelGGL(k_finalize_rowwise<FMT>, dim3((unsigned)(nbr + nbc)), dim3(256), 0,
                         stream, rowpart, colpart, R, C, (int)g.tiles_c, (int)g.tiles_r,
                         (int)nbr, scale, scale_t, amax_out);
  } else if (nparts == 0) {
    hipLaunchKernelGGL(k_finalize_tw_empty<FMT>, dim3(1), dim3(64), 0, stream, scale,
                       scale_t, amax_out);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ct_r = cdiv(rows, CT_T), ct_c = cdiv(cols, CT_T);
  if (ct_r * ct_c > 0) {
    if (!rowwise)
      hipLaunchKernelGGL((k_cast_transpose<MODE_TW, FMT>), dim3((unsigned)(ct_r * ct_c)),
                         dim3(CT_THREADS), 0, stream, xb, R, C, (int)ct_c, scale, scale_t,
                         static_cast<const uint32_t *>(workspace), nparts, amax_out,
                         static_cast<uint8_t *>(q), static_cast<uint8_t *>(qt));
    else
      hipLaunchKernelGGL((k_cast_transpose<MODE_RW, FMT>), dim3((unsigned)(ct_r * ct_c)),
                         dim3(CT_THREADS), 0, stream, xb, R, C, (int)ct_c, scale, scale_t,
                         nullptr, 0, nullptr, static_cast<uint8_t *>(q),
                         static_cast<uint8_t *>(qt));
  }
  return hipGetLastError();
}

// first pass (amax partial maxima of x), then the second half
template <int FMT>
hipError_t quantize_launch_fmt(const void *x, int64_t rows, int64_t cols, bool rowwise,
                               void *q, void *qt, float *scale, float *scale_t,
                               float *amax_out, void *workspace, hipStream_t stream) {
  const AmaxGeom g = amax_geom(rows, cols);
  const int64_t ntiles = g.tiles_r * g.tiles_c;
  const int64_t nb = rowwise ? 0 : tw_blocks(rows, cols);
  if (!rowwise) {
    if (nb > 0)
      hipLaunchKernelGGL(k_amax_tw, dim3((unsigned)nb), dim3(AM_THREADS), 0, stream,
                         static_cast<const uint4 *>(x), rows * cols / 8,
                         static_cast<uint32_t *>(workspace));
  } else if (ntiles > 0) {
    uint16_t *rowpart, *colpart;
    quantize_rowwise_partials(workspace, rows, cols, &rowpart, &colpart);
    hipLaunchKernelGGL(k_amax_partial, dim3((unsigned)ntiles), dim3(AM_THREADS), 0, stream,
                       static_cast<const uint16_t *>(x), (int)rows, (int)cols,
                       (int)g.tiles_c, rowpart, colpart);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish_fmt<FMT>(x, rows, cols, rowwise, (int)nb, q, qt, scale, scale_t, amax_out,
                         workspace, stream);
}

}  // namespace

void quantize_rowwise_partials(void *workspace, int64_t rows, int64_t cols,
                               uint16_t **rowpart, uint16_t **colpart) {
  const AmaxGeom g = amax_geom(rows, cols);
  // column partials start on a 256-byte boundary after the row partials
  const size_t off = ((size_t)(g.tiles_c * rows) * sizeof(uint16_t) + 255) & ~(size_t)255;
  *rowpart = static_cast<uint16_t *>(workspace);
  *colpart = reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(workspace) + off);
}

hipError_t quantize_finish_launch(const void *x, int64_t rows, int64_t cols, int scaling,
                                  int nparts, void *q, void *qt, float *scale,
                                  float *scale_t, float *amax_out, void *workspace,
                                  hipStream_t stream) {
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  if (scaling & FP8L_E5M2)
    return finish_fmt<1>(x, rows, cols, rw, nparts, q, qt, scale, scale_t, amax_out,
                         workspace, stream);
  return finish_fmt<0>(x, rows, cols, rw, nparts, q, qt, scale, scale_t, amax_out, workspace,
                       stream);
}

hipError_t quantize_launch(const void *x, int64_t rows, int64_t cols,
                           int scaling, void *q, void *qt, float *scale,
                           float *scale_t, float *amax_out, void *workspace,
                           hipStream_t stream) {
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  if (scaling & FP8L_E5M2)
    return quantize_launch_fmt<1>(x, rows, cols, rw, q, qt, scale, scale_t, amax_out,
                                  workspace, stream);
  return quantize_launch_fmt<0>(x, rows, cols, rw, q, qt, scale, scale_t, amax_out,
                                workspace, stream);
}

hipError_t amax_launch(const void *x, int64_t rows, int64_t cols, float *amax_out,
                       void *workspace, hipStream_t stream) {
  const int64_t nb = tw_blocks(rows, cols);
  uint32_t *part = static_cast<uint32_t *>(workspace);
  if (nb > 0)
    hipLaunchKernelGGL(k_amax_tw, dim3((unsigned)nb), dim3(AM_THREADS), 0, stream,
                       static_cast<const uint4 *>(x), rows * cols / 8, part);
  hipLaunchKernelGGL(k_amax_finish, dim3(1), dim3(AM_THREADS), 0, stream, part, (int)nb,
                     amax_out);
  return hipGetLastError();
}

hipError_t quantize_scaled_launch(const void *x, int64_t rows, int64_t cols,
                                  const float *scale, void *q, void *qt, hipStream_t stream) {
  const int64_t ct_r = cdiv(rows, CT_T), ct_c = cdiv(cols, CT_T);
  if (ct_r * ct_c > 0)
    hipLaunchKernelGGL((k_cast_transpose<MODE_GIVEN, 0>), dim3((unsigned)(ct_r * ct_c)),
                       dim3(CT_THREADS), 0, stream, static_cast<const uint16_t *>(x), (int)rows,
                       (int)cols, (int)ct_c, const_cast<float *>(scale), nullptr, nullptr, 0,
                       nullptr, static_cast<uint8_t *>(q), static_cast<uint8_t *>(qt));
  return hipGetLastError();
}

hipError_t encode_launch(const float *in, uint8_t *out, int64_t n, int fmt,
                         hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = cdiv(n / 4 + 1, 256);
  if (blocks > 8192) blocks = 8192;
  if (fmt)
    hipLaunchKernelGGL(k_encode<1>, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
  else
    hipLaunchKernelGGL(k_encode<0>, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
  return hipGetLastError();
}

}  // namespace fp8l
