// SwiGLU elementwise of the Llama 3.1 feed-forward on gfx950, as the
// producer of the next fp8 operands.  The block's dataflow (the Llama 3.1
// model the "torchtitan" tutorial page trains, Part II, "Using it"; Float8
// training of its linears, "Torchtitan: A PyTorch Library for Parallelism
// Techniques explained", section 3):
//
//   a = x W1^T, b = x W3^T          two fp8 linears sharing one quantize of x
//   h = silu(a) * b                 this file, forward
//   out = h W2^T                    fp8 linear whose input is h
//   dh = d_out W2                   (backward of w2)
//   da = dh * b * silu'(a),  db = dh * silu(a)      this file, backward
//
// Each kernel here writes its bf16 outputs and, on the way, the amax partial
// maxima of what it wrote, in the layouts the quantize's second half reads
// (fp8l_internal.h).  The quantize of h (and of da, db) then needs only the
// cast pass: the separate amax read pass of a plain quantize is gone.
//
// Numerics (the oracle states the same definitions):
//   h  = bf16( fl32( fl32(silu(a)) * b ) )
//   da = bf16( fl32( fl32(dh * b) * fl32(silu'(a)) ) )
//   db = bf16( fl32( dh * fl32(silu(a)) ) )
// with silu(a) = a / (1 + e^-a) and silu'(a) = s (1 + a (1 - s)),
// s = 1 / (1 + e^-a), evaluated in fp64 and rounded once to fp32, so the
// fp32 values are the correctly rounded ones except where the exact value
// lies within a few fp64 ulps of an fp32 rounding boundary.
//
// silu and silu' of the bf16 gate come from a table the call first fills
// with those fp64 evaluations (see "silu table" below).
//
// Layout: a, b, h, dh, da, db are separate dense [rows, hidden] bf16
// matrices.  Tensorwise kernels walk them as flat arrays of 16-byte chunks
// (8 values) in a grid-stride loop, one partial maximum per workgroup and
// output; rowwise kernels walk tiles of AM_TR x AM_TC grid-stride and write
// row and column maxima per tile.  Workspace: the partial maxima of each
// output (two shares), then the table (72 KB).
#include "fp8l_internal.h"

namespace fp8l {
namespace {

// ------------------------------------------------------------------ math --

// fp32 -> bf16 bits, round to nearest even (exact for subnormals and
// overflow to infinity); NaN -> quiet NaN with its sign
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// sigma(x) = 1 / (1 + e^-x) in fp64: library exp, then the reciprocal from
// the hardware estimate and two Newton steps (relative error a few fp64
// ulps; x / (1 + e^-x) is taken as x * sigma).  Below -700, e^-x overflows
// or nearly does and sigma is below 2^-1000: it is taken as 0, which keeps
// silu(-inf) = -inf * 0 = NaN as the quotient gives it.
__device__ __forceinline__ double sigmoid64(double x) {
#pragma clang fp contract(off)
  const double d = 1.0 + exp(-x);
  double y = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, y, 1.0);
  y = __builtin_fma(y, e, y);
  e = __builtin_fma(-d, y, 1.0);
  y = __builtin_fma(y, e, y);
  return x < -700.0 ? 0.0 : y;
}

__device__ __forceinline__ float silu32(float a) {
#pragma clang fp contract(off)
  const double x = a;
  return (float)(x * sigmoid64(x));
}

__device__ __forceinline__ void silu_and_deriv32(float a, float &s, float &ds) {
#pragma clang fp contract(off)
  const double x = a;
  const double sg = sigmoid64(x);
  s = (float)(x * sg);
  ds = (float)(sg * (1.0 + x * (1.0 - sg)));
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

__device__ __forceinline__ uint32_t dword(const U4 &v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ U4 pack(const uint32_t w[4]) { return {w[0], w[1], w[2], w[3]}; }

// |values| of a chunk, per-half maxima folded into one dword
__device__ __forceinline__ uint32_t chunk_absmax(const U4 &v) {
  const uint32_t m = 0x7FFF7FFFu;
  return max_u16x2(max_u16x2(v.x & m, v.y & m), max_u16x2(v.z & m, v.w & m));
}

// ----------------------------------------------------------- silu table --
//
// The gate input a is bf16, so silu(a) and silu'(a) take one value per bf16
// pattern.  Each call first fills a table of both, with the fp64 functions
// above, for the patterns of exponent field [TAB_E0, TAB_E0 + TAB_NE)
// (2^-19 <= |a| < 2^17, both signs; 36 KB per function, so that two
// backward or four forward workgroups fit a compute unit's LDS); every
// workgroup of the producers copies it to LDS and looks the values up.
// Other patterns (zeros, |a| < 2^-19 or >= 2^17, infinities, NaN) take the
// fp64 path per element.  The table holds that path's own results, so an output does not
// depend on which way its element went.
constexpr int TAB_E0 = 108;
constexpr int TAB_NE = 36;
constexpr int TAB_N = 2 * TAB_NE * 128;      // entries per function

// index of a bf16 pattern in the table, or -1 outside it
__device__ __forceinline__ int tab_index(uint32_t h16) {
  const int e = (int)((h16 >> 7) & 0xFFu) - TAB_E0;
  if ((unsigned)e >= (unsigned)TAB_NE) return -1;
  return (int)((h16 >> 15) * TAB_NE + e) * 128 + (int)(h16 & 127u);
}

// the bf16 pattern of table index i
__device__ __forceinline__ uint32_t tab_pattern(int i) {
  const int t = i >> 7;
  return (uint32_t)((t / TAB_NE) << 15 | (t % TAB_NE + TAB_E0) << 7 | (i & 127));
}

// tab[0 .. TAB_N) = silu, tab[TAB_N .. 2 TAB_N) = silu'; grid covers TAB_N
__global__ __launch_bounds__(256) void k_silu_table(float *__restrict__ tab) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  float s, ds;
  silu_and_deriv32(bf16_to_f32(tab_pattern(i)), s, ds);
  tab[i] = s;
  tab[TAB_N + i] = ds;
}

// ------------------------------------------------------------- the ops --
// An op maps NIN input values (bf16 bits) to NOUT output values: fast()
// with the table (NTAB functions of it in LDS), flagging an element whose
// gate is outside it; exact() with the fp64 path.

struct FwdOp {
  static constexpr int NIN = 2, NOUT = 1, NTAB = 1;   // in: a, b; out: h
  __device__ static bool fast(const uint32_t *in, uint32_t *out, const float *tab) {
    const int i = tab_index(in[0]);
    out[0] = bf16_rne(tab[i < 0 ? 0 : i] * bf16_to_f32(in[1]));
    return i < 0;
  }
  __device__ static void exact(const uint32_t *in, uint32_t *out) {
    out[0] = bf16_rne(silu32(bf16_to_f32(in[0])) * bf16_to_f32(in[1]));
  }
};

struct BwdOp {
  static constexpr int NIN = 3, NOUT = 2, NTAB = 2;   // in: dh, a, b; out: da, db
  __device__ static bool fast(const uint32_t *in, uint32_t *out, const float *tab) {
    const int i = tab_index(in[1]);
    const int ic = i < 0 ? 0 : i;
    const float g = bf16_to_f32(in[0]);
    const float gb = g * bf16_to_f32(in[2]);
    out[0] = bf16_rne(gb * tab[TAB_N + ic]);
    out[1] = bf16_rne(g * tab[ic]);
    return i < 0;
  }
  __device__ static void exact(const uint32_t *in, uint32_t *out) {
    float s, ds;
    silu_and_deriv32(bf16_to_f32(in[1]), s, ds);
    const float g = bf16_to_f32(in[0]);
    const float gb = g * bf16_to_f32(in[2]);
    out[0] = bf16_rne(gb * ds);
    out[1] = bf16_rne(g * s);
  }
};

// Element e (0..7) of a chunk, and the chunk with element e replaced.
__device__ __forceinline__ uint32_t elem(const U4 &v, int e) {
  const uint32_t w = dword(v, e >> 1);
  return (e & 1) ? hi16(w) : lo16(w);
}

__device__ __forceinline__ void set_elem(U4 &v, int e, uint32_t h) {
  const int k = e >> 1;
  const uint32_t w = dword(v, k);
  const uint32_t nw = (e & 1) ? (lo16(w) | (h << 16)) : ((w & 0xFFFF0000u) | h);
  if (k == 0) v.x = nw;
  else if (k == 1) v.y = nw;
  else if (k == 2) v.z = nw;
  else v.w = nw;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o);
  return v;
}

// A group of G chunks (8 G elements per thread, G <= 4): the table path on
// every element, then the fp64 path for the flagged ones.  The flags of the
// whole wave are OR'ed so that the loop over flagged element slots is
// wave-uniform and holds one copy of the fp64 path; an element's inputs and
// results move through selects on the uniform slot index.  valid[c] false:
// chunk c is outside the arrays (its results are not used).
template <class OP, int G>
__device__ __forceinline__ void apply_group(const U4 (*v)[OP::NIN], U4 (*o)[OP::NOUT],
                                            const bool *valid, const float *tab) {
  uint32_t slow = 0;
#pragma unroll
  for (int c = 0; c < G; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t in[OP::NIN], out[OP::NOUT];
#pragma unroll
      for (int k = 0; k < OP::NIN; ++k) in[k] = elem(v[c][k], e);
      const bool f = OP::fast(in, out, tab);
#pragma unroll
      for (int j = 0; j < OP::NOUT; ++j) set_elem(o[c][j], e, out[j]);
      slow |= (f && valid[c] ? 1u : 0u) << (c * 8 + e);
    }
  }
  uint32_t todo = __builtin_amdgcn_readfirstlane(wave_or(slow));
  while (todo) {
    const int sl = __builtin_ctz(todo);           // wave-uniform slot
    todo &= todo - 1;
    if (slow & (1u << sl)) {
      uint32_t in[OP::NIN], out[OP::NOUT];
#pragma unroll
      for (int k = 0; k < OP::NIN; ++k) in[k] = 0;
#pragma unroll
      for (int c = 0; c < G; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (sl == c * 8 + e)
#pragma unroll
            for (int k = 0; k < OP::NIN; ++k) in[k] = elem(v[c][k], e);
      OP::exact(in, out);
#pragma unroll
      for (int c = 0; c < G; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (sl == c * 8 + e)
#pragma unroll
            for (int j = 0; j < OP::NOUT; ++j) set_elem(o[c][j], e, out[j]);
    }
  }
}

struct SwArgs {
  const uint16_t *in[3];
  uint16_t *out[2];
  uint32_t *part[2];        // tensorwise block maxima, one array per output
  uint16_t *rowpart[2];     // rowwise tile maxima, per output
  uint16_t *colpart[2];
  const float *tab;         // silu table (k_silu_table)
};

// the table's first NTAB functions into LDS
template <class OP>
__device__ __forceinline__ void load_table(float *lds_tab, const float *tab) {
  constexpr int N4 = OP::NTAB * TAB_N / 4;
  for (int i = threadIdx.x; i < N4; i += AM_THREADS)
    reinterpret_cast<float4 *>(lds_tab)[i] = reinterpret_cast<const float4 *>(tab)[i];
  __syncthreads();
}

// ----------------------------------------------------------- tensorwise --
//
// Chunks of 256 threads x SW_UNROLL 16-byte vectors; every load is issued
// unconditionally (index clamped into the arrays), stores and maxima only
// for indices inside.  The grid is a few workgroups per compute unit, each
// loading the table once.
constexpr int SW_UNROLL = 4;
constexpr int SW_CHUNK = AM_THREADS * SW_UNROLL;

template <class OP>
__global__ __launch_bounds__(AM_THREADS) void k_swiglu_tw(SwArgs p, int64_t n16) {
  __shared__ __attribute__((aligned(16))) float tab[OP::NTAB * TAB_N];
  load_table<OP>(tab, p.tab);
  const int tid = threadIdx.x;
  uint32_t acc[OP::NOUT];
#pragma unroll
  for (int j = 0; j < OP::NOUT; ++j) acc[j] = 0;
  const int64_t nchunks = (n16 + SW_CHUNK - 1) / SW_CHUNK;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const int64_t base = ch * SW_CHUNK + tid;
    U4 v[SW_UNROLL][OP::NIN];
    U4 o[SW_UNROLL][OP::NOUT];
    bool valid[SW_UNROLL];
#pragma unroll
    for (int u = 0; u < SW_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * AM_THREADS;
      valid[u] = i < n16;
      const int64_t ic = valid[u] ? i : n16 - 1;
#pragma unroll
      for (int k = 0; k < OP::NIN; ++k) v[u][k] = load16(p.in[k] + ic * 8);
    }
#pragma unroll
    for (int u = 0; u < SW_UNROLL; ++u) {
      apply_group<OP, 1>(&v[u], &o[u], &valid[u], tab);
      const int64_t i = base + (int64_t)u * AM_THREADS;
      if (valid[u]) {
#pragma unroll
        for (int j = 0; j < OP::NOUT; ++j) {
          *reinterpret_cast<uint4 *>(p.out[j] + i * 8) =
              make_uint4(o[u][j].x, o[u][j].y, o[u][j].z, o[u][j].w);
          acc[j] = max_u16x2(acc[j], chunk_absmax(o[u][j]));
        }
      }
    }
  }
  __shared__ uint32_t red[OP::NOUT][AM_THREADS / 64];
#pragma unroll
  for (int j = 0; j < OP::NOUT; ++j) {
    const uint32_t m = wave_max(hmax16(acc[j]));
    if ((tid & 63) == 0) red[j][tid >> 6] = m;
  }
  __syncthreads();
  if (tid < OP::NOUT) {
    uint32_t t = red[tid][0];
#pragma unroll
    for (int w = 1; w < AM_THREADS / 64; ++w) t = max(t, red[tid][w]);
    p.part[tid][blockIdx.x] = t;
  }
}

// -------------------------------------------------------------- rowwise --
//
// Tiles of AM_TR rows x AM_TC columns, walked grid-stride (each workgroup
// loads the table once); thread (cx, ry): cx = tid % 32 picks an 8-column
// chunk, ry = tid / 32 a row phase; the thread walks rows ry + 8 i of a
// tile, in two batches of four rows whose loads are in flight together (row
// clamped into the matrix, column chunk to 0, results masked).
template <class OP>
__global__ __launch_bounds__(AM_THREADS) void k_swiglu_rw(SwArgs p, int rows, int cols,
                                                          int tiles_c, int ntiles) {
  __shared__ __attribute__((aligned(16))) float tab[OP::NTAB * TAB_N];
  __shared__ uint32_t cred[8][AM_TC / 2];
  load_table<OP>(tab, p.tab);
  const int tid = threadIdx.x;
  const int cx = tid & 31;
  const int ry = tid >> 5;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int tile_c = t % tiles_c;
    const int tile_r = t / tiles_c;
    const int r0 = tile_r * AM_TR;
    const int c = tile_c * AM_TC + cx * 8;
    const bool col_ok = c < cols;
    const int cl = col_ok ? c : 0;

    uint32_t cm[OP::NOUT][4];
#pragma unroll
    for (int j = 0; j < OP::NOUT; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) cm[j][k] = 0;

#pragma unroll
    for (int bt = 0; bt < AM_TR / 8; bt += 4) {
      U4 v[4][OP::NIN];
      U4 o[4][OP::NOUT];
      bool valid[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + ry + 8 * (bt + i);
        valid[i] = col_ok && r < rows;
        const int rc = min(r, rows - 1);
#pragma unroll
        for (int k = 0; k < OP::NIN; ++k) v[i][k] = load16(p.in[k] + (size_t)rc * cols + cl);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        apply_group<OP, 1>(&v[i], &o[i], &valid[i], tab);
        const int r = r0 + ry + 8 * (bt + i);
        const bool ok = valid[i];
#pragma unroll
        for (int j = 0; j < OP::NOUT; ++j) {
          if (ok)
            *reinterpret_cast<uint4 *>(p.out[j] + (size_t)r * cols + c) =
                make_uint4(o[i][j].x, o[i][j].y, o[i][j].z, o[i][j].w);
          const uint32_t keep = ok ? 0x7FFF7FFFu : 0u;
          const uint32_t x0 = o[i][j].x & keep, x1 = o[i][j].y & keep;
          const uint32_t x2 = o[i][j].z & keep, x3 = o[i][j].w & keep;
          cm[j][0] = max_u16x2(cm[j][0], x0);
          cm[j][1] = max_u16x2(cm[j][1], x1);
          cm[j][2] = max_u16x2(cm[j][2], x2);
          cm[j][3] = max_u16x2(cm[j][3], x3);
          // the 32 lanes of a half-wave share row r
          const uint32_t rm =
              half_wave_max(hmax16(max_u16x2(max_u16x2(x0, x1), max_u16x2(x2, x3))));
          if (cx == 0 && r < rows) p.rowpart[j][(size_t)tile_c * rows + r] = (uint16_t)rm;
        }
      }
    }

    // column maxima: reduce over the 8 row phases through LDS, one output
    // at a time; the barriers also keep the next tile's writes of cred
    // behind this tile's reads
#pragma unroll
    for (int j = 0; j < OP::NOUT; ++j) {
#pragma unroll
      for (int k = 0; k < 4; ++k) cred[ry][cx * 4 + k] = cm[j][k];
      __syncthreads();
      if (tid < AM_TC / 2) {
        uint32_t m = cred[0][tid];
#pragma unroll
        for (int ph = 1; ph < 8; ++ph) m = max_u16x2(m, cred[ph][tid]);
        const int cc = tile_c * AM_TC + tid * 2;
        if (cc < cols) {
          uint16_t *dst = p.colpart[j] + (size_t)tile_r * cols + cc;
          dst[0] = (uint16_t)(m & 0xFFFFu);
          dst[1] = (uint16_t)(m >> 16);
        }
      }
      __syncthreads();
    }
  }
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// bytes of one output's share of the workspace (256-byte aligned)
size_t share_bytes(int64_t rows, int64_t hidden, int scaling) {
  size_t b = quantize_workspace_bytes(rows, hidden, scaling & FP8L_ROWWISE);
  const size_t tw = (size_t)TW_MAX_BLOCKS * sizeof(uint32_t);
  if (b < tw) b = tw;
  return (b + 255) & ~(size_t)255;
}

constexpr size_t TAB_BYTES = 2 * TAB_N * sizeof(float);

// workgroups of the producers: a few per compute unit (each loads the
// table once), as many as their LDS lets run together
template <class OP>
int64_t producer_blocks() {
  return OP::NTAB == 1 ? 1024 : 512;
}

// The producer pass: writes the NOUT outputs and their partial maxima into
// the output's workspace share; returns the tensorwise partial count.
template <class OP>
hipError_t produce(SwArgs p, int64_t rows, int64_t hidden, bool rowwise, void *workspace,
                   size_t share, int *nparts, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  *nparts = 0;
  if (rows * hidden == 0) return hipSuccess;
  float *tab = reinterpret_cast<float *>(ws + 2 * share);
  hipLaunchKernelGGL(k_silu_table, dim3(TAB_N / 256), dim3(256), 0, stream, tab);
  p.tab = tab;
  const int64_t cap = producer_blocks<OP>();
  if (!rowwise) {
    const int64_t n16 = rows * hidden / 8;
    const int64_t nb = cdiv(n16, SW_CHUNK) < cap ? cdiv(n16, SW_CHUNK) : cap;
    for (int j = 0; j < OP::NOUT; ++j) p.part[j] = reinterpret_cast<uint32_t *>(ws + j * share);
    hipLaunchKernelGGL(k_swiglu_tw<OP>, dim3((unsigned)nb), dim3(AM_THREADS), 0, stream, p,
                       n16);
    *nparts = (int)nb;
  } else {
    for (int j = 0; j < OP::NOUT; ++j)
      quantize_rowwise_partials(ws + j * share, rows, hidden, &p.rowpart[j], &p.colpart[j]);
    const int64_t tiles_c = cdiv(hidden, AM_TC), tiles_r = cdiv(rows, AM_TR);
    const int64_t ntiles = tiles_r * tiles_c;
    hipLaunchKernelGGL(k_swiglu_rw<OP>, dim3((unsigned)(ntiles < cap ? ntiles : cap)),
                       dim3(AM_THREADS), 0, stream, p, (int)rows, (int)hidden, (int)tiles_c,
                       (int)ntiles);
  }
  return hipGetLastError();
}

}  // namespace

size_t swiglu_workspace_bytes(int64_t rows, int64_t hidden, int scaling) {
  return 2 * share_bytes(rows, hidden, scaling) + TAB_BYTES;
}

hipError_t swiglu_fwd_launch(const void *a, const void *b, int64_t rows, int64_t hidden,
                             int scaling, void *h, void *hq, void *hqt, float *scale,
                             float *scale_t, float *amax_out, void *workspace,
                             hipStream_t stream) {
  SwArgs p = {};
  p.in[0] = static_cast<const uint16_t *>(a);
  p.in[1] = static_cast<const uint16_t *>(b);
  p.out[0] = static_cast<uint16_t *>(h);
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  int nparts = 0;
  hipError_t e = produce<FwdOp>(p, rows, hidden, rw, workspace,
                                share_bytes(rows, hidden, scaling), &nparts, stream);
  if (e != hipSuccess) return e;
  return quantize_finish_launch(h, rows, hidden, scaling, nparts, hq, hqt, scale, scale_t,
                                amax_out, workspace, stream);
}

hipError_t swiglu_bwd_launch(const void *dh, const void *a, const void *b, int64_t rows,
                             int64_t hidden, int scaling, void *da, void *db,
                             const Fp8Out &qa, const Fp8Out &qb, void *workspace,
                             hipStream_t stream) {
  SwArgs p = {};
  p.in[0] = static_cast<const uint16_t *>(dh);
  p.in[1] = static_cast<const uint16_t *>(a);
  p.in[2] = static_cast<const uint16_t *>(b);
  p.out[0] = static_cast<uint16_t *>(da);
  p.out[1] = static_cast<uint16_t *>(db);
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  const size_t share = share_bytes(rows, hidden, scaling);
  int nparts = 0;
  hipError_t e = produce<BwdOp>(p, rows, hidden, rw, workspace, share, &nparts, stream);
  if (e != hipSuccess) return e;
  e = quantize_finish_launch(da, rows, hidden, scaling, nparts, qa.q, qa.qt, qa.scale,
                             qa.scale_t, qa.amax, workspace, stream);
  if (e != hipSuccess) return e;
  return quantize_finish_launch(db, rows, hidden, scaling, nparts, qb.q, qb.qt, qb.scale,
                                qb.scale_t, qb.amax, static_cast<uint8_t *>(workspace) + share,
                                stream);
}

}  // namespace fp8l
