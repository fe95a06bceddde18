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
// Layout: a, b, h, dh, da, db are separate dense [rows, hidden] bf16
// matrices.  Tensorwise kernels walk them as flat arrays of 16-byte chunks
// (8 values) in a grid-stride loop with at most TW_MAX_BLOCKS workgroups,
// one partial maximum per workgroup and output; rowwise kernels walk tiles
// of AM_TR x AM_TC and write row and column maxima per tile.
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

// ------------------------------------------------------------- the ops --
// An op maps NIN input chunks (8 bf16 each) to NOUT output chunks.

struct FwdOp {
  static constexpr int NIN = 2, NOUT = 1;   // in: a, b; out: h
  __device__ static void apply(const U4 *in, U4 *out) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = dword(in[0], k), b = dword(in[1], k);
      const uint32_t h0 = bf16_rne(silu32(bf16_to_f32(lo16(a))) * bf16_to_f32(lo16(b)));
      const uint32_t h1 = bf16_rne(silu32(bf16_to_f32(hi16(a))) * bf16_to_f32(hi16(b)));
      w[k] = h0 | (h1 << 16);
    }
    out[0] = pack(w);
  }
};

struct BwdOp {
  static constexpr int NIN = 3, NOUT = 2;   // in: dh, a, b; out: da, db
  __device__ static void one(uint32_t g16, uint32_t a16, uint32_t b16, uint32_t &da,
                             uint32_t &db) {
    float s, ds;
    silu_and_deriv32(bf16_to_f32(a16), s, ds);
    const float g = bf16_to_f32(g16);
    const float gb = g * bf16_to_f32(b16);
    da = bf16_rne(gb * ds);
    db = bf16_rne(g * s);
  }
  __device__ static void apply(const U4 *in, U4 *out) {
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t g = dword(in[0], k), a = dword(in[1], k), b = dword(in[2], k);
      uint32_t a0, b0, a1, b1;
      one(lo16(g), lo16(a), lo16(b), a0, b0);
      one(hi16(g), hi16(a), hi16(b), a1, b1);
      wa[k] = a0 | (a1 << 16);
      wb[k] = b0 | (b1 << 16);
    }
    out[0] = pack(wa);
    out[1] = pack(wb);
  }
};

struct SwArgs {
  const uint16_t *in[3];
  uint16_t *out[2];
  uint32_t *part[2];        // tensorwise block maxima, one array per output
  uint16_t *rowpart[2];     // rowwise tile maxima, per output
  uint16_t *colpart[2];
};

// ----------------------------------------------------------- tensorwise --
//
// Chunks of 256 threads x SW_UNROLL 16-byte vectors; every load is issued
// unconditionally (index clamped into the arrays), stores and maxima only
// for indices inside.
constexpr int SW_UNROLL = 4;
constexpr int SW_CHUNK = AM_THREADS * SW_UNROLL;

template <class OP>
__global__ __launch_bounds__(AM_THREADS) void k_swiglu_tw(SwArgs p, int64_t n16) {
  const int tid = threadIdx.x;
  uint32_t acc[OP::NOUT];
#pragma unroll
  for (int j = 0; j < OP::NOUT; ++j) acc[j] = 0;
  const int64_t nchunks = (n16 + SW_CHUNK - 1) / SW_CHUNK;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const int64_t base = ch * SW_CHUNK + tid;
    U4 v[SW_UNROLL][OP::NIN];
#pragma unroll
    for (int u = 0; u < SW_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * AM_THREADS;
      const int64_t ic = i < n16 ? i : n16 - 1;
#pragma unroll
      for (int k = 0; k < OP::NIN; ++k) v[u][k] = load16(p.in[k] + ic * 8);
    }
#pragma unroll
    for (int u = 0; u < SW_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * AM_THREADS;
      if (i < n16) {
        U4 o[OP::NOUT];
        OP::apply(v[u], o);
#pragma unroll
        for (int j = 0; j < OP::NOUT; ++j) {
          *reinterpret_cast<uint4 *>(p.out[j] + i * 8) = make_uint4(o[j].x, o[j].y, o[j].z, o[j].w);
          acc[j] = max_u16x2(acc[j], chunk_absmax(o[j]));
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
// Tile of AM_TR rows x AM_TC columns; thread (cx, ry): cx = tid % 32 picks
// an 8-column chunk, ry = tid / 32 a row phase; the thread walks rows
// ry + 8 i, in two batches of four rows whose loads are in flight together
// (row clamped into the matrix, column chunk to 0, results masked).
template <class OP>
__global__ __launch_bounds__(AM_THREADS) void k_swiglu_rw(SwArgs p, int rows, int cols,
                                                          int tiles_c) {
  const int tid = threadIdx.x;
  const int tile_c = blockIdx.x % tiles_c;
  const int tile_r = blockIdx.x / tiles_c;
  const int cx = tid & 31;
  const int ry = tid >> 5;
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(r0 + ry + 8 * (bt + i), rows - 1);
#pragma unroll
      for (int k = 0; k < OP::NIN; ++k) v[i][k] = load16(p.in[k] + (size_t)r * cols + cl);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + ry + 8 * (bt + i);
      const bool ok = col_ok && r < rows;
      U4 o[OP::NOUT];
      OP::apply(v[i], o);
#pragma unroll
      for (int j = 0; j < OP::NOUT; ++j) {
        if (ok)
          *reinterpret_cast<uint4 *>(p.out[j] + (size_t)r * cols + c) =
              make_uint4(o[j].x, o[j].y, o[j].z, o[j].w);
        const uint32_t keep = ok ? 0x7FFF7FFFu : 0u;
        const uint32_t x0 = o[j].x & keep, x1 = o[j].y & keep;
        const uint32_t x2 = o[j].z & keep, x3 = o[j].w & keep;
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

  // column maxima: reduce over the 8 row phases through LDS, one output at
  // a time
  __shared__ uint32_t cred[8][AM_TC / 2];
#pragma unroll
  for (int j = 0; j < OP::NOUT; ++j) {
    if (j > 0) __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) cred[ry][cx * 4 + k] = cm[j][k];
    __syncthreads();
    if (tid < AM_TC / 2) {
      uint32_t t = cred[0][tid];
#pragma unroll
      for (int ph = 1; ph < 8; ++ph) t = max_u16x2(t, cred[ph][tid]);
      const int cc = tile_c * AM_TC + tid * 2;
      if (cc < cols) {
        uint16_t *dst = p.colpart[j] + (size_t)tile_r * cols + cc;
        dst[0] = (uint16_t)(t & 0xFFFFu);
        dst[1] = (uint16_t)(t >> 16);
      }
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

// The producer pass: writes the NOUT outputs and their partial maxima into
// the output's workspace share; returns the tensorwise partial count.
template <class OP>
hipError_t produce(SwArgs p, int64_t rows, int64_t hidden, bool rowwise, void *workspace,
                   size_t share, int *nparts, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  *nparts = 0;
  if (rows * hidden == 0) return hipSuccess;
  if (!rowwise) {
    const int64_t n16 = rows * hidden / 8;
    const int64_t nb = cdiv(n16, SW_CHUNK) < TW_MAX_BLOCKS ? cdiv(n16, SW_CHUNK) : TW_MAX_BLOCKS;
    for (int j = 0; j < OP::NOUT; ++j) p.part[j] = reinterpret_cast<uint32_t *>(ws + j * share);
    hipLaunchKernelGGL(k_swiglu_tw<OP>, dim3((unsigned)nb), dim3(AM_THREADS), 0, stream, p,
                       n16);
    *nparts = (int)nb;
  } else {
    for (int j = 0; j < OP::NOUT; ++j)
      quantize_rowwise_partials(ws + j * share, rows, hidden, &p.rowpart[j], &p.colpart[j]);
    const int64_t tiles_c = cdiv(hidden, AM_TC), tiles_r = cdiv(rows, AM_TR);
    hipLaunchKernelGGL(k_swiglu_rw<OP>, dim3((unsigned)(tiles_r * tiles_c)), dim3(AM_THREADS),
                       0, stream, p, (int)rows, (int)hidden, (int)tiles_c);
  }
  return hipGetLastError();
}

}  // namespace

size_t swiglu_workspace_bytes(int64_t rows, int64_t hidden, int scaling) {
  return 2 * share_bytes(rows, hidden, scaling);
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
