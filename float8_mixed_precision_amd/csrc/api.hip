// C ABI of the Float8 linear library (declared in include/fp8_linear.h):
// argument validation on the host, then asynchronous launches on the
// caller's stream.  Nothing here allocates or synchronizes; the only state
// is the per-device address of the no-allocation entry point's scratch
// array, looked up once per device.
#include "fp8l_internal.h"

#include <atomic>
#include <mutex>

namespace {

bool bad_dim(int64_t d) { return d < 0 || (d % 16) != 0 || d > (int64_t)1 << 30; }

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// FP8L_TENSORWISE or FP8L_ROWWISE, optionally with the FP8L_E5M2 flag
bool bad_scaling(int scaling) { return (scaling & ~(FP8L_ROWWISE | FP8L_E5M2)) != 0; }

// Dimensions are capped at 2^30 so that every 32-bit index in the kernels
// stays in range (addresses are formed in 64 bits), and a matrix at 2^40
// elements so that grid sizes fit in 32 bits.
constexpr int64_t kMaxElems = (int64_t)1 << 40;
// GEMM operands and outputs are addressed through buffer resources with
// 32-bit byte offsets: each must stay below 2^31 bytes.
constexpr int64_t kMaxGemmBytes = ((int64_t)1 << 31) - 1;

bool bad_gemm_sizes(int64_t m, int64_t n, int64_t k) {
  return m * k > kMaxGemmBytes || n * k > kMaxGemmBytes || 2 * m * n > kMaxGemmBytes;
}

// C[m,n] = A[m,k] . B[n,k]^T: a pointer may be NULL only where its matrix
// is empty; the scales are read whenever an output element is written.
int check_gemm_operands(const void *a, const float *sa, const void *b,
                        const float *sb, const void *c, int64_t m, int64_t n,
                        int64_t k) {
  if ((!a && m * k > 0) || (!b && n * k > 0) || (!c && m * n > 0)) return FP8L_EINVAL;
  if ((!sa || !sb) && m * n > 0) return FP8L_EINVAL;
  if (misaligned(a) || misaligned(b) || misaligned(c)) return FP8L_EALIGN;
  if ((reinterpret_cast<uintptr_t>(sa) & 3u) || (reinterpret_cast<uintptr_t>(sb) & 3u))
    return FP8L_EALIGN;
  return FP8L_OK;
}

// ---- scratch of fp8_linear_quantize_noalloc -------------------------------
// One array per GPU, held until the process ends; every noalloc call on a
// GPU uses that GPU's copy.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): it passes the
// device address that hipGetSymbolAddress returns for the device, taken
// once per device with that device current and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[FP8L_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch address on the device of `stream` (the current device for the
// default stream); FP8L_EHIP if it cannot be found.
int scratch_address(hipStream_t stream, void **out) {
  int dev = -1;
  if (stream) {
    hipDevice_t d;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return FP8L_EHIP;
    dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FP8L_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FP8L_EHIP;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return FP8L_EHIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return FP8L_EHIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return FP8L_EHIP;
      if (e != hipSuccess || !p) return FP8L_EHIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8L_OK;
}

// Argument checks shared by the quantize entry points (everything but the
// workspace); FP8L_OK if the call is valid.
int check_quantize_args(const void *x, int64_t rows, int64_t cols, int scaling, const void *q,
                        const void *qt, const float *scale, const float *scale_t,
                        const float *amax_out) {
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  if (bad_dim(rows) || bad_dim(cols) || rows * cols > kMaxElems) return FP8L_ESHAPE;
  const bool empty = rows == 0 || cols == 0;
  // scale vectors may be NULL only where they have no entries (rowwise, 0 rows
  // or 0 columns); tensorwise scales always have one entry
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  if ((!scale && (!rw || rows > 0)) || (!scale_t && (!rw || cols > 0))) return FP8L_EINVAL;
  if (!empty && (!x || !q || !qt)) return FP8L_EINVAL;
  if (misaligned(x) || misaligned(q) || misaligned(qt)) return FP8L_EALIGN;
  if ((reinterpret_cast<uintptr_t>(scale) & 3u) || (reinterpret_cast<uintptr_t>(scale_t) & 3u) ||
      (reinterpret_cast<uintptr_t>(amax_out) & 3u))
    return FP8L_EALIGN;
  return FP8L_OK;
}

}  // namespace

extern "C" {

size_t fp8_linear_workspace_bytes(int64_t rows, int64_t cols, int scaling) {
  if (bad_dim(rows) || bad_dim(cols)) return 0;
  if (bad_scaling(scaling)) return 0;
  return fp8l::quantize_workspace_bytes(rows, cols, scaling);
}

int fp8_linear_quantize(const void *x, int64_t rows, int64_t cols, int scaling,
                        void *q, void *qt, float *scale, float *scale_t,
                        float *amax_out, void *workspace, size_t workspace_bytes,
                        void *stream) {
  const int s = check_quantize_args(x, rows, cols, scaling, q, qt, scale, scale_t, amax_out);
  if (s != FP8L_OK) return s;
  const size_t need = fp8l::quantize_workspace_bytes(rows, cols, scaling);
  if (need > 0 && !workspace) return FP8L_EINVAL;
  if (workspace_bytes < need) return FP8L_EWORKSPACE;
  if (misaligned(workspace)) return FP8L_EALIGN;
  hipError_t e = fp8l::quantize_launch(x, rows, cols, scaling, q, qt, scale, scale_t,
                                       amax_out, workspace,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_quantize_noalloc(const void *x, int64_t rows, int64_t cols, int scaling,
                                void *q, void *qt, float *scale, float *scale_t,
                                float *amax_out, void *stream) {
  const int s = check_quantize_args(x, rows, cols, scaling, q, qt, scale, scale_t, amax_out);
  if (s != FP8L_OK) return s;
  // checked before any HIP call: an oversized request fails on the host
  if (fp8l::quantize_workspace_bytes(rows, cols, scaling) > FP8L_NOALLOC_MAX_WORKSPACE)
    return FP8L_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  const int sa = scratch_address(st, &ws);
  if (sa != FP8L_OK) return sa;
  // every partial maximum the cast reads is written by this call's amax
  // pass first, so the array needs no clearing between calls
  hipError_t e = fp8l::quantize_launch(x, rows, cols, scaling, q, qt, scale, scale_t, amax_out,
                                       ws, st);
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_fwd(const void *xq, const float *sx, const void *wq,
                   const float *sw, int64_t M, int64_t N, int64_t K,
                   int scaling, void *out, void *stream) {
  if (scaling != FP8L_TENSORWISE && scaling != FP8L_ROWWISE) return FP8L_EINVAL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8L_ESHAPE;
  if (bad_gemm_sizes(M, N, K)) return FP8L_ESHAPE;
  int s = check_gemm_operands(xq, sx, wq, sw, out, M, N, K);
  if (s != FP8L_OK) return s;
  const int vec = scaling == FP8L_ROWWISE;
  hipError_t e = fp8l::gemm_launch(static_cast<const uint8_t *>(xq), sx,
                                   static_cast<const uint8_t *>(wq), sw, vec, 0, M, N, K,
                                   static_cast<uint16_t *>(out),
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_bwd(const void *dyq, const float *sdy, const void *dytq,
                   const float *sdyt, const void *wtq, const float *swt,
                   const void *xtq, const float *sxt, int64_t M, int64_t N,
                   int64_t K, int scaling, void *grad_x, void *grad_w,
                   void *stream) {
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8L_ESHAPE;
  // grad_x: [M,K] from [M,N] x [K,N]; grad_w: [N,K] from [N,M] x [K,M]
  if (bad_gemm_sizes(M, K, N) || bad_gemm_sizes(N, K, M)) return FP8L_ESHAPE;
  if (!grad_x && !grad_w) return FP8L_EINVAL;
  int s;
  if (grad_x && (s = check_gemm_operands(dyq, sdy, wtq, swt, grad_x, M, K, N)) != FP8L_OK)
    return s;
  if (grad_w && (s = check_gemm_operands(dytq, sdyt, xtq, sxt, grad_w, N, K, M)) != FP8L_OK)
    return s;
  const int vec = (scaling & FP8L_ROWWISE) != 0;
  const int fa = (scaling & FP8L_E5M2) != 0;     // dY operands in E5M2
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (grad_x)  // [M,K] = dYq[M,N] . WTq[K,N]^T
    e = fp8l::gemm_launch(static_cast<const uint8_t *>(dyq), sdy,
                          static_cast<const uint8_t *>(wtq), swt, vec, fa, M, K, N,
                          static_cast<uint16_t *>(grad_x), st);
  if (e == hipSuccess && grad_w)  // [N,K] = dYTq[N,M] . XTq[K,M]^T
    e = fp8l::gemm_launch(static_cast<const uint8_t *>(dytq), sdyt,
                          static_cast<const uint8_t *>(xtq), sxt, vec, fa, N, K, M,
                          static_cast<uint16_t *>(grad_w), st);
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_amax(const void *x, int64_t rows, int64_t cols, float *amax_out,
                    void *workspace, size_t workspace_bytes, void *stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols > kMaxElems) return FP8L_ESHAPE;
  if (!amax_out || (rows * cols > 0 && !x)) return FP8L_EINVAL;
  const size_t need = fp8l::quantize_workspace_bytes(rows, cols, FP8L_TENSORWISE);
  if (need > 0 && !workspace) return FP8L_EINVAL;
  if (workspace_bytes < need) return FP8L_EWORKSPACE;
  if (misaligned(x) || misaligned(workspace) || (reinterpret_cast<uintptr_t>(amax_out) & 3u))
    return FP8L_EALIGN;
  hipError_t e = fp8l::amax_launch(x, rows, cols, amax_out, workspace,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_quantize_scaled(const void *x, int64_t rows, int64_t cols, const float *scale,
                               void *q, void *qt, void *stream) {
  if (bad_dim(rows) || bad_dim(cols) || rows * cols > kMaxElems) return FP8L_ESHAPE;
  if (rows * cols == 0) return FP8L_OK;
  if (!x || !scale || !q || !qt) return FP8L_EINVAL;
  if (misaligned(x) || misaligned(q) || misaligned(qt) ||
      (reinterpret_cast<uintptr_t>(scale) & 3u))
    return FP8L_EALIGN;
  hipError_t e = fp8l::quantize_scaled_launch(x, rows, cols, scale, q, qt,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_bwd_w_f32(const void *dytq, const float *sdyt, const void *xtq,
                         const float *sxt, int64_t M, int64_t N, int64_t K, int scaling,
                         float *grad_w, void *stream) {
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8L_ESHAPE;
  // [N,K] fp32 = dYTq[N,M] . XTq[K,M]^T: 4-byte outputs under the same
  // 32-bit offset limit
  if (bad_gemm_sizes(N, K, M) || 4 * N * K > kMaxGemmBytes) return FP8L_ESHAPE;
  int s = check_gemm_operands(dytq, sdyt, xtq, sxt, grad_w, N, K, M);
  if (s != FP8L_OK) return s;
  hipError_t e = fp8l::gemm_f32_launch(static_cast<const uint8_t *>(dytq), sdyt,
                                       static_cast<const uint8_t *>(xtq), sxt,
                                       (scaling & FP8L_ROWWISE) != 0,
                                       (scaling & FP8L_E5M2) != 0, N, K, M, grad_w,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_gemm_grouped(const fp8l_gemm_problem *problems, int count, int scaling,
                            void *stream) {
  if (!problems || count < 1 || count > FP8L_MAX_GROUP) return FP8L_EINVAL;
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  fp8l::GemmDesc d[FP8L_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    const fp8l_gemm_problem &p = problems[i];
    if (bad_dim(p.m) || bad_dim(p.n) || bad_dim(p.k)) return FP8L_ESHAPE;
    if (bad_gemm_sizes(p.m, p.n, p.k)) return FP8L_ESHAPE;
    int s = check_gemm_operands(p.a, p.sa, p.b, p.sb, p.c, p.m, p.n, p.k);
    if (s != FP8L_OK) return s;
    d[i] = {static_cast<const uint8_t *>(p.a), p.sa, static_cast<const uint8_t *>(p.b), p.sb,
            p.c, p.m, p.n, p.k};
  }
  // outputs pairwise disjoint
  for (int i = 0; i < count; ++i)
    for (int j = i + 1; j < count; ++j) {
      const uintptr_t a0 = reinterpret_cast<uintptr_t>(problems[i].c);
      const uintptr_t a1 = a0 + (uintptr_t)(2 * problems[i].m * problems[i].n);
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(problems[j].c);
      const uintptr_t b1 = b0 + (uintptr_t)(2 * problems[j].m * problems[j].n);
      if (a0 < b1 && b0 < a1) return FP8L_EINVAL;
    }
  hipError_t e = fp8l::gemm_group_launch(d, count, (scaling & FP8L_ROWWISE) != 0,
                                         (scaling & FP8L_E5M2) != 0,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_bwd_x_acc(const void *dyq, const float *sdy, const void *wtq, const float *swt,
                         int64_t M, int64_t N, int64_t K, int scaling, void *grad_x,
                         void *stream) {
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  if (bad_dim(M) || bad_dim(N) || bad_dim(K)) return FP8L_ESHAPE;
  if (bad_gemm_sizes(M, K, N)) return FP8L_ESHAPE;
  int s = check_gemm_operands(dyq, sdy, wtq, swt, grad_x, M, K, N);
  if (s != FP8L_OK) return s;
  hipError_t e = fp8l::gemm_acc_launch(static_cast<const uint8_t *>(dyq), sdy,
                                       static_cast<const uint8_t *>(wtq), swt,
                                       (scaling & FP8L_ROWWISE) != 0,
                                       (scaling & FP8L_E5M2) != 0, M, K, N,
                                       static_cast<uint16_t *>(grad_x),
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

size_t fp8_swiglu_workspace_bytes(int64_t rows, int64_t hidden, int scaling) {
  if (bad_dim(rows) || bad_dim(hidden) || bad_scaling(scaling)) return 0;
  return fp8l::swiglu_workspace_bytes(rows, hidden, scaling);
}

int fp8_swiglu_fwd(const void *a, const void *b, int64_t rows, int64_t hidden, int scaling,
                   void *h, void *hq, void *hqt, float *scale, float *scale_t, float *amax_out,
                   void *workspace, size_t workspace_bytes, void *stream) {
  if (scaling != FP8L_TENSORWISE && scaling != FP8L_ROWWISE) return FP8L_EINVAL;
  if (bad_dim(rows) || bad_dim(hidden) || rows * hidden > kMaxElems) return FP8L_ESHAPE;
  const bool rw = scaling == FP8L_ROWWISE;
  if ((!scale && (!rw || rows > 0)) || (!scale_t && (!rw || hidden > 0))) return FP8L_EINVAL;
  if (rows * hidden > 0 && (!a || !b || !h || !hq || !hqt)) return FP8L_EINVAL;
  const size_t need = fp8l::swiglu_workspace_bytes(rows, hidden, scaling);
  if (!workspace) return FP8L_EINVAL;
  if (workspace_bytes < need) return FP8L_EWORKSPACE;
  if (misaligned(a) || misaligned(b) || misaligned(h) || misaligned(hq) || misaligned(hqt) ||
      misaligned(workspace))
    return FP8L_EALIGN;
  if ((reinterpret_cast<uintptr_t>(scale) & 3u) || (reinterpret_cast<uintptr_t>(scale_t) & 3u) ||
      (reinterpret_cast<uintptr_t>(amax_out) & 3u))
    return FP8L_EALIGN;
  hipError_t e = fp8l::swiglu_fwd_launch(a, b, rows, hidden, scaling, h, hq, hqt, scale,
                                         scale_t, amax_out, workspace,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_swiglu_bwd(const void *dh, const void *a, const void *b, int64_t rows, int64_t hidden,
                   int scaling, void *da, void *db, void *daq, void *daqt, float *da_scale,
                   float *da_scale_t, float *da_amax, void *dbq, void *dbqt, float *db_scale,
                   float *db_scale_t, float *db_amax, void *workspace, size_t workspace_bytes,
                   void *stream) {
  if (bad_scaling(scaling)) return FP8L_EINVAL;
  if (bad_dim(rows) || bad_dim(hidden) || rows * hidden > kMaxElems) return FP8L_ESHAPE;
  const bool rw = (scaling & FP8L_ROWWISE) != 0;
  if ((!da_scale || !db_scale) && (!rw || rows > 0)) return FP8L_EINVAL;
  if ((!da_scale_t || !db_scale_t) && (!rw || hidden > 0)) return FP8L_EINVAL;
  if (rows * hidden > 0 &&
      (!dh || !a || !b || !da || !db || !daq || !daqt || !dbq || !dbqt))
    return FP8L_EINVAL;
  const size_t need = fp8l::swiglu_workspace_bytes(rows, hidden, scaling);
  if (!workspace) return FP8L_EINVAL;
  if (workspace_bytes < need) return FP8L_EWORKSPACE;
  if (misaligned(dh) || misaligned(a) || misaligned(b) || misaligned(da) || misaligned(db) ||
      misaligned(daq) || misaligned(daqt) || misaligned(dbq) || misaligned(dbqt) ||
      misaligned(workspace))
    return FP8L_EALIGN;
  for (const float *f : {da_scale, da_scale_t, da_amax, db_scale, db_scale_t, db_amax})
    if (reinterpret_cast<uintptr_t>(f) & 3u) return FP8L_EALIGN;
  const fp8l::Fp8Out qa = {daq, daqt, da_scale, da_scale_t, da_amax};
  const fp8l::Fp8Out qb = {dbq, dbqt, db_scale, db_scale_t, db_amax};
  hipError_t e = fp8l::swiglu_bwd_launch(dh, a, b, rows, hidden, scaling, da, db, qa, qb,
                                         workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_encode_e4m3(const float *in, uint8_t *out, int64_t n, void *stream) {
  if (n < 0 || n > kMaxElems) return FP8L_ESHAPE;
  if (n == 0) return FP8L_OK;
  if (!in || !out) return FP8L_EINVAL;
  if (misaligned(in) || misaligned(out)) return FP8L_EALIGN;
  hipError_t e = fp8l::encode_launch(in, out, n, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

int fp8_linear_encode_e5m2(const float *in, uint8_t *out, int64_t n, void *stream) {
  if (n < 0 || n > kMaxElems) return FP8L_ESHAPE;
  if (n == 0) return FP8L_OK;
  if (!in || !out) return FP8L_EINVAL;
  if (misaligned(in) || misaligned(out)) return FP8L_EALIGN;
  hipError_t e = fp8l::encode_launch(in, out, n, 1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8L_OK : FP8L_EHIP;
}

const char *fp8_linear_status_string(int status) {
  switch (status) {
    case FP8L_OK: return "ok";
    case FP8L_EINVAL: return "invalid argument (null pointer or unknown enum)";
    case FP8L_ESHAPE: return "invalid shape (dimension < 0 or not a multiple of 16)";
    case FP8L_EALIGN: return "misaligned pointer (tensors need 16-byte alignment)";
    case FP8L_EWORKSPACE: return "workspace too small";
    case FP8L_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

const char *fp8_linear_version(void) { return "fp8_linear 0.1 gfx950"; }

}  // extern "C"
