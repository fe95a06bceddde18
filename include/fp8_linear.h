/*
 * fp8_linear.h -- C ABI of the MI355X (gfx950) Float8 training linear layer.
 *
 * The operation is Float8 training of a linear layer inside a bf16
 * mixed-precision step: the layer's large GEMMs run with 8-bit operands
 * ("Torchtitan: A PyTorch Library for Parallelism Techniques explained",
 * section 3, "Float8 Training"; the forum index "torchtitan", topic
 * "Enabling Float8 All-Gather in FSDP2": fp8 is used because it speeds up
 * large GEMMs).  The 8-bit format is E4M3 from the FP8 formats paper named on
 * the "torchtitan" tutorial page, Part XI, item 9; inputs and outputs are
 * bf16 as in the tutorial page's mixed-precision policy (Part IV, Stage 5).
 *
 * One linear with X [M,K] (tokens x in-features), W [N,K] (out x in) and the
 * output gradient dY [M,N] runs as:
 *   quantize(X), quantize(W), quantize(dY)          -> fp8 copies + scales
 *   fwd:  out    [M,N] = X  . W^T                   (Xq,   Wq)
 *   bwd:  grad_X [M,K] = dY . W                     (dYq,  WTq)
 *         grad_W [N,K] = dY^T . X                   (dYTq, XTq)
 * Every GEMM reads two operands stored contiguous along the contraction
 * index; quantize writes the transposed copy that makes this true.
 *
 * Conventions shared by every entry point
 *  - All matrices are row-major and dense (leading dimension = #columns).
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA memory),
 *    16-byte aligned.  The caller owns every buffer; the library allocates
 *    nothing, never synchronizes and keeps no state between calls (apart
 *    from fp8_linear_quantize_noalloc's per-GPU scratch array).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; results are ready when the stream reaches them.
 *    Calls on different streams may run concurrently if their buffers do not
 *    overlap.
 *  - Dimensions must be >= 0 and multiples of 16 (FP8L_ESHAPE otherwise);
 *    every fp8 GEMM operand and every bf16 GEMM output must be smaller than
 *    2^31 bytes.
 *    A zero dimension is an empty matrix: the call is valid and writes only
 *    what its definition gives (scales of the empty set, zero outputs).
 *  - Argument errors are detected on the host before anything is enqueued
 *    and returned as a status code; nothing is written in that case.  A
 *    failed launch returns FP8L_EHIP.  Non-finite input values are not
 *    errors: they propagate into amax (NaN if any NaN, else inf if any inf)
 *    so the caller can test it; the fp8 bytes are then unspecified.
 */
#ifndef FP8_LINEAR_H
#define FP8_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP8L_API __attribute__((visibility("default")))
#else
#define FP8L_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (return value of every int-returning entry point). */
#define FP8L_OK          0
#define FP8L_EINVAL      1   /* null required pointer or unknown enum value */
#define FP8L_ESHAPE      2   /* dimension < 0 or not a multiple of 16       */
#define FP8L_EALIGN      3   /* a tensor pointer is not 16-byte aligned     */
#define FP8L_EWORKSPACE  4   /* workspace smaller than required             */
#define FP8L_EHIP        5   /* a HIP launch or runtime call failed         */

/* Scaling granularity. */
#define FP8L_TENSORWISE  0   /* one scale per tensor                          */
#define FP8L_ROWWISE     1   /* one scale per row of q, one per column of x
                                (i.e. per row of qt)                         */
/* Format flag, OR'ed into a `scaling` argument: E5M2 codes (the second FP8
 * encoding the pages name, "torchtitan" tutorial, Part XI, item 9) for the
 * gradient dY.  fp8_linear_quantize with it writes E5M2 q / qt whose scale
 * maps amax onto 57344; fp8_linear_bwd and fp8_linear_bwd_w_f32 with it
 * read dyq / dytq as E5M2 (the weight and activation operands stay E4M3).
 * fp8_linear_fwd and fp8_linear_quantize_scaled take E4M3 only. */
#define FP8L_E5M2        2

/* Largest finite E4M3 value; the scale maps a tensor's amax onto it. */
#define FP8L_E4M3_MAX    448.0f
/* Largest finite E5M2 value (the gradient format, FP8L_E5M2 below). */
#define FP8L_E5M2_MAX    57344.0f
/* Lower clamp of amax in the scale, keeping the scale finite. */
#define FP8L_AMAX_EPS    1e-12f

/*
 * Bytes of device workspace fp8_linear_quantize needs for an x of
 * [rows, cols] with the given scaling (partial maxima of the amax pass;
 * 0 for an empty tensorwise x).  Returns 0 for invalid arguments.
 */
FP8L_API size_t fp8_linear_workspace_bytes(int64_t rows, int64_t cols, int scaling);

/*
 * Quantize a bf16 matrix to E4M3 with dynamic scaling (amax of the current
 * tensor; the pages leave the recipe open, this is the reading taken).
 * With FP8L_E5M2 OR'ed into scaling, the codes are E5M2 and 448 below
 * reads 57344:
 *
 *   a        = max |x| over the tensor (tensorwise), or per row of x for
 *              q and per column of x for qt (rowwise)
 *   s        = fp32( 448 / max(a, 1e-12) )        one IEEE fp32 division
 *   q[r][c]  = e4m3_sat_rne( fp32(x[r][c] * s_row[r]) )
 *   qt[c][r] = e4m3_sat_rne( fp32(x[r][c] * s_col[c]) )
 *
 * where e4m3_sat_rne rounds to the nearest E4M3 value (ties to the even
 * code), clamps magnitudes >= 448 to 448 and keeps the sign (so -0 -> 0x80).
 * Tensorwise: s_row = s_col = s, so qt is exactly q transposed.
 *
 *   x        [rows, cols] bf16 (device, read only)
 *   q        [rows, cols] e4m3 bytes (device, written)
 *   qt       [cols, rows] e4m3 bytes (device, written)
 *   scale    tensorwise [1]; rowwise [rows]  fp32 multipliers s of q
 *   scale_t  tensorwise [1]; rowwise [cols]  fp32 multipliers s of qt
 *   amax_out NULL, or tensorwise [1]; rowwise [rows + cols] (rows first)
 *   workspace / workspace_bytes: >= fp8_linear_workspace_bytes(...) bytes of
 *            device scratch, owned by the caller, contents undefined on
 *            entry and exit; must not be shared by calls in flight together.
 * The stored scale is the multiplier (q = x * s); the GEMMs divide it out.
 */
FP8L_API int fp8_linear_quantize(const void *x, int64_t rows, int64_t cols, int scaling,
                        void *q, void *qt, float *scale, float *scale_t,
                        float *amax_out, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * fp8_linear_quantize without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same definition, arguments and results
 * as fp8_linear_quantize; the partial maxima go to a scratch array that the
 * library holds on each GPU it runs on (FP8L_NOALLOC_MAX_WORKSPACE bytes,
 * held until the process ends) instead of a caller's workspace.  The call
 * allocates nothing (no hipMalloc, no allocating library call).
 *
 *   Limit: fp8_linear_workspace_bytes(rows, cols, scaling) must not exceed
 *   FP8L_NOALLOC_MAX_WORKSPACE (16 MiB: any tensorwise x; rowwise x up to
 *   about 4e8 elements, e.g. [8192, 28672]); larger requests return
 *   FP8L_EWORKSPACE before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's one array.  Calls that may
 *   run at the same time on one GPU (different streams without ordering)
 *   race on it and must be serialised by the caller (one stream, or events);
 *   calls in stream order are safe.  Nothing in the array needs clearing:
 *   each call writes every partial maximum it reads before reading it.
 *   The first call on a device (with that device's stream) looks the
 *   array's address up once; FP8L_EHIP if that fails.
 */
#define FP8L_NOALLOC_MAX_WORKSPACE (16u << 20)
FP8L_API int fp8_linear_quantize_noalloc(const void *x, int64_t rows, int64_t cols, int scaling,
                                         void *q, void *qt, float *scale, float *scale_t,
                                         float *amax_out, void *stream);

/*
 * Tensorwise amax of one bf16 matrix alone: one GPU's share of the global
 * amax that Float8 all-gather of FSDP2 weights needs ("Enabling Float8
 * All-Gather in FSDP2" on the torchtitan forum index: each rank reduces its
 * shard, an all-reduce(max) of the 4-byte amax makes the tensorwise scale
 * global, then every rank casts its shard with that scale).
 *
 *   x         [rows, cols] bf16 (device, read only)
 *   amax_out  [1] fp32 (device, written): max |x|, NaN if x holds a NaN,
 *             0 for an empty x
 *   workspace / workspace_bytes: as for fp8_linear_quantize with
 *             FP8L_TENSORWISE and the same shape.
 */
FP8L_API int fp8_linear_amax(const void *x, int64_t rows, int64_t cols, float *amax_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Cast with a scale given by the caller (single read pass, 4 bytes of HBM
 * traffic per element): the second half of the Float8 all-gather flow above,
 * or any recipe whose scale is known before the cast.
 *
 *   q[r][c]  = e4m3_sat_rne( fp32(x[r][c] * scale[0]) ),  qt[c][r] = q[r][c]
 *
 *   x      [rows, cols] bf16 (device, read only)
 *   scale  [1] fp32 multiplier (device, read only), e.g.
 *          448 / max(global_amax, 1e-12) computed as one fp32 division
 *   q      [rows, cols] e4m3 bytes (device, written)
 *   qt     [cols, rows] e4m3 bytes (device, written)
 * An empty x writes nothing.  Same shape and alignment rules as
 * fp8_linear_quantize.
 */
FP8L_API int fp8_linear_quantize_scaled(const void *x, int64_t rows, int64_t cols,
                                        const float *scale, void *q, void *qt, void *stream);

/*
 * Forward GEMM of the linear (out = X . W^T) on the quantized operands: the
 * fp8 GEMM that is the point of the method (the forum index "torchtitan",
 * topic "Enabling Float8 All-Gather in FSDP2": fp8 speeds up large GEMMs),
 * with bf16 output as under the mixed-precision policy of the "torchtitan"
 * tutorial page, Part IV, Stage 5:
 *
 *   out[m][n] = bf16( fp32( fp32(acc * (1/sx)) * (1/sw) ) ),
 *   acc       = sum_k value(xq[m][k]) * value(wq[n][k])     (fp32 accumulate)
 *
 *   xq [M, K] e4m3 (q of X), sx: tensorwise [1], rowwise [M] (scale of X)
 *   wq [N, K] e4m3 (q of W), sw: tensorwise [1], rowwise [N] (scale of W)
 *   out [M, N] bf16 (device, written; rounded to nearest even)
 * The order of the fp32 additions is unspecified.
 */
FP8L_API int fp8_linear_fwd(const void *xq, const float *sx, const void *wq,
                   const float *sw, int64_t M, int64_t N, int64_t K,
                   int scaling, void *out, void *stream);

/*
 * Backward GEMMs of the linear on the quantized operands (the same fp8 GEMM,
 * forum topic "Enabling Float8 All-Gather in FSDP2"; bf16 gradients as under
 * the tutorial page's mixed-precision policy, Part IV, Stage 5):
 *
 *   grad_x[m][k] = bf16((sum_n dyq[m][n]  * wtq[k][n]) / sdy[m]  / swt[k])
 *   grad_w[n][k] = bf16((sum_m dytq[n][m] * xtq[k][m]) / sdyt[n] / sxt[k])
 *
 * (each "/ s" is a multiplication by the fp32 reciprocal, as in fwd)
 *
 *   dyq  [M, N] (q of dY),  sdy  tensorwise [1], rowwise [M]
 *   dytq [N, M] (qt of dY), sdyt tensorwise [1], rowwise [N]
 *   wtq  [K, N] (qt of W),  swt  tensorwise [1], rowwise [K]
 *   xtq  [K, M] (qt of X),  sxt  tensorwise [1], rowwise [K]
 *   grad_x [M, K] bf16, grad_w [N, K] bf16.
 * Either output may be NULL to skip that GEMM (its inputs may then be NULL).
 */
FP8L_API int fp8_linear_bwd(const void *dyq, const float *sdy, const void *dytq,
                   const float *sdyt, const void *wtq, const float *swt,
                   const void *xtq, const float *sxt, int64_t M, int64_t N,
                   int64_t K, int scaling, void *grad_x, void *grad_w,
                   void *stream);

/*
 * grad_W of the linear with an fp32 output: the value before bf16 rounding,
 * for a grad_W that is reduce-scattered in fp32 (the torchtitan tutorial,
 * Part IV, Stage 5: gradients are reduced in float32 under the default
 * mixed-precision policy).
 *
 *   grad_w[n][k] = fp32( fp32(acc / sdyt) / sxt ),
 *   acc = sum_m value(dytq[n][m]) * value(xtq[k][m])     (fp32 accumulate)
 *
 * with the reciprocals 1/sdyt, 1/sxt taken in fp32 and multiplied as in
 * fp8_linear_bwd (so bf16(grad_w) is fp8_linear_bwd's grad_w).  Operands,
 * scales and scaling as for fp8_linear_bwd's grad_w; grad_w [N, K] fp32
 * (device, written), 16-byte aligned, N * K * 4 < 2^31 bytes.
 */
FP8L_API int fp8_linear_bwd_w_f32(const void *dytq, const float *sdyt, const void *xtq,
                                  const float *sxt, int64_t M, int64_t N, int64_t K,
                                  int scaling, float *grad_w, void *stream);

/*
 * Several independent GEMMs of fp8_linear_fwd's form in one launch:
 *
 *   c[i][j] = bf16( fp32( fp32(acc * (1/sa)) * (1/sb) ) ),
 *   acc     = sum_t value(a[i][t]) * value(b[j][t])        (fp32 accumulate)
 *
 * for each problem, a [m, k] (E4M3, or E5M2 with FP8L_E5M2 in scaling),
 * b [n, k] E4M3, sa / sb tensorwise [1] or rowwise [m] / [n], c [m, n]
 * bf16 written.  One launch lets a problem whose output tiles leave the
 * chip's last round partly idle (896 tiles of 256 x 256 on 256 compute
 * units) share that round with another: e.g. the grad_W of w1 and w3 of
 * the SwiGLU feed-forward, or any of fp8_linear_bwd's GEMMs.  Each
 * problem's result is the one its own fp8_linear_fwd-style call gives.
 *
 *   problems  host array of count descriptors (read during the call only)
 *   count     1..FP8L_MAX_GROUP
 *   scaling   FP8L_TENSORWISE or FP8L_ROWWISE, optionally | FP8L_E5M2,
 *             for every problem
 * Dimension, alignment and size rules as for fp8_linear_fwd, per problem;
 * the outputs must not overlap one another (FP8L_EINVAL).
 */
#define FP8L_MAX_GROUP 4
typedef struct fp8l_gemm_problem {
    const void *a;
    const float *sa;
    const void *b;
    const float *sb;
    void *c;
    int64_t m, n, k;
} fp8l_gemm_problem;

FP8L_API int fp8_linear_gemm_grouped(const fp8l_gemm_problem *problems, int count, int scaling,
                                     void *stream);

/*
 * grad_X added into an existing bf16 grad_x: for an x that feeds two linears
 * (w1 and w3 of the SwiGLU feed-forward below), whose gradient is the sum of
 * the two contributions as bf16 tensors add (autograd accumulates the
 * gradient of a tensor used twice):
 *
 *   grad_x[m][k] = bf16( fl32(grad_x[m][k]) + fl32(g[m][k]) ),
 *   g[m][k]      = fp8_linear_bwd's grad_x for these operands (bf16)
 *
 * dyq, sdy, wtq, swt, M, N, K, scaling as for fp8_linear_bwd's grad_x;
 * grad_x [M, K] bf16 (device, read and written).
 */
FP8L_API int fp8_linear_bwd_x_acc(const void *dyq, const float *sdy, const void *wtq,
                                  const float *swt, int64_t M, int64_t N, int64_t K,
                                  int scaling, void *grad_x, void *stream);

/*
 * SwiGLU feed-forward of the Llama 3.1 model the pages train (the
 * "torchtitan" tutorial page, Part II, "Using it", llama3_8b; Part V splits
 * its hidden dimension across tensor-parallel ranks):
 *
 *   a = x W1^T,  b = x W3^T   [rows, hidden]   (two Float8 linears; x is
 *                                               quantized once for both)
 *   h = silu(a) * b           [rows, hidden]   (fp8_swiglu_fwd)
 *   out = h W2^T                               (Float8 linear on h)
 *
 * The SwiGLU elementwise is the producer of w2's input, and of the output
 * gradients of w1 and w3 in the backward; these entry points write the
 * bf16 result and take its amax partial maxima in the same pass, so its
 * quantize needs only the cast pass afterwards (one read of the tensor
 * fewer than fp8_linear_quantize on the bf16 result).
 *
 * Elementwise definitions (silu(a) = a / (1 + e^-a); sigma(a) = 1/(1+e^-a);
 * silu'(a) = sigma(a) (1 + a (1 - sigma(a))); silu and silu' are the fp32
 * roundings of their exact values -- computed in fp64 -- and each other
 * operation is one fp32 operation):
 *   h  = bf16( fl32( silu(a) * b ) )
 *   da = bf16( fl32( fl32(dh * b) * silu'(a) ) )
 *   db = bf16( fl32( dh * silu(a) ) )
 * followed by fp8_linear_quantize's definition applied to h (E4M3), or to
 * da and db separately (E4M3, or E5M2 with that flag), each with its own
 * scales.
 *
 * Every matrix is a separate dense [rows, hidden] array; rows and hidden
 * are multiples of 16.  The workspace (>= fp8_swiglu_workspace_bytes) holds
 * the partial maxima; contents undefined on entry and exit, not shared by
 * calls in flight together.  An empty matrix writes only the scales of the
 * empty set.
 */
FP8L_API size_t fp8_swiglu_workspace_bytes(int64_t rows, int64_t hidden, int scaling);

/*
 *   a, b      [rows, hidden] bf16 (device, read only)
 *   h         [rows, hidden] bf16 (device, written)
 *   hq, hqt, scale, scale_t, amax_out: as fp8_linear_quantize's q, qt, scale,
 *             scale_t, amax_out for x = h (scaling: FP8L_TENSORWISE or
 *             FP8L_ROWWISE; codes E4M3)
 */
FP8L_API int fp8_swiglu_fwd(const void *a, const void *b, int64_t rows, int64_t hidden,
                            int scaling, void *h, void *hq, void *hqt, float *scale,
                            float *scale_t, float *amax_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 *   dh, a, b  [rows, hidden] bf16 (device, read only): dh is the gradient of h
 *   da, db    [rows, hidden] bf16 (device, written)
 *   daq, daqt, da_scale, da_scale_t, da_amax: the quantize of da, as
 *             fp8_linear_quantize's outputs for x = da; likewise db*
 *   scaling   FP8L_TENSORWISE or FP8L_ROWWISE, optionally | FP8L_E5M2
 */
FP8L_API int fp8_swiglu_bwd(const void *dh, const void *a, const void *b, int64_t rows,
                            int64_t hidden, int scaling, void *da, void *db, void *daq,
                            void *daqt, float *da_scale, float *da_scale_t, float *da_amax,
                            void *dbq, void *dbqt, float *db_scale, float *db_scale_t,
                            float *db_amax, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * The element conversion the quantize kernels use, exposed for testing it on
 * every fp32 input: out[i] = e4m3_sat_rne(in[i]) (definition above; a NaN
 * input gives a NaN code).  in: n fp32, out: n bytes, both device pointers.
 * n >= 0, no multiple-of-16 requirement.
 */
FP8L_API int fp8_linear_encode_e4m3(const float *in, uint8_t *out, int64_t n,
                           void *stream);

/* The E5M2 counterpart (saturating at 57344, ties to even, NaN -> a NaN
 * code), for testing the gradient conversion the same way. */
FP8L_API int fp8_linear_encode_e5m2(const float *in, uint8_t *out, int64_t n,
                                    void *stream);

/* Human-readable text of a status code (static storage, never NULL). */
FP8L_API const char *fp8_linear_status_string(int status);

/* Library version and target, e.g. "fp8_linear 0.1 gfx950". */
FP8L_API const char *fp8_linear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8_LINEAR_H */
