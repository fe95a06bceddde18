/*
 * CPU oracle for the Float8 training linear layer: TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library under
 * float8_mixed_precision_amd/csrc) shares no code, header, table or constant
 * generator with this file, and neither side includes or links the other.
 *
 * What it computes, and where it comes from:
 *   - The method is Float8 training of the linear layers of a bf16
 *     mixed-precision transformer step ("Torchtitan: A PyTorch Library for
 *     Parallelism Techniques explained", section 3, "Float8 Training";
 *     "TorchTitan: One-stop PyTorch native solution ...", Approach).
 *   - The 8-bit format is E4M3 from the FP8 formats paper named on the
 *     "torchtitan" tutorial page, Part XI (Papers and further reading),
 *     item 9.  The value of a code is the closed form of the OCP E4M3 ("fn")
 *     encoding: no infinities, one NaN mantissa pattern, largest finite 448.
 *   - Inputs are bf16 (the tutorial page, Part IV, Stage 5: parameters travel
 *     in bfloat16 under the default mixed-precision policy).
 *   - The pages leave the scaling recipe open.  The reading taken here:
 *     dynamic scaling from the current tensor's absolute maximum (per tensor,
 *     or per row / per column of the non-contracted index), scale
 *     s = 448 / max(amax, 1e-12) as a correctly rounded fp32 quotient,
 *     y = fl32(x * s), then a saturating round-to-nearest-even encode.
 *   - The GEMMs accumulate products of decoded codes in fp32, in ascending
 *     order of the contraction index, and are dequantised by fp32
 *     reciprocals of the two scales and rounded to bf16 (ties to even).
 *   - The feed-forward block the linears sit in is the Llama 3.1 MLP that
 *     the tutorial page trains (Part II, "Using it", llama3_8b; Part V
 *     splits its hidden dimension): SwiGLU, h = silu(x W1^T) * (x W3^T),
 *     out = h W2^T.  Its elementwise part and the bf16 sum of the two
 *     gradient contributions of x are at the end of this file.
 *
 * Nothing here is blocked, fused or reordered beyond these definitions.  The
 * only concession to speed is the OpenMP pragma on the outermost loops, which
 * splits independent output elements over threads and changes no result.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off
 *        (no -ffast-math: the divisions and products must be IEEE fp32).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_E4M3_MAX 448.0
#define ORC_E5M2_MAX 57344.0
#define ORC_EPS 1e-12f

/* ---------------------------------------------------------------- e4m3 -- */

/* Value of an E4M3 code from its closed form (OCP "fn" variant):
 *   S = bit 7, E = bits 6..3, F = bits 2..0
 *   E == 15 and F == 7      -> NaN (no infinities in this format)
 *   E == 0                  -> (-1)^S * F * 2^-9          (subnormals, +-0)
 *   otherwise               -> (-1)^S * (8 + F) * 2^(E-10)                  */
double orc_e4m3_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, f = code & 7;
    double mag;
    if (e == 15 && f == 7) return NAN;
    if (e == 0) mag = ldexp((double)f, -9);
    else        mag = ldexp((double)(8 + f), e - 10);
    return s ? -mag : mag;
}

/* Value of an E5M2 code from its closed form (OCP E5M2, the second
 * encoding of the same FP8 formats paper, IEEE-like):
 *   S = bit 7, E = bits 6..2, F = bits 1..0
 *   E == 31: F == 0 -> (-1)^S * inf, otherwise NaN
 *   E == 0          -> (-1)^S * F * 2^-16          (subnormals, +-0)
 *   otherwise       -> (-1)^S * (4 + F) * 2^(E-17)                         */
double orc_e5m2_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 2) & 31, f = code & 3;
    double mag;
    if (e == 31) mag = f == 0 ? INFINITY : NAN;
    else if (e == 0) mag = ldexp((double)f, -16);
    else mag = ldexp((double)(4 + f), e - 17);
    return s ? -mag : mag;
}

/* The closed forms evaluated once per code, so the hot loops below read a
 * table instead of calling ldexp. */
static double val64[256];
static float val32[256];
static double e5_val64[256];
static float e5_val32[256];
static int tables_ready;

static void tables_init(void)
{
    if (tables_ready) return;
    for (int c = 0; c < 256; c++) {
        val64[c] = orc_e4m3_value((uint8_t)c);
        val32[c] = (float)val64[c];
        e5_val64[c] = orc_e5m2_value((uint8_t)c);
        e5_val32[c] = (float)e5_val64[c];
    }
    tables_ready = 1;
}

/* Saturating round-to-nearest-even encode of one fp32 value, written as the
 * definition: the code of the finite E4M3 value nearest to y, with ties going
 * to the code whose last bit is 0; magnitudes at or above 448 (and +-inf)
 * clamp to the largest finite code; the sign bit is the sign of y, so -0 and
 * negative values that round to zero give 0x80; NaN gives the NaN code. */
uint8_t orc_e4m3_encode(float y)
{
    tables_init();
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    double m = fabs((double)y);
    if (m >= ORC_E4M3_MAX) return (uint8_t)(sign | 0x7E);
    /* The non-negative finite codes 0x00..0x7E have strictly increasing
     * values, so the nearest one is found by bisection for the last code
     * whose value is <= m, then comparing with its successor. */
    int lo = 0, hi = 0x7E;            /* value(lo) <= m < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (val64[mid] <= m) lo = mid; else hi = mid;
    }
    double dlo = m - val64[lo];   /* exact in fp64 */
    double dhi = val64[hi] - m;
    int code;
    if (dlo < dhi)      code = lo;
    else if (dhi < dlo) code = hi;
    else                code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | code);
}

void orc_e4m3_encode_array(const float *y, uint8_t *out, int64_t n)
{
    tables_init();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_e4m3_encode(y[i]);
}

/* Saturating round-to-nearest-even E5M2 encode, the same definition as for
 * E4M3 with this format's finite values: nearest finite value, ties to the
 * code whose last bit is 0, magnitudes at or above 57344 (and +-inf) clamp
 * to the largest finite code 0x7B, the sign bit from y, NaN -> 0x7F. */
uint8_t orc_e5m2_encode(float y)
{
    tables_init();
    uint8_t sgn = signbit(y) ? (uint8_t)0x80 : (uint8_t)0x00;
    if (isnan(y)) return (uint8_t)(sgn | 0x7F);
    double m = fabs((double)y);
    if (m >= ORC_E5M2_MAX) return (uint8_t)(sgn | 0x7B);
    int lo = 0, hi = 0x7B;            /* e5 value(lo) <= m < e5 value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e5_val64[mid] <= m) lo = mid; else hi = mid;
    }
    double dlo = m - e5_val64[lo];
    double dhi = e5_val64[hi] - m;
    int code;
    if (dlo < dhi)      code = lo;
    else if (dhi < dlo) code = hi;
    else                code = (lo & 1) ? hi : lo;
    return (uint8_t)(sgn | code);
}

void orc_e5m2_encode_array(const float *y, uint8_t *out, int64_t n)
{
    tables_init();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = orc_e5m2_encode(y[i]);
}

/* ---------------------------------------------------------------- bf16 -- */

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;       /* bf16 is the top half of fp32 */
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* Nearest bf16 to v, ties to the even pattern; values past the largest
 * finite bf16 round to infinity as IEEE rounding does; NaN stays a quiet NaN
 * with its sign. */
uint16_t orc_f32_to_bf16(float v)
{
    uint32_t bits;
    memcpy(&bits, &v, 4);
    if (isnan(v)) return (uint16_t)((bits >> 16) | 0x0040);
    uint16_t down = (uint16_t)(bits >> 16);          /* truncation toward 0 */
    if ((bits & 0xFFFFu) == 0) return down;          /* already a bf16 */
    uint16_t up = (uint16_t)(down + 1);              /* next away from 0 */
    double dv = fabs((double)v);
    double dd = dv - fabs((double)orc_bf16_to_f32(down));
    /* the successor of the largest finite bf16 is infinity; the rounding
     * boundary is then the midpoint to the next (unrepresentable) step */
    double du;
    if ((up & 0x7FFF) == 0x7F80) {
        double step = fabs((double)orc_bf16_to_f32(down)) -
                      fabs((double)orc_bf16_to_f32((uint16_t)(down - 1)));
        du = fabs((double)orc_bf16_to_f32(down)) + step - dv;
    } else {
        du = fabs((double)orc_bf16_to_f32(up)) - dv;
    }
    if (dd < du) return down;
    if (du < dd) return up;
    return (down & 1) ? up : down;
}

void orc_f32_to_bf16_array(const float *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_f32_to_bf16(v[i]);
}

/* ------------------------------------------------------------ quantize -- */

/* max |v| over a set, NaN-propagating (a NaN anywhere makes the result NaN);
 * the max of the empty set is 0. */
static float amax_update(float a, float v)
{
    if (isnan(a) || isnan(v)) return NAN;
    float m = fabsf(v);
    return m > a ? m : a;
}

/* s = 448 / max(a, eps) as one IEEE fp32 division.  A NaN amax gives NaN. */
float orc_scale_from_amax(float a)
{
    float d = (a < ORC_EPS) ? ORC_EPS : a;   /* NaN compares false: d = NaN */
    return (float)ORC_E4M3_MAX / d;
}

/* Quantize a bf16 matrix x[rows][cols] (row-major).
 *   rowwise == 0 (tensorwise): one amax over the tensor, one scale; q and qt
 *       both use it, so qt[c][r] == q[r][c].  scale[0] = scale_t[0] = s,
 *       amax[0] = a.
 *   rowwise == 1: q[r][c] uses the scale of row r (amax over the row) and
 *       qt[c][r] uses the scale of column c (amax over the column).
 *       scale[rows], scale_t[cols], amax[rows + cols] (rows first).
 * The stored scale is the multiplier: q = enc(fl32(x * s)).  */
void orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int rowwise,
                  uint8_t *q, uint8_t *qt, float *scale, float *scale_t,
                  float *amax)
{
    tables_init();
    if (!rowwise) {
        float a = 0.0f;
        for (int64_t i = 0; i < rows * cols; i++)
            a = amax_update(a, orc_bf16_to_f32(x[i]));
        float s = orc_scale_from_amax(a);
        #pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; r++)
            for (int64_t c = 0; c < cols; c++) {
                uint8_t code = orc_e4m3_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
                q[r * cols + c] = code;
                qt[c * rows + r] = code;
            }
        scale[0] = s;
        scale_t[0] = s;
        if (amax) amax[0] = a;
        return;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float a = 0.0f;
        for (int64_t c = 0; c < cols; c++)
            a = amax_update(a, orc_bf16_to_f32(x[r * cols + c]));
        float s = orc_scale_from_amax(a);
        for (int64_t c = 0; c < cols; c++)
            q[r * cols + c] = orc_e4m3_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
        scale[r] = s;
        if (amax) amax[r] = a;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float a = 0.0f;
        for (int64_t r = 0; r < rows; r++)
            a = amax_update(a, orc_bf16_to_f32(x[r * cols + c]));
        float s = orc_scale_from_amax(a);
        for (int64_t r = 0; r < rows; r++)
            qt[c * rows + r] = orc_e4m3_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
        scale_t[c] = s;
        if (amax) amax[rows + c] = a;
    }
}

/* max |x| over a bf16 tensor of n elements (NaN-propagating; 0 when empty):
 * one rank's share of the global tensorwise amax. */
float orc_amax(const uint16_t *x, int64_t n)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; i++)
        a = amax_update(a, orc_bf16_to_f32(x[i]));
    return a;
}

/* Cast with a scale given by the caller (one tensorwise multiplier s, e.g.
 * from a global amax): q[r][c] = enc(fl32(x[r][c] * s)) and qt[c][r] = the
 * same code.  With s = scale_from_amax(amax(x)) this is the tensorwise
 * quantize above. */
void orc_quantize_scaled(const uint16_t *x, int64_t rows, int64_t cols, float s,
                         uint8_t *q, uint8_t *qt)
{
    tables_init();
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            float y = orc_bf16_to_f32(x[r * cols + c]) * s;
            uint8_t code = orc_e4m3_encode(y);
            q[r * cols + c] = code;
            qt[c * rows + r] = code;
        }
}

/* s = 57344 / max(a, eps) as one IEEE fp32 division (E5M2's largest finite
 * value in place of E4M3's 448). */
float orc_scale_from_amax_e5m2(float a)
{
    float d = (a < ORC_EPS) ? ORC_EPS : a;
    return (float)ORC_E5M2_MAX / d;
}

/* The quantize of orc_quantize with E5M2 codes (gradients): the same
 * amax / scale / cast steps, the scale mapping amax onto 57344. */
void orc_quantize_e5m2(const uint16_t *x, int64_t rows, int64_t cols, int rowwise,
                       uint8_t *q, uint8_t *qt, float *scale, float *scale_t,
                       float *amax)
{
    tables_init();
    if (!rowwise) {
        float a = 0.0f;
        for (int64_t i = 0; i < rows * cols; i++)
            a = amax_update(a, orc_bf16_to_f32(x[i]));
        float s = orc_scale_from_amax_e5m2(a);
        #pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; r++)
            for (int64_t c = 0; c < cols; c++) {
                uint8_t code = orc_e5m2_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
                q[r * cols + c] = code;
                qt[c * rows + r] = code;
            }
        scale[0] = s;
        scale_t[0] = s;
        if (amax) amax[0] = a;
        return;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float a = 0.0f;
        for (int64_t c = 0; c < cols; c++)
            a = amax_update(a, orc_bf16_to_f32(x[r * cols + c]));
        float s = orc_scale_from_amax_e5m2(a);
        for (int64_t c = 0; c < cols; c++)
            q[r * cols + c] = orc_e5m2_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
        scale[r] = s;
        if (amax) amax[r] = a;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float a = 0.0f;
        for (int64_t r = 0; r < rows; r++)
            a = amax_update(a, orc_bf16_to_f32(x[r * cols + c]));
        float s = orc_scale_from_amax_e5m2(a);
        for (int64_t r = 0; r < rows; r++)
            qt[c * rows + r] = orc_e5m2_encode(orc_bf16_to_f32(x[r * cols + c]) * s);
        scale_t[c] = s;
        if (amax) amax[rows + c] = a;
    }
}

/* ---------------------------------------------------------------- GEMM -- */

/* One output element of a scaled fp8 GEMM with both operands contiguous
 * along the contraction index:
 *   acc = sum_{t=0..k-1} value(a[i][t]) * value(b[j][t])   (fp32, ascending t)
 *   out = bf16( fl32( fl32(acc * (1/sa)) * (1/sb) ) )
 * Every fp8 x fp8 product is exact in fp32, so the only roundings are the
 * k additions, the two reciprocals, the two scalings and the final bf16. */
static float gemm_element_f32(const uint8_t *arow, const uint8_t *brow,
                              int64_t k, float sa, float sb, float *acc_out)
{
    float acc = 0.0f;
    for (int64_t t = 0; t < k; t++)
        acc += val32[arow[t]] * val32[brow[t]];
    if (acc_out) *acc_out = acc;
    float inv_a = 1.0f / sa;
    float inv_b = 1.0f / sb;
    float v = acc * inv_a;
    return v * inv_b;
}

static uint16_t gemm_element(const uint8_t *arow, const uint8_t *brow,
                             int64_t k, float sa, float sb, float *acc_out)
{
    return orc_f32_to_bf16(gemm_element_f32(arow, brow, k, sa, sb, acc_out));
}

/* Full GEMM: out[i][j] (row-major, m x n) from a[m][k] and b[n][k].
 * sa has m entries when a_vec != 0, else one; likewise sb with n / b_vec.
 * acc (optional, m x n) receives the fp32 sums before scaling. */
void orc_gemm_tn(const uint8_t *a, const float *sa, int a_vec,
                 const uint8_t *b, const float *sb, int b_vec,
                 int64_t m, int64_t n, int64_t k, uint16_t *out, float *acc)
{
    tables_init();
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            out[i * n + j] = gemm_element(a + i * k, b + j * k, k,
                                          a_vec ? sa[i] : sa[0],
                                          b_vec ? sb[j] : sb[0],
                                          acc ? &acc[i * n + j] : 0);
}

/* The same definition evaluated only at the listed (ii[s], jj[s]) outputs. */
void orc_gemm_tn_sampled(const uint8_t *a, const float *sa, int a_vec,
                         const uint8_t *b, const float *sb, int b_vec,
                         int64_t k, const int64_t *ii, const int64_t *jj,
                         int64_t ns, uint16_t *out, float *acc)
{
    tables_init();
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t s = 0; s < ns; s++) {
        int64_t i = ii[s], j = jj[s];
        out[s] = gemm_element(a + i * k, b + j * k, k,
                              a_vec ? sa[i] : sa[0], b_vec ? sb[j] : sb[0],
                              acc ? &acc[s] : 0);
    }
}

/* The fp32-output form of the same GEMM (the value before the final bf16
 * rounding), as a grad_W that is reduce-scattered in fp32 would need:
 *   out[i][j] = fl32( fl32(acc * (1/sa)) * (1/sb) )                         */
void orc_gemm_tn_f32(const uint8_t *a, const float *sa, int a_vec,
                     const uint8_t *b, const float *sb, int b_vec,
                     int64_t m, int64_t n, int64_t k, float *out)
{
    tables_init();
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            out[i * n + j] = gemm_element_f32(a + i * k, b + j * k, k,
                                              a_vec ? sa[i] : sa[0],
                                              b_vec ? sb[j] : sb[0], 0);
}

void orc_gemm_tn_f32_sampled(const uint8_t *a, const float *sa, int a_vec,
                             const uint8_t *b, const float *sb, int b_vec,
                             int64_t k, const int64_t *ii, const int64_t *jj,
                             int64_t ns, float *out)
{
    tables_init();
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t s = 0; s < ns; s++) {
        int64_t i = ii[s], j = jj[s];
        out[s] = gemm_element_f32(a + i * k, b + j * k, k,
                                  a_vec ? sa[i] : sa[0], b_vec ? sb[j] : sb[0], 0);
    }
}

/* The GEMM with a format per operand (0 = E4M3, 1 = E5M2), e.g. an E5M2
 * gradient times an E4M3 weight or activation; every E4M3 x E5M2 product
 * has at most 7 significant bits and is exact in fp32, so the definition is
 * otherwise the same: fp32 sum in ascending t, fp32 reciprocals, bf16. */
static uint16_t gemm_element_mixed(const uint8_t *arow, const float *ta,
                                   const uint8_t *brow, const float *tb,
                                   int64_t k, float sa, float sb)
{
    float sum = 0.0f;
    for (int64_t t = 0; t < k; ++t)
        sum += ta[arow[t]] * tb[brow[t]];
    float ra = 1.0f / sa;
    float rb = 1.0f / sb;
    float v = sum * ra;
    v = v * rb;
    return orc_f32_to_bf16(v);
}

void orc_gemm_tn_mixed(const uint8_t *a, int fmt_a, const float *sa, int a_vec,
                       const uint8_t *b, int fmt_b, const float *sb, int b_vec,
                       int64_t m, int64_t n, int64_t k, uint16_t *out)
{
    tables_init();
    const float *ta = fmt_a ? e5_val32 : val32;
    const float *tb = fmt_b ? e5_val32 : val32;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            out[i * n + j] = gemm_element_mixed(a + i * k, ta, b + j * k, tb, k,
                                                a_vec ? sa[i] : sa[0], b_vec ? sb[j] : sb[0]);
}

void orc_gemm_tn_mixed_sampled(const uint8_t *a, int fmt_a, const float *sa, int a_vec,
                               const uint8_t *b, int fmt_b, const float *sb, int b_vec,
                               int64_t k, const int64_t *ii, const int64_t *jj,
                               int64_t ns, uint16_t *out)
{
    tables_init();
    const float *ta = fmt_a ? e5_val32 : val32;
    const float *tb = fmt_b ? e5_val32 : val32;
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t s = 0; s < ns; s++) {
        int64_t i = ii[s], j = jj[s];
        out[s] = gemm_element_mixed(a + i * k, ta, b + j * k, tb, k,
                                    a_vec ? sa[i] : sa[0], b_vec ? sb[j] : sb[0]);
    }
}

/* ------------------------------------------------------------- SwiGLU -- */

/* The SwiGLU feed-forward of the Llama 3.1 model the tutorial page trains:
 *   h = silu(a) * b,  silu(a) = a * sigma(a) = a / (1 + e^-a)
 * with a = x.W1^T and b = x.W3^T, each [rows, cols].  Reading: bf16 inputs
 * are widened to fp32, silu is the fp32 rounding of its exact value, one
 * fp32 product, one bf16 rounding:
 *   h = bf16( fl32( fl32(silu(a)) * b ) )
 * Backward, with the derivative silu'(a) = sigma(a) (1 + a (1 - sigma(a))):
 *   da = bf16( fl32( fl32(dh * b) * fl32(silu'(a)) ) )
 *   db = bf16( fl32( dh * fl32(silu(a)) ) )
 * silu and silu' are evaluated in float64 and rounded once to fp32.       */
float orc_silu(float a)
{
    double x = (double)a;
    return (float)(x / (1.0 + exp(-x)));
}

float orc_dsilu(float a)
{
    double x = (double)a;
    double sg = 1.0 / (1.0 + exp(-x));
    return (float)(sg * (1.0 + x * (1.0 - sg)));
}

/* a, b, h: bf16 [n] (any shape, element by element) */
void orc_swiglu_fwd(const uint16_t *a, const uint16_t *b, int64_t n, uint16_t *h)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float av = orc_bf16_to_f32(a[i]);
        float bv = orc_bf16_to_f32(b[i]);
        h[i] = orc_f32_to_bf16(orc_silu(av) * bv);
    }
}

/* dh, a, b, da, db: bf16 [n] */
void orc_swiglu_bwd(const uint16_t *dh, const uint16_t *a, const uint16_t *b, int64_t n,
                    uint16_t *da, uint16_t *db)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        float g = orc_bf16_to_f32(dh[i]);
        float av = orc_bf16_to_f32(a[i]);
        float bv = orc_bf16_to_f32(b[i]);
        float gb = g * bv;
        da[i] = orc_f32_to_bf16(gb * orc_dsilu(av));
        db[i] = orc_f32_to_bf16(g * orc_silu(av));
    }
}

/* x feeds two linears of the block (w1 and w3), so its gradient is the sum
 * of their two bf16 grad_X outputs, added as bf16 tensors are: widened to
 * fp32, one fp32 addition, one bf16 rounding. */
void orc_add_bf16(const uint16_t *x, const uint16_t *y, int64_t n, uint16_t *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_f32_to_bf16(orc_bf16_to_f32(x[i]) + orc_bf16_to_f32(y[i]));
}
