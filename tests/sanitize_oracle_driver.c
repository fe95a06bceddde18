/* The oracle (oracle/oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: tests/test_sanitize.py compiles the two files
 * together with both and runs the result on the host.
 *
 * Every function runs on small inputs held in buffers of exactly the size
 * its definition gives (so a read or write one element out of range is
 * reported), over shapes that include empty matrices, a single 16 x 16
 * block and ragged ones, and over inputs that include every bf16 class
 * (zeros of both signs, subnormals, the largest finite values, infinities,
 * NaNs).  A few identities that hold for any input are checked on the way:
 * a tensorwise transposed copy holds the same codes as the plain one, a
 * sampled GEMM equals the full one where both are defined, and the fp32
 * GEMM rounds to the bf16 one.  Exits with the number of failed checks. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's entry points (plain C, defined in oracle/oracle.c) */
double orc_e4m3_value(uint8_t code);
double orc_e5m2_value(uint8_t code);
uint8_t orc_e4m3_encode(float y);
uint8_t orc_e5m2_encode(float y);
void orc_e4m3_encode_array(const float *y, uint8_t *out, int64_t n);
void orc_e5m2_encode_array(const float *y, uint8_t *out, int64_t n);
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float v);
void orc_f32_to_bf16_array(const float *v, uint16_t *out, int64_t n);
float orc_scale_from_amax(float a);
float orc_scale_from_amax_e5m2(float a);
void orc_quantize(const uint16_t *x, int64_t rows, int64_t cols, int rowwise, uint8_t *q,
                  uint8_t *qt, float *scale, float *scale_t, float *amax);
void orc_quantize_e5m2(const uint16_t *x, int64_t rows, int64_t cols, int rowwise, uint8_t *q,
                       uint8_t *qt, float *scale, float *scale_t, float *amax);
float orc_amax(const uint16_t *x, int64_t n);
void orc_quantize_scaled(const uint16_t *x, int64_t rows, int64_t cols, float s, uint8_t *q,
                         uint8_t *qt);
void orc_gemm_tn(const uint8_t *a, const float *sa, int a_vec, const uint8_t *b,
                 const float *sb, int b_vec, int64_t m, int64_t n, int64_t k, uint16_t *out,
                 float *acc);
void orc_gemm_tn_sampled(const uint8_t *a, const float *sa, int a_vec, const uint8_t *b,
                         const float *sb, int b_vec, int64_t k, const int64_t *ii,
                         const int64_t *jj, int64_t ns, uint16_t *out, float *acc);
void orc_gemm_tn_f32(const uint8_t *a, const float *sa, int a_vec, const uint8_t *b,
                     const float *sb, int b_vec, int64_t m, int64_t n, int64_t k, float *out);
void orc_gemm_tn_f32_sampled(const uint8_t *a, const float *sa, int a_vec, const uint8_t *b,
                             const float *sb, int b_vec, int64_t k, const int64_t *ii,
                             const int64_t *jj, int64_t ns, float *out);
void orc_gemm_tn_mixed(const uint8_t *a, int fmt_a, const float *sa, int a_vec,
                       const uint8_t *b, int fmt_b, const float *sb, int b_vec, int64_t m,
                       int64_t n, int64_t k, uint16_t *out);
void orc_gemm_tn_mixed_sampled(const uint8_t *a, int fmt_a, const float *sa, int a_vec,
                               const uint8_t *b, int fmt_b, const float *sb, int b_vec,
                               int64_t k, const int64_t *ii, const int64_t *jj, int64_t ns,
                               uint16_t *out);
float orc_silu(float a);
float orc_dsilu(float a);
void orc_swiglu_fwd(const uint16_t *a, const uint16_t *b, int64_t n, uint16_t *h);
void orc_swiglu_bwd(const uint16_t *dh, const uint16_t *a, const uint16_t *b, int64_t n,
                    uint16_t *da, uint16_t *db);
void orc_add_bf16(const uint16_t *x, const uint16_t *y, int64_t n, uint16_t *out);

static int fails;

#define CHECK(cond)                                                      \
    do {                                                                 \
        if (!(cond)) {                                                   \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

/* exact-size allocation; a zero-size request still returns a distinct
 * pointer that must not be dereferenced */
static void *alloc(size_t n) { return malloc(n ? n : 1); }

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 32);
}

/* bf16 inputs: mostly N(0, 1)-like magnitudes, with every special class */
static uint16_t *bf16_input(int64_t n)
{
    static const uint16_t special[] = {0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F,
                                       0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x3F80, 0x0080};
    uint16_t *x = alloc((size_t)n * 2);
    for (int64_t i = 0; i < n; i++) {
        uint32_t r = next_u32();
        if (r % 97 == 0)
            x[i] = special[(r >> 8) % (sizeof special / sizeof special[0])];
        else
            x[i] = (uint16_t)(0x3C00 + (r >> 16) % 0x0700) ^ (uint16_t)((r & 1) << 15);
    }
    return x;
}

/* bf16 inputs without NaN or infinity (for the GEMM operands' quantize) */
static uint16_t *bf16_finite(int64_t n)
{
    uint16_t *x = bf16_input(n);
    for (int64_t i = 0; i < n; i++)
        if ((x[i] & 0x7F80) == 0x7F80) x[i] = 0x3F80;
    return x;
}

static void conversions(void)
{
    for (int c = 0; c < 256; c++) {
        double v = orc_e4m3_value((uint8_t)c);
        double w = orc_e5m2_value((uint8_t)c);
        if (!isnan(v)) CHECK(orc_e4m3_value(orc_e4m3_encode((float)v)) == v);
        if (!isnan(w) && !isinf(w)) CHECK(orc_e5m2_value(orc_e5m2_encode((float)w)) == w);
    }
    /* every bf16 value through the encoders and back through bf16 */
    float *y = alloc(65536 * sizeof(float));
    uint8_t *e4 = alloc(65536), *e5 = alloc(65536);
    uint16_t *hb = alloc(65536 * 2);
    for (int i = 0; i < 65536; i++) y[i] = orc_bf16_to_f32((uint16_t)i);
    orc_e4m3_encode_array(y, e4, 65536);
    orc_e5m2_encode_array(y, e5, 65536);
    orc_f32_to_bf16_array(y, hb, 65536);
    for (int i = 0; i < 65536; i++)
        if (!isnan(y[i])) CHECK(hb[i] == (uint16_t)i);
    for (int i = 0; i < 65536; i++) {
        float s = orc_silu(y[i]), d = orc_dsilu(y[i]);
        (void)s;
        (void)d;
    }
    CHECK(orc_scale_from_amax(0.0f) > 0.0f);
    CHECK(orc_scale_from_amax_e5m2(0.0f) > 0.0f);
    CHECK(isnan(orc_scale_from_amax(NAN)));
    free(y);
    free(e4);
    free(e5);
    free(hb);
}

static void quantize_shape(int64_t rows, int64_t cols)
{
    const int64_t n = rows * cols;
    uint16_t *x = bf16_input(n);
    for (int rw = 0; rw < 2; rw++)
        for (int e5 = 0; e5 < 2; e5++) {
            uint8_t *q = alloc((size_t)n), *qt = alloc((size_t)n);
            const int64_t ns = rw ? rows : 1, nst = rw ? cols : 1;
            float *s = alloc((size_t)ns * 4), *st = alloc((size_t)nst * 4);
            float *am = alloc((size_t)(rw ? rows + cols : 1) * 4);
            if (e5)
                orc_quantize_e5m2(x, rows, cols, rw, q, qt, s, st, am);
            else
                orc_quantize(x, rows, cols, rw, q, qt, s, st, am);
            if (!rw)
                for (int64_t r = 0; r < rows; r++)
                    for (int64_t c = 0; c < cols; c++)
                        CHECK(q[r * cols + c] == qt[c * rows + r]);
            free(q);
            free(qt);
            free(s);
            free(st);
            free(am);
        }
    uint8_t *q = alloc((size_t)n), *qt = alloc((size_t)n);
    float a = orc_amax(x, n);
    orc_quantize_scaled(x, rows, cols, orc_scale_from_amax(a), q, qt);
    free(q);
    free(qt);
    free(x);
}

static void gemm_shape(int64_t m, int64_t n, int64_t k)
{
    uint16_t *xa = bf16_finite(m * k), *xb = bf16_finite(n * k);
    for (int rw = 0; rw < 2; rw++) {
        uint8_t *a = alloc((size_t)(m * k)), *at = alloc((size_t)(m * k));
        uint8_t *b = alloc((size_t)(n * k)), *bt = alloc((size_t)(n * k));
        float *sa = alloc((size_t)(rw ? m : 1) * 4), *sat = alloc((size_t)(rw ? k : 1) * 4);
        float *sb = alloc((size_t)(rw ? n : 1) * 4), *sbt = alloc((size_t)(rw ? k : 1) * 4);
        orc_quantize(xa, m, k, rw, a, at, sa, sat, NULL);
        orc_quantize(xb, n, k, rw, b, bt, sb, sbt, NULL);

        uint16_t *out = alloc((size_t)(m * n) * 2), *mix = alloc((size_t)(m * n) * 2);
        float *acc = alloc((size_t)(m * n) * 4), *o32 = alloc((size_t)(m * n) * 4);
        orc_gemm_tn(a, sa, rw, b, sb, rw, m, n, k, out, acc);
        orc_gemm_tn(a, sa, rw, b, sb, rw, m, n, k, out, NULL);
        orc_gemm_tn_f32(a, sa, rw, b, sb, rw, m, n, k, o32);
        orc_gemm_tn_mixed(a, 0, sa, rw, b, 0, sb, rw, m, n, k, mix);
        for (int64_t i = 0; i < m * n; i++) {
            CHECK(orc_f32_to_bf16(o32[i]) == out[i]);
            CHECK(mix[i] == out[i]);
        }
        /* samples: the corners and a few inner points, where the matrix has any */
        const int64_t ns = (m && n) ? 6 : 0;
        int64_t *ii = alloc((size_t)ns * 8), *jj = alloc((size_t)ns * 8);
        for (int64_t s = 0; s < ns; s++) {
            ii[s] = (s & 1) ? m - 1 : (int64_t)(next_u32() % (uint32_t)m);
            jj[s] = (s & 2) ? n - 1 : (int64_t)(next_u32() % (uint32_t)n);
        }
        uint16_t *so = alloc((size_t)ns * 2), *sm = alloc((size_t)ns * 2);
        float *sacc = alloc((size_t)ns * 4), *s32 = alloc((size_t)ns * 4);
        orc_gemm_tn_sampled(a, sa, rw, b, sb, rw, k, ii, jj, ns, so, sacc);
        orc_gemm_tn_f32_sampled(a, sa, rw, b, sb, rw, k, ii, jj, ns, s32);
        orc_gemm_tn_mixed_sampled(a, 0, sa, rw, b, 0, sb, rw, k, ii, jj, ns, sm);
        for (int64_t s = 0; s < ns; s++) {
            const int64_t at_ = ii[s] * n + jj[s];
            CHECK(so[s] == out[at_]);
            CHECK(sm[s] == out[at_]);
            CHECK(memcmp(&s32[s], &o32[at_], 4) == 0);
            CHECK(memcmp(&sacc[s], &acc[at_], 4) == 0);
        }
        free(a); free(at); free(b); free(bt);
        free(sa); free(sat); free(sb); free(sbt);
        free(out); free(mix); free(acc); free(o32);
        free(ii); free(jj); free(so); free(sm); free(sacc); free(s32);
    }
    free(xa);
    free(xb);
}

static void swiglu_n(int64_t n)
{
    uint16_t *a = bf16_input(n), *b = bf16_input(n), *dh = bf16_input(n);
    uint16_t *h = alloc((size_t)n * 2), *da = alloc((size_t)n * 2), *db = alloc((size_t)n * 2);
    uint16_t *sum = alloc((size_t)n * 2);
    orc_swiglu_fwd(a, b, n, h);
    orc_swiglu_bwd(dh, a, b, n, da, db);
    orc_add_bf16(da, db, n, sum);
    free(a); free(b); free(dh); free(h); free(da); free(db); free(sum);
}

int main(void)
{
    conversions();
    static const int64_t qshape[][2] = {{0, 0}, {0, 16}, {16, 0}, {16, 16}, {48, 32}, {33, 7}};
    for (size_t s = 0; s < sizeof qshape / sizeof qshape[0]; s++)
        quantize_shape(qshape[s][0], qshape[s][1]);
    static const int64_t gshape[][3] = {{0, 16, 16}, {16, 0, 16}, {16, 16, 0},
                                        {16, 16, 16}, {48, 32, 80}, {17, 5, 33}};
    for (size_t s = 0; s < sizeof gshape / sizeof gshape[0]; s++)
        gemm_shape(gshape[s][0], gshape[s][1], gshape[s][2]);
    swiglu_n(0);
    swiglu_n(1);
    swiglu_n(4099);
    printf("oracle under sanitizers: %d failed checks\n", fails);
    return fails;
}
