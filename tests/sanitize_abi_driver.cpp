// The C ABI's host-side argument validation, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; tests/test_sanitize.py builds
// the library's host code with both and links this driver against it).
//
// Every call below is rejected before any HIP call or launch: the device
// addresses are fake (never dereferenced) and each case breaks one rule of
// include/fp8_linear.h.  Dimensions up to 2^62 check that the size
// arithmetic of the validation itself does not overflow.  Prints one line
// per mismatch and exits with the number of mismatches.
#include "fp8_linear.h"

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

namespace {

int fails = 0;

#define EXPECT(call, want)                                                          \
  do {                                                                              \
    const long long got_ = (long long)(call);                                       \
    if (got_ != (long long)(want)) {                                                \
      std::fprintf(stderr, "line %d: %s gave %lld, expected %lld\n", __LINE__, #call, \
                   got_, (long long)(want));                                        \
      ++fails;                                                                      \
    }                                                                               \
  } while (0)

constexpr uintptr_t A16 = 0x10000;   // 16-byte aligned fake device address
constexpr uintptr_t A_BAD = 0x10004; // misaligned
constexpr int64_t HUGE_DIM = (int64_t)1 << 62;

void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }
float *F(uintptr_t a) { return reinterpret_cast<float *>(a); }

int quant(uintptr_t x = A16, int64_t rows = 16, int64_t cols = 16, int scaling = 0,
          uintptr_t q = A16, uintptr_t qt = A16, uintptr_t s = A16, uintptr_t st = A16,
          uintptr_t amax = 0, uintptr_t ws = A16, size_t wsb = 1 << 20) {
  return fp8_linear_quantize(P(x), rows, cols, scaling, P(q), P(qt), F(s), F(st), F(amax),
                             P(ws), wsb, nullptr);
}

int fwd(int64_t M, int64_t N, int64_t K, int scaling = 0, uintptr_t out = A16,
        uintptr_t wq = A16) {
  return fp8_linear_fwd(P(A16), F(A16), P(wq), F(A16), M, N, K, scaling, P(out), nullptr);
}

int bwd(int64_t M, int64_t N, int64_t K, uintptr_t gx = A16, uintptr_t gw = A16,
        uintptr_t wtq = A_BAD, int scaling = 0) {
  return fp8_linear_bwd(P(A16), F(A16), P(A16), F(A16), P(wtq), F(A16), P(A16), F(A16), M, N,
                        K, scaling, P(gx), P(gw), nullptr);
}

void status_and_sizes() {
  EXPECT(std::strcmp(fp8_linear_status_string(FP8L_OK), "ok"), 0);
  for (int s : {-1, 6, 99, INT_MIN, INT_MAX})
    EXPECT(std::strcmp(fp8_linear_status_string(s), "unknown status"), 0);
  EXPECT(std::strstr(fp8_linear_version(), "gfx950") != nullptr, 1);

  EXPECT(fp8_linear_workspace_bytes(0, 0, 0), 0);
  EXPECT(fp8_linear_workspace_bytes(17, 16, 0), 0);
  EXPECT(fp8_linear_workspace_bytes(16, 16, 5), 0);
  EXPECT(fp8_linear_workspace_bytes(-16, 16, 0), 0);
  EXPECT(fp8_linear_workspace_bytes(HUGE_DIM, HUGE_DIM, 0), 0);
  EXPECT(fp8_linear_workspace_bytes(HUGE_DIM, HUGE_DIM, FP8L_ROWWISE), 0);
  EXPECT(fp8_linear_workspace_bytes(16, INT64_MIN, 0), 0);
  EXPECT(fp8_linear_workspace_bytes(8192, 14336, 0) % 256, 0);
  EXPECT(fp8_linear_workspace_bytes(8192, 14336, 0) <
             fp8_linear_workspace_bytes(8192, 14336, FP8L_ROWWISE), 1);
  EXPECT(fp8_swiglu_workspace_bytes(24, 16, 0), 0);
  EXPECT(fp8_swiglu_workspace_bytes(HUGE_DIM, HUGE_DIM, FP8L_ROWWISE), 0);
}

void quantize_cases() {
  EXPECT(quant(A16, 16, 16, 4), FP8L_EINVAL);
  EXPECT(quant(A16, 16, 16, -1), FP8L_EINVAL);
  EXPECT(quant(A16, 17, 16), FP8L_ESHAPE);
  EXPECT(quant(A16, 16, -16), FP8L_ESHAPE);
  EXPECT(quant(A16, (int64_t)1 << 31, 16), FP8L_ESHAPE);
  EXPECT(quant(A16, HUGE_DIM, HUGE_DIM), FP8L_ESHAPE);
  EXPECT(quant(A16, HUGE_DIM, HUGE_DIM, FP8L_ROWWISE), FP8L_ESHAPE);
  EXPECT(quant(0), FP8L_EINVAL);
  EXPECT(quant(A16, 16, 16, 0, 0), FP8L_EINVAL);
  EXPECT(quant(A16, 16, 16, 0, A16, A16, A16, A16, 0, 0), FP8L_EINVAL);
  EXPECT(quant(A16, 16, 16, 0, A16, A16, A16, A16, 0, A16, 0), FP8L_EWORKSPACE);
  EXPECT(quant(A16, 8192, 4096, 0, A16, A16, A16, A16, 0, A16, 100), FP8L_EWORKSPACE);
  EXPECT(quant(A_BAD), FP8L_EALIGN);
  EXPECT(quant(A16, 16, 16, 0, A16, A_BAD), FP8L_EALIGN);
  EXPECT(quant(A16, 16, 16, 0, A16, A16, A16 + 2), FP8L_EALIGN);
  EXPECT(quant(A16, 16, 16, 0, A16, A16, A16, A16, A16 + 1), FP8L_EALIGN);

  EXPECT(fp8_linear_quantize_noalloc(P(A16), 17, 16, 0, P(A16), P(A16), F(A16), F(A16),
                                     nullptr, nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_quantize_noalloc(P(A16), 65536, 32768, FP8L_ROWWISE, P(A16), P(A16),
                                     F(A16), F(A16), nullptr, nullptr), FP8L_EWORKSPACE);
  EXPECT(fp8_linear_quantize_noalloc(P(A16), HUGE_DIM, HUGE_DIM, FP8L_ROWWISE, P(A16),
                                     P(A16), F(A16), F(A16), nullptr, nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_quantize_noalloc(P(A16), 16, 16, 0, P(A16), P(A_BAD), F(A16), F(A16),
                                     nullptr, nullptr), FP8L_EALIGN);

  EXPECT(fp8_linear_amax(P(A16), 24, 16, F(A16), P(A16), 1 << 20, nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_amax(P(A16), HUGE_DIM, HUGE_DIM, F(A16), P(A16), 1 << 20, nullptr),
         FP8L_ESHAPE);
  EXPECT(fp8_linear_amax(P(A16), 16, 16, nullptr, P(A16), 1 << 20, nullptr), FP8L_EINVAL);
  EXPECT(fp8_linear_amax(P(A16), 16, 16, F(A16), P(A16), 0, nullptr), FP8L_EWORKSPACE);
  EXPECT(fp8_linear_amax(P(A_BAD), 16, 16, F(A16), P(A16), 1 << 20, nullptr), FP8L_EALIGN);

  EXPECT(fp8_linear_quantize_scaled(P(A16), 16, 8, F(A16), P(A16), P(A16), nullptr),
         FP8L_ESHAPE);
  EXPECT(fp8_linear_quantize_scaled(nullptr, 0, 16, nullptr, nullptr, nullptr, nullptr),
         FP8L_OK);
  EXPECT(fp8_linear_quantize_scaled(P(A16), HUGE_DIM, HUGE_DIM, F(A16), P(A16), P(A16),
                                    nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_quantize_scaled(P(A16), 16, 16, nullptr, P(A16), P(A16), nullptr),
         FP8L_EINVAL);
  EXPECT(fp8_linear_quantize_scaled(P(A16), 16, 16, F(A16), P(A16), P(A_BAD), nullptr),
         FP8L_EALIGN);

  EXPECT(fp8_linear_encode_e4m3(F(A16), reinterpret_cast<uint8_t *>(A16), -1, nullptr),
         FP8L_ESHAPE);
  EXPECT(fp8_linear_encode_e4m3(nullptr, reinterpret_cast<uint8_t *>(A16), 4, nullptr),
         FP8L_EINVAL);
  EXPECT(fp8_linear_encode_e5m2(F(A_BAD), reinterpret_cast<uint8_t *>(A16), 4, nullptr),
         FP8L_EALIGN);
  EXPECT(fp8_linear_encode_e5m2(nullptr, nullptr, 0, nullptr), FP8L_OK);
}

void gemm_cases() {
  EXPECT(fwd(16, 16, 16, -1), FP8L_EINVAL);
  EXPECT(fwd(16, 16, 16, FP8L_E5M2), FP8L_EINVAL);
  EXPECT(fwd(8, 16, 16), FP8L_ESHAPE);
  EXPECT(fwd(16, 16, -16), FP8L_ESHAPE);
  EXPECT(fwd(32768, 32768, 16), FP8L_ESHAPE);            // bf16 output of 2^31 bytes
  EXPECT(fwd(32752, 32768, 16, 0, A_BAD), FP8L_EALIGN);  // one row less passes the size check
  EXPECT(fwd(65536, 16, 32768), FP8L_ESHAPE);            // xq of 2^31 bytes
  EXPECT(fwd((int64_t)1 << 31, 16, 16), FP8L_ESHAPE);
  EXPECT(fwd(HUGE_DIM, HUGE_DIM, HUGE_DIM), FP8L_ESHAPE);
  EXPECT(fwd(16, HUGE_DIM, 16), FP8L_ESHAPE);
  EXPECT(fwd(16, 16, 16, 0, A_BAD), FP8L_EALIGN);
  EXPECT(fwd(16, 16, 16, 0, A16, A_BAD), FP8L_EALIGN);

  EXPECT(bwd(16, 16, 16, 0, 0), FP8L_EINVAL);
  EXPECT(bwd(16, 24, 16), FP8L_ESHAPE);
  EXPECT(bwd(16, 16, 16), FP8L_EALIGN);
  EXPECT(bwd(16, 16, 16, A16, A_BAD, A16), FP8L_EALIGN);
  EXPECT(bwd(16, 16, 16, A16, A16, A16, 4), FP8L_EINVAL);
  EXPECT(bwd(32768, 16, 32768), FP8L_ESHAPE);
  EXPECT(bwd(HUGE_DIM, HUGE_DIM, HUGE_DIM), FP8L_ESHAPE);

  EXPECT(fp8_linear_bwd_w_f32(P(A16), F(A16), P(A16), F(A16), 16, 32768, 32768, 0, F(A16),
                              nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_bwd_w_f32(P(A16), F(A16), P(A16), F(A16), HUGE_DIM, HUGE_DIM, HUGE_DIM, 0,
                              F(A16), nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_bwd_w_f32(P(A16), F(A16), P(A16), nullptr, 16, 16, 16, 0, F(A16),
                              nullptr), FP8L_EINVAL);
  EXPECT(fp8_linear_bwd_w_f32(P(A16), F(A16), P(A16), F(A16), 16, 16, 16, 0, F(A_BAD),
                              nullptr), FP8L_EALIGN);

  EXPECT(fp8_linear_bwd_x_acc(P(A16), F(A16), P(A16), F(A16), 16, 16, 20, 0, P(A16), nullptr),
         FP8L_ESHAPE);
  EXPECT(fp8_linear_bwd_x_acc(P(A16), F(A16), P(A16), F(A16), HUGE_DIM, HUGE_DIM, HUGE_DIM, 0,
                              P(A16), nullptr), FP8L_ESHAPE);
  EXPECT(fp8_linear_bwd_x_acc(P(A16), F(A16), P(A16), F(A16), 16, 16, 16, 0, P(A_BAD),
                              nullptr), FP8L_EALIGN);

  fp8l_gemm_problem pr[5];
  for (auto &p : pr) p = {P(A16), F(A16), P(A16), F(A16), P(A16), 16, 16, 16};
  EXPECT(fp8_linear_gemm_grouped(nullptr, 1, 0, nullptr), FP8L_EINVAL);
  EXPECT(fp8_linear_gemm_grouped(pr, 0, 0, nullptr), FP8L_EINVAL);
  EXPECT(fp8_linear_gemm_grouped(pr, 5, 0, nullptr), FP8L_EINVAL);
  EXPECT(fp8_linear_gemm_grouped(pr, 1, 4, nullptr), FP8L_EINVAL);
  pr[1].c = P(A16 + 256);                                // outputs overlap
  EXPECT(fp8_linear_gemm_grouped(pr, 2, 0, nullptr), FP8L_EINVAL);
  pr[1].c = P(0x20000);
  pr[1].m = pr[1].n = pr[1].k = HUGE_DIM;
  EXPECT(fp8_linear_gemm_grouped(pr, 2, 0, nullptr), FP8L_ESHAPE);
  pr[1].m = pr[1].n = pr[1].k = 16;
  pr[1].c = P(A_BAD);
  EXPECT(fp8_linear_gemm_grouped(pr, 2, 0, nullptr), FP8L_EALIGN);
}

void swiglu_cases() {
  auto sfwd = [](int64_t rows, int64_t hidden, int scaling, uintptr_t h, size_t wsb) {
    return fp8_swiglu_fwd(P(A16), P(A16), rows, hidden, scaling, P(h), P(A16), P(A16), F(A16),
                          F(A16), nullptr, P(A16), wsb, nullptr);
  };
  EXPECT(sfwd(16, 16, FP8L_E5M2, A16, 1 << 20), FP8L_EINVAL);
  EXPECT(sfwd(16, 40, 0, A16, 1 << 20), FP8L_ESHAPE);
  EXPECT(sfwd(HUGE_DIM, HUGE_DIM, 0, A16, 1 << 20), FP8L_ESHAPE);
  EXPECT(sfwd(16, 16, 0, 0, 1 << 20), FP8L_EINVAL);
  EXPECT(sfwd(16, 16, 0, A16, 16), FP8L_EWORKSPACE);
  EXPECT(sfwd(16, 16, 0, A_BAD, 1 << 20), FP8L_EALIGN);

  auto sbwd = [](int64_t rows, int64_t hidden, int scaling, uintptr_t da, size_t wsb) {
    return fp8_swiglu_bwd(P(A16), P(A16), P(A16), rows, hidden, scaling, P(da), P(A16), P(A16),
                          P(A16), F(A16), F(A16), nullptr, P(A16), P(A16), F(A16), F(A16),
                          nullptr, P(A16), wsb, nullptr);
  };
  EXPECT(sbwd(16, 16, 8, A16, 1 << 20), FP8L_EINVAL);
  EXPECT(sbwd(8, 16, 0, A16, 1 << 20), FP8L_ESHAPE);
  EXPECT(sbwd(HUGE_DIM, HUGE_DIM, FP8L_ROWWISE, A16, 1 << 20), FP8L_ESHAPE);
  EXPECT(sbwd(16, 16, 0, 0, 1 << 20), FP8L_EINVAL);
  EXPECT(sbwd(16, 16, 0, A16, 0), FP8L_EWORKSPACE);
  EXPECT(sbwd(16, 16, 0, A_BAD, 1 << 20), FP8L_EALIGN);
}

}  // namespace

int main() {
  status_and_sizes();
  quantize_cases();
  gemm_cases();
  swiglu_cases();
  std::printf("abi validation under sanitizers: %d mismatches\n", fails);
  return fails;
}
