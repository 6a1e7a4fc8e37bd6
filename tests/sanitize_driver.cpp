// Host-side argument checks of the GDPA C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every call below is refused (or is an empty
// problem) before anything reaches the GPU, so it runs on a machine without
// one.  Extreme sizes exercise the overflow-safe size arithmetic of the checks
// and the workspace queries.  Prints "ok" and exits 0 when every status
// matches.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "gdpa.h"

namespace {
int failures = 0;
void expect(const char* what, gdpa_status_t got, gdpa_status_t want) {
  if (got != want) {
    std::printf("FAIL %s: got %d (%s), want %d\n", what, (int)got, gdpa_status_string(got), (int)want);
    ++failures;
  }
}
void* const FAKE = reinterpret_cast<void*>(0x1000);  // never dereferenced
const int32_t* const CU = reinterpret_cast<const int32_t*>(0x1000);

gdpa_status_t fwd(int32_t B, int32_t Lq, int32_t Lk, int32_t Hq, int32_t Hkv, int32_t D, int32_t Dv, float scale,
                  int32_t mask, int32_t wl, int32_t wr, int32_t act, int32_t qk = GDPA_DTYPE_BF16,
                  int32_t vd = GDPA_DTYPE_BF16, int32_t od = GDPA_DTYPE_FP32) {
  return gdpa_fwd(FAKE, FAKE, FAKE, FAKE, B, Lq, Lk, Hq, Hkv, D, Dv, scale, mask, wl, wr, act, 0.01f, qk, vd, od,
                  1.0f, 1.0f, nullptr, 0, nullptr);
}
gdpa_status_t vfwd(int32_t B, int32_t mq, int32_t mk, int64_t tq, int64_t tk, int32_t Hq, int32_t Hkv, int32_t D,
                   void* ws, size_t nws) {
  return gdpa_varlen_fwd(FAKE, FAKE, FAKE, FAKE, CU, CU, B, mq, mk, tq, tk, Hq, Hkv, D, D, 0.1f, 0, -1, -1, 3, 0.01f,
                         GDPA_DTYPE_BF16, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, 1.0f, 1.0f, ws, nws, nullptr);
}
gdpa_status_t bwd(int32_t B, int32_t Lq, int32_t Lk, int32_t Hq, int32_t Hkv, int32_t D, int32_t in_dtype,
                  int32_t gd, void* dq, void* dk, void* dv, void* ws, size_t nws) {
  return gdpa_bwd(FAKE, FAKE, FAKE, FAKE, dq, dk, dv, B, Lq, Lk, Hq, Hkv, D, D, 0.1f, 0, -1, -1, 8, 0.01f, in_dtype,
                  gd, ws, nws, nullptr);
}
gdpa_status_t vbwd(int32_t B, int32_t mq, int32_t mk, int64_t tq, int64_t tk, int32_t Hq, int32_t Hkv, int32_t D,
                   void* ws, size_t nws) {
  return gdpa_varlen_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, CU, CU, B, mq, mk, tq, tk, Hq, Hkv, D, D, 0.1f, 0,
                         -1, -1, 8, 0.01f, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, ws, nws, nullptr);
}
}  // namespace

int main() {
  const gdpa_status_t OK = GDPA_OK, INV = GDPA_ERR_INVALID_ARG, UNS = GDPA_ERR_UNSUPPORTED,
                      WS = GDPA_ERR_WORKSPACE_TOO_SMALL;
  // forward: shapes, head dims, enums, dtypes
  expect("fwd Hq % Hkv", fwd(2, 128, 128, 3, 2, 128, 128, 0.1f, 0, -1, -1, 3), INV);
  expect("fwd Hkv 0", fwd(2, 128, 128, 4, 0, 128, 128, 0.1f, 0, -1, -1, 3), INV);
  expect("fwd D 80", fwd(2, 128, 128, 4, 2, 80, 80, 0.1f, 0, -1, -1, 3), UNS);
  expect("fwd (192,192)", fwd(2, 128, 128, 4, 2, 192, 192, 0.1f, 0, -1, -1, 3), UNS);
  expect("fwd B -1", fwd(-1, 128, 128, 4, 2, 128, 128, 0.1f, 0, -1, -1, 3), INV);
  expect("fwd act 11", fwd(2, 128, 128, 4, 2, 128, 128, 0.1f, 0, -1, -1, 11), INV);
  expect("fwd mask 3", fwd(2, 128, 128, 4, 2, 128, 128, 0.1f, 3, -1, -1, 3), INV);
  expect("fwd window -2", fwd(2, 128, 128, 4, 2, 128, 128, 0.1f, 2, -2, 0, 3), INV);
  expect("fwd nan scale", fwd(2, 128, 128, 4, 2, 128, 128, NAN, 0, -1, -1, 3), INV);
  expect("fwd fp16 Q/K, bf16 V", fwd(2, 128, 128, 4, 2, 128, 128, 0.1f, 0, -1, -1, 3, GDPA_DTYPE_FP16), UNS);
  expect("fwd fp8 (192,128)",
         fwd(2, 128, 128, 4, 2, 192, 128, 0.1f, 0, -1, -1, 3, GDPA_DTYPE_FP8_E4M3, GDPA_DTYPE_BF16), UNS);
  expect("fwd empty", fwd(0, 128, 128, 4, 2, 128, 128, 0.1f, 0, -1, -1, 3), OK);
  expect("fwd Lq 0", fwd(2, 0, 128, 4, 2, 128, 128, 0.1f, 0, -1, -1, 3), OK);
  // sizes at the 32-bit limits: refused, with no overflow in the checks
  expect("fwd huge batch", fwd(INT32_MAX, INT32_MAX, INT32_MAX, 64, 64, 128, 128, 0.1f, 0, -1, -1, 3), UNS);
  expect("fwd huge heads", fwd(INT32_MAX, 1024, 1024, INT32_MAX, INT32_MAX, 128, 128, 0.1f, 0, -1, -1, 3), UNS);
  expect("vfwd no workspace", vfwd(2, 128, 128, 200, 200, 4, 4, 64, nullptr, 0), WS);
  expect("vfwd small workspace", vfwd(2, 128, 128, 200, 200, 4, 4, 64, FAKE, 255), WS);
  expect("vfwd total beyond batch x max", vfwd(2, 128, 128, 257, 200, 4, 4, 64, FAKE, 1 << 20), INV);
  expect("vfwd huge totals", vfwd(INT32_MAX, INT32_MAX, INT32_MAX, INT64_MAX, INT64_MAX, 4, 4, 64, FAKE, 1 << 20),
         INV);
  // backward
  expect("bwd no workspace", bwd(2, 128, 128, 4, 2, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, FAKE, FAKE, FAKE,
                                 nullptr, 0), WS);
  expect("bwd fp8 input", bwd(2, 128, 128, 4, 2, 128, GDPA_DTYPE_FP8_E4M3, GDPA_DTYPE_FP32, FAKE, FAKE, FAKE,
                              FAKE, 1 << 20), UNS);
  expect("bwd fp8 grads", bwd(2, 128, 128, 4, 2, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP8_E4M3, FAKE, FAKE, FAKE,
                              FAKE, 1 << 20), INV);
  expect("bwd dk without dv", bwd(2, 128, 128, 4, 2, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, FAKE, FAKE, nullptr,
                                  FAKE, 1 << 20), INV);
  expect("bwd nothing wanted", bwd(2, 128, 128, 4, 2, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, nullptr, nullptr,
                                   nullptr, FAKE, 1 << 20), INV);
  expect("bwd empty", bwd(0, 128, 128, 4, 2, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, FAKE, FAKE, FAKE, nullptr, 0),
         OK);
  expect("bwd huge", bwd(INT32_MAX, INT32_MAX, INT32_MAX, 64, 64, 128, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, FAKE, FAKE,
                         FAKE, FAKE, 1 << 20), UNS);
  expect("vbwd small workspace", vbwd(2, 128, 128, 200, 200, 4, 2, 128, FAKE, 8), WS);
  expect("vbwd huge totals", vbwd(INT32_MAX, INT32_MAX, INT32_MAX, INT64_MAX, INT64_MAX, 4, 2, 128, FAKE, 1 << 20),
         INV);
  expect("vbwd noalloc bad heads",
         gdpa_varlen_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, CU, CU, 2, 128, 128, 200, 200, 3, 2, 128,
                                 128, 0.1f, 0, -1, -1, 8, 0.01f, GDPA_DTYPE_BF16, GDPA_DTYPE_FP32, nullptr),
         INV);
  // workspace queries at the limits (no overflow; plausible sizes)
  const size_t q1 = gdpa_varlen_bwd_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX, INT64_MAX / 2, INT32_MAX,
                                                   INT32_MAX, 128, GDPA_DTYPE_BF16);
  const size_t q2 = gdpa_bwd_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 128,
                                            GDPA_DTYPE_FP32);
  const size_t q3 = gdpa_varlen_fwd_workspace_size(INT32_MAX, INT32_MAX, INT32_MAX, 1, 1, 64);
  std::printf("queries at the limits: %zu %zu %zu\n", q1, q2, q3);
  expect("query negative batch", gdpa_bwd_workspace_size(-1, 128, 128, 4, 4, 128, GDPA_DTYPE_FP32) == 0 ? OK : INV,
         OK);
  for (int s = -1; s < 8; ++s)
    if (gdpa_status_string((gdpa_status_t)s) == nullptr) ++failures;
  if (gdpa_abi_version() != GDPA_ABI_VERSION) ++failures;
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
