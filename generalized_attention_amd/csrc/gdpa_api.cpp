// Host side of the GDPA C ABI: argument validation, variant selection and
// kernel launches on the caller's stream.  Every check runs before the first
// HIP call, so invalid arguments are reported without touching a device.
#include "../../include/gdpa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <vector>

#include "gdpa_kernels.hpp"

namespace {

using gdpa::BwdArgs;
using gdpa::FwdArgs;

// A dispatch packet counts work-items in 32 bits: at most 2^32 - 1 threads of 256.
constexpr int64_t kMaxGrid = ((1LL << 32) - 1) / 256;

bool debug_log() {
  static const bool on = [] {
    const char* e = std::getenv("GDPA_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

// Folds the enum aliases onto the kernel's activation kinds; -1 if invalid.
int act_kind_of(int32_t act) {
  switch (act) {
    case GDPA_ACT_IDENTITY: return gdpa::ACT_IDENTITY;
    case GDPA_ACT_GELU: return gdpa::ACT_GELU;
    case GDPA_ACT_GELU_TANH:
    case GDPA_ACT_FAST_GELU:
    case GDPA_ACT_FAST_GELU_BF16: return gdpa::ACT_GELU_TANH;
    case GDPA_ACT_RELU: return gdpa::ACT_RELU;
    case GDPA_ACT_RELU2: return gdpa::ACT_RELU2;
    case GDPA_ACT_LEAKY_RELU: return gdpa::ACT_LEAKY;
    case GDPA_ACT_SILU:
    case GDPA_ACT_FAST_SILU: return gdpa::ACT_SILU;
    case GDPA_ACT_HARDSWISH: return gdpa::ACT_HARDSWISH;
    default: return -1;
  }
}

struct Common {
  int32_t batch, max_lq, max_lk, hq, hkv, d, dv;  // d: head dim of Q and K, dv: of V and O
  int64_t total_q, total_k;
  int act_kind;
  int32_t wl, wr;
};

// Shape/enum checks shared by all four entry points.
gdpa_status_t check_common(int32_t batch, int32_t max_lq, int32_t max_lk, int64_t total_q,
                           int64_t total_k, int32_t hq, int32_t hkv, int32_t d, int32_t dv, float scale,
                           int32_t mask, int32_t window_left, int32_t window_right, int32_t act,
                           float act_param, Common* c) {
  if (batch < 0 || max_lq < 0 || max_lk < 0 || total_q < 0 || total_k < 0) return GDPA_ERR_INVALID_ARG;
  // no sequence is longer than its max_seqlen (an empty batch is an empty call)
  if (batch > 0 && (total_q > (int64_t)batch * max_lq || total_k > (int64_t)batch * max_lk))
    return GDPA_ERR_INVALID_ARG;
  if (total_q > INT32_MAX || total_k > INT32_MAX) return GDPA_ERR_UNSUPPORTED;
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return GDPA_ERR_INVALID_ARG;
  if (d <= 0 || dv <= 0) return GDPA_ERR_INVALID_ARG;
  // (Q/K, V) head dims: (64, 64), (96, 96), (128, 128), (192, 128)
  if (!(d == dv && (d == 64 || d == 96 || d == 128)) && !(d == 192 && dv == 128)) return GDPA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !std::isfinite(act_param)) return GDPA_ERR_INVALID_ARG;
  const int kind = act_kind_of(act);
  if (kind < 0) return GDPA_ERR_INVALID_ARG;
  int32_t wl = -1, wr = -1;
  switch (mask) {
    case GDPA_MASK_NONE: break;
    case GDPA_MASK_CAUSAL: wr = 0; break;
    case GDPA_MASK_SLIDING_WINDOW:
      if (window_left < -1 || window_right < -1) return GDPA_ERR_INVALID_ARG;
      wl = window_left;
      wr = window_right;
      break;
    default: return GDPA_ERR_INVALID_ARG;
  }
  // Row offsets inside the kernels are 32-bit; tensor offsets are 64-bit.
  const int64_t dmax = std::max(d, dv);
  if ((int64_t)total_q * hq * dmax > (int64_t)1 << 40 || (int64_t)total_k * hkv * dmax > (int64_t)1 << 40)
    return GDPA_ERR_UNSUPPORTED;
  *c = Common{batch, max_lq, max_lk, hq, hkv, d, dv, total_q, total_k, kind, wl, wr};
  return GDPA_OK;
}

// Kernels built per input element kind and (Q/K, V) head dims: 16-bit inputs
// at (64, 64), (96, 96), (128, 128) and, forward only, (192, 128); FP8 Q/K
// (forward only) at (64, 64), (96, 96) and (128, 128).  Every entry point
// checks its combination here, before the schedule kernel or any other HIP
// call is queued.
bool fwd_built(int in_kind, int32_t d, int32_t dv) {
  if (in_kind == gdpa::EL_MX8 || in_kind == gdpa::EL_MX4)
    return d == dv && (d == 64 || d == 128);  // 32-wide blocks on the K = 64 MFMA
  if (d == dv && (d == 64 || d == 96 || d == 128)) return true;
  return in_kind != gdpa::EL_FP8 && d == 192 && dv == 128;
}
bool bwd_built(int in_kind, int32_t d, int32_t dv) {
  return in_kind != gdpa::EL_FP8 && ((d == dv && (d == 64 || d == 96 || d == 128)) || (d == 192 && dv == 128));
}

// Output dtype -> kernel output kind (-1: not an output type).
int out_kind_of(int32_t dtype) {
  switch (dtype) {
    case GDPA_DTYPE_FP32: return gdpa::OUT_F32;
    case GDPA_DTYPE_BF16: return gdpa::OUT_BF16;
    case GDPA_DTYPE_FP16: return gdpa::OUT_F16;
    default: return -1;
  }
}

// Upper bound on the number of products summed into one output row: `len`
// rows of the other operand times `heads` query heads, with `len` capped by the
// window width when both window sides are bounded.
constexpr int64_t kFewTerms = 128;
bool few_terms(int64_t len, int64_t heads, const Common& c) {
  if (c.wl >= 0 && c.wr >= 0) len = std::min<int64_t>(len, (int64_t)c.wl + c.wr + 1);
  return len * heads <= kFewTerms;
}

// Activation constants for the kernels: act(c s) = pscale * y(s), the score
// scale c folded into the constants (the formulas are listed in
// gdpa_common.hpp next to the device code that uses them).
gdpa::ActConsts make_act(int kind, double c, double alpha) {
  const double log2e = 1.4426950408889634, sqrt2opi = 0.7978845608028654, cubic = 0.044715;
  gdpa::ActConsts k{};
  k.alpha = (float)alpha;
  k.gscale = (float)c;
  k.pscale = 1.0f;
  switch (kind) {
    case gdpa::ACT_IDENTITY: k.pscale = (float)c; break;
    case gdpa::ACT_GELU:
      k.k0 = (float)(c / std::sqrt(2.0));
      k.a0 = (float)(c / std::sqrt(2.0 * M_PI));
      k.a1 = (float)(-0.5 * c * c * log2e);
      k.pscale = (float)(0.5 * c);
      break;
    case gdpa::ACT_GELU_TANH: {
      const double c0 = -2.0 * sqrt2opi * log2e;  // sigmoid(2u) = 1 / (1 + 2^(x (c0 + c1 x^2)))
      k.k0 = (float)(c * c0);
      k.k1 = (float)(c * c * c * c0 * cubic);
      k.a0 = (float)(2.0 * sqrt2opi * c);            // x 2u'(x) = s (a0 + a1 s^2)
      k.a1 = (float)(2.0 * sqrt2opi * 3.0 * cubic * c * c * c);
      k.pscale = (float)c;
      break;
    }
    case gdpa::ACT_RELU:
      k.k0 = (float)c;
      k.pscale = (float)c;
      k.a0 = c >= 0 ? 0.0f : -INFINITY;
      k.a1 = c >= 0 ? INFINITY : 0.0f;
      break;
    case gdpa::ACT_RELU2: k.k0 = (float)c; break;
    case gdpa::ACT_LEAKY: {
      // leaky(c s) = A max(s, 0) + B min(s, 0)
      const double A = c > 0 ? c : alpha * c, B = c > 0 ? alpha * c : c;
      k.k0 = (float)c;
      if (std::fabs(A) >= std::fabs(B)) {  // y = s + (B/A - 1) min(s, 0)
        k.pscale = (float)A;
        k.k1 = A != 0 ? (float)(B / A - 1.0) : 0.0f;
        k.a0 = -INFINITY;
        k.a1 = 0.0f;
      } else {  // y = s + (A/B - 1) max(s, 0)
        k.pscale = (float)B;
        k.k1 = (float)(A / B - 1.0);
        k.a0 = 0.0f;
        k.a1 = INFINITY;
      }
      break;
    }
    case gdpa::ACT_SILU:
      k.k0 = (float)(-log2e * c);
      k.a0 = (float)c;
      k.pscale = (float)c;
      break;
    case gdpa::ACT_HARDSWISH:
      k.k0 = (float)c;
      k.pscale = (float)(c / 6.0);
      break;
    default: break;
  }
  return k;
}

gdpa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GDPA_OK;
  if (debug_log()) std::fprintf(stderr, "[gdpa] %s failed: %s\n", what, hipGetErrorString(e));
  return GDPA_ERR_HIP;
}

// Workspace of a jagged call: the costliest-first sequence order (int32 per
// sequence) and the work-queue counters, built on the device before the main
// kernels.  Batches beyond kSortMax keep index order and need no workspace.
size_t schedule_bytes(int64_t batch) {
  if (batch <= 0 || batch > gdpa::kSortMax) return 0;
  return (size_t)(((batch + gdpa::kNumCounters) * 4 + 255) / 256 * 256);
}

// Backward workspace, each part 256-byte aligned:
//   order  int32 [batch]        costliest-first sequence order (jagged calls of up
//                                to kSortMax sequences; index order otherwise)
//   queues int32 [kQWords]      per-XCD queue heads and owners, then the flag a
//                                dQ turn wait sets when it gives up
//   turns  int32 [tiles * hq]   dQ turn counters per (64-row query tile, head):
//                                tiles = total_q / 64 + batch + 1 (jagged) or
//                                batch * ceil(seqlen_q / 64)
//   acc    fp32 [total_q, hq, d] dQ accumulator, when dQ is stored in 16 bits
// How a backward call produces dQ: GDPA_BWD_DQ=fused|separate (read at every
// call, also by the workspace queries) overrides the default choice.
enum DqMode { DQ_AUTO, DQ_FUSED, DQ_SEPARATE };
DqMode dq_mode() {
  const char* m = std::getenv("GDPA_BWD_DQ");
  if (m == nullptr) return DQ_AUTO;
  if (std::strcmp(m, "fused") == 0) return DQ_FUSED;
  if (std::strcmp(m, "separate") == 0) return DQ_SEPARATE;
  return DQ_AUTO;
}
// A 16-bit dQ needs the fp32 accumulator only when the fused pass reduces
// partial sums of several key blocks; by default that pass runs only when
// every sequence's keys fit one block (dQ then written directly).
bool bwd_acc16(bool grads16, int64_t max_lk) {
  return grads16 && max_lk > gdpa::kBwdBN && dq_mode() == DQ_FUSED;
}

struct BwdLayout {
  size_t order, queues, turns, acc, bytes;
  int64_t nturn;  // turn counters
};
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
// Sizes past kMaxWorkspace (far beyond any GPU's memory) are reported as
// SIZE_MAX: no call can be given that much, and the arithmetic stays in range
// for any argument values.
constexpr int64_t kMaxWorkspace = int64_t(1) << 60;
BwdLayout bwd_layout(int64_t batch, bool jagged, int64_t max_lq, int64_t total_q, int64_t hq, int64_t d,
                     bool acc16) {
  BwdLayout l{};
  if (batch <= 0) return l;
  const __int128 tiles = jagged ? (__int128)total_q / gdpa::kDqTile + batch + 1
                                : (__int128)batch * ((max_lq + gdpa::kDqTile - 1) / gdpa::kDqTile);
  const __int128 turn_bytes = tiles * hq * 4;
  const __int128 acc_bytes = acc16 ? (__int128)total_q * hq * d * 4 : 0;
  if (turn_bytes > kMaxWorkspace || acc_bytes > kMaxWorkspace) {
    l.bytes = SIZE_MAX;
    return l;
  }
  l.nturn = (int64_t)(tiles * hq);
  l.order = 0;
  l.queues = jagged && batch <= gdpa::kSortMax ? align256((size_t)batch * 4) : 0;
  l.turns = l.queues + align256(gdpa::kQWords * 4);
  l.acc = l.turns + align256((size_t)turn_bytes);
  l.bytes = l.acc + (acc16 ? align256((size_t)acc_bytes) : 0);
  return l;
}

// GDPA_DEBUG_CHECKS=1 (read at every call): jagged calls copy cu_seqlens to the
// host, synchronising the caller's stream, and reject device data that the
// kernels would otherwise take on trust.
bool debug_checks() {
  const char* e = std::getenv("GDPA_DEBUG_CHECKS");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

// cu[0] = 0, non-decreasing, cu[batch] = total, every length <= max_len.
gdpa_status_t check_cu_on_host(const int32_t* cu, int32_t batch, int32_t max_len, int64_t total, void* stream) {
  std::vector<int32_t> h((size_t)batch + 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "cu_seqlens check copy");
  if (h[0] != 0 || (int64_t)h[batch] != total) return GDPA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)h[b + 1] - h[b];
    if (len < 0 || len > max_len) return GDPA_ERR_INVALID_ARG;
  }
  return GDPA_OK;
}

gdpa_status_t debug_check_jagged(const int32_t* cu_q, const int32_t* cu_k, const Common& c, void* stream) {
  if (cu_q == nullptr || !debug_checks()) return GDPA_OK;
  gdpa_status_t st = check_cu_on_host(cu_q, c.batch, c.max_lq, c.total_q, stream);
  if (st == GDPA_OK) st = check_cu_on_host(cu_k, c.batch, c.max_lk, c.total_k, stream);
  if (st == GDPA_ERR_INVALID_ARG && debug_log()) std::fprintf(stderr, "[gdpa] invalid cu_seqlens\n");
  return st;
}

// Compute units of the current device (0 if unknown), cached per device.  The
// cache entries are atomics: concurrent callers on other threads may both
// query the attribute, and both store the same value.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  static std::atomic<int> cache[64];
  if (dev >= 0 && dev < 64) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Builds the schedule into the workspace when this is a jagged call that has
// one; *perm and *counters stay nullptr otherwise (index order, one workgroup
// per item).
gdpa_status_t build_schedule(const int32_t* cu_q, const int32_t* cu_k, const Common& c, void* workspace,
                             size_t workspace_bytes, void* stream, const int32_t** perm, int32_t** counters,
                             int32_t* ncu) {
  const int32_t batch = c.batch;
  *perm = nullptr;
  *counters = nullptr;
  *ncu = 0;
  if (cu_q == nullptr) return GDPA_OK;
  const size_t need = schedule_bytes(batch);
  if (need == 0) return GDPA_OK;
  if (workspace == nullptr || workspace_bytes < need) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  int32_t* p = static_cast<int32_t*>(workspace);
  int32_t* cnt = p + batch;
  const gdpa_status_t st = hip_status(
      gdpa::launch_schedule(cu_q, cu_k, batch, c.wl, c.wr, p, cnt, static_cast<hipStream_t>(stream)), "schedule launch");
  if (st != GDPA_OK) return st;
  *perm = p;
  const int n = device_cu_count();
  if (n > 0) {
    *counters = cnt;
    *ncu = n;
  }
  return GDPA_OK;
}

gdpa_status_t run_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* cu_q,
                      const int32_t* cu_k, const Common& c, float scale, float act_param,
                      int32_t qk_dtype, int32_t v_dtype, int32_t out_dtype, float q_descale,
                      float k_descale, void* workspace, size_t workspace_bytes, void* stream,
                      const uint8_t* q_mx = nullptr, const uint8_t* k_mx = nullptr) {
  if (qk_dtype != GDPA_DTYPE_BF16 && qk_dtype != GDPA_DTYPE_FP16 && qk_dtype != GDPA_DTYPE_FP8_E4M3 &&
      qk_dtype != GDPA_DTYPE_MXFP8_E4M3 && qk_dtype != GDPA_DTYPE_MXFP4_E2M1)
    return GDPA_ERR_INVALID_ARG;
  // MXFP8 / MXFP4 Q/K carry their scales in q_mx / k_mx (and only they do)
  const bool mx4 = qk_dtype == GDPA_DTYPE_MXFP4_E2M1;
  const bool mx = qk_dtype == GDPA_DTYPE_MXFP8_E4M3 || mx4;
  if (mx != (q_mx != nullptr || k_mx != nullptr) && !(mx && c.batch == 0)) return GDPA_ERR_INVALID_ARG;
  if (v_dtype != GDPA_DTYPE_BF16 && v_dtype != GDPA_DTYPE_FP16)
    return v_dtype == GDPA_DTYPE_FP8_E4M3 ? GDPA_ERR_UNSUPPORTED : GDPA_ERR_INVALID_ARG;
  const int out_kind = out_kind_of(out_dtype);
  if (out_kind < 0) return GDPA_ERR_INVALID_ARG;
  // bf16 Q/K with bf16 V, fp16 with fp16, or FP8 Q/K with bf16 V (P takes V's type).
  const bool fp8 = qk_dtype == GDPA_DTYPE_FP8_E4M3 || mx;
  const bool f16 = v_dtype == GDPA_DTYPE_FP16;
  if (f16 != (qk_dtype == GDPA_DTYPE_FP16)) return GDPA_ERR_UNSUPPORTED;
  const int in_kind = mx4  ? gdpa::EL_MX4
                      : mx ? gdpa::EL_MX8
                      : fp8 ? gdpa::EL_FP8
                      : f16 ? gdpa::EL_F16
                            : gdpa::EL_BF16;
  if (fp8 && (!std::isfinite(q_descale) || !std::isfinite(k_descale))) return GDPA_ERR_INVALID_ARG;
  if (!fwd_built(in_kind, c.d, c.dv)) return GDPA_ERR_UNSUPPORTED;
  if (c.batch == 0 || c.total_q == 0) return GDPA_OK;
  if (q == nullptr || o == nullptr) return GDPA_ERR_INVALID_ARG;
  if (c.total_k > 0 && (k == nullptr || v == nullptr)) return GDPA_ERR_INVALID_ARG;
  if (mx && (q_mx == nullptr || (c.total_k > 0 && k_mx == nullptr))) return GDPA_ERR_INVALID_ARG;
  const int64_t mblocks = ((int64_t)c.max_lq + gdpa::kFwdBM - 1) / gdpa::kFwdBM;
  if (mblocks == 0) return GDPA_OK;

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.batch = c.batch;
  a.lq_fixed = c.max_lq;
  a.lk_fixed = c.max_lk;
  a.hq = c.hq;
  a.hkv = c.hkv;
  a.group = c.hq / c.hkv;
  a.mblocks = (int32_t)mblocks;
  a.act = make_act(c.act_kind, fp8 ? (double)scale * q_descale * k_descale : (double)scale, act_param);
  a.wl = c.wl;
  a.wr = c.wr;
  a.out_kind = out_kind;
  a.q_mx = q_mx;
  a.k_mx = k_mx;
  // When an output row sums at most kFewTerms products, the bf16 rounding of P
  // no longer averages out; P is then carried as hi + lo (such short rows are
  // bandwidth-bound, so the second MFMA is free).  fp16's 3 extra mantissa
  // bits keep a single word within tolerance.
  a.psplit = !f16 && few_terms(c.max_lk, 1, c) ? 1 : 0;
  if (gdpa::fwd_grid(a) > kMaxGrid) return GDPA_ERR_UNSUPPORTED;
  // The forward kernel addresses one sequence's K and V rows with 32-bit byte offsets.
  if ((int64_t)c.max_lk * c.hkv * std::max(c.d, c.dv) * 2 > INT32_MAX) return GDPA_ERR_UNSUPPORTED;
  int32_t* counters = nullptr;  // the forward keeps one workgroup per item
  int32_t ncu = 0;
  gdpa_status_t sst = debug_check_jagged(cu_q, cu_k, c, stream);
  if (sst != GDPA_OK) return sst;
  sst = build_schedule(cu_q, cu_k, c, workspace, workspace_bytes, stream, &a.perm, &counters, &ncu);
  if (sst != GDPA_OK) return sst;
  if (debug_log())
    std::fprintf(stderr, "[gdpa] fwd B=%d maxLq=%d maxLk=%d Hq=%d Hkv=%d D=%d act=%d in=%d wl=%d wr=%d psplit=%d grid=%lld\n",
                 c.batch, c.max_lq, c.max_lk, c.hq, c.hkv, c.d, c.act_kind, in_kind, c.wl, c.wr,
                 a.psplit, (long long)gdpa::fwd_grid(a));
  return hip_status(gdpa::launch_fwd(a, c.d, c.dv, c.act_kind, in_kind, static_cast<hipStream_t>(stream)),
                    "forward launch");
}

// Polls of a dQ turn wait before it gives up; GDPA_DEBUG_SPIN_LIMIT (read in
// the debug mode only) overrides it, a negative value making every wait give
// up at once (to exercise the error path).
int32_t spin_limit() {
  if (debug_checks()) {
    const char* e = std::getenv("GDPA_DEBUG_SPIN_LIMIT");
    if (e != nullptr && e[0] != '\0') return (int32_t)std::strtol(e, nullptr, 10);
  }
  return 1 << 21;
}

// qd / kd: per-tensor scales of Q and K whose codes are passed as q / k (the
// FP8 backward); S folds both in, dQ and dK the other operand's.  check_only:
// return after the argument checks, before any HIP call.
gdpa_status_t run_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                      void* dv, const int32_t* cu_q, const int32_t* cu_k, const Common& c, float scale,
                      float act_param, int32_t in_dtype, int32_t grad_dtype, void* workspace,
                      size_t workspace_bytes, void* stream, float qd = 1.0f, float kd = 1.0f,
                      bool check_only = false) {
  if (in_dtype == GDPA_DTYPE_FP8_E4M3) return GDPA_ERR_UNSUPPORTED;  // FP8 is forward-only
  if (in_dtype != GDPA_DTYPE_BF16 && in_dtype != GDPA_DTYPE_FP16) return GDPA_ERR_INVALID_ARG;
  if (!bwd_built(in_dtype == GDPA_DTYPE_FP16 ? gdpa::EL_F16 : gdpa::EL_BF16, c.d, c.dv)) return GDPA_ERR_UNSUPPORTED;
  const int out_kind = out_kind_of(grad_dtype);
  if (out_kind < 0) return GDPA_ERR_INVALID_ARG;
  const bool f16 = in_dtype == GDPA_DTYPE_FP16;
  // dq == NULL skips dQ; dk == dv == NULL skips dK and dV; at least one is wanted.
  const bool want_dq = dq != nullptr;
  const bool want_dkv = dk != nullptr;
  if ((dk == nullptr) != (dv == nullptr) || (!want_dq && !want_dkv)) return GDPA_ERR_INVALID_ARG;
  if (c.batch == 0 || (c.total_q == 0 && c.total_k == 0)) return GDPA_OK;
  if (c.total_q > 0 && (q == nullptr || dout == nullptr)) return GDPA_ERR_INVALID_ARG;
  if (c.total_k > 0 && (k == nullptr || v == nullptr)) return GDPA_ERR_INVALID_ARG;
  // The backward kernels address one sequence's rows with 32-bit byte offsets.
  if ((int64_t)c.max_lq * c.hq * c.d * 2 > INT32_MAX || (int64_t)c.max_lk * c.hkv * c.d * 2 > INT32_MAX)
    return GDPA_ERR_UNSUPPORTED;
  const int64_t mblocks = ((int64_t)c.max_lq + gdpa::kBwdBM - 1) / gdpa::kBwdBM;
  const int64_t nblocks = std::max<int64_t>(1, ((int64_t)c.max_lk + gdpa::kBwdBN - 1) / gdpa::kBwdBN);
  if (gdpa::pair_grid(c.batch, c.hkv, (long)(c.hq / c.hkv) * mblocks) > kMaxGrid ||
      gdpa::pair_grid(c.batch, c.hkv, nblocks) > kMaxGrid)
    return GDPA_ERR_UNSUPPORTED;
  const bool jagged = cu_q != nullptr;
  const BwdLayout lay =
      bwd_layout(c.batch, jagged, c.max_lq, c.total_q, c.hq, c.d, bwd_acc16(out_kind != gdpa::OUT_F32, c.max_lk));
  if (workspace == nullptr || workspace_bytes < lay.bytes) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  if (check_only) return GDPA_OK;

  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.batch = c.batch;
  a.lq_fixed = c.max_lq;
  a.lk_fixed = c.max_lk;
  a.hq = c.hq;
  a.hkv = c.hkv;
  a.group = c.hq / c.hkv;
  a.mblocks = (int32_t)mblocks;
  a.nblocks = (int32_t)nblocks;
  a.act = make_act(c.act_kind, (double)scale * qd * kd, act_param);
  // dQ = scale dS K and dK = scale dS^T Q: with K (Q) given as codes of
  // per-tensor scale kd (qd), each takes scale times that scale
  a.dq_scale = (float)((double)scale * kd);
  a.dk_scale = (float)((double)scale * qd);
  a.wl = c.wl;
  a.wr = c.wr;
  a.out_kind = out_kind;
  a.dsplit = !f16 && few_terms(c.max_lk, 1, c) ? 1 : 0;
  a.kvsplit = !f16 && few_terms(c.max_lq, a.group, c) ? 1 : 0;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.qstate = reinterpret_cast<int32_t*>(ws + lay.queues);
  a.turn = reinterpret_cast<int32_t*>(ws + lay.turns);
  a.dq_acc = out_kind == gdpa::OUT_F32 ? static_cast<float*>(dq) : reinterpret_cast<float*>(ws + lay.acc);
  a.mt_fixed = (int32_t)(((int64_t)c.max_lq + gdpa::kDqTile - 1) / gdpa::kDqTile);
  a.spin_limit = spin_limit();
  a.ncu = device_cu_count();
  // dQ comes from the dK/dV pass (five products; partial sums of a query tile
  // from several key blocks meet in an ordered fp32 reduction) or from a
  // separate kernel that recomputes S and dP (seven products, no reduction).
  // Each key block that reaches a query tile adds a read and a write of the
  // tile's fp32 partial sums, which cost more than the recomputation once a
  // tile has several contributors, so the fused pass is the default only when
  // every sequence's keys fit one block; GDPA_BWD_DQ=fused|separate overrides.
  // The fused pass also needs all three gradients, at most one of the two
  // word splits and a sequence's fp32 dQ rows within 32-bit offsets.
  const DqMode mode = dq_mode();
  const bool force_fused = mode == DQ_FUSED;
  const bool force_separate = mode == DQ_SEPARATE;
  const bool fused = want_dq && want_dkv && c.d == c.dv && !(a.dsplit && a.kvsplit) && a.ncu > 0 && !force_separate &&
                     (force_fused || c.max_lk <= gdpa::kBwdBN) &&
                     ((int64_t)c.max_lq + gdpa::kDqTile) * c.hq * c.d * 4 <= INT32_MAX;
  gdpa_status_t sst = debug_check_jagged(cu_q, cu_k, c, stream);
  if (sst != GDPA_OK) return sst;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (jagged && c.batch <= gdpa::kSortMax) {
    // costliest-first order; also zeroes the first queue words
    sst = hip_status(gdpa::launch_schedule(cu_q, cu_k, c.batch, c.wl, c.wr,
                                           reinterpret_cast<int32_t*>(ws + lay.order), a.qstate, hs),
                     "schedule launch");
    if (sst != GDPA_OK) return sst;
    a.perm = reinterpret_cast<const int32_t*>(ws + lay.order);
  }
  if (fused) {
    // queue heads and owners, the error flag and the turn counters start at zero
    sst = hip_status(gdpa::launch_zero(a.qstate, (long)((lay.acc - lay.queues) / 4), hs), "workspace clear");
    if (sst != GDPA_OK) return sst;
  } else if (a.perm != nullptr && a.ncu > 0) {
    a.counters = a.qstate;  // the dK/dV kernel's work queues (zeroed by the schedule)
  }
  if (debug_log())
    std::fprintf(stderr, "[gdpa] bwd B=%d maxLq=%d maxLk=%d Hq=%d Hkv=%d D=%d act=%d wl=%d wr=%d fused=%d\n", c.batch,
                 c.max_lq, c.max_lk, c.hq, c.hkv, c.d, c.act_kind, c.wl, c.wr, (int)fused);
  sst = hip_status(gdpa::launch_bwd(a, c.d, c.act_kind, f16 ? gdpa::EL_F16 : gdpa::EL_BF16, want_dq, want_dkv, fused,
                                    hs),
                   "backward launch");
  if (sst != GDPA_OK || !fused || !debug_checks()) return sst;
  // debug mode: wait for the kernel and report a dQ turn wait that gave up
  int32_t flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, a.qstate + gdpa::kQErr, sizeof(flag), hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_status(e, "wait-flag readback");
  return flag != 0 ? GDPA_ERR_DEVICE_WAIT : GDPA_OK;
}

}  // namespace

// ------------------------------------------------ allocation-free backward
// The backward's workspace for callers that cannot allocate device memory:
// one copy of this array per GPU, alive until the process ends.  Host code
// uses only the address looked up per device (the array's name on the host
// is a stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[GDPA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Address of the current device's scratch array (looked up once per device,
// with that device current).
gdpa_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return GDPA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "scratch address");
    if (p == nullptr) return GDPA_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return GDPA_OK;
}
}  // namespace

extern "C" {

gdpa_status_t gdpa_fwd(const void* q, const void* k, const void* v, void* o, int32_t batch, int32_t seqlen_q,
                       int32_t seqlen_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v, float scale,
                       int32_t mask, int32_t window_left, int32_t window_right, int32_t act, float act_param,
                       int32_t qk_dtype, int32_t v_dtype, int32_t out_dtype, float q_descale, float k_descale,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Common c;
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return GDPA_ERR_INVALID_ARG;
  gdpa_status_t st = check_common(batch, seqlen_q, seqlen_k, (int64_t)batch * seqlen_q, (int64_t)batch * seqlen_k,
                                  num_heads_q, num_heads_kv, head_dim, head_dim_v, scale, mask, window_left, window_right, act,
                                  act_param, &c);
  if (st != GDPA_OK) return st;
  return run_fwd(q, k, v, o, nullptr, nullptr, c, scale, act_param, qk_dtype, v_dtype, out_dtype, q_descale,
                 k_descale, workspace, workspace_bytes, stream);
}

gdpa_status_t gdpa_varlen_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int64_t total_q, int64_t total_k, int32_t num_heads_q, int32_t num_heads_kv,
                              int32_t head_dim, int32_t head_dim_v, float scale, int32_t mask, int32_t window_left,
                       int32_t window_right,
                              int32_t act, float act_param, int32_t qk_dtype, int32_t v_dtype, int32_t out_dtype,
                              float q_descale, float k_descale, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Common c;
  gdpa_status_t st = check_common(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                  head_dim, head_dim_v, scale, mask, window_left, window_right, act, act_param, &c);
  if (st != GDPA_OK) return st;
  if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return GDPA_ERR_INVALID_ARG;
  return run_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, c, scale, act_param, qk_dtype, v_dtype, out_dtype,
                 q_descale, k_descale, workspace, workspace_bytes, stream);
}

namespace {
gdpa_status_t varlen_fwd_mx(int32_t qk_dtype, const void* q, const void* q_scale, const void* k,
                            const void* k_scale, const void* v, void* o, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int64_t total_q, int64_t total_k, int32_t num_heads_q, int32_t num_heads_kv,
                            int32_t head_dim, float scale, int32_t mask, int32_t window_left, int32_t window_right,
                            int32_t act, float act_param, int32_t out_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  Common c;
  gdpa_status_t st = check_common(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                  head_dim, head_dim, scale, mask, window_left, window_right, act, act_param, &c);
  if (st != GDPA_OK) return st;
  if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return GDPA_ERR_INVALID_ARG;
  if (batch > 0 && total_q > 0 && (q_scale == nullptr || (total_k > 0 && k_scale == nullptr)))
    return GDPA_ERR_INVALID_ARG;
  return run_fwd(q, k, v, o, cu_seqlens_q, cu_seqlens_k, c, scale, act_param, qk_dtype, GDPA_DTYPE_BF16,
                 out_dtype, 1.0f, 1.0f, workspace, workspace_bytes, stream, static_cast<const uint8_t*>(q_scale),
                 static_cast<const uint8_t*>(k_scale));
}
}  // namespace

gdpa_status_t gdpa_varlen_fwd_mxfp8(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                    const void* v, void* o, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q,
                                    int64_t total_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                    int32_t act, float act_param, int32_t out_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return varlen_fwd_mx(GDPA_DTYPE_MXFP8_E4M3, q, q_scale, k, k_scale, v, o, cu_seqlens_q, cu_seqlens_k, batch,
                       max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv, head_dim, scale,
                       mask, window_left, window_right, act, act_param, out_dtype, workspace, workspace_bytes, stream);
}

gdpa_status_t gdpa_varlen_fwd_mxfp4(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                    const void* v, void* o, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q,
                                    int64_t total_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    float scale, int32_t mask, int32_t window_left, int32_t window_right,
                                    int32_t act, float act_param, int32_t out_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return varlen_fwd_mx(GDPA_DTYPE_MXFP4_E2M1, q, q_scale, k, k_scale, v, o, cu_seqlens_q, cu_seqlens_k, batch,
                       max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv, head_dim, scale,
                       mask, window_left, window_right, act, act_param, out_dtype, workspace, workspace_bytes, stream);
}

gdpa_status_t gdpa_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                       int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q, int32_t num_heads_kv,
                       int32_t head_dim, int32_t head_dim_v, float scale, int32_t mask, int32_t window_left,
                       int32_t window_right,
                       int32_t act, float act_param, int32_t in_dtype, int32_t grad_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Common c;
  if (batch < 0 || seqlen_q < 0 || seqlen_k < 0) return GDPA_ERR_INVALID_ARG;
  gdpa_status_t st = check_common(batch, seqlen_q, seqlen_k, (int64_t)batch * seqlen_q, (int64_t)batch * seqlen_k,
                                  num_heads_q, num_heads_kv, head_dim, head_dim_v, scale, mask, window_left, window_right, act,
                                  act_param, &c);
  if (st != GDPA_OK) return st;
  return run_bwd(q, k, v, dout, dq, dk, dv, nullptr, nullptr, c, scale, act_param, in_dtype, grad_dtype, workspace,
                 workspace_bytes, stream);
}

gdpa_status_t gdpa_varlen_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                              void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q, int64_t total_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, int32_t head_dim_v, float scale, int32_t mask,
                              int32_t window_left, int32_t window_right, int32_t act, float act_param,
                              int32_t in_dtype, int32_t grad_dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Common c;
  gdpa_status_t st = check_common(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                  head_dim, head_dim_v, scale, mask, window_left, window_right, act, act_param, &c);
  if (st != GDPA_OK) return st;
  if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return GDPA_ERR_INVALID_ARG;
  return run_bwd(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, c, scale, act_param, in_dtype, grad_dtype,
                 workspace, workspace_bytes, stream);
}

gdpa_status_t gdpa_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* dout, void* dq,
                                      void* dk, void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q,
                                      int64_t total_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                      int32_t head_dim_v, float scale, int32_t mask, int32_t window_left,
                                      int32_t window_right, int32_t act, float act_param, int32_t in_dtype,
                                      int32_t grad_dtype, void* stream) {
  Common c;
  gdpa_status_t st = check_common(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                  head_dim, head_dim_v, scale, mask, window_left, window_right, act, act_param, &c);
  if (st != GDPA_OK) return st;
  const size_t need = gdpa_varlen_bwd_workspace_size(batch, max_seqlen_q, max_seqlen_k, total_q, num_heads_q,
                                                     num_heads_kv, head_dim, grad_dtype);
  if (need > GDPA_NOALLOC_SCRATCH_BYTES) return GDPA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != GDPA_OK) return st;
  }
  return gdpa_varlen_bwd(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                         total_q, total_k, num_heads_q, num_heads_kv, head_dim, head_dim_v, scale, mask, window_left,
                         window_right, act, act_param, in_dtype, grad_dtype, ws,
                         need > 0 ? (size_t)GDPA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t gdpa_fwd_workspace_size(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }
size_t gdpa_varlen_fwd_workspace_size(int32_t batch, int32_t, int32_t, int32_t, int32_t, int32_t) {
  return schedule_bytes(batch);
}
size_t gdpa_bwd_workspace_size(int32_t batch, int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads_q, int32_t,
                               int32_t head_dim, int32_t grad_dtype) {
  if (batch <= 0 || seqlen_q < 0 || num_heads_q <= 0 || head_dim <= 0) return 0;
  return bwd_layout(batch, false, seqlen_q, (int64_t)batch * seqlen_q, num_heads_q, head_dim,
                    bwd_acc16(grad_dtype != GDPA_DTYPE_FP32, seqlen_k))
      .bytes;
}
size_t gdpa_varlen_bwd_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q,
                                      int32_t num_heads_q, int32_t, int32_t head_dim, int32_t grad_dtype) {
  if (batch <= 0 || max_seqlen_q < 0 || total_q < 0 || num_heads_q <= 0 || head_dim <= 0) return 0;
  return bwd_layout(batch, true, max_seqlen_q, total_q, num_heads_q, head_dim,
                    bwd_acc16(grad_dtype != GDPA_DTYPE_FP32, max_seqlen_k))
      .bytes;
}

namespace {
// Workspace of the backward from 8- or 4-bit Q/K: the 16-bit backward's, then
// bf16 copies of Q and K; SIZE_MAX past kMaxWorkspace.
struct LowpLayout {
  size_t base, qdec, kdec, bytes;
};
LowpLayout lowp_layout(int32_t batch, int32_t max_lq, int32_t max_lk, int64_t total_q, int64_t total_k, int32_t hq,
                       int32_t hkv, int32_t d, int32_t grad_dtype) {
  LowpLayout l{};
  l.base = gdpa_varlen_bwd_workspace_size(batch, max_lq, max_lk, total_q, hq, hkv, d, grad_dtype);
  const __int128 qb = (__int128)std::max<int64_t>(total_q, 0) * hq * d * 2;
  const __int128 kb = (__int128)std::max<int64_t>(total_k, 0) * hkv * d * 2;
  if (l.base == SIZE_MAX || qb > kMaxWorkspace || kb > kMaxWorkspace) {
    l.bytes = SIZE_MAX;
    return l;
  }
  l.qdec = align256(l.base);
  l.kdec = l.qdec + align256((size_t)qb);
  l.bytes = l.kdec + align256((size_t)kb);
  return l;
}
}  // namespace

size_t gdpa_varlen_bwd_lowp_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                           int64_t total_q, int64_t total_k, int32_t num_heads_q,
                                           int32_t num_heads_kv, int32_t head_dim, int32_t qk_dtype,
                                           int32_t grad_dtype) {
  (void)qk_dtype;
  if (batch <= 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0 || num_heads_q <= 0 || num_heads_kv <= 0 ||
      head_dim <= 0)
    return 0;
  return lowp_layout(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv, head_dim,
                     grad_dtype)
      .bytes;
}

gdpa_status_t gdpa_varlen_bwd_lowp(const void* q, const void* q_scale, const void* k, const void* k_scale,
                                   const void* v, const void* dout, void* dq, void* dk, void* dv,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                                   int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q, int64_t total_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim, float scale,
                                   int32_t mask, int32_t window_left, int32_t window_right, int32_t act,
                                   float act_param, int32_t qk_dtype, float q_descale, float k_descale,
                                   int32_t grad_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  Common c;
  gdpa_status_t st = check_common(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                  head_dim, head_dim, scale, mask, window_left, window_right, act, act_param, &c);
  if (st != GDPA_OK) return st;
  int in_kind = -1;
  if (qk_dtype == GDPA_DTYPE_FP8_E4M3) in_kind = gdpa::EL_FP8;
  if (qk_dtype == GDPA_DTYPE_MXFP8_E4M3) in_kind = gdpa::EL_MX8;
  if (qk_dtype == GDPA_DTYPE_MXFP4_E2M1) in_kind = gdpa::EL_MX4;
  if (in_kind < 0) return GDPA_ERR_INVALID_ARG;
  // the head dims the forward of the format is built for
  if (!fwd_built(in_kind, c.d, c.dv) || c.d % 32 != 0) return GDPA_ERR_UNSUPPORTED;
  const bool mx = in_kind != gdpa::EL_FP8;
  // FP8 codes carry per-tensor scales, the MX formats block scales (and only they)
  if (!mx && (q_scale != nullptr || k_scale != nullptr)) return GDPA_ERR_INVALID_ARG;
  if (!mx && (!std::isfinite(q_descale) || !std::isfinite(k_descale))) return GDPA_ERR_INVALID_ARG;
  if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr)) return GDPA_ERR_INVALID_ARG;
  if (mx && batch > 0 && ((total_q > 0 && q_scale == nullptr) || (total_k > 0 && k_scale == nullptr)))
    return GDPA_ERR_INVALID_ARG;
  const LowpLayout lay = lowp_layout(batch, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads_q, num_heads_kv,
                                     head_dim, grad_dtype);
  const float qd = mx ? 1.0f : q_descale, kd = mx ? 1.0f : k_descale;
  // every check of the 16-bit backward (q and k stand in for their decoded
  // copies), then the workspace with the copies, before any launch
  st = run_bwd(q, k, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, c, scale, act_param, GDPA_DTYPE_BF16,
               grad_dtype, workspace, lay.base, stream, qd, kd, /*check_only=*/true);
  const bool work = batch > 0 && (total_q > 0 || total_k > 0);
  if (st != GDPA_OK || !work) return st;
  if (workspace == nullptr || lay.bytes == SIZE_MAX || workspace_bytes < lay.bytes)
    return GDPA_ERR_WORKSPACE_TOO_SMALL;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const void* qdec = total_q > 0 ? ws + lay.qdec : nullptr;
  const void* kdec = total_k > 0 ? ws + lay.kdec : nullptr;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = hip_status(gdpa::launch_decode_bf16(static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(q_scale),
                                           reinterpret_cast<uint16_t*>(ws + lay.qdec), (long)total_q * num_heads_q,
                                           head_dim, in_kind, hs),
                  "q decode launch");
  if (st != GDPA_OK) return st;
  st = hip_status(gdpa::launch_decode_bf16(static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(k_scale),
                                           reinterpret_cast<uint16_t*>(ws + lay.kdec), (long)total_k * num_heads_kv,
                                           head_dim, in_kind, hs),
                  "k decode launch");
  if (st != GDPA_OK) return st;
  return run_bwd(qdec, kdec, v, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, c, scale, act_param, GDPA_DTYPE_BF16,
                 grad_dtype, workspace, lay.base, stream, qd, kd);
}

const char* gdpa_status_string(gdpa_status_t s) {
  // read as the int the C caller passed (a value outside the enumeration
  // would be undefined behaviour if loaded as the C++ enum type)
  int code = 0;
  std::memcpy(&code, &s, sizeof(code));
  switch (code) {
    case GDPA_OK: return "GDPA_OK";
    case GDPA_ERR_INVALID_ARG: return "GDPA_ERR_INVALID_ARG";
    case GDPA_ERR_UNSUPPORTED: return "GDPA_ERR_UNSUPPORTED";
    case GDPA_ERR_WORKSPACE_TOO_SMALL: return "GDPA_ERR_WORKSPACE_TOO_SMALL";
    case GDPA_ERR_HIP: return "GDPA_ERR_HIP";
    case GDPA_ERR_DEVICE_WAIT: return "GDPA_ERR_DEVICE_WAIT";
    default: return "GDPA_ERR_UNKNOWN";
  }
}

int32_t gdpa_abi_version(void) { return GDPA_ABI_VERSION; }

}  // extern "C"
