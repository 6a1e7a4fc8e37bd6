// Kernel argument blocks and host-side launchers of the GDPA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdpa {

// Activation kinds after folding the enum aliases (FAST_GELU*, GELU_TANH -> GELU_TANH;
// FAST_SILU -> SILU).  Values match gdpa_act_t.
enum ActKind : int {
  ACT_IDENTITY = 0,
  ACT_GELU = 1,
  ACT_GELU_TANH = 2,
  ACT_RELU = 5,
  ACT_RELU2 = 6,
  ACT_LEAKY = 7,
  ACT_SILU = 8,
  ACT_HARDSWISH = 10,
};


// Activation constants with the score scale folded in (computed on the host).
// With c = scale (times the FP8 descales) and s the raw dot product q.k, the
// kernels evaluate y(s) such that act(c s) = pscale * y(s), and d(s) =
// act'(c s); the chain-rule factor c of dQ and dK is applied once, as gscale,
// to the accumulators.  k0, k1, a0, a1 are per-activation (see gdpa_common.hpp).
struct ActConsts {
  float k0, k1, a0, a1;
  float alpha;    // LeakyReLU slope
  float pscale;   // act(c s) = pscale * y(s)
  float gscale;   // = c
};

// One forward launch.  Sequence b of a jagged batch owns query rows
// cu_q[b]..cu_q[b+1]-1 and key rows cu_k[b]..cu_k[b+1]-1; with cu_q == nullptr
// the batch is fixed-length (lq_fixed / lk_fixed rows per sequence).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t lq_fixed;
  int32_t lk_fixed;
  int32_t hq;
  int32_t hkv;
  int32_t group;      // hq / hkv
  int32_t mblocks;    // ceil(max_seqlen_q / 128)
  ActConsts act;      // activation constants (c = scale * q_descale * k_descale)
  int32_t wl;         // window left  (-1: unbounded)
  int32_t wr;         // window right (-1: unbounded)
  int32_t out_f32;    // 1: fp32 output, 0: bf16
  int32_t psplit;     // 1: P carried as a bf16 hi/lo pair (two MFMAs for P V)
};

// One backward launch (both kernels take the same block).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch;
  int32_t lq_fixed;
  int32_t lk_fixed;
  int32_t hq;
  int32_t hkv;
  int32_t group;
  int32_t mblocks;    // dQ kernel: ceil(max_seqlen_q / 128)
  int32_t nblocks;    // dK/dV kernel: ceil(max_seqlen_k / 128)
  ActConsts act;      // activation constants (c = scale)
  int32_t wl;
  int32_t wr;
  int32_t out_f32;
  int32_t dsplit;     // 1: dS carried as a bf16 hi/lo pair in dQ = dS K
  int32_t kvsplit;    // 1: P and dS carried as bf16 hi/lo pairs in dV, dK
};

// Forward workgroup shape: kFwdNW waves, each owning kFwdNQB blocks of 32 query rows.
constexpr int kFwdNW = 4, kFwdNQB = 1;
constexpr int kFwdBM = 32 * kFwdNW * kFwdNQB;
// XCDs per MI355X; workgroup ids are dealt to them round-robin.
constexpr int kNumXcd = 8;

// Forward grid: (sequence, KV head) pairs rounded up to a multiple of the XCD
// count, times query heads per KV head, times query blocks.
inline long fwd_grid(const FwdArgs& a) {
  const long pairs = ((long)a.batch * a.hkv + kNumXcd - 1) / kNumXcd * kNumXcd;
  return pairs * a.group * a.mblocks;
}
// Backward: dK/dV blocks cover 128 key rows, dQ blocks 128 query rows.
constexpr int kBwdBN = 128;
constexpr int kBwdBM = 128;

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int act_kind, bool fp8, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int head_dim, int act_kind, bool want_dq, bool want_dkv,
                      hipStream_t stream);

}  // namespace gdpa
