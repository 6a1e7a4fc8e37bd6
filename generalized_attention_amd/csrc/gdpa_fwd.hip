// GDPA forward kernel for gfx950.
//
// Computes O = M .* act(scale * Q K^T) V per (sequence, query head): the GDPA
// definition of the GDPA README (intro; softmax replaced by an activation, no
// normaliser).  Because nothing is normalised, every KV tile adds an exact
// partial sum to O: there is no running maximum, no rescaling and no final
// division, unlike softmax flash attention.
//
// Work decomposition: one workgroup of NW waves per (sequence, query head,
// BM-row query block), BM = 32 * NQB * NW; wave w owns NQB blocks of 32 query
// rows.  Per KV tile of BN = 8192/D keys:
//   * K and V are copied HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging), row-major with 16-byte chunks XOR-swizzled by the row index;
//     tiles are double-buffered, the next tile's copy is in flight while the
//     current tile is computed;
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (Q^T stays in registers as the B
//     operand for the whole loop; each K operand read from LDS feeds the NQB
//     query blocks), then scale, mask and activation in registers;
//   * P^T is packed to bf16 straight from the accumulators and is the B
//     operand of O^T += V^T P^T.  The V^T operand comes from the row-major V
//     tile through ds_read_b64_tr_b16, whose 16-lane transpose hands each lane
//     4 consecutive keys of one head-dim column, in exactly the key order of
//     the accumulator rows; each V^T operand also feeds the NQB query blocks.
// Query blocks are dispatched last-block-first: for self-attention the late
// blocks exist only in long sequences and carry the most KV tiles, so the
// hardware dispatcher sees roughly longest-processing-time-first order (the
// README's "Features" names load-balanced tile scheduling for jagged inputs).
#include "gdpa_common.hpp"
#include "gdpa_kernels.hpp"

namespace gdpa {

template <int D, int ACT, bool FP8, bool PSPLIT, int NW, int NQB>
struct FwdKernel {
  static constexpr int BM = 32 * NQB * NW;
  static constexpr int BN = 8192 / D;     // keys per KV tile
  static constexpr int NKB = BN / 32;     // 32-key blocks per tile
  static constexpr int KS = D / 16;       // k-steps of Q K^T
  static constexpr int NDB = D / 32;      // 32-row blocks of O^T
  static constexpr int KROWB = FP8 ? D : 2 * D;
  static constexpr int VROWB = 2 * D;
  static constexpr int NQR = FP8 ? 1 : KS;   // bf16 Q registers per query block
  static constexpr int NQR8 = FP8 ? KS : 1;  // FP8 Q registers per query block

  // One KV tile for this wave: S^T = K Q^T, P = act(S) (masked to each
  // lane's [jlo, jhi] when MASK), O^T += V^T P^T.  qact: query blocks with at
  // least one valid row.
  template <bool MASK>
  static __device__ __forceinline__ void tile(const uint8_t* kl, const uint8_t* vl, const u32x4 (*qreg)[NQR],
                                              const u32x2 (*qreg8)[NQR8], f32x16 (*oacc)[NDB], int lane, int n0,
                                              const int* jlo, const int* jhi, int qact, const FwdArgs& a) {
    const int hf = lane >> 5;
    f32x16 sacc[NQB][NKB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[qb][kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + (lane & 31);
        if constexpr (FP8) {
          const u32x2 aop = *reinterpret_cast<const u32x2*>(kl + lds_off<KROWB>(row, s) + hf * 8);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            if (qb < qact) sacc[qb][kb] = mfma_fp8(aop, qreg8[qb][s], sacc[qb][kb]);
        } else {
          const u32x4 aop = *reinterpret_cast<const u32x4*>(kl + lds_off<KROWB>(row, 2 * s + hf));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            if (qb < qact) sacc[qb][kb] = mfma_bf16(aop, qreg[qb][s], sacc[qb][kb]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // V^T operands of this 32-key block, read (transposed) from the row-major
      // V tile before the activation so the LDS latency hides behind it.
      bf16x8 vop[2][NDB];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < NDB; ++db) vop[t][db] = tr_operand<VROWB>(vl, kb * 32 + 16 * t, db * 32, lane);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (qb >= qact) continue;
        // allowed keys of this lane relative to the block's first key for this lane
        const int base = n0 + kb * 32 + hf * 4;
        const int lo = jlo[qb] - base, hi = jhi[qb] - base;
        u32x4 phi[2], plo[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * t + 2 * w + u;
              float v = Act<ACT>::f(sacc[qb][kb][r], a.act);
              if constexpr (MASK) v = in_range(r, lo, hi) ? v : 0.0f;
              y[u] = v;
            }
            const uint32_t hi2 = pack_bf16x2(y[0], y[1]);
            phi[t][w] = hi2;
            if constexpr (PSPLIT) plo[t][w] = split_lo(y[0], y[1], hi2);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][db], __builtin_bit_cast(bf16x8, phi[t]),
                                                                   oacc[qb][db], 0, 0, 0);
            if constexpr (PSPLIT)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][db], __builtin_bit_cast(bf16x8, plo[t]),
                                                                     oacc[qb][db], 0, 0, 0);
          }
        }
      }
    }
  }
};

template <int D, int ACT, bool FP8, bool PSPLIT, int NW, int NQB>
__global__ __launch_bounds__(64 * NW) void gdpa_fwd_kernel(const FwdArgs a) {
  using K = FwdKernel<D, ACT, FP8, PSPLIT, NW, NQB>;
  constexpr int BM = K::BM, BN = K::BN, KS = K::KS, NDB = K::NDB;
  constexpr int KBYTES = BN * K::KROWB, VBYTES = BN * K::VROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[VBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // One work item: sequence b, KV head g, query head h, query block m.
  auto process = [&](int b, int g, int h, int m) __attribute__((always_inline)) {
  int qs, lq, ks, lk;
  if (a.cu_q != nullptr) {
    qs = a.cu_q[b];
    lq = a.cu_q[b + 1] - qs;
    ks = a.cu_k[b];
    lk = a.cu_k[b + 1] - ks;
  } else {
    qs = b * a.lq_fixed;
    lq = a.lq_fixed;
    ks = b * a.lk_fixed;
    lk = a.lk_fixed;
  }
  const int row0 = m * BM;
  if (row0 >= lq) return;
  const int off = lk - lq;  // bottom-right alignment of masks
  const int rlast = min(row0 + BM, lq) - 1;
  int j_lo = 0, j_hi = lk;
  if (a.wl >= 0) j_lo = max(0, row0 + off - a.wl);
  if (a.wr >= 0) j_hi = min(lk, rlast + off + a.wr + 1);
  const int nb_begin = j_lo / BN;
  const int nb_end = (j_hi > j_lo) ? (j_hi + BN - 1) / BN : nb_begin;

  const int q0w = row0 + wave * 32 * NQB;  // first query row of this wave
  const bool wave_active = q0w < lq;
  const int qmax_w = min(q0w + 32 * NQB - 1, lq - 1);
  const int qact = min(NQB, (lq - q0w + 31) / 32);  // query blocks with valid rows
  const int hf = lane >> 5;
  int qi[NQB], jlo[NQB], jhi[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    qi[qb] = q0w + qb * 32 + (lane & 31);
    // keys this lane's query may see: [jlo, jhi]
    jlo[qb] = a.wl >= 0 ? qi[qb] + off - a.wl : 0;
    jhi[qb] = min(lk - 1, a.wr >= 0 ? qi[qb] + off + a.wr : lk - 1);
  }

  // Q^T as the B operand of S^T = K Q^T: lane holds query qi, 8 head-dim values per k-step.
  const long q_ld = (long)a.hq * D;
  u32x4 qreg[NQB][K::NQR];
  u32x2 qreg8[NQB][K::NQR8];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const long qrow = (long)(qs + min(qi[qb], lq - 1)) * q_ld + h * D + hf * 8;
    if constexpr (FP8) {
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qrow;
#pragma unroll
      for (int s = 0; s < KS; ++s) qreg8[qb][s] = load8_or_zero(qp + s * 16, qi[qb] < lq);
    } else {
      const __bf16* qp = static_cast<const __bf16*>(a.q) + qrow;
#pragma unroll
      for (int s = 0; s < KS; ++s) qreg[qb][s] = load16_or_zero(qp + s * 16, qi[qb] < lq);
    }
  }

  f32x16 oacc[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[qb][i] = f32x16{};

  const int esz = FP8 ? 1 : 2;
  const long kv_ld = (long)a.hkv * D;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + ((long)ks * kv_ld + g * D) * esz;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + ((long)ks * kv_ld + g * D) * 2;

  // Byte ranges of this sequence's K and V rows (all KV heads), addressed by
  // 32-bit offsets; the host keeps them below 2^31.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, lk * (int)kv_ld * esz);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, lk * (int)kv_ld * 2);
  auto stage = [&](int nb, uint8_t* kl, uint8_t* vl) {
    const int n0 = nb * BN;
    stage_tile_buf<BN, K::KROWB, NW>(krs, n0 * (int)kv_ld * esz, (int)kv_ld * esz, lk - n0, kl, wave, lane);
    stage_tile_buf<BN, K::VROWB, NW>(vrs, n0 * (int)kv_ld * 2, (int)kv_ld * 2, lk - n0, vl, wave, lane);
  };
  // One tile of math for this wave; the mask is applied only where the
  // window cuts the tile or the tile runs past the last key.
  auto compute = [&](int nb, const uint8_t* kl, const uint8_t* vl) {
    const int n0 = nb * BN;
    bool empty = false, full = n0 + BN <= lk;
    if (a.wr >= 0) {
      empty |= n0 > qmax_w + off + a.wr;
      full &= n0 + BN - 1 <= q0w + off + a.wr;
    }
    if (a.wl >= 0) {
      empty |= n0 + BN - 1 < q0w + off - a.wl;
      full &= n0 >= qmax_w + off - a.wl;
    }
    if (!wave_active || empty) return;
    if (full)
      K::template tile<false>(kl, vl, qreg, qreg8, oacc, lane, n0, jlo, jhi, qact, a);
    else
      K::template tile<true>(kl, vl, qreg, qreg8, oacc, lane, n0, jlo, jhi, qact, a);
  };

  if (nb_begin < nb_end) stage(nb_begin, k_lds0, v_lds0);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): tile copy landed
  __syncthreads();
  for (int nb = nb_begin; nb < nb_end; nb += 2) {
    if (nb + 1 < nb_end) stage(nb + 1, k_lds1, v_lds1);
    compute(nb, k_lds0, v_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nb + 1 >= nb_end) break;
    if (nb + 2 < nb_end) stage(nb + 2, k_lds0, v_lds0);
    compute(nb + 1, k_lds1, v_lds1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: lane stores 4 consecutive head-dim values per register group
  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    if (qi[qb] >= lq) continue;
    const long orow = ((long)(qs + qi[qb]) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float ps = a.act.pscale;
        const float o0 = oacc[qb][db][4 * i4] * ps, o1 = oacc[qb][db][4 * i4 + 1] * ps;
        const float o2 = oacc[qb][db][4 * i4 + 2] * ps, o3 = oacc[qb][db][4 * i4 + 3] * ps;
        if (a.out_f32)
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d) = f32x4{o0, o1, o2, o3};
        else
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      }
    }
  }
  };

  // Block -> work item: (sequence, KV head) pair on one XCD, longest
  // sequences first; within a pair, query blocks run last-first.
  WorkItem w;
  if (!map_work(blockIdx.x, a.batch, a.hkv, a.group * a.mblocks, a.perm, w)) return;
  process(w.b, w.g, w.g * a.group + w.rest / a.mblocks, a.mblocks - 1 - w.rest % a.mblocks);
}

template <int D, bool FP8>
static hipError_t launch_fwd_d(const FwdArgs& a, int act_kind, hipStream_t stream) {
  dim3 g((unsigned)fwd_grid(a)), blk(64 * kFwdNW);
  switch (act_kind) {
#define GDPA_FWD_CASE(K)                                                                                  \
  case K:                                                                                                 \
    if (a.psplit)                                                                                         \
      hipLaunchKernelGGL((gdpa_fwd_kernel<D, K, FP8, true, kFwdNW, kFwdNQB>), g, blk, 0, stream, a);      \
    else                                                                                                  \
      hipLaunchKernelGGL((gdpa_fwd_kernel<D, K, FP8, false, kFwdNW, kFwdNQB>), g, blk, 0, stream, a);     \
    break;
    GDPA_FWD_CASE(ACT_IDENTITY)
    GDPA_FWD_CASE(ACT_GELU)
    GDPA_FWD_CASE(ACT_GELU_TANH)
    GDPA_FWD_CASE(ACT_RELU)
    GDPA_FWD_CASE(ACT_RELU2)
    GDPA_FWD_CASE(ACT_LEAKY)
    GDPA_FWD_CASE(ACT_SILU)
    GDPA_FWD_CASE(ACT_HARDSWISH)
#undef GDPA_FWD_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int act_kind, bool fp8, hipStream_t stream) {
  if (head_dim == 64) return fp8 ? launch_fwd_d<64, true>(a, act_kind, stream) : launch_fwd_d<64, false>(a, act_kind, stream);
  if (head_dim == 128) return fp8 ? launch_fwd_d<128, true>(a, act_kind, stream) : launch_fwd_d<128, false>(a, act_kind, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdpa
