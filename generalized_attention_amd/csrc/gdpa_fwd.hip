// GDPA forward kernel for gfx950.
//
// Computes O = M .* act(scale * Q K^T) V per (sequence, query head): the GDPA
// definition of the GDPA README (intro; softmax replaced by an activation, no
// normaliser).  Because nothing is normalised, every KV tile adds an exact
// partial sum to O: there is no running maximum, no rescaling and no final
// division, unlike softmax flash attention.
//
// Work decomposition: one workgroup (4 waves) per (sequence, query head,
// 128-row query block); wave w owns query rows 32w..32w+31 of the block.
// Per KV tile of BN = 8192/D keys:
//   * K (row-major) and V^T (transposed, accumulator column order) are staged
//     in LDS, double-buffered: the next tile's global loads are issued before
//     the current tile's MFMAs and written to the other buffer afterwards;
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (Q^T held in registers as the B
//     operand for the whole loop), scaled, masked and activated in registers;
//   * P^T is packed to bf16 straight from the accumulators and used as the B
//     operand of O^T += V^T P^T (fp32 accumulation in registers).
// Query blocks are dispatched last-block-first: for self-attention the late
// blocks exist only in long sequences and carry the most KV tiles, so the
// hardware dispatcher sees roughly longest-processing-time-first order (the
// README's "Features" names load-balanced tile scheduling for jagged inputs).
#include "gdpa_common.hpp"
#include "gdpa_kernels.hpp"

namespace gdpa {

template <int D, int ACT, bool FP8>
__global__ __launch_bounds__(256) void gdpa_fwd_kernel(const FwdArgs a) {
  constexpr int BM = kFwdBM;
  constexpr int BN = 8192 / D;          // keys per KV tile
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int KS = D / 16;            // k-steps of Q K^T
  constexpr int NDB = D / 32;           // 32-row blocks of O^T
  constexpr int KBYTES = FP8 ? BN * D : BN * D * 2;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][KBYTES];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[2][D * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int idx = blockIdx.x;
  const int h = idx % a.hq;
  idx /= a.hq;
  const int b = idx % a.batch;
  const int m = a.mblocks - 1 - idx / a.batch;

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
  const int g = h / a.group;
  const int off = lk - lq;  // bottom-right alignment of masks
  const int rlast = min(row0 + BM, lq) - 1;
  int j_lo = 0, j_hi = lk;
  if (a.wl >= 0) j_lo = max(0, row0 + off - a.wl);
  if (a.wr >= 0) j_hi = min(lk, rlast + off + a.wr + 1);
  const int nb_begin = j_lo / BN;
  const int nb_end = (j_hi > j_lo) ? (j_hi + BN - 1) / BN : nb_begin;

  const int q0w = row0 + wave * 32;
  const bool wave_active = q0w < lq;
  const int qmax_w = min(q0w + 31, lq - 1);
  const int qi = q0w + (lane & 31);
  const int hf = lane >> 5;

  // Q^T as the B operand of S^T = K Q^T: lane holds query qi, 8 head-dim values per k-step.
  const long q_ld = (long)a.hq * D;
  u32x4 qreg[FP8 ? 1 : KS];
  u32x2 qreg8[FP8 ? KS : 1];
  if constexpr (FP8) {
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (long)(qs + qi) * q_ld + h * D + hf * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qreg8[s] = (qi < lq) ? *reinterpret_cast<const u32x2*>(qp + s * 16) : u32x2{0u, 0u};
  } else {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + (long)(qs + qi) * q_ld + h * D + hf * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qreg[s] = (qi < lq) ? *reinterpret_cast<const u32x4*>(qp + s * 16) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};

  const long kv_ld = (long)a.hkv * D;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + (long)ks * kv_ld + g * D;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + (long)ks * kv_ld + g * D;
  const uint8_t* kbase8 = static_cast<const uint8_t*>(a.k) + (long)ks * kv_ld + g * D;

  RowTileRegs<BN, D> kregs;
  RowTile8Regs<BN, D> kregs8;
  TrTileRegs<BN, D> vregs;

  auto load_tile = [&](int nb) {
    const int n0 = nb * BN;
    if constexpr (FP8)
      kregs8.load(kbase8 + (long)n0 * kv_ld, kv_ld, lk - n0, tid);
    else
      kregs.load(kbase + (long)n0 * kv_ld, kv_ld, lk - n0, tid);
    vregs.load(vbase + (long)n0 * kv_ld, kv_ld, lk - n0, tid);
  };
  auto store_tile = [&](int buf) {
    if constexpr (FP8)
      kregs8.store(k_lds[buf], tid);
    else
      kregs.store(reinterpret_cast<__bf16*>(k_lds[buf]), tid);
    vregs.store(vt_lds[buf], tid);
  };

  if (nb_begin < nb_end) {
    load_tile(nb_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int nb = nb_begin; nb < nb_end; ++nb) {
    const int buf = (nb - nb_begin) & 1;
    const bool has_next = nb + 1 < nb_end;
    if (has_next) load_tile(nb + 1);

    const int n0 = nb * BN;
    // wave-level mask classification of this tile
    bool empty = false, full = true;
    if (a.wr >= 0) {
      empty |= n0 > qmax_w + off + a.wr;
      full &= n0 + BN - 1 <= q0w + off + a.wr;
    }
    if (a.wl >= 0) {
      empty |= n0 + BN - 1 < q0w + off - a.wl;
      full &= n0 >= qmax_w + off - a.wl;
    }
    if (wave_active && !empty) {
      // ---- S^T = K Q^T
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + (lane & 31);
          if constexpr (FP8) {
            u32x2 aop = *reinterpret_cast<const u32x2*>(k_lds[buf] + row_tile8_off<D>(row, 2 * s + hf));
            sacc[kb] = mfma_fp8(aop, qreg8[s], sacc[kb]);
          } else {
            const __bf16* kl = reinterpret_cast<const __bf16*>(k_lds[buf]);
            u32x4 aop = *reinterpret_cast<const u32x4*>(kl + row_tile_off<D>(row, 2 * s + hf));
            sacc[kb] = mfma_bf16(aop, qreg[s], sacc[kb]);
          }
        }
      }
      // ---- P = M .* act(scale S), packed to bf16 (hi, and lo = remainder if split)
      u32x4 phi[NKB][2], plo[NKB][2];
      const int ip = qi + off;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * a.s_scale;
          float y = Act<ACT>::f(x, a.act_param);
          if (!full) {
            const int j = n0 + kb * 32 + hf * 4 + 8 * (r >> 2) + (r & 3);
            bool ok = true;
            if (a.wl >= 0) ok &= j >= ip - a.wl;
            if (a.wr >= 0) ok &= j <= ip + a.wr;
            y = ok ? y : 0.0f;
          }
          p[r] = y;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float x0 = p[8 * t + 2 * w], x1 = p[8 * t + 2 * w + 1];
            const uint32_t hi = pack_bf16x2(x0, x1);
            phi[kb][t][w] = hi;
            if (a.psplit) plo[kb][t][w] = pack_bf16x2(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
          }
        }
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int chunk = kb * 4 + 2 * t + hf;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = db * 32 + (lane & 31);
            u32x4 aop = *reinterpret_cast<const u32x4*>(vt_lds[buf] + tr_tile_off<BN>(d, chunk));
            oacc[db] = mfma_bf16(aop, phi[kb][t], oacc[db]);
            if (a.psplit) oacc[db] = mfma_bf16(aop, plo[kb][t], oacc[db]);
          }
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane stores 4 consecutive head-dim values per register group
  if (wave_active && qi < lq) {
    const long orow = ((long)(qs + qi) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        if (a.out_f32) {
          f32x4 val{oacc[db][4 * i4], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d) = val;
        } else {
          u32x2 val{pack_bf16x2(oacc[db][4 * i4], oacc[db][4 * i4 + 1]),
                    pack_bf16x2(oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3])};
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.o) + orow + d) = val;
        }
      }
    }
  }
}

template <int D, bool FP8>
static hipError_t launch_fwd_d(const FwdArgs& a, int act_kind, hipStream_t stream) {
  const long grid = (long)a.batch * a.hq * a.mblocks;
  dim3 g((unsigned)grid), blk(256);
  switch (act_kind) {
#define GDPA_FWD_CASE(K) \
  case K: hipLaunchKernelGGL((gdpa_fwd_kernel<D, K, FP8>), g, blk, 0, stream, a); break;
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
