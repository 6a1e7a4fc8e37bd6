// GDPA backward kernels for gfx950.
//
// Gradients of L = sum(O .* dO) for O = M .* act(scale Q K^T) V (GDPA README,
// intro: softmax replaced by an activation, no normaliser).  With
// S = scale Q K^T, P = M .* act(S):
//   dV = P^T dO,  dP = dO V^T,  dS = M .* act'(S) .* dP,
//   dK = scale dS^T Q,  dQ = scale dS K,
// with dK/dV summed over the query heads of a GQA group.  Without a softmax
// there is no row-sum term (no "D = rowsum(dO .* O)" as in flash attention).
//
// Two kernels, each writing its outputs exactly once (no atomics, so results
// are bitwise reproducible):
//  * dK/dV kernel (KV-outer): one workgroup per (sequence, KV head, 128-key
//    block), wave w owns keys 32w..32w+31 with K and V held in registers.  It
//    loops over the group's query heads and 32-row query blocks; Q and dO
//    tiles are staged in LDS both row-major (A operands of S = Q K^T and
//    dP = dO V^T) and transposed (A operands of dK^T += Q^T dS and
//    dV^T += dO^T P).  S and dP come out of the MFMAs with the query index on
//    the accumulator rows, so P and dS feed the next products straight from
//    registers.
//  * dQ kernel (Q-outer): one workgroup per (sequence, query head, 128-row
//    block) recomputes S^T = K Q^T and dP^T = V dO^T per KV tile and
//    accumulates dQ^T += K^T dS^T in a fixed key order.
// This costs 7 matrix products per (query, key) pair instead of the 5 the
// gradient needs, in exchange for a deterministic dQ without a reduction
// buffer.
#include "gdpa_common.hpp"
#include "gdpa_kernels.hpp"

namespace gdpa {

__device__ __forceinline__ void seq_bounds(const BwdArgs& a, int b, int& qs, int& lq, int& ks, int& lk) {
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
}

// ------------------------------------------------------------------ dK / dV
template <int D, int ACT>
__global__ __launch_bounds__(256) void gdpa_bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int BNB = kBwdBN;  // keys per workgroup (32 per wave)
  constexpr int BQ = 32;       // query rows per step
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 q_lds[2][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 qt_lds[2][D * BQ];
  __shared__ __attribute__((aligned(16))) __bf16 do_lds[2][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 dot_lds[2][D * BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  int idx = blockIdx.x;
  const int g = idx % a.hkv;
  idx /= a.hkv;
  const int b = idx % a.batch;
  const int nblk = a.nblocks - 1 - idx / a.batch;
  int qs, lq, ks, lk;
  seq_bounds(a, b, qs, lq, ks, lk);
  const int n0 = nblk * BNB;
  if (n0 >= lk) return;
  const int off = lk - lq;
  const int k0w = n0 + wave * 32;
  const bool wave_active = k0w < lk;
  const int kj = k0w + (lane & 31);  // this lane's key
  const int kmax_w = min(k0w + 31, lk - 1);
  const int klast = min(n0 + BNB, lk) - 1;

  // query rows that can see any key of this block
  int i_lo = 0, i_hi = lq;
  if (a.wr >= 0) i_lo = max(0, n0 - a.wr - off);
  if (a.wl >= 0) i_hi = min(lq, klast + a.wl - off + 1);
  const int mb_begin = i_lo / BQ;
  const int mb_end = (i_hi > i_lo) ? (i_hi + BQ - 1) / BQ : mb_begin;
  const int nsteps = (mb_end - mb_begin) * a.group;

  // K and V of this lane's key as B operands (column = key, 8 head-dim values per k-step)
  const long kv_ld = (long)a.hkv * D;
  u32x4 kreg[KS], vreg[KS];
  {
    const long krow = (long)(ks + min(kj, lk - 1)) * kv_ld + g * D + hf * 8;
    const __bf16* kp = static_cast<const __bf16*>(a.k) + krow;
    const __bf16* vp = static_cast<const __bf16*>(a.v) + krow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kreg[s] = load16_or_zero(kp + s * 16, kj < lk);
      vreg[s] = load16_or_zero(vp + s * 16, kj < lk);
    }
  }
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  const long q_ld = (long)a.hq * D;
  TrTileRegs<BQ, D> qregs, doregs;
  auto load_step = [&](int step) {
    const int h = g * a.group + step % a.group;
    const int m0 = (mb_begin + step / a.group) * BQ;
    const __bf16* qb = static_cast<const __bf16*>(a.q) + (long)(qs + m0) * q_ld + h * D;
    const __bf16* db = static_cast<const __bf16*>(a.dout) + (long)(qs + m0) * q_ld + h * D;
    qregs.load(qb, q_ld, lq - m0, tid);
    doregs.load(db, q_ld, lq - m0, tid);
  };
  auto store_step = [&](int buf) {
    qregs.store_rows(q_lds[buf], tid);
    qregs.store(qt_lds[buf], tid);
    doregs.store_rows(do_lds[buf], tid);
    doregs.store(dot_lds[buf], tid);
  };

  if (nsteps > 0) {
    load_step(0);
    store_step(0);
  }
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool has_next = step + 1 < nsteps;
    if (has_next) load_step(step + 1);
    const int m0 = (mb_begin + step / a.group) * BQ;
    const int mmax = min(m0 + BQ - 1, lq - 1);
    // wave-level mask classification of (queries m0.., keys k0w..)
    bool empty = false, full = true;
    if (a.wr >= 0) {
      empty |= k0w > mmax + off + a.wr;
      full &= kmax_w <= m0 + off + a.wr;
    }
    if (a.wl >= 0) {
      empty |= kmax_w < m0 + off - a.wl;
      full &= k0w >= mmax + off - a.wl;
    }
    if (wave_active && !empty) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int row = lane & 31;
        u32x4 qa = *reinterpret_cast<const u32x4*>(q_lds[buf] + row_tile_off<D>(row, 2 * s + hf));
        u32x4 da = *reinterpret_cast<const u32x4*>(do_lds[buf] + row_tile_off<D>(row, 2 * s + hf));
        sacc = mfma_bf16(qa, kreg[s], sacc);
        dpacc = mfma_bf16(da, vreg[s], dpacc);
      }
      // accumulator element r: query m0 + 4hf + 8(r/4) + r%4, key kj
      u32x4 pb[2], dsb[2], pbl[2], dsbl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 8 * t + 2 * w + u;
            float dy;
            float y = Act<ACT>::f_df(sacc[r] * a.scale, a.act_param, dy);
            float ds = dpacc[r] * dy;
            if (!full) {
              const int ip = m0 + hf * 4 + 8 * (r >> 2) + (r & 3) + off;
              bool ok = true;
              if (a.wl >= 0) ok &= kj >= ip - a.wl;
              if (a.wr >= 0) ok &= kj <= ip + a.wr;
              y = ok ? y : 0.0f;
              ds = ok ? ds : 0.0f;
            }
            pv[u] = y;
            dsv[u] = ds;
          }
          const uint32_t ph = pack_bf16x2(pv[0], pv[1]);
          const uint32_t dh = pack_bf16x2(dsv[0], dsv[1]);
          pb[t][w] = ph;
          dsb[t][w] = dh;
          if (a.kvsplit) {
            pbl[t][w] = pack_bf16x2(pv[0] - bf16_lo_to_f32(ph), pv[1] - bf16_hi_to_f32(ph));
            dsbl[t][w] = pack_bf16x2(dsv[0] - bf16_lo_to_f32(dh), dsv[1] - bf16_hi_to_f32(dh));
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + (lane & 31);
          u32x4 doa = *reinterpret_cast<const u32x4*>(dot_lds[buf] + tr_tile_off<BQ>(d, 2 * t + hf));
          u32x4 qta = *reinterpret_cast<const u32x4*>(qt_lds[buf] + tr_tile_off<BQ>(d, 2 * t + hf));
          dvacc[db] = mfma_bf16(doa, pb[t], dvacc[db]);
          dkacc[db] = mfma_bf16(qta, dsb[t], dkacc[db]);
          if (a.kvsplit) {
            dvacc[db] = mfma_bf16(doa, pbl[t], dvacc[db]);
            dkacc[db] = mfma_bf16(qta, dsbl[t], dkacc[db]);
          }
        }
      }
    }
    if (has_next) store_step(buf ^ 1);
    __syncthreads();
  }

  if (wave_active && kj < lk) {
    const long orow = ((long)(ks + kj) * a.hkv + g) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float k0 = dkacc[db][4 * i4] * a.scale, k1 = dkacc[db][4 * i4 + 1] * a.scale;
        const float k2 = dkacc[db][4 * i4 + 2] * a.scale, k3 = dkacc[db][4 * i4 + 3] * a.scale;
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.dk) + orow + d) = f32x4{k0, k1, k2, k3};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.dv) + orow + d) =
              f32x4{dvacc[db][4 * i4], dvacc[db][4 * i4 + 1], dvacc[db][4 * i4 + 2], dvacc[db][4 * i4 + 3]};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.dk) + orow + d) = u32x2{pack_bf16x2(k0, k1), pack_bf16x2(k2, k3)};
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.dv) + orow + d) =
              u32x2{pack_bf16x2(dvacc[db][4 * i4], dvacc[db][4 * i4 + 1]),
                    pack_bf16x2(dvacc[db][4 * i4 + 2], dvacc[db][4 * i4 + 3])};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------- dQ
template <int D, int ACT>
__global__ __launch_bounds__(256) void gdpa_bwd_dq_kernel(const BwdArgs a) {
  constexpr int BM = kBwdBM;
  constexpr int BN = 4096 / D;  // keys per KV tile
  constexpr int NKB = BN / 32;
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][BN * D];
  __shared__ __attribute__((aligned(16))) __bf16 kt_lds[2][D * BN];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][BN * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  int idx = blockIdx.x;
  const int h = idx % a.hq;
  idx /= a.hq;
  const int b = idx % a.batch;
  const int m = a.mblocks - 1 - idx / a.batch;
  int qs, lq, ks, lk;
  seq_bounds(a, b, qs, lq, ks, lk);
  const int row0 = m * BM;
  if (row0 >= lq) return;
  const int g = h / a.group;
  const int off = lk - lq;
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

  const long q_ld = (long)a.hq * D;
  u32x4 qreg[KS], doreg[KS];
  {
    const long qrow = (long)(qs + min(qi, lq - 1)) * q_ld + h * D + hf * 8;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + qrow;
    const __bf16* dp = static_cast<const __bf16*>(a.dout) + qrow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qreg[s] = load16_or_zero(qp + s * 16, qi < lq);
      doreg[s] = load16_or_zero(dp + s * 16, qi < lq);
    }
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};

  const long kv_ld = (long)a.hkv * D;
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + (long)ks * kv_ld + g * D;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + (long)ks * kv_ld + g * D;
  TrTileRegs<BN, D> kregs;
  RowTileRegs<BN, D> vregs;
  auto load_tile = [&](int nb) {
    const int n0 = nb * BN;
    kregs.load(kbase + (long)n0 * kv_ld, kv_ld, lk - n0, tid);
    vregs.load(vbase + (long)n0 * kv_ld, kv_ld, lk - n0, tid);
  };
  auto store_tile = [&](int buf) {
    kregs.store_rows(k_lds[buf], tid);
    kregs.store(kt_lds[buf], tid);
    vregs.store(v_lds[buf], tid);
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
      f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16{};
        dpacc[kb] = f32x16{};
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + (lane & 31);
          u32x4 ka = *reinterpret_cast<const u32x4*>(k_lds[buf] + row_tile_off<D>(row, 2 * s + hf));
          u32x4 va = *reinterpret_cast<const u32x4*>(v_lds[buf] + row_tile_off<D>(row, 2 * s + hf));
          sacc[kb] = mfma_bf16(ka, qreg[s], sacc[kb]);
          dpacc[kb] = mfma_bf16(va, doreg[s], dpacc[kb]);
        }
      }
      const int ip = qi + off;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        u32x4 dsh[2], dsl[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * t + 2 * w + u;
              float dy;
              (void)Act<ACT>::f_df(sacc[kb][r] * a.scale, a.act_param, dy);
              float ds = dpacc[kb][r] * dy;
              if (!full) {
                const int j = n0 + kb * 32 + hf * 4 + 8 * (r >> 2) + (r & 3);
                bool ok = true;
                if (a.wl >= 0) ok &= j >= ip - a.wl;
                if (a.wr >= 0) ok &= j <= ip + a.wr;
                ds = ok ? ds : 0.0f;
              }
              dsv[u] = ds;
            }
            const uint32_t hi = pack_bf16x2(dsv[0], dsv[1]);
            dsh[t][w] = hi;
            if (a.dsplit) dsl[t][w] = pack_bf16x2(dsv[0] - bf16_lo_to_f32(hi), dsv[1] - bf16_hi_to_f32(hi));
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int chunk = kb * 4 + 2 * t + hf;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = db * 32 + (lane & 31);
            u32x4 kta = *reinterpret_cast<const u32x4*>(kt_lds[buf] + tr_tile_off<BN>(d, chunk));
            dqacc[db] = mfma_bf16(kta, dsh[t], dqacc[db]);
            if (a.dsplit) dqacc[db] = mfma_bf16(kta, dsl[t], dqacc[db]);
          }
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (wave_active && qi < lq) {
    const long orow = ((long)(qs + qi) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float x0 = dqacc[db][4 * i4] * a.scale, x1 = dqacc[db][4 * i4 + 1] * a.scale;
        const float x2 = dqacc[db][4 * i4 + 2] * a.scale, x3 = dqacc[db][4 * i4 + 3] * a.scale;
        if (a.out_f32)
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.dq) + orow + d) = f32x4{x0, x1, x2, x3};
        else
          *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.dq) + orow + d) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
      }
    }
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, hipStream_t stream) {
  const long grid_kv = want_dkv ? (long)a.batch * a.hkv * a.nblocks : 0;
  const long grid_q = want_dq ? (long)a.batch * a.hq * a.mblocks : 0;
  dim3 blk(256);
  switch (act_kind) {
#define GDPA_BWD_CASE(K)                                                                             \
  case K:                                                                                            \
    if (grid_kv > 0) hipLaunchKernelGGL((gdpa_bwd_dkdv_kernel<D, K>), dim3((unsigned)grid_kv), blk, 0, stream, a); \
    if (grid_q > 0) hipLaunchKernelGGL((gdpa_bwd_dq_kernel<D, K>), dim3((unsigned)grid_q), blk, 0, stream, a);     \
    break;
    GDPA_BWD_CASE(ACT_IDENTITY)
    GDPA_BWD_CASE(ACT_GELU)
    GDPA_BWD_CASE(ACT_GELU_TANH)
    GDPA_BWD_CASE(ACT_RELU)
    GDPA_BWD_CASE(ACT_RELU2)
    GDPA_BWD_CASE(ACT_LEAKY)
    GDPA_BWD_CASE(ACT_SILU)
    GDPA_BWD_CASE(ACT_HARDSWISH)
#undef GDPA_BWD_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, int act_kind, bool want_dq, bool want_dkv,
                      hipStream_t stream) {
  if (head_dim == 64) return launch_bwd_d<64>(a, act_kind, want_dq, want_dkv, stream);
  if (head_dim == 128) return launch_bwd_d<128>(a, act_kind, want_dq, want_dkv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdpa
