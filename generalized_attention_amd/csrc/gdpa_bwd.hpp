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
//    block), wave w owns keys 32w..32w+31 with K and V held in registers as B
//    operands.  It loops over the group's query heads and 64-row query
//    blocks; each Q and dO tile is copied HBM -> LDS once (row-major) and read
//    both row-wise (A operands of S = Q K^T and dP = dO V^T) and through the
//    transposing LDS read (A operands of dK^T += Q^T dS and dV^T += dO^T P).
//    S and dP come out of the MFMAs with the query index on the accumulator
//    rows, so P and dS feed the next products straight from registers.
//  * dQ kernel (Q-outer): one workgroup per (sequence, query head, 128-row
//    block), Q and dO in registers; per KV tile it recomputes S^T = K Q^T and
//    dP^T = V dO^T and accumulates dQ^T += K^T dS^T in a fixed key order, the
//    K^T operand again read transposed from the row-major K tile.
// This costs 7 matrix products per (query, key) pair instead of the 5 the
// gradient needs, in exchange for a deterministic dQ without a reduction
// buffer.
#pragma once

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
// Per wave: 32 keys (B operands K, V in registers), per step one 64-row query
// block of one query head (two 32-row blocks qb = 0, 1):
//   S/dP:  S = Q K^T, dP = dO V^T                (2 KS MFMAs per block)
//   pairs: P = act(S), dS = act'(S) dP, packed   (VALU, 8 pairs per block)
//   dV/dK: dV^T += dO^T P, dK^T += Q^T dS       (2 NDB MFMAs x 2 per block)
// One wave per SIMD (dK, dV, K and V stay in registers), so the wave itself
// must keep its matrix core busy while its vector ALU works: a step is issued
// as one stream of "units" (2 MFMAs each, their LDS operands read PREF units
// ahead) in the order S/dP(0), S/dP(1), dV/dK(0), dV/dK(1), and the pairs of
// block 0 ride under S/dP(1), those of block 1 under dV/dK(0).
template <int D, int ACT, int EL, bool SPLIT>
struct DkdvKernel {
  static constexpr int BQ = 64;                      // query rows per step
  static constexpr int KS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int ROWB = 2 * lds_dim(D);        // LDS row bytes (96 padded to 128)
  static constexpr int TB = BQ * ROWB;               // bytes of one Q (or dO) tile
  static constexpr int LPS = 2 * TB / (256 * 16);    // LDS copies per wave per step
  static constexpr int NP = SPLIT ? 2 : 1;           // 16-bit words per P / dS element
  static constexpr int NA = KS;                      // S/dP units per query block (2 MFMAs each)
  static constexpr int NB = 2 * NDB;                 // dV/dK units per query block
  static constexpr int NU = 2 * NA + 2 * NB;
  static constexpr int PREF = 2;                     // units of operand prefetch

  using LaneOffs = TileOffs<ROWB>;
  struct Words {  // packed P and dS of one 32-query block: [hi/lo][t] x 4 words
    u32x4 p[NP][2];
    u32x4 ds[NP][2];
  };

  // One pair of accumulator elements (rows 8t+2w, +1) -> P, dS words.
  template <bool MASK>
  static __device__ __forceinline__ void pair(const f32x16& s, const f32x16& dp, int t, int w, int lo, int hi,
                                              Words& wd, const ActConsts& k) {
    float pv[2], dsv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * t + 2 * w + u;
      float dy;
      float y = Act<ACT>::f_df(s[r], k, dy);
      float ds = dp[r] * dy;
      if constexpr (MASK) {
        const bool ok = in_range(r, lo, hi);
        y = ok ? y : 0.0f;
        ds = ok ? ds : 0.0f;
      }
      pv[u] = y;
      dsv[u] = ds;
    }
    const uint32_t ph = pack2<EL>(pv[0], pv[1]), dh = pack2<EL>(dsv[0], dsv[1]);
    wd.p[0][t][w] = ph;
    wd.ds[0][t][w] = dh;
    if constexpr (SPLIT) {
      wd.p[1][t][w] = split2<EL>(pv[0], pv[1], ph);
      wd.ds[1][t][w] = split2<EL>(dsv[0], dsv[1], dh);
    }
  }

  // Unit u of a step: u < 2 NA: S/dP of block u / NA, k-step u % NA;
  // else dV/dK of block (u - 2 NA) / NB, key-row half t and head-dim block db.
  static __device__ __forceinline__ void load_unit(int u, const uint8_t* ql, const uint8_t* dl, const LaneOffs& lo,
                                                   u32x4& o0, u32x4& o1) {
    if (u < 2 * NA) {
      const int qb = u / NA, s = u % NA;
      o0 = row_at(ql, lo.row[s] + qb * 32 * ROWB);
      o1 = row_at(dl, lo.row[s] + qb * 32 * ROWB);
    } else {
      const int v = u - 2 * NA, qb = v / NB, t = (v % NB) / NDB, db = v % NDB;
      const int base = (qb * 32 + 16 * t) * ROWB;
      o0 = tr_at(dl, lo.tr[db], base);
      o1 = tr_at(ql, lo.tr[db], base);
    }
  }
  static __device__ __forceinline__ void mma_unit(int u, const u32x4& o0, const u32x4& o1, const u32x4* kreg,
                                                  const u32x4* vreg, f32x16* sacc, f32x16* dpacc, const Words* wd,
                                                  f32x16* dkacc, f32x16* dvacc) {
    if (u < 2 * NA) {
      const int qb = u / NA, s = u % NA;
      sacc[qb] = mfma16<EL>(o0, kreg[s], sacc[qb]);
      dpacc[qb] = mfma16<EL>(o1, vreg[s], dpacc[qb]);
    } else {
      const int v = u - 2 * NA, qb = v / NB, t = (v % NB) / NDB, db = v % NDB;
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        dvacc[db] = mfma16<EL>(o0, wd[qb].p[h][t], dvacc[db]);
        dkacc[db] = mfma16<EL>(o1, wd[qb].ds[h][t], dkacc[db]);
      }
    }
  }

  // One step.  lo/hi[qb]: this lane's allowed-query range relative to the
  // accumulator base of block qb (used when MASK).
  template <bool MASK>
  static __device__ __forceinline__ void step(const uint8_t* ql, const uint8_t* dl, const LaneOffs& lo,
                                              const u32x4* kreg, const u32x4* vreg, f32x16* dkacc, f32x16* dvacc,
                                              const int* mlo, const int* mhi, const ActConsts& k) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
    Words wd[2];
    u32x4 ring[PREF + 1][2];
#pragma unroll
    for (int u = 0; u < PREF; ++u) load_unit(u, ql, dl, lo, ring[u][0], ring[u][1]);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + PREF < NU)
        load_unit(u + PREF, ql, dl, lo, ring[(u + PREF) % (PREF + 1)][0], ring[(u + PREF) % (PREF + 1)][1]);
      mma_unit(u, ring[u % (PREF + 1)][0], ring[u % (PREF + 1)][1], kreg, vreg, sacc, dpacc, wd, dkacc, dvacc);
      // pairs of block qb ride under the NA (or NB) units that follow its last S/dP unit
      if (u >= NA && u < 2 * NA + NB) {
        const int qb = u < 2 * NA ? 0 : 1;
        const int v = u < 2 * NA ? u - NA : u - 2 * NA;
        const int span = u < 2 * NA ? NA : NB;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (pair_at(j, v, span)) pair<MASK>(sacc[qb], dpacc[qb], j >> 2, j & 3, mlo[qb], mhi[qb], wd[qb], k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// One workgroup (4 waves; one per SIMD at D = 128, two at D = 64) per (sequence, KV head, 128-key
// block).  Q / dO tiles of the steps are double-buffered in LDS: the next
// step's copy is in flight while the current step is computed.
// Workgroups per CU of the dK/dV kernel: two at D = 64 (K, V, dK, dV take 128
// registers), except where the activation's gradient needs more registers
// than two waves per SIMD leave (exact GELU, and the hi/lo split).
template <int D, int ACT, bool SPLIT>
constexpr int dkdv_occupancy() {
  return (D == 64 && !SPLIT && ACT != ACT_GELU) ? 2 : 1;
}

template <int D, int ACT, int EL, bool SPLIT>
__global__ __launch_bounds__(256, (dkdv_occupancy<D, ACT, SPLIT>())) void gdpa_bwd_dkdv_kernel(const BwdArgs a) {
  using K = DkdvKernel<D, ACT, EL, SPLIT>;
  constexpr int BNB = kBwdBN;  // keys per workgroup (32 per wave)
  constexpr int BQ = K::BQ, KS = K::KS, NDB = K::NDB, ROWB = K::ROWB, TB = K::TB;
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  // One work item: sequence b, KV head g, key block nblk.
  auto process = [&](int b, int g, int nblk) __attribute__((always_inline)) {
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
  // queries that may see this lane's key: [ilo_l, ihi_l]
  const int ilo_l = a.wr >= 0 ? kj - a.wr - off : 0;
  const int ihi_l = min(lq - 1, a.wl >= 0 ? kj + a.wl - off : lq - 1);

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
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + krow;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + krow;
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
  const TileOffs<ROWB> loffs = TileOffs<ROWB>::make(lane);

  const int q_ld_b = a.hq * D * 2;  // bytes per token row of q / dO
  // this sequence's q and dO rows (all heads); 32-bit offsets, bounded on the host
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(static_cast<const uint8_t*>(a.q) + (long)qs * q_ld_b, lq * q_ld_b);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(static_cast<const uint8_t*>(a.dout) + (long)qs * q_ld_b, lq * q_ld_b);
  auto step_m0 = [&](int i) { return (mb_begin + i / a.group) * BQ; };
  auto stage = [&](int i, uint8_t* ql, uint8_t* dl) {
    const int h = g * a.group + i % a.group;
    const int m0 = step_m0(i);
    const int o = m0 * q_ld_b + h * D * 2;
    stage_tile_buf<BQ, ROWB, 4, D / 8>(qrs, o, q_ld_b, lq - m0, ql, wave, lane);
    stage_tile_buf<BQ, ROWB, 4, D / 8>(drs, o, q_ld_b, lq - m0, dl, wave, lane);
  };
  auto compute = [&](int i, const uint8_t* ql, const uint8_t* dl) {
    if (!wave_active) return;
    const int m0 = step_m0(i), mhi = m0 + BQ - 1;
    // wave-level classification of (queries m0..mhi, keys k0w..kmax_w)
    bool empty = false, full = true;  // Q / dO rows past the last query are zeros
    if (a.wr >= 0) {
      empty |= k0w > min(mhi, lq - 1) + off + a.wr;
      full &= kmax_w <= m0 + off + a.wr;
    }
    if (a.wl >= 0) {
      empty |= kmax_w < m0 + off - a.wl;
      full &= k0w >= mhi + off - a.wl;
    }
    if (empty) return;
    int mlo[2], mhi2[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int base = m0 + qb * 32 + hf * 4;
      mlo[qb] = ilo_l - base;
      mhi2[qb] = ihi_l - base;
    }
    // With one wave per SIMD, K and V (MFMA B operands) live in AGPRs; tying
    // them to one register each step stops the allocator from copying them
    // between AGPR groups inside the step (one move per register and step).
    // At D = 64 they fit among the arch VGPRs, and are left there.
    if constexpr (D > 64) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        asm volatile("" : "+a"(kreg[s]));
        asm volatile("" : "+a"(vreg[s]));
      }
    }
    if (full)
      K::template step<false>(ql, dl, loffs, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act);
    else
      K::template step<true>(ql, dl, loffs, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act);
  };

  if (nsteps > 0) stage(0, q_lds0, do_lds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < nsteps; i += 2) {
    if (i + 1 < nsteps) stage(i + 1, q_lds1, do_lds1);
    compute(i, q_lds0, do_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 1 >= nsteps) break;
    if (i + 2 < nsteps) stage(i + 2, q_lds0, do_lds0);
    compute(i + 1, q_lds1, do_lds1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (wave_active && kj < lk) {
    const long orow = ((long)(ks + kj) * a.hkv + g) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float gs = a.act.gscale, ps = a.act.pscale;
        store4(a.dk, orow + d, dkacc[db][4 * i4] * gs, dkacc[db][4 * i4 + 1] * gs, dkacc[db][4 * i4 + 2] * gs,
               dkacc[db][4 * i4 + 3] * gs, a.out_kind);
        store4(a.dv, orow + d, dvacc[db][4 * i4] * ps, dvacc[db][4 * i4 + 1] * ps, dvacc[db][4 * i4 + 2] * ps,
               dvacc[db][4 * i4 + 3] * ps, a.out_kind);
      }
    }
  }
  };

  if (a.counters == nullptr) {
    // Block -> work item: (sequence, KV head) pair on one XCD, longest
    // sequences first; within a pair, key blocks run last-first.
    WorkItem w;
    if (!map_work(blockIdx.x, a.batch, a.hkv, a.nblocks, a.perm, w)) return;
    process(w.b, w.g, a.nblocks - 1 - w.rest);
  } else {
    // Per-XCD work queue over the same pairs, longest sequence first (one
    // workgroup per CU here, so the dispatcher's in-order hand-out of one
    // item per workgroup would leave CUs idle between items).
    run_queue(a.counters + (blockIdx.x & (kNumXcd - 1)), xcd_items(a.batch, a.hkv, a.nblocks),
              [&](int j) __attribute__((always_inline)) {
                WorkItem w;
                xcd_item(j, a.hkv, a.nblocks, a.perm, w);
                process(w.b, w.g, a.nblocks - 1 - w.rest);
              });
  }
}

// ----------------------------------------------------------------------- dQ
template <int D, int ACT, int EL, bool SPLIT>
struct DqKernel {
  static constexpr int BN = 8192 / lds_dim(D);  // keys per KV tile
  static constexpr int NKB = BN / 32;
  static constexpr int KS = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int ROWB = 2 * lds_dim(D);  // LDS row bytes (96 padded to 128)

  static constexpr int NP = SPLIT ? 2 : 1;   // 16-bit words per dS element
  static constexpr int NA = KS;               // S/dP units per key block (2 MFMAs each)
  static constexpr int NB = 2 * NDB;          // dQ units per key block (NP MFMAs each)
  static constexpr int NU = 2 * NA + 2 * NB;  // units of a pair of key blocks
  static constexpr int PREF = 2;              // units of operand prefetch
  using LaneOffs = TileOffs<ROWB>;

  // One pair of accumulator elements (key rows 8t+2w, +1) -> dS words.
  template <bool MASK>
  static __device__ __forceinline__ void pair(const f32x16& s, const f32x16& dp, int t, int w, int lo, int hi,
                                              u32x4 (*ds)[2], const ActConsts& k) {
    float dsv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * t + 2 * w + u;
      float dy;
      (void)Act<ACT>::f_df(s[r], k, dy);
      float v = dp[r] * dy;
      if constexpr (MASK) v = in_range(r, lo, hi) ? v : 0.0f;
      dsv[u] = v;
    }
    const uint32_t dh = pack2<EL>(dsv[0], dsv[1]);
    ds[0][t][w] = dh;
    if constexpr (SPLIT) ds[1][t][w] = split2<EL>(dsv[0], dsv[1], dh);
  }

  // Unit u of a block pair (blocks kb0, kb0+1 of the tile): u < 2 NA: S/dP of
  // block u / NA, k-step u % NA; else dQ of block (u - 2 NA) / NB, key-row half
  // t and head-dim block db.
  static __device__ __forceinline__ void load_unit(int u, int kb0, const uint8_t* kl, const uint8_t* vl,
                                                   const LaneOffs& lo, u32x4& o0, u32x4& o1) {
    if (u < 2 * NA) {
      const int kb = kb0 + u / NA, s = u % NA;
      o0 = row_at(kl, lo.row[s] + kb * 32 * ROWB);
      o1 = row_at(vl, lo.row[s] + kb * 32 * ROWB);
    } else {
      const int v = u - 2 * NA, kb = kb0 + v / NB, t = (v % NB) / NDB, db = v % NDB;
      o0 = tr_at(kl, lo.tr[db], (kb * 32 + 16 * t) * ROWB);
      o1 = o0;
    }
  }

  // S^T/dP^T of two 32-key blocks against this wave's 32 queries, their dS,
  // and dQ^T += K^T dS^T, as one stream of units (LDS operands PREF units
  // ahead); the dS pairs of block 0 ride under block 1's S/dP units, those of
  // block 1 under block 0's dQ units.  lo/hi[j]: this lane's allowed-key range
  // relative to block j's accumulator base (used when MASK).
  template <bool MASK>
  static __device__ __forceinline__ void block_pair(const uint8_t* kl, const uint8_t* vl, int kb0, const LaneOffs& lo,
                                                    const u32x4* qreg, const u32x4* doreg, f32x16* dqacc,
                                                    const int* mlo, const int* mhi, const ActConsts& k) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
    u32x4 ds[2][NP][2];
    u32x4 ring[PREF + 1][2];
#pragma unroll
    for (int u = 0; u < PREF; ++u) load_unit(u, kb0, kl, vl, lo, ring[u][0], ring[u][1]);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + PREF < NU)
        load_unit(u + PREF, kb0, kl, vl, lo, ring[(u + PREF) % (PREF + 1)][0], ring[(u + PREF) % (PREF + 1)][1]);
      const u32x4& o0 = ring[u % (PREF + 1)][0];
      const u32x4& o1 = ring[u % (PREF + 1)][1];
      if (u < 2 * NA) {
        const int j = u / NA, s = u % NA;
        sacc[j] = mfma16<EL>(o0, qreg[s], sacc[j]);
        dpacc[j] = mfma16<EL>(o1, doreg[s], dpacc[j]);
      } else {
        const int v = u - 2 * NA, j = v / NB, t = (v % NB) / NDB, db = v % NDB;
#pragma unroll
        for (int h = 0; h < NP; ++h) dqacc[db] = mfma16<EL>(o0, ds[j][h][t], dqacc[db]);
      }
      if (u >= NA && u < 2 * NA + NB) {
        const int j = u < 2 * NA ? 0 : 1;
        const int v = u < 2 * NA ? u - NA : u - 2 * NA;
        const int span = u < 2 * NA ? NA : NB;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (pair_at(q, v, span)) pair<MASK>(sacc[j], dpacc[j], q >> 2, q & 3, mlo[j], mhi[j], ds[j], k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Two workgroups per CU, except where the activation gradient needs more
// registers than two waves per SIMD leave at D = 128 (exact GELU, and SiLU
// with dS carried as a hi/lo pair).
template <int D, int ACT, bool SPLIT>
constexpr int dq_occupancy() {
  return (D == 128 && (ACT == ACT_GELU || (SPLIT && ACT == ACT_SILU))) ? 1 : 2;
}

template <int D, int ACT, int EL, bool SPLIT>
__global__ __launch_bounds__(256, (dq_occupancy<D, ACT, SPLIT>())) void gdpa_bwd_dq_kernel(const BwdArgs a) {
  using K = DqKernel<D, ACT, EL, SPLIT>;
  constexpr int BM = kBwdBM;
  constexpr int BN = K::BN, NKB = K::NKB, KS = K::KS, NDB = K::NDB, ROWB = K::ROWB;
  constexpr int TB = BN * ROWB;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  // One work item: sequence b, KV head g, query head h, query block m.
  auto process = [&](int b, int g, int h, int m) __attribute__((always_inline)) {
  int qs, lq, ks, lk;
  seq_bounds(a, b, qs, lq, ks, lk);
  const int row0 = m * BM;
  if (row0 >= lq) return;
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
  // keys this lane's query may see: [jlo, jhi]
  const int jlo = a.wl >= 0 ? qi + off - a.wl : 0;
  const int jhi = min(lk - 1, a.wr >= 0 ? qi + off + a.wr : lk - 1);

  const long q_ld = (long)a.hq * D;
  u32x4 qreg[KS], doreg[KS];
  {
    const long qrow = (long)(qs + min(qi, lq - 1)) * q_ld + h * D + hf * 8;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow;
    const uint16_t* dp = static_cast<const uint16_t*>(a.dout) + qrow;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qreg[s] = load16_or_zero(qp + s * 16, qi < lq);
      doreg[s] = load16_or_zero(dp + s * 16, qi < lq);
    }
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};
  const TileOffs<ROWB> loffs = TileOffs<ROWB>::make(lane);

  const long kv_ld_b = (long)a.hkv * D * 2;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (long)ks * kv_ld_b + (long)g * D * 2;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (long)ks * kv_ld_b + (long)g * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, lk * (int)kv_ld_b);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, lk * (int)kv_ld_b);
  auto stage = [&](int nb, uint8_t* kl, uint8_t* vl) {
    const int n0 = nb * BN;
    stage_tile_buf<BN, ROWB, 4, D / 8>(krs, n0 * (int)kv_ld_b, (int)kv_ld_b, lk - n0, kl, wave, lane);
    stage_tile_buf<BN, ROWB, 4, D / 8>(vrs, n0 * (int)kv_ld_b, (int)kv_ld_b, lk - n0, vl, wave, lane);
  };
  auto compute = [&](int nb, const uint8_t* kl, const uint8_t* vl) __attribute__((always_inline)) {
    if (!wave_active) return;
    const int n0 = nb * BN;
#pragma unroll
    for (int kb0 = 0; kb0 < NKB; kb0 += 2) {
      // wave-level classification of the two 32-key blocks
      bool any = false, all_full = true;
      int mlo[2], mhi[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int b_lo = n0 + (kb0 + j) * 32, b_hi = b_lo + 31;  // keys of this 32-key block
        bool empty = b_lo >= lk, full = true;  // K / V rows past the last key are zeros
        if (a.wr >= 0) {
          empty |= b_lo > qmax_w + off + a.wr;
          full &= b_hi <= q0w + off + a.wr;
        }
        if (a.wl >= 0) {
          empty |= b_hi < q0w + off - a.wl;
          full &= b_lo >= qmax_w + off - a.wl;
        }
        any |= !empty;
        all_full &= full;
        // accumulator element r: key b_lo + 4hf + 8(r/4) + r%4, this lane's query
        mlo[j] = jlo - (b_lo + hf * 4);
        mhi[j] = jhi - (b_lo + hf * 4);
      }
      if (!any) continue;
      if (all_full)
        K::template block_pair<false>(kl, vl, kb0, loffs, qreg, doreg, dqacc, mlo, mhi, a.act);
      else
        K::template block_pair<true>(kl, vl, kb0, loffs, qreg, doreg, dqacc, mlo, mhi, a.act);
    }
  };

  if (nb_begin < nb_end) stage(nb_begin, k_lds0, v_lds0);
  __builtin_amdgcn_s_waitcnt(0);
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

  if (wave_active && qi < lq) {
    const long orow = ((long)(qs + qi) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float gs = a.act.gscale;
        store4(a.dq, orow + d, dqacc[db][4 * i4] * gs, dqacc[db][4 * i4 + 1] * gs, dqacc[db][4 * i4 + 2] * gs,
               dqacc[db][4 * i4 + 3] * gs, a.out_kind);
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

template <int D, int EL, bool SPLIT_KV, bool SPLIT_Q>
static hipError_t launch_bwd_ds(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, hipStream_t stream) {
  // dK/dV work queue: as many workgroups as are resident at once
  const bool queue = a.counters != nullptr;
  const long grid_kv = !want_dkv ? 0 : queue ? -1 : pair_grid(a.batch, a.hkv, a.nblocks);
  const long grid_q = !want_dq ? 0 : pair_grid(a.batch, a.hkv, a.group * a.mblocks);
  dim3 blk(256);
  switch (act_kind) {
#define GDPA_BWD_CASE(K)                                                                                       \
  case K:                                                                                                      \
    if (grid_kv != 0)                                                                                          \
      hipLaunchKernelGGL((gdpa_bwd_dkdv_kernel<D, K, EL, SPLIT_KV>),                                               \
                         dim3((unsigned)(grid_kv > 0 ? grid_kv                                                 \
                                                     : queue_grid(a.ncu, dkdv_occupancy<D, K, SPLIT_KV>()))), \
                         blk, 0, stream, a);                                                                   \
    if (grid_q > 0)                                                                                            \
      hipLaunchKernelGGL((gdpa_bwd_dq_kernel<D, K, EL, SPLIT_Q>), dim3((unsigned)grid_q), blk, 0, stream, a);     \
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

template <int D, int EL>
static hipError_t launch_bwd_d(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, hipStream_t stream) {
  // fp16 never splits P or dS (the host keeps a single word within tolerance)
  if constexpr (EL == EL_F16) {
    if (a.kvsplit || a.dsplit) return hipErrorInvalidValue;
    return launch_bwd_ds<D, EL, false, false>(a, act_kind, want_dq, want_dkv, stream);
  }
  if (a.kvsplit)
    return a.dsplit ? launch_bwd_ds<D, EL, true, true>(a, act_kind, want_dq, want_dkv, stream)
                    : launch_bwd_ds<D, EL, true, false>(a, act_kind, want_dq, want_dkv, stream);
  return a.dsplit ? launch_bwd_ds<D, EL, false, true>(a, act_kind, want_dq, want_dkv, stream)
                  : launch_bwd_ds<D, EL, false, false>(a, act_kind, want_dq, want_dkv, stream);
}

// Backward launches of one input element kind (each kind is instantiated in
// its own translation unit).
template <int EL>
static hipError_t launch_bwd_el(const BwdArgs& a, int head_dim, int act_kind, bool want_dq, bool want_dkv,
                                hipStream_t stream) {
  if (head_dim == 64) return launch_bwd_d<64, EL>(a, act_kind, want_dq, want_dkv, stream);
  if (head_dim == 96) return launch_bwd_d<96, EL>(a, act_kind, want_dq, want_dkv, stream);
  if (head_dim == 128) return launch_bwd_d<128, EL>(a, act_kind, want_dq, want_dkv, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdpa
