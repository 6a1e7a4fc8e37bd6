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
// Three kernels.  The fused kernel (below the two others) computes dK, dV
// and dQ in one pass with an ordered dQ reduction; the call uses it whenever
// all three gradients are wanted.  The two separate kernels write their
// outputs exactly once (no atomics, so results are bitwise reproducible) and
// serve calls that want only dQ or only dK and dV, short rows whose dS needs
// a hi/lo pair, and comparisons:
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
//
// With DQ (the fused backward), the step also writes its dS to an LDS tile
// [128 keys][64 queries] and computes the previous step's dQ = dS K for one
// 32-column head-dim block of the workgroup's 128 keys (the A operand dS and
// the B operand K both arrive through the transposing LDS read, so their key
// orders agree): NQU more units of 2 MFMAs, spread over the two regions that
// carry activation work, so the matrix core has more to do while the vector
// ALU evaluates the activation.  With DSPL (few keys per dQ row, where the
// bf16 rounding of dS no longer averages out) dS is carried as hi + lo words
// in two LDS tiles and each dQ product is taken twice.
// D is the head dim of Q and K (S, dK), DV that of V and dO (dP, dV); they
// differ only at (192, 128), where the S units of k-steps >= DV / 16 carry no
// dP product and the dK blocks >= DV / 32 no dV product.
template <int D, int ACT, int EL, bool SPLIT, bool DQ = false, bool DSPL = false, int DV = D>
struct DkdvKernel {
  static constexpr int BQ = 64;                      // query rows per step
  static constexpr int KS = D / 16;                  // k-steps of S (Q, K head dim)
  static constexpr int NDB = D / 32;                 // 32-column blocks of dK
  static constexpr int KSV = DV / 16;                // k-steps of dP (dO, V head dim)
  static constexpr int NDBV = DV / 32;               // 32-column blocks of dV
  static constexpr int ROWB = 2 * lds_dim(D);        // LDS row bytes of a Q tile (96 padded to 128)
  static constexpr int ROWBV = 2 * lds_dim(DV);      // LDS row bytes of a dO tile
  static constexpr int TB = BQ * ROWB;               // bytes of one Q tile
  static constexpr int TBV = BQ * ROWBV;             // bytes of one dO tile
  static_assert(KSV <= KS && NDBV <= NDB, "V's head dim is at most Q's");
  static_assert(!DQ || DV == D, "the fused pass is built for equal head dims");
  static constexpr int NP = SPLIT ? 2 : 1;           // 16-bit words per P / dS element (dV, dK)
  static constexpr int NPD = SPLIT || DSPL ? 2 : 1;  // 16-bit words per dS element kept
  static constexpr int NA = KS;                      // S/dP units per query block (2 MFMAs each)
  static constexpr int NB = 2 * NDB;                 // dV/dK units per query block
  // dQ of one step, per wave: both 32-row query blocks x one head-dim block
  // (head dims 96, 128), or one query block x one head-dim block (64), over
  // 8 key steps of 16: each unit is one key step of both blocks, or two key
  // steps of the one block.
  static constexpr int DQB = D == 64 ? 1 : 2;
  static constexpr int NQH = DQ ? (DQB == 2 ? 8 : 4) : 0;  // dQ units per dS word
  static constexpr int NQU = NQH * (DSPL ? 2 : 1);
  static constexpr int NQ1 = NQU / 2, NQ2 = NQU - NQ1;
  static constexpr int L1 = NA + NQ1, L2 = NB + NQ2;  // lengths of the two activation regions
  static constexpr int U1 = NA, U2 = U1 + L1, U3 = U2 + L2;
  static constexpr int NU = U3 + NB;
  static constexpr int PREF = 2;                     // units of operand prefetch
  static constexpr int DS_ROWB = 2 * BQ;             // dS tile row (one key): 64 queries
  static constexpr int DS_BYTES = 128 * DS_ROWB;     // dS tile of the workgroup's 128 keys
  static constexpr int DS_TILE = DS_BYTES * (DSPL ? 2 : 1);  // hi (and lo) tiles of one step

  using LaneOffs = TileOffs<ROWB>;
  using LaneOffsV = TileOffs<ROWBV>;
  using DsOffs = TileOffs<DS_ROWB>;
  struct Words {  // packed P and dS of one 32-query block: [hi/lo][t] x 4 words
    u32x4 p[NP][2];
    u32x4 ds[NPD][2];
  };

  // Unit kinds: S/dP of block qb, k-step s; dV/dK of block qb, key-row half t,
  // head-dim block db; dQ unit q.  Region 1 (S/dP of block 1) and region 2
  // (dV/dK of block 0) interleave NQ1 and NQ2 dQ units evenly.
  enum { U_SDP = 0, U_DVK = 1, U_DQ = 2 };
  struct Unit {
    int kind, qb, s, t, db, q;
  };
  static constexpr Unit unit(int u) {
    if (u < U1) return Unit{U_SDP, 0, u, 0, 0, 0};
    if (u < U2) {
      const int p = u - U1, before = p * NQ1 / L1;
      if ((p + 1) * NQ1 / L1 > before) return Unit{U_DQ, 0, 0, 0, 0, before};
      return Unit{U_SDP, 1, p - before, 0, 0, 0};
    }
    if (u < U3) {
      const int p = u - U2, before = p * NQ2 / L2;
      if ((p + 1) * NQ2 / L2 > before) return Unit{U_DQ, 0, 0, 0, 0, NQ1 + before};
      const int v = p - before;
      return Unit{U_DVK, 0, 0, v / NDB, v % NDB, 0};
    }
    const int v = u - U3;
    return Unit{U_DVK, 1, 0, v / NDB, v % NDB, 0};
  }

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
    if constexpr (SPLIT) wd.p[1][t][w] = split2<EL>(pv[0], pv[1], ph);
    if constexpr (NPD == 2) wd.ds[1][t][w] = split2<EL>(dsv[0], dsv[1], dh);
  }

  // dS of query block qb -> this lane's key row of the dS tile (the lo words
  // to the second tile with DSPL).  Words t of
  // block qb hold queries 32 qb + 4 hf + 16 t + {0..3} (words 0, 1) and
  // + {8..11} (words 2, 3): two 8-byte pieces, 16-byte chunks 4 qb + 2 t and
  // 4 qb + 2 t + 1 at byte 8 hf.
  static __device__ __forceinline__ void write_ds(uint8_t* dsl, int krow, int hf, int qb, const Words& wd) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = lds_off<DS_ROWB>(krow, 4 * qb + 2 * t + h) + 8 * hf;
        *reinterpret_cast<u32x2*>(dsl + off) = u32x2{wd.ds[0][t][2 * h], wd.ds[0][t][2 * h + 1]};
        if constexpr (DSPL)
          *reinterpret_cast<u32x2*>(dsl + DS_BYTES + off) = u32x2{wd.ds[1][t][2 * h], wd.ds[1][t][2 * h + 1]};
      }
  }
  static __device__ __forceinline__ void zero_ds(uint8_t* dsl, int krow, int hf) {
#pragma unroll
    for (int w = 0; w < DS_TILE / DS_BYTES; ++w)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x2*>(dsl + w * DS_BYTES + lds_off<DS_ROWB>(krow, c) + 8 * hf) = u32x2{0u, 0u};
  }

  // The dQ operands of the previous step: A = dS rows (query block) from the
  // transposed dS tile, key steps 16 ks.  dsa/dsb: this lane's transposed-read
  // offsets of the two query blocks (the same block twice at head dim 64).
  // Units q >= NQH read the lo tile.
  static __device__ __forceinline__ void load_dq(int qu, const uint8_t* dsl, const int* dsa, const int* dsb,
                                                 u32x4& o0, u32x4& o1) {
    const int q = NQH > 0 ? qu % NQH : 0;  // (no dQ units without DQ)
    dsl += (NQH > 0 ? qu / NQH : 0) * DS_BYTES;
    const int a2[2] = {dsa[0], dsa[1]};
    if constexpr (DQB == 2) {
      const int b2[2] = {dsb[0], dsb[1]};
      o0 = tr_at(dsl, a2, 16 * q * DS_ROWB);
      o1 = tr_at(dsl, b2, 16 * q * DS_ROWB);
    } else {
      o0 = tr_at(dsl, a2, 32 * q * DS_ROWB);
      o1 = tr_at(dsl, a2, (32 * q + 16) * DS_ROWB);
    }
  }
  static __device__ __forceinline__ void mma_dq(int qu, const u32x4& o0, const u32x4& o1, const u32x4* ktr,
                                                f32x16* dqacc) {
    const int q = NQH > 0 ? qu % NQH : 0;
    if constexpr (DQB == 2) {
      dqacc[0] = mfma16<EL>(o0, ktr[q], dqacc[0]);
      dqacc[1] = mfma16<EL>(o1, ktr[q], dqacc[1]);
    } else {
      dqacc[0] = mfma16<EL>(o0, ktr[2 * q], dqacc[0]);
      dqacc[0] = mfma16<EL>(o1, ktr[2 * q + 1], dqacc[0]);
    }
  }

  static __device__ __forceinline__ void load_unit(int u, const uint8_t* ql, const uint8_t* dl, const LaneOffs& lo,
                                                   const LaneOffsV& lov, const uint8_t* dsl, const int* dsa,
                                                   const int* dsb, u32x4& o0, u32x4& o1) {
    const Unit x = unit(u);
    if (x.kind == U_SDP) {
      o0 = row_at(ql, lo.row[x.s] + x.qb * 32 * ROWB);
      o1 = x.s < KSV ? row_at(dl, lov.row[x.s < KSV ? x.s : 0] + x.qb * 32 * ROWBV) : o0;
    } else if (x.kind == U_DVK) {
      const int base = (x.qb * 32 + 16 * x.t) * ROWB;
      o0 = x.db < NDBV ? tr_at(dl, lov.tr[x.db < NDBV ? x.db : 0], (x.qb * 32 + 16 * x.t) * ROWBV)
                       : u32x4{0u, 0u, 0u, 0u};
      o1 = tr_at(ql, lo.tr[x.db], base);
    } else {
      load_dq(x.q, dsl, dsa, dsb, o0, o1);
    }
  }
  static __device__ __forceinline__ void mma_unit(int u, const u32x4& o0, const u32x4& o1, const u32x4* kreg,
                                                  const u32x4* vreg, f32x16* sacc, f32x16* dpacc, const Words* wd,
                                                  f32x16* dkacc, f32x16* dvacc, const u32x4* ktr, f32x16* dqacc) {
    const Unit x = unit(u);
    if (x.kind == U_SDP) {
      sacc[x.qb] = mfma16<EL>(o0, kreg[x.s], sacc[x.qb]);
      if (x.s < KSV) dpacc[x.qb] = mfma16<EL>(o1, vreg[x.s < KSV ? x.s : 0], dpacc[x.qb]);
    } else if (x.kind == U_DVK) {
#pragma unroll
      for (int h = 0; h < NP; ++h) {
        if (x.db < NDBV) dvacc[x.db < NDBV ? x.db : 0] = mfma16<EL>(o0, wd[x.qb].p[h][x.t], dvacc[x.db < NDBV ? x.db : 0]);
        dkacc[x.db] = mfma16<EL>(o1, wd[x.qb].ds[h][x.t], dkacc[x.db]);
      }
    } else {
      mma_dq(x.q, o0, o1, ktr, dqacc);
    }
  }

  // One step.  lo/hi[qb]: this lane's allowed-query range relative to the
  // accumulator base of block qb (used when MASK).  With DQ: dsw receives
  // this step's dS (row krow = the lane's key), and dqacc accumulates the
  // previous step's dQ from dsr.
  template <bool MASK>
  static __device__ __forceinline__ void step(const uint8_t* ql, const uint8_t* dl, const LaneOffs& lo,
                                              const LaneOffsV& lov, const u32x4* kreg, const u32x4* vreg, f32x16* dkacc, f32x16* dvacc,
                                              const int* mlo, const int* mhi, const ActConsts& k,
                                              uint8_t* dsw = nullptr, const uint8_t* dsr = nullptr,
                                              const int* dsa = nullptr, const int* dsb = nullptr,
                                              const u32x4* ktr = nullptr, f32x16* dqacc = nullptr, int krow = 0,
                                              int hf = 0) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
    Words wd[2];
    u32x4 ring[PREF + 1][2];
#pragma unroll
    for (int u = 0; u < PREF; ++u) load_unit(u, ql, dl, lo, lov, dsr, dsa, dsb, ring[u][0], ring[u][1]);
    auto unit_body = [&](const int u) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + PREF < NU)
        load_unit(u + PREF, ql, dl, lo, lov, dsr, dsa, dsb, ring[(u + PREF) % (PREF + 1)][0],
                  ring[(u + PREF) % (PREF + 1)][1]);
      mma_unit(u, ring[u % (PREF + 1)][0], ring[u % (PREF + 1)][1], kreg, vreg, sacc, dpacc, wd, dkacc, dvacc, ktr,
               dqacc);
      // pairs of block qb ride under the units of its region
      if (u >= U1 && u < U3) {
        const int qb = u < U2 ? 0 : 1;
        const int v = u < U2 ? u - U1 : u - U2;
        const int span = u < U2 ? L1 : L2;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (pair_at(j, v, span)) pair<MASK>(sacc[qb], dpacc[qb], j >> 2, j & 3, mlo[qb], mhi[qb], wd[qb], k);
      }
      if constexpr (DQ) {
        if (u == U2 - 1) write_ds(dsw, krow, hf, 0, wd[0]);
        if (u == U3 - 1) write_ds(dsw, krow, hf, 1, wd[1]);
      }
    };
    if constexpr (DQ || D != DV) {
      // the longer streams (dQ units; head dim 192) exceed the unroller's
      // threshold: issue them with compile-time unit indices
      static_for<0, NU>([&](auto uc) __attribute__((always_inline)) { unit_body(decltype(uc)::value); });
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) unit_body(u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // dQ units only (a step whose S/dP this wave skips, and the drain after the
  // last step).
  static __device__ __forceinline__ void dq_only(const uint8_t* dsr, const int* dsa, const int* dsb,
                                                 const u32x4* ktr, f32x16* dqacc) {
    u32x4 ring[PREF + 1][2];
#pragma unroll
    for (int u = 0; u < PREF && u < NQU; ++u) load_dq(u, dsr, dsa, dsb, ring[u][0], ring[u][1]);
    static_for<0, NQU>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u + PREF < NQU)
        load_dq(u + PREF, dsr, dsa, dsb, ring[(u + PREF) % (PREF + 1)][0], ring[(u + PREF) % (PREF + 1)][1]);
      mma_dq(u, ring[u % (PREF + 1)][0], ring[u % (PREF + 1)][1], ktr, dqacc);
    });
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

template <int D, int ACT, int EL, bool SPLIT, int DV = D>
__global__ __launch_bounds__(256, (dkdv_occupancy<D, ACT, SPLIT>())) void gdpa_bwd_dkdv_kernel(const BwdArgs a) {
  using K = DkdvKernel<D, ACT, EL, SPLIT, false, false, DV>;
  constexpr int BNB = kBwdBN;  // keys per workgroup (32 per wave)
  constexpr int BQ = K::BQ, KS = K::KS, NDB = K::NDB, ROWB = K::ROWB, TB = K::TB;
  constexpr int KSV = K::KSV, NDBV = K::NDBV, ROWBV = K::ROWBV, TBV = K::TBV;
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds0[TBV];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds1[TBV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  // One work item: sequence b, KV head g, key block nblk.  In queue mode
  // fetch (non-null) takes the next index as the last step starts; returns
  // whether it did (there was a step).
  auto process = [&](int b, int g, int nblk, QueueFetch* fetch) __attribute__((always_inline)) -> bool {
  int qs, lq, ks, lk;
  seq_bounds(a, b, qs, lq, ks, lk);
  const int n0 = nblk * BNB;
  if (n0 >= lk) return false;
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
  const long kv_ld = (long)a.hkv * D, vv_ld = (long)a.hkv * DV;
  u32x4 kreg[KS], vreg[KSV];
  {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + (long)(ks + min(kj, lk - 1)) * kv_ld + g * D + hf * 8;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + (long)(ks + min(kj, lk - 1)) * vv_ld + g * DV + hf * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) kreg[s] = load16_or_zero(kp + s * 16, kj < lk);
#pragma unroll
    for (int s = 0; s < KSV; ++s) vreg[s] = load16_or_zero(vp + s * 16, kj < lk);
  }
  f32x16 dkacc[NDB], dvacc[NDBV];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dkacc[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < NDBV; ++i) dvacc[i] = f32x16{};
  const TileOffs<ROWB> loffs = TileOffs<ROWB>::make(lane);
  const TileOffs<ROWBV> loffsv = TileOffs<ROWBV>::make(lane);

  const int q_ld_b = a.hq * D * 2;    // bytes per token row of q
  const int do_ld_b = a.hq * DV * 2;  // bytes per token row of dO
  // this sequence's q and dO rows (all heads); 32-bit offsets, bounded on the host
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(static_cast<const uint8_t*>(a.q) + (long)qs * q_ld_b, lq * q_ld_b);
  const __amdgpu_buffer_rsrc_t drs =
      make_rsrc(static_cast<const uint8_t*>(a.dout) + (long)qs * do_ld_b, lq * do_ld_b);
  auto step_m0 = [&](int i) { return (mb_begin + i / a.group) * BQ; };
  auto stage = [&](int i, uint8_t* ql, uint8_t* dl) {
    const int h = g * a.group + i % a.group;
    const int m0 = step_m0(i);
    stage_tile_buf<BQ, ROWB, 4, D / 8>(qrs, m0 * q_ld_b + h * D * 2, q_ld_b, lq - m0, ql, wave, lane);
    stage_tile_buf<BQ, ROWBV, 4, DV / 8>(drs, m0 * do_ld_b + h * DV * 2, do_ld_b, lq - m0, dl, wave, lane);
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
      for (int s = 0; s < KS; ++s) asm volatile("" : "+a"(kreg[s]));
#pragma unroll
      for (int s = 0; s < KSV; ++s) asm volatile("" : "+a"(vreg[s]));
    }
    const auto& lov = [&]() -> const auto& {
      if constexpr (D == DV) return loffs; else return loffsv;
    }();
    if (full)
      K::template step<false>(ql, dl, loffs, lov, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act);
    else
      K::template step<true>(ql, dl, loffs, lov, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act);
  };

  if (nsteps > 0) stage(0, q_lds0, do_lds0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int i = 0; i < nsteps; i += 2) {
    if (i + 1 < nsteps) stage(i + 1, q_lds1, do_lds1);
    if (fetch != nullptr && i + 1 == nsteps) fetch->issue();  // (uniform)
    compute(i, q_lds0, do_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 1 >= nsteps) break;
    if (i + 2 < nsteps) stage(i + 2, q_lds0, do_lds0);
    if (fetch != nullptr && i + 2 == nsteps) fetch->issue();
    compute(i + 1, q_lds1, do_lds1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Each wave stores its 32 keys' dK and dV rows through one of the (now
  // idle) tile buffers, rows in consecutive lanes.
  constexpr int ST_BYTES = TileStore<NDB>::BYTES > TileStore<NDBV>::BYTES ? TileStore<NDB>::BYTES
                                                                          : TileStore<NDBV>::BYTES;
  if constexpr (ST_BYTES <= TB && ST_BYTES <= TBV) {
    if (wave_active) {
      uint8_t* sl = wave == 0 ? q_lds0 : wave == 1 ? q_lds1 : wave == 2 ? do_lds0 : do_lds1;
      const int nrows = min(32, lk - k0w);
      TileStore<NDB>::store(dkacc, a.dk_scale, sl, a.dk, ((long)(ks + k0w) * a.hkv + g) * D, (long)a.hkv * D,
                            nrows, a.out_kind, lane);
      TileStore<NDBV>::store(dvacc, a.act.pscale, sl, a.dv, ((long)(ks + k0w) * a.hkv + g) * DV, (long)a.hkv * DV,
                             nrows, a.out_kind, lane);
    }
  } else if (wave_active && kj < lk) {
    const long orow = ((long)(ks + kj) * a.hkv + g) * D, vrow = ((long)(ks + kj) * a.hkv + g) * DV;
    const float gs = a.dk_scale, ps = a.act.pscale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        store4(a.dk, orow + d, dkacc[db][4 * i4] * gs, dkacc[db][4 * i4 + 1] * gs, dkacc[db][4 * i4 + 2] * gs,
               dkacc[db][4 * i4 + 3] * gs, a.out_kind);
        if (db < NDBV)
          store4(a.dv, vrow + d, dvacc[db < NDBV ? db : 0][4 * i4] * ps, dvacc[db < NDBV ? db : 0][4 * i4 + 1] * ps,
                 dvacc[db < NDBV ? db : 0][4 * i4 + 2] * ps, dvacc[db < NDBV ? db : 0][4 * i4 + 3] * ps,
                 a.out_kind);
      }
    }
  }
  return nsteps > 0;
  };

  if (a.counters == nullptr) {
    // Block -> work item: (sequence, KV head) pair on one XCD, costliest
    // sequences first; within a pair, key blocks run in ascending order: a
    // bottom-right causal mask shows a key block to no more queries than the
    // blocks before it, and without a mask a partial last block goes last.
    WorkItem w;
    if (!map_work(blockIdx.x, a.batch, a.hkv, a.nblocks, a.perm, w)) return;
    process(w.b, w.g, w.rest, nullptr);
  } else {
    // Per-XCD work queue over the same pairs, costliest sequence first (one
    // workgroup per CU here, so the dispatcher's in-order hand-out of one
    // item per workgroup would leave CUs idle between items).
    run_queue(a.counters + (blockIdx.x & (kNumXcd - 1)), xcd_items(a.batch, a.hkv, a.nblocks),
              [&](int j, QueueFetch& fetch) __attribute__((always_inline)) {
                WorkItem w;
                xcd_item(j, a.hkv, a.nblocks, a.perm, w);
                return process(w.b, w.g, w.rest, &fetch);
              });
  }
}

// ------------------------------------------------------------ fused backward
// dK, dV and dQ in one pass (the five products of the gradient, no
// recomputation).  Work items are the dK/dV kernel's (sequence, KV head,
// 128-key block); each step also adds the workgroup's partial dQ of one
// (64-row query tile, query head) into an fp32 accumulator.  The partials of a
// tile are added in a fixed order (the contributing key blocks in descending
// order; the first one stores, a sole contributor stores the final value), so
// the sum is bitwise reproducible: a per-tile turn counter says how many
// contributors have finished, and a workgroup waits for its turn before it
// reads the tile.  The flash-attention summary describes deterministic
// backward passes built on such semaphore-ordered reductions.
//
// The tile's read-modify-write is a plain load / add / store in L2: every
// workgroup that adds into a tile runs on the same XCD (one L2), because work
// is handed out from per-XCD queues that only workgroups of the owning XCD
// (hardware XCC id) drain.  Loads bypass the per-CU L1; a workgroup's stores
// complete (vmcnt(0)) before a barrier, after which one thread stores the
// tile's next turn into its counter, which waiters poll in L2 (see poll_l2).  Queue order equals turn order (key blocks
// descending within a (sequence, KV head) pair), and a workgroup takes its
// next item only once it has finished the current one, so a workgroup only
// ever waits for items handed out before its own, which are running: the
// waits cannot deadlock.  Each wait is bounded anyway; one that gives up sets
// an error flag (read back by the host in its debug mode) and goes on.
//
// Pipeline per step i: the stream computes S, dP, dV, dK of step i, writes
// dS_i to the LDS dS tile, and computes dQ of step i-1 from the other dS tile;
// after the stream the workgroup waits for the turn of tile i-1 and issues the
// loads of its current sums; after the end-of-step barrier it adds and stores
// them; the counter is bumped after the next step's barrier.

// Hardware id of the XCD (XCC) the workgroup runs on.
__device__ __forceinline__ int hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & (kNumXcd - 1);
}

// Key blocks [n_lo, n_hi] that contribute to 64-row query tile m of a
// sequence (empty when n_lo > n_hi): block n reaches the tile iff its first
// visible query lies in or before it (128 n < 64 m + 64 + wr + off) and its
// last visible query in or after it (128 n + 128 + wl - off > 64 m).
// Arithmetic shifts are floor divisions of the possibly negative numerators.
__device__ __forceinline__ void dq_contributors(int m, int lk, int off, int wl, int wr, int& n_lo, int& n_hi) {
  n_hi = (lk + kBwdBN - 1) / kBwdBN - 1;
  if (wr >= 0) n_hi = min(n_hi, (kDqTile * m + kDqTile - 1 + wr + off) >> 7);
  n_lo = wl >= 0 ? max(0, (kDqTile * m - wl + off) >> 7) : 0;
}

// Turn counters live in L2 like the sums they order: every workgroup that
// polls or bumps the counter of a tile runs on the XCD that owns the tile's
// queue.  A release is a plain store of the next turn (one writer per turn)
// after the tile's sums were stored and acknowledged (vmcnt(0)) and the
// workgroup's barrier; a poll is a load with the sc1 policy.  Measured on
// gfx950: a load with sc1 (or nt) misses the CU's L1 and reads the XCD's L2,
// so it sees another CU's plain store on the same XCD, while a plain or sc0
// load can keep hitting a stale L1 line; stores in one XCD's L2 are not seen
// from another XCD's, and agent-scope atomics, which are, each take a round
// trip past L2.  The counters are zeroed by a separate kernel before each
// call; kernel boundaries make memory coherent across XCDs.
__device__ __forceinline__ int32_t poll_l2(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16);
}
// Atomic read (add 0) of a word shared across XCDs (the queue state and the
// error flag).
__device__ __forceinline__ int32_t poll(int32_t* p) {
  return __hip_atomic_fetch_add(p, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until the counter at byte offset `off` of `ctr` equals want; false if
// it gave up after `limit` polls (a negative limit gives up at once), or
// because another wait already gave up (every later wait then ends quickly).
__device__ __forceinline__ bool wait_turn(__amdgpu_buffer_rsrc_t ctr, unsigned off, int want, int32_t* err, int limit) {
  int it = 0;
  for (;;) {
    if (poll_l2(ctr, off) == want) break;
    if (++it > limit || ((it & 255) == 0 && poll(err) != 0)) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    // a memory fence in the loop keeps the compiler from hoisting the poll
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_s_sleep(2);
  }
  // later loads of the tile stay behind the poll
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return true;
}

// fp32 loads that miss the CU's L1 and read the XCD's L2 (sc1 policy), so they
// see the sums other CUs of the XCD stored.
__device__ __forceinline__ float load_l2(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16));
}
__device__ __forceinline__ void store_f32(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void store_16(__amdgpu_buffer_rsrc_t r, unsigned off, float v, int kind) {
  const uint32_t w = kind == OUT_F16 ? pack2<EL_F16>(v, 0.0f) : pack2<EL_BF16>(v, 0.0f);
  __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w & 0xffffu), r, (int)off, 0, 0);
}

// Items of queue q: the (sequence, KV head) pairs p with p % 8 == q, per_pair
// items each.
__device__ __forceinline__ int queue_items(int q, int batch, int hkv, int per_pair) {
  const int pairs = batch * hkv;
  return pairs > q ? (pairs - q + kNumXcd - 1) / kNumXcd * per_pair : 0;
}

// Next item for a workgroup on XCD xcc: from its own queue, else from a queue
// that no XCD has claimed yet (claimed for xcc) or that xcc already owns.
// Returns the queue (or -1 when no work is left) and the item index in *j.
__device__ __forceinline__ int fused_fetch(int32_t* qs, int xcc, int batch, int hkv, int per_pair, int* j) {
  for (int k = 0; k < kNumXcd; ++k) {
    const int q = (xcc + k) & (kNumXcd - 1);
    int own = poll(qs + kQOwner + q);
    if (own == 0) {
      int expected = 0;
      __hip_atomic_compare_exchange_strong(qs + kQOwner + q, &expected, xcc + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      own = expected == 0 ? xcc + 1 : expected;
    }
    if (own != xcc + 1) continue;
    const int total = queue_items(q, batch, hkv, per_pair);
    if (poll(qs + kQNext + q) >= total) continue;
    const int i = __hip_atomic_fetch_add(qs + kQNext + q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < total) {
      *j = i;
      return q;
    }
  }
  return -1;
}

template <int D, int ACT, int EL, bool SPLIT, bool DSPL>
__global__ __launch_bounds__(256, 1) void gdpa_bwd_fused_kernel(const BwdArgs a) {
  using K = DkdvKernel<D, ACT, EL, SPLIT, true, DSPL>;
  constexpr int BNB = kBwdBN;  // keys per workgroup (32 per wave)
  constexpr int BQ = K::BQ, KS = K::KS, NDB = K::NDB, ROWB = K::ROWB, TB = K::TB, DQB = K::DQB;
  constexpr int DSB = K::DS_TILE;
  static_assert(BQ == kDqTile, "dQ tiles are the steps' query blocks");
  static_assert(BNB * ROWB <= 2 * DSB, "the K tile is staged in the dS tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t do_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t ds_lds[2 * DSB];
  __shared__ int32_t s_item[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;
  const int xcc = hw_xcc_id();
  // This wave's share of dQ: head-dim block dbw of both query blocks (head
  // dims 96, 128; at 96 the fourth wave repeats block 2 and stores nothing),
  // or of query block qbw (head dim 64).
  const int dbw = D == 64 ? (wave & 1) : min(wave, NDB - 1);
  const int qbw = D == 64 ? (wave >> 1) : 0;
  const bool dq_owner = D == 64 || wave < NDB;
  const TileOffs<ROWB> loffs = TileOffs<ROWB>::make(lane);
  int dsa[2], dsb[2], ktro[2];
  K::DsOffs::tr_of(lane, qbw, dsa);
  K::DsOffs::tr_of(lane, 1, dsb);
  TileOffs<ROWB>::tr_of(lane, dbw, ktro);  // K^T operand of this wave's head-dim block
  const int esz_out = a.out_kind == OUT_F32 ? 4 : 2;

  auto process = [&](int b, int g, int nblk) __attribute__((always_inline)) {
    int qs, lq, ks, lk;
    seq_bounds(a, b, qs, lq, ks, lk);
    const int off = lk - lq;
    const int tile0 = a.cu_q != nullptr ? (qs >> 6) + b : b * a.mt_fixed;  // first turn-counter tile
    const long qrow_f = (long)a.hq * D;                                    // elements per token row of dq
    // Output rows of this sequence (all heads), range-checked: rows past the
    // sequence's end are dropped by the resource bounds.
    const __amdgpu_buffer_rsrc_t dqo_rs =
        make_rsrc(static_cast<uint8_t*>(a.dq) + (long)qs * qrow_f * esz_out, lq * (int)qrow_f * esz_out);
    const __amdgpu_buffer_rsrc_t acc_rs = make_rsrc(a.dq_acc + (long)qs * qrow_f, lq * (int)qrow_f * 4);

    // Query tiles no key block contributes to (queries that see no key):
    // written as zeros by the sequence's first key block item.
    if (nblk == 0) {
      const int mt = (lq + kDqTile - 1) / kDqTile;
      constexpr int RB = D * 2;  // bytes of one (row, head) in a 16-bit output; doubled for fp32
      for (int m = 0; m < mt; ++m) {
        int n_lo, n_hi;
        dq_contributors(m, lk, off, a.wl, a.wr, n_lo, n_hi);
        if (n_lo <= n_hi) continue;
        const int rowb = RB * esz_out / 2, chunks = rowb / 16;
        for (int idx = tid; idx < kDqTile * a.group * chunks; idx += 256) {
          const int r = idx / (a.group * chunks), rest = idx % (a.group * chunks);
          const int h = g * a.group + rest / chunks, c = rest % chunks;
          const unsigned o = (unsigned)(((kDqTile * m + r) * a.hq + h) * rowb + 16 * c);
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, dqo_rs, (int)o, 0, 0);
        }
      }
    }
    const int n0 = nblk * BNB;
    if (n0 >= lk) return;
    const int k0w = n0 + wave * 32;
    const bool wave_active = k0w < lk;
    const int kj = k0w + (lane & 31);  // this lane's key
    const int kmax_w = min(k0w + 31, lk - 1);
    const int klast = min(n0 + BNB, lk) - 1;
    const int ilo_l = a.wr >= 0 ? kj - a.wr - off : 0;
    const int ihi_l = min(lq - 1, a.wl >= 0 ? kj + a.wl - off : lq - 1);
    int i_lo = 0, i_hi = lq;
    if (a.wr >= 0) i_lo = max(0, n0 - a.wr - off);
    if (a.wl >= 0) i_hi = min(lq, klast + a.wl - off + 1);
    const int mb_begin = i_lo / BQ;
    const int mb_end = (i_hi > i_lo) ? (i_hi + BQ - 1) / BQ : mb_begin;
    const int nsteps = (mb_end - mb_begin) * a.group;

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

    if (nsteps > 0) {
      const int q_ld_b = a.hq * D * 2;
      const __amdgpu_buffer_rsrc_t qrs =
          make_rsrc(static_cast<const uint8_t*>(a.q) + (long)qs * q_ld_b, lq * q_ld_b);
      const __amdgpu_buffer_rsrc_t drs =
          make_rsrc(static_cast<const uint8_t*>(a.dout) + (long)qs * q_ld_b, lq * q_ld_b);
      auto step_m0 = [&](int i) __attribute__((always_inline)) { return (mb_begin + i / a.group) * BQ; };
      auto stage = [&](int i, uint8_t* ql, uint8_t* dl) __attribute__((always_inline)) {
        const int h = g * a.group + i % a.group;
        const int m0 = step_m0(i);
        const int o = m0 * q_ld_b + h * D * 2;
        stage_tile_buf<BQ, ROWB, 4, D / 8>(qrs, o, q_ld_b, lq - m0, ql, wave, lane);
        stage_tile_buf<BQ, ROWB, 4, D / 8>(drs, o, q_ld_b, lq - m0, dl, wave, lane);
      };
      // K of the block, staged in the dS tiles, read once as the B operand of
      // dQ (this wave's head-dim block, 8 steps of 16 keys)
      const long kv_ld_b = kv_ld * 2;
      const __amdgpu_buffer_rsrc_t krs =
          make_rsrc(static_cast<const uint8_t*>(a.k) + (long)ks * kv_ld_b + (long)g * D * 2, lk * (int)kv_ld_b);
      stage_tile_buf<BNB, ROWB, 4, D / 8>(krs, n0 * (int)kv_ld_b, (int)kv_ld_b, lk - n0, ds_lds, wave, lane);
      stage(0, q_lds0, do_lds0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      u32x4 ktr[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) ktr[s] = tr_at(ds_lds, ktro, 16 * s * ROWB);
      __syncthreads();

      f32x16 dqacc[DQB];
      float old[DQB][16];
      // flush state of the tile whose dQ sits in dqacc (uniform per workgroup)
      int fl_idx = -1, fl_m = 0, fl_h = 0, fl_turn = 0;
      bool fl_first = false, fl_last = false, fl_single = false;
      int rel = -1, rel_val = 0;  // turn counter to set (to rel_val) after the current step's barrier

      // Element (query block j, register r) of this lane lies at element
      // base(m, h, j) + roff[r] of the sequence's dQ rows: query row
      // 64 m + 32 qb + 4 hf + 8 (r / 4) + r % 4, column 32 dbw + lane % 32.
      const int row_el = a.hq * D;  // elements per token row
      const int lane_el = 4 * hf * row_el + dbw * 32 + (lane & 31);
      auto base = [&](int m, int h, int j) __attribute__((always_inline)) {
        const int qb = DQB == 2 ? j : qbw;
        return (unsigned)((kDqTile * m + 32 * qb) * row_el + h * D + lane_el);
      };
      auto roff = [&](int r) __attribute__((always_inline)) { return (unsigned)((8 * (r >> 2) + (r & 3)) * row_el); };
      const __amdgpu_buffer_rsrc_t turn_rs = make_rsrc(a.turn, 0x7fffffff);
      auto start_flush = [&](int i) __attribute__((always_inline)) {  // dqacc holds dQ of step i
        const int m = mb_begin + i / a.group, h = g * a.group + i % a.group;
        int n_lo, n_hi;
        dq_contributors(m, lk, off, a.wl, a.wr, n_lo, n_hi);
        fl_m = m;
        fl_h = h;
        fl_idx = (tile0 + m) * a.hq + h;
        fl_turn = n_hi - nblk;
        fl_first = nblk == n_hi;
        fl_last = nblk == n_lo;
        fl_single = n_lo == n_hi;
        if (dq_owner && !fl_first) {
          wait_turn(turn_rs, 4u * (unsigned)fl_idx, fl_turn, a.qstate + kQErr, a.spin_limit);
#pragma unroll
          for (int j = 0; j < DQB; ++j) {
            const unsigned b0 = base(m, h, j);
#pragma unroll
            for (int r = 0; r < 16; ++r) old[j][r] = load_l2(acc_rs, 4 * (b0 + roff(r)));
          }
        }
      };
      auto finish_flush = [&]() __attribute__((always_inline)) {
        if (fl_idx < 0) return;
        if (dq_owner) {
          const float gs = a.dq_scale;
          const bool out16 = a.out_kind != OUT_F32 && (fl_single || fl_last);
#pragma unroll
          for (int j = 0; j < DQB; ++j) {
            const unsigned b0 = base(fl_m, fl_h, j);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float v = fl_first ? dqacc[j][r] * gs : __builtin_fmaf(dqacc[j][r], gs, old[j][r]);
              if (out16)
                store_16(dqo_rs, 2 * (b0 + roff(r)), v, a.out_kind);
              else
                store_f32(acc_rs, 4 * (b0 + roff(r)), v);
            }
          }
        }
        if (!fl_last) {  // hand the tile to the next contributor
          rel = fl_idx;
          rel_val = fl_turn + 1;
        }
        fl_idx = -1;
      };
      auto end_step = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (rel >= 0 && tid == 0)
          __builtin_amdgcn_raw_buffer_store_b32((uint32_t)rel_val, turn_rs, (int)(4u * (unsigned)rel), 0, 0);
        rel = -1;
      };
      auto compute = [&](int i, const uint8_t* ql, const uint8_t* dl, uint8_t* dsw, const uint8_t* dsr)
                         __attribute__((always_inline)) {
        const int krow = wave * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < DQB; ++j) dqacc[j] = f32x16{};
        const int m0 = step_m0(i), mhi = m0 + BQ - 1;
        bool empty = !wave_active, full = true;
        if (a.wr >= 0) {
          empty |= k0w > min(mhi, lq - 1) + off + a.wr;
          full &= kmax_w <= m0 + off + a.wr;
        }
        if (a.wl >= 0) {
          empty |= kmax_w < m0 + off - a.wl;
          full &= k0w >= mhi + off - a.wl;
        }
        if (empty) {
          // this wave's keys see none of the step's queries: dS = 0
          K::zero_ds(dsw, krow, hf);
          K::dq_only(dsr, dsa, dsb, ktr, dqacc);
          return;
        }
        int mlo[2], mhi2[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int base = m0 + qb * 32 + hf * 4;
          mlo[qb] = ilo_l - base;
          mhi2[qb] = ihi_l - base;
        }
        if constexpr (D > 64) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            asm volatile("" : "+a"(kreg[s]));
            asm volatile("" : "+a"(vreg[s]));
          }
        }
        if (full)
          K::template step<false>(ql, dl, loffs, loffs, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act, dsw, dsr, dsa,
                                  dsb, ktr, dqacc, krow, hf);
        else
          K::template step<true>(ql, dl, loffs, loffs, kreg, vreg, dkacc, dvacc, mlo, mhi2, a.act, dsw, dsr, dsa,
                                 dsb, ktr, dqacc, krow, hf);
      };
      // one step over fixed LDS buffers: (ql, dl) this step's tiles, (qn, dn)
      // the next step's, dsw / dsr the dS tiles written / read
      auto half = [&](int i, const uint8_t* ql, const uint8_t* dl, uint8_t* qn, uint8_t* dn, uint8_t* dsw,
                      const uint8_t* dsr) __attribute__((always_inline)) {
        finish_flush();
        if (i + 1 < nsteps) stage(i + 1, qn, dn);
        compute(i, ql, dl, dsw, dsr);
        if (i >= 1) start_flush(i - 1);
        end_step();
      };
      uint8_t* ds0 = ds_lds;
      uint8_t* ds1 = ds_lds + DSB;
      for (int i = 0; i < nsteps; i += 2) {
        half(i, q_lds0, do_lds0, q_lds1, do_lds1, ds0, ds1);
        if (i + 1 >= nsteps) break;
        half(i + 1, q_lds1, do_lds1, q_lds0, do_lds0, ds1, ds0);
      }
      // drain: dQ of the last step
      finish_flush();
#pragma unroll
      for (int j = 0; j < DQB; ++j) dqacc[j] = f32x16{};
      K::dq_only(((nsteps - 1) & 1) ? ds1 : ds0, dsa, dsb, ktr, dqacc);
      start_flush(nsteps - 1);
      end_step();
      finish_flush();
      end_step();
    }

    if (wave_active && kj < lk) {
      const long orow = ((long)(ks + kj) * a.hkv + g) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = db * 32 + hf * 4 + 8 * i4;
          const float gs = a.dk_scale, ps = a.act.pscale;
          store4(a.dk, orow + d, dkacc[db][4 * i4] * gs, dkacc[db][4 * i4 + 1] * gs, dkacc[db][4 * i4 + 2] * gs,
                 dkacc[db][4 * i4 + 3] * gs, a.out_kind);
          store4(a.dv, orow + d, dvacc[db][4 * i4] * ps, dvacc[db][4 * i4 + 1] * ps, dvacc[db][4 * i4 + 2] * ps,
                 dvacc[db][4 * i4 + 3] * ps, a.out_kind);
        }
      }
    }
  };

  // Items in queue order: pairs (sequence, KV head) p with p % 8 == q in rank
  // order, key blocks last-first; the next item is taken once the current
  // one is done.
  for (;;) {
    if (tid == 0) {
      int j = 0;
      const int q = fused_fetch(a.qstate, xcc, a.batch, a.hkv, a.nblocks, &j);
      s_item[0] = q;
      s_item[1] = j;
    }
    __syncthreads();
    const int q = s_item[0], j = s_item[1];
    __syncthreads();
    if (q < 0) break;
    const int pair = (j / a.nblocks) * kNumXcd + q;
    const int rank = pair / a.hkv;
    process(a.perm != nullptr ? a.perm[rank] : rank, pair % a.hkv, a.nblocks - 1 - j % a.nblocks);
  }
}

// ----------------------------------------------------------------------- dQ
// D: head dim of Q and K (S, dQ); DV: that of V and dO (dP), smaller only at
// (192, 128).
template <int D, int ACT, int EL, bool SPLIT, int DV = D>
struct DqKernel {
  static constexpr int BN = 8192 / lds_dim(D) < 64 ? 64 : 8192 / lds_dim(D);  // keys per KV tile
  static constexpr int NKB = BN / 32;
  static constexpr int KS = D / 16;              // k-steps of S
  static constexpr int KSV = DV / 16;            // k-steps of dP
  static constexpr int NDB = D / 32;
  static constexpr int ROWB = 2 * lds_dim(D);    // LDS row bytes of a K tile (96 padded to 128)
  static constexpr int ROWBV = 2 * lds_dim(DV);  // LDS row bytes of a V tile
  static_assert(KSV <= KS, "V's head dim is at most K's");

  static constexpr int NP = SPLIT ? 2 : 1;   // 16-bit words per dS element
  static constexpr int NA = KS;               // S/dP units per key block (2 MFMAs each)
  static constexpr int NB = 2 * NDB;          // dQ units per key block (NP MFMAs each)
  static constexpr int NU = 2 * NA + 2 * NB;  // units of a pair of key blocks
  static constexpr int PREF = 2;              // units of operand prefetch
  using LaneOffs = TileOffs<ROWB>;
  using LaneOffsV = TileOffs<ROWBV>;

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
                                                   const LaneOffs& lo, const LaneOffsV& lov, u32x4& o0, u32x4& o1) {
    if (u < 2 * NA) {
      const int kb = kb0 + u / NA, s = u % NA;
      o0 = row_at(kl, lo.row[s] + kb * 32 * ROWB);
      o1 = s < KSV ? row_at(vl, lov.row[s < KSV ? s : 0] + kb * 32 * ROWBV) : o0;
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
                                                    const LaneOffsV& lov, const u32x4* qreg, const u32x4* doreg,
                                                    f32x16* dqacc,
                                                    const int* mlo, const int* mhi, const ActConsts& k) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}}, dpacc[2] = {f32x16{}, f32x16{}};
    u32x4 ds[2][NP][2];
    u32x4 ring[PREF + 1][2];
#pragma unroll
    for (int u = 0; u < PREF; ++u) load_unit(u, kb0, kl, vl, lo, lov, ring[u][0], ring[u][1]);
    auto unit_body = [&](const int u) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      if (u + PREF < NU)
        load_unit(u + PREF, kb0, kl, vl, lo, lov, ring[(u + PREF) % (PREF + 1)][0],
                  ring[(u + PREF) % (PREF + 1)][1]);
      const u32x4& o0 = ring[u % (PREF + 1)][0];
      const u32x4& o1 = ring[u % (PREF + 1)][1];
      if (u < 2 * NA) {
        const int j = u / NA, s = u % NA;
        sacc[j] = mfma16<EL>(o0, qreg[s], sacc[j]);
        if (s < KSV) dpacc[j] = mfma16<EL>(o1, doreg[s < KSV ? s : 0], dpacc[j]);
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
    };
    if constexpr (D != DV) {
      // the 48-unit stream of head dim 192 exceeds the unroller's threshold:
      // issue it with compile-time unit indices
      static_for<0, NU>([&](auto uc) __attribute__((always_inline)) { unit_body(decltype(uc)::value); });
    } else {
#pragma unroll
      for (int u = 0; u < NU; ++u) unit_body(u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Two workgroups per CU, except where the activation gradient needs more
// registers than two waves per SIMD leave at D = 128 (exact GELU, and SiLU
// with dS carried as a hi/lo pair).
template <int D, int ACT, bool SPLIT>
constexpr int dq_occupancy() {
  return D > 128 || (D == 128 && (ACT == ACT_GELU || (SPLIT && ACT == ACT_SILU))) ? 1 : 2;
}

template <int D, int ACT, int EL, bool SPLIT, int DV = D>
__global__ __launch_bounds__(256, (dq_occupancy<D, ACT, SPLIT>())) void gdpa_bwd_dq_kernel(const BwdArgs a) {
  using K = DqKernel<D, ACT, EL, SPLIT, DV>;
  constexpr int BM = kBwdBM;
  constexpr int BN = K::BN, NKB = K::NKB, KS = K::KS, KSV = K::KSV, NDB = K::NDB, ROWB = K::ROWB;
  constexpr int ROWBV = K::ROWBV;
  constexpr int TB = BN * ROWB, TBV = BN * ROWBV;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TBV];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TBV];

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

  const long q_ld = (long)a.hq * D, do_ld = (long)a.hq * DV;
  u32x4 qreg[KS], doreg[KSV];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (long)(qs + min(qi, lq - 1)) * q_ld + h * D + hf * 8;
    const uint16_t* dp =
        static_cast<const uint16_t*>(a.dout) + (long)(qs + min(qi, lq - 1)) * do_ld + h * DV + hf * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = load16_or_zero(qp + s * 16, qi < lq);
#pragma unroll
    for (int s = 0; s < KSV; ++s) doreg[s] = load16_or_zero(dp + s * 16, qi < lq);
  }
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};
  const TileOffs<ROWB> loffs = TileOffs<ROWB>::make(lane);
  const TileOffs<ROWBV> loffsv = TileOffs<ROWBV>::make(lane);
  const auto& lov = [&]() -> const auto& {
    if constexpr (D == DV) return loffs; else return loffsv;
  }();

  const long kv_ld_b = (long)a.hkv * D * 2, vv_ld_b = (long)a.hkv * DV * 2;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + (long)ks * kv_ld_b + (long)g * D * 2;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + (long)ks * vv_ld_b + (long)g * DV * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, lk * (int)kv_ld_b);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, lk * (int)vv_ld_b);
  auto stage = [&](int nb, uint8_t* kl, uint8_t* vl) {
    const int n0 = nb * BN;
    stage_tile_buf<BN, ROWB, 4, D / 8>(krs, n0 * (int)kv_ld_b, (int)kv_ld_b, lk - n0, kl, wave, lane);
    stage_tile_buf<BN, ROWBV, 4, DV / 8>(vrs, n0 * (int)vv_ld_b, (int)vv_ld_b, lk - n0, vl, wave, lane);
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
        K::template block_pair<false>(kl, vl, kb0, loffs, lov, qreg, doreg, dqacc, mlo, mhi, a.act);
      else
        K::template block_pair<true>(kl, vl, kb0, loffs, lov, qreg, doreg, dqacc, mlo, mhi, a.act);
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

  // Each wave stores its 32 query rows of dQ through one of the (now idle)
  // tile buffers, rows in consecutive lanes.
  if constexpr (TileStore<NDB>::BYTES <= TB && TileStore<NDB>::BYTES <= TBV) {
    if (wave_active) {
      uint8_t* sl = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
      TileStore<NDB>::store(dqacc, a.dq_scale, sl, a.dq, ((long)(qs + q0w) * a.hq + h) * D, (long)a.hq * D,
                            min(32, lq - q0w), a.out_kind, lane);
    }
  } else if (wave_active && qi < lq) {
    const long orow = ((long)(qs + qi) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + hf * 4 + 8 * i4;
        const float gs = a.dq_scale;
        store4(a.dq, orow + d, dqacc[db][4 * i4] * gs, dqacc[db][4 * i4 + 1] * gs, dqacc[db][4 * i4 + 2] * gs,
               dqacc[db][4 * i4 + 3] * gs, a.out_kind);
      }
    }
  }
  };

  // Block -> work item: (sequence, KV head) pair on one XCD, costliest
  // sequences first; within a pair, query blocks run last-first.
  WorkItem w;
  if (!map_work(blockIdx.x, a.batch, a.hkv, a.group * a.mblocks, a.perm, w)) return;
  process(w.b, w.g, w.g * a.group + w.rest / a.mblocks, a.mblocks - 1 - w.rest % a.mblocks);
}

template <int D, int EL, bool SPLIT_KV, bool SPLIT_DS>
static hipError_t launch_bwd_fused(const BwdArgs& a, int act_kind, hipStream_t stream) {
  // as many workgroups as are resident at once (one per CU), drawing from
  // the per-XCD queues
  const dim3 g((unsigned)queue_grid(a.ncu, 1)), blk(256);
  switch (act_kind) {
#define GDPA_FUSED_CASE(K)                                                                      \
  case K:                                                                                       \
    hipLaunchKernelGGL((gdpa_bwd_fused_kernel<D, K, EL, SPLIT_KV, SPLIT_DS>), g, blk, 0, stream, a); \
    break;
    GDPA_FUSED_CASE(ACT_IDENTITY)
    GDPA_FUSED_CASE(ACT_GELU)
    GDPA_FUSED_CASE(ACT_GELU_TANH)
    GDPA_FUSED_CASE(ACT_RELU)
    GDPA_FUSED_CASE(ACT_RELU2)
    GDPA_FUSED_CASE(ACT_LEAKY)
    GDPA_FUSED_CASE(ACT_SILU)
    GDPA_FUSED_CASE(ACT_HARDSWISH)
#undef GDPA_FUSED_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Fused launches of one input element kind and head dim, instantiated in
// their own translation units (gdpa_bwdf_<type>_<dim>.hip): hipcc's pass that
// rewrites MFMA register forms fails on the fused kernels' long unit streams
// when MFMA results are forced into architectural VGPRs, so those units are
// built with the compiler's own choice of MFMA register form.
template <int EL, int D>
hipError_t launch_bwd_fused_ed(const BwdArgs& a, int act_kind, hipStream_t stream) {
  // P / dS split for dK and dV (few queries) or dS split for dQ (few keys),
  // not both
  if (a.kvsplit && a.dsplit) return hipErrorInvalidValue;
  if constexpr (EL == EL_F16) {
    if (a.kvsplit || a.dsplit) return hipErrorInvalidValue;
    return launch_bwd_fused<D, EL, false, false>(a, act_kind, stream);
  } else {
    if (a.kvsplit) return launch_bwd_fused<D, EL, true, false>(a, act_kind, stream);
    return a.dsplit ? launch_bwd_fused<D, EL, false, true>(a, act_kind, stream)
                    : launch_bwd_fused<D, EL, false, false>(a, act_kind, stream);
  }
}
#define GDPA_BWDF_EXTERN(EL, D) extern template hipError_t launch_bwd_fused_ed<EL, D>(const BwdArgs&, int, hipStream_t);
GDPA_BWDF_EXTERN(EL_BF16, 64)
GDPA_BWDF_EXTERN(EL_BF16, 96)
GDPA_BWDF_EXTERN(EL_BF16, 128)
GDPA_BWDF_EXTERN(EL_F16, 64)
GDPA_BWDF_EXTERN(EL_F16, 96)
GDPA_BWDF_EXTERN(EL_F16, 128)
#undef GDPA_BWDF_EXTERN

template <int D, int EL, bool SPLIT_KV, bool SPLIT_Q, int DV = D>
static hipError_t launch_bwd_ds(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, bool fused,
                                hipStream_t stream) {
  if (fused) {
    // dQ accumulated in the dK/dV pass (equal head dims only)
    if (!want_dq || !want_dkv) return hipErrorInvalidValue;
    if constexpr (D == DV)
      return launch_bwd_fused_ed<EL, D>(a, act_kind, stream);
    else
      return hipErrorInvalidValue;
  }
  // dK/dV work queue: as many workgroups as are resident at once
  const bool queue = a.counters != nullptr;
  const long grid_kv = !want_dkv ? 0 : queue ? -1 : pair_grid(a.batch, a.hkv, a.nblocks);
  const long grid_q = !want_dq ? 0 : pair_grid(a.batch, a.hkv, a.group * a.mblocks);
  dim3 blk(256);
  switch (act_kind) {
#define GDPA_BWD_CASE(K)                                                                                       \
  case K:                                                                                                      \
    if (grid_kv != 0)                                                                                          \
      hipLaunchKernelGGL((gdpa_bwd_dkdv_kernel<D, K, EL, SPLIT_KV, DV>),                                           \
                         dim3((unsigned)(grid_kv > 0 ? grid_kv                                                 \
                                                     : queue_grid(a.ncu, dkdv_occupancy<D, K, SPLIT_KV>()))), \
                         blk, 0, stream, a);                                                                   \
    if (grid_q > 0)                                                                                            \
      hipLaunchKernelGGL((gdpa_bwd_dq_kernel<D, K, EL, SPLIT_Q, DV>), dim3((unsigned)grid_q), blk, 0, stream, a); \
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

template <int D, int EL, int DV = D>
static hipError_t launch_bwd_d(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, bool fused,
                               hipStream_t stream) {
  // fp16 never splits P or dS (the host keeps a single word within tolerance)
  if constexpr (EL == EL_F16) {
    if (a.kvsplit || a.dsplit) return hipErrorInvalidValue;
    return launch_bwd_ds<D, EL, false, false, DV>(a, act_kind, want_dq, want_dkv, fused, stream);
  }
  if (a.kvsplit)
    return a.dsplit ? launch_bwd_ds<D, EL, true, true, DV>(a, act_kind, want_dq, want_dkv, fused, stream)
                    : launch_bwd_ds<D, EL, true, false, DV>(a, act_kind, want_dq, want_dkv, fused, stream);
  return a.dsplit ? launch_bwd_ds<D, EL, false, true, DV>(a, act_kind, want_dq, want_dkv, fused, stream)
                  : launch_bwd_ds<D, EL, false, false, DV>(a, act_kind, want_dq, want_dkv, fused, stream);
}

// Backward launches of one input element kind and (Q/K, V) head dims.  Each
// is instantiated in its own translation unit (gdpa_bwd_<type>_<dim>.hip), so
// the library's kernels compile in parallel; gdpa_bwd.hip dispatches.
template <int EL, int D, int DV = D>
hipError_t launch_bwd_ed(const BwdArgs& a, int act_kind, bool want_dq, bool want_dkv, bool fused,
                         hipStream_t stream) {
  return launch_bwd_d<D, EL, DV>(a, act_kind, want_dq, want_dkv, fused, stream);
}
#define GDPA_BWD_EXTERN(EL, D, DV)                                                                            \
  extern template hipError_t launch_bwd_ed<EL, D, DV>(const BwdArgs&, int, bool, bool, bool, hipStream_t);
GDPA_BWD_EXTERN(EL_BF16, 64, 64)
GDPA_BWD_EXTERN(EL_BF16, 96, 96)
GDPA_BWD_EXTERN(EL_BF16, 128, 128)
GDPA_BWD_EXTERN(EL_BF16, 192, 128)
GDPA_BWD_EXTERN(EL_F16, 64, 64)
GDPA_BWD_EXTERN(EL_F16, 96, 96)
GDPA_BWD_EXTERN(EL_F16, 128, 128)
GDPA_BWD_EXTERN(EL_F16, 192, 128)
#undef GDPA_BWD_EXTERN

}  // namespace gdpa
