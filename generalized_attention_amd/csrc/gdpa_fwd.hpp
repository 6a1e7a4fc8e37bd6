// GDPA forward kernel for gfx950.
//
// Computes O = M .* act(scale * Q K^T) V per (sequence, query head): the GDPA
// definition of the GDPA README (intro; softmax replaced by an activation, no
// normaliser).  Because nothing is normalised, every KV tile adds an exact
// partial sum to O: there is no running maximum, no rescaling and no final
// division, unlike softmax flash attention.
//
// Work decomposition: one workgroup of 4 waves per (sequence, query head,
// 128-row query block); wave w owns 32 query rows.  Per KV tile of
// BN = 8192/D keys:
//   * K and V are copied HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging), row-major with 16-byte chunks XOR-swizzled by the row index;
//     tiles are double-buffered, the next tile's copy is in flight while the
//     current tile is computed;
//   * S^T = K Q^T on v_mfma_f32_32x32x16 (Q^T stays in registers as the B
//     operand for the whole loop), then scale, mask and activation in
//     registers;
//   * P^T is packed to V's 16-bit type straight from the accumulators and is the B
//     operand of O^T += V^T P^T.  The V^T operand comes from the row-major V
//     tile through ds_read_b64_tr_b16, whose 16-lane transpose hands each lane
//     4 consecutive keys of one head-dim column, in exactly the key order of
//     the accumulator rows.
// Two 32-key blocks are issued as one interleaved stream so the activation
// of one block runs on the vector ALU under the other block's MFMAs.
// Work items are taken (sequence, KV head) pair by pair, each pair's blocks on
// one XCD, costliest sequences first, query blocks last-first (the README's
// "Features" names load-balanced tile scheduling for jagged inputs).
#pragma once

#include "gdpa_common.hpp"
#include "gdpa_kernels.hpp"

namespace gdpa {

// The N E8M0 scale bytes of one MXFP8 row (N = 2 or 4; the row's scales start
// at a multiple of N bytes), in one 32-bit value, byte b for head-dim block b.
template <int N>
__device__ __forceinline__ uint32_t load_scales(const uint8_t* p) {
  static_assert(N == 2 || N == 4, "head dims 64 and 128");
  if constexpr (N == 4)
    return *reinterpret_cast<const uint32_t*>(p);
  else
    return *reinterpret_cast<const uint16_t*>(p);
}

// D: head dim of Q and K; DV: head dim of V and O.
template <int D, int ACT, int IN, bool PSPLIT, int NW, int DV = D>
struct FwdKernel {
  static constexpr bool MX4 = IN == EL_MX4;   // MXFP4 Q/K: E2M1 pairs per byte with an E8M0 scale per 32 head dims
  static constexpr bool MX = IN == EL_MX8 || MX4;  // block-scaled (MXFP8: E4M3 codes with an E8M0 scale per 32)
  static constexpr bool FP8 = IN == EL_FP8 || IN == EL_MX8;  // one byte per Q/K element
  static constexpr bool NARROW = FP8 || MX4;                // Q K^T on the K = 64 MFMA
  static constexpr int EL = IN == EL_F16 ? EL_F16 : EL_BF16;  // V, P (and 16-bit Q, K)
  static_assert(!MX || D % 64 == 0, "MX formats: every head-dim block of 32 on the K = 64 MFMA");
  static constexpr int BM = 32 * NW;
  static constexpr int DPK = lds_dim(D);  // head dims of the LDS rows of K and V
  static constexpr int DPV = lds_dim(DV);
  static constexpr int BN = 8192 / (DPK > DPV ? DPK : DPV) < 64 ? 64 : 8192 / (DPK > DPV ? DPK : DPV);  // keys per tile
  static constexpr int NKB = BN / 32;     // 32-key blocks per tile
  static constexpr int KS = D / 16;       // k-steps of Q K^T
  static constexpr int NDB = DV / 32;     // 32-row blocks of O^T
  static constexpr int KROWB = MX4 ? DPK / 2 : FP8 ? DPK : 2 * DPK;
  static constexpr int VROWB = 2 * DPV;
  // FP8 Q K^T: the first 64 * NK64 head-dim bytes on the K = 64 MFMA (lane
  // half h of unit s < NK64 holds bytes [64 s + 32 h, +32) of its K row and of
  // its Q row, two 16-byte pieces each), the remaining 16 * NK16 bytes on the
  // K = 16 MFMA (8 bytes per lane half, as for 16-bit inputs)
  // (MXFP4: unit s on the K = 64 MFMA takes bytes [32 s + 16 h, +16) in lane half h)
  static constexpr int NK64 = NARROW ? D / 64 : 0;
  static constexpr int NK16 = FP8 ? (D % 64) / 16 : 0;
  static constexpr int NQR = MX4 ? NK64 : FP8 ? (NK64 > 0 ? 2 * NK64 : 1) : KS;  // 16-byte Q registers
  static constexpr int NQR8 = NK16 > 0 ? NK16 : 1;                  // 8-byte FP8 Q registers
  static constexpr int NP = PSPLIT ? 2 : 1;  // 16-bit words per P element (hi, lo)
  static constexpr int NA = NARROW ? NK64 + NK16 : KS;  // S units per key block (1 MFMA each)
  static constexpr int NB = 2 * NDB;         // P V units per key block (NP MFMAs each)
  static constexpr int NU = 2 * NA + 2 * NB;
  // units of operand prefetch (8- and 4-bit Q K^T: one MFMA per key block,
  // so a deeper ring covers more of the LDS latency; measured 2 % faster)
  static constexpr int PREF = NARROW ? 3 : 2;
  using KOffs = TileOffs<NARROW ? VROWB : KROWB>;  // row reads of 16-bit K (unused for 8- and 4-bit K)
  using VOffs = TileOffs<VROWB>;                 // transposed reads of V

  // One pair of accumulator elements (key rows 8t+2w, +1) -> packed P words.
  template <bool MASK>
  static __device__ __forceinline__ void pair(const f32x16& s, int t, int w, uint32_t mbits, u32x4 (*p)[2],
                                              const ActConsts& k) {
    float y[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * t + 2 * w + u;
      float v = Act<ACT>::f(s[r], k);
      if constexpr (MASK) v = keep_bits(v, mbits, r);
      y[u] = v;
    }
    const uint32_t h2 = pack2<EL>(y[0], y[1]);
    p[0][t][w] = h2;
    if constexpr (PSPLIT) p[1][t][w] = split2<EL>(y[0], y[1], h2);
  }

  // Unit u of a key-block pair (blocks kb0, kb0+1): u < 2 NA: S of block
  // u / NA, k-step u % NA (A operand: K rows); else P V of block
  // (u - 2 NA) / NB, key-row half t, head-dim block db (A operand: V^T).
  static __device__ __forceinline__ u32x4 load_unit(int u, int kb0, const uint8_t* kl, const uint8_t* vl,
                                                    const KOffs& lo, const VOffs& vo, int lane, u32x4& hi) {
    if (u < 2 * NA) {
      const int kb = kb0 + u / NA, s = u % NA;
      if constexpr (MX4) {
        // head-dim block 2 s + h: bytes [32 s + 16 h, +16) of the K row
        hi = u32x4{0u, 0u, 0u, 0u};
        return *reinterpret_cast<const u32x4*>(kl + lds_off<KROWB>(kb * 32 + (lane & 31), 2 * s + (lane >> 5)));
      } else if constexpr (FP8) {
        const int row = kb * 32 + (lane & 31);
        if (s < NK64) {
          // FP8: bytes [64 s + 32 h, +32) in lane half h.  MXFP8: the block
          // scales apply per 32 k-values made of the first 16 bytes of both
          // lane halves (block 2 s, scale from half 0) and their last 16 bytes
          // (block 2 s + 1, from half 1), so half h holds head dims
          // [64 s + 16 h, +16) and [64 s + 32 + 16 h, +16)
          const int h = lane >> 5;
          const int c = MX ? 4 * s + h : 4 * s + 2 * h;
          hi = *reinterpret_cast<const u32x4*>(kl + lds_off<KROWB>(row, MX ? c + 2 : c + 1));
          return *reinterpret_cast<const u32x4*>(kl + lds_off<KROWB>(row, c));
        }
        const u32x2 v = *reinterpret_cast<const u32x2*>(kl + lds_off<KROWB>(row, 4 * NK64 + s - NK64) +
                                                         (lane >> 5) * 8);
        return u32x4{v[0], v[1], 0u, 0u};
      } else {
        return row_at(kl, lo.row[s] + kb * 32 * KROWB);
      }
    }
    const int v = u - 2 * NA, kb = kb0 + v / NB, t = (v % NB) / NDB, db = v % NDB;
    return tr_at(vl, vo.tr[db], (kb * 32 + 16 * t) * VROWB);
  }

  // S^T = K Q^T of two 32-key blocks against this wave's 32 queries, P =
  // act(S) (masked to each lane's allowed keys when MASK), and O^T += V^T P^T,
  // as one stream of units whose LDS operands are read PREF units ahead; the
  // activation of block 0 rides under block 1's S units, that of block 1
  // under block 0's P V units.  mlo/mhi[j]: this lane's allowed-key range
  // relative to block j's accumulator base.
  template <bool MASK>
  static __device__ __forceinline__ void block_pair(const uint8_t* kl, const uint8_t* vl, int kb0, const KOffs& lo,
                                                    const VOffs& vo, int lane, const u32x4* qreg, const u32x2* qreg8, f32x16* oacc,
                                                    const int* mlo, const int* mhi, const ActConsts& k,
                                                    const uint32_t* ksc = nullptr, uint32_t qsc = 0) {
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    u32x4 p[2][NP][2];
    uint32_t mbits[2] = {0u, 0u};
    if constexpr (MASK) {
      mbits[0] = range_bits(mlo[0], mhi[0]);
      mbits[1] = range_bits(mlo[1], mhi[1]);
    }
    u32x4 ring[PREF + 1], ring_hi[PREF + 1];  // ring_hi: second 16 bytes of K = 64 FP8 units
#pragma unroll
    for (int u = 0; u < PREF; ++u) ring[u] = load_unit(u, kb0, kl, vl, lo, vo, lane, ring_hi[u]);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      // the units with no activation work (S of block 0, P V of block 1) run
      // at raised priority, so the other wave on the SIMD fills the vector
      // ALU with its activation while these keep the matrix core busy
      // (measured: 2-4 % shorter 16-bit forwards at two waves per SIMD; the
      // 8- and 4-bit forwards, at three waves per SIMD and one S MFMA per
      // key block, ran 1-4 % faster without it)
      if (!NARROW && (u == 0 || u == 2 * NA + NB)) __builtin_amdgcn_s_setprio(3);
      if (!NARROW && u == NA) __builtin_amdgcn_s_setprio(0);
      if (u + PREF < NU)
        ring[(u + PREF) % (PREF + 1)] =
            load_unit(u + PREF, kb0, kl, vl, lo, vo, lane, ring_hi[(u + PREF) % (PREF + 1)]);
      const u32x4& op = ring[u % (PREF + 1)];
      if (u < 2 * NA) {
        const int j = u / NA, s = u % NA;
        if constexpr (MX4) {
          const int sh = 16 * s + 8 * (lane >> 5);
          sacc[j] = mfma_fp4_k64_scaled(op, qreg[s], sacc[j], (ksc[j] >> sh) & 0xffu, (qsc >> sh) & 0xffu);
        } else if constexpr (FP8) {
          if constexpr (MX) {
            // lane half h supplies the scale of head-dim block 2 s + h (its key's / query's)
            const int sh = 16 * s + 8 * (lane >> 5);
            sacc[j] = mfma_fp8_k64_scaled(op, ring_hi[u % (PREF + 1)], qreg[2 * s], qreg[2 * s + 1], sacc[j],
                                          (ksc[j] >> sh) & 0xffu, (qsc >> sh) & 0xffu);
          } else if (s < NK64)
            sacc[j] = mfma_fp8_k64(op, ring_hi[u % (PREF + 1)], qreg[2 * s], qreg[2 * s + 1], sacc[j]);
          else
            sacc[j] = mfma_fp8(u32x2{op[0], op[1]}, qreg8[s - NK64], sacc[j]);
        }
        else
          sacc[j] = mfma16<EL>(op, qreg[s], sacc[j]);
      } else {
        const int v = u - 2 * NA, j = v / NB, t = (v % NB) / NDB, db = v % NDB;
#pragma unroll
        for (int h = 0; h < NP; ++h) oacc[db] = mfma16<EL>(op, p[j][h][t], oacc[db]);
      }
      if (u >= NA && u < 2 * NA + NB) {
        const int j = u < 2 * NA ? 0 : 1;
        const int v = u < 2 * NA ? u - NA : u - 2 * NA;
        const int span = u < 2 * NA ? NA : NB;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (pair_at(q, v, span)) pair<MASK>(sacc[j], q >> 2, q & 3, mbits[j], p[j], k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  }
};

template <int D, int ACT, int IN, bool PSPLIT, int NW, int DV>
__global__ __launch_bounds__(64 * NW) void gdpa_fwd_kernel(const FwdArgs a) {
  using K = FwdKernel<D, ACT, IN, PSPLIT, NW, DV>;
  constexpr bool FP8 = K::FP8;
  constexpr int BM = K::BM, BN = K::BN, KS = K::KS, NDB = K::NDB, NKB = K::NKB;
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

  const int q0w = row0 + wave * 32;  // first query row of this wave
  const bool wave_active = q0w < lq;
  const int qmax_w = min(q0w + 31, lq - 1);
  const int hf = lane >> 5;
  const int qi = q0w + (lane & 31);
  // keys this lane's query may see: [jlo, jhi]
  const int jlo = a.wl >= 0 ? qi + off - a.wl : 0;
  const int jhi = min(lk - 1, a.wr >= 0 ? qi + off + a.wr : lk - 1);

  // Q^T as the B operand of S^T = K Q^T: lane holds query qi, 8 head-dim values per k-step
  // (FP8: 32 bytes [64 s + 32 hf, +32) per K = 64 unit, then 8 bytes per K = 16 unit).
  const long q_ld = (long)a.hq * D;
  u32x4 qreg[K::NQR];
  u32x2 qreg8[K::NQR8];
  {
    const long qrow = (long)(qs + min(qi, lq - 1)) * q_ld + h * D + hf * 8;
    if constexpr (K::MX4) {
      // MXFP4 (two elements per byte): bytes [32 s + 16 hf, +16) of the row, as for K
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (qrow - hf * 8) / 2;
#pragma unroll
      for (int s = 0; s < K::NK64; ++s) qreg[s] = load16_or_zero(qp + 32 * s + 16 * hf, qi < lq);
    } else if constexpr (FP8) {
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + (qrow - hf * 8);
#pragma unroll
      for (int s = 0; s < K::NK64; ++s) {
        // the same byte layout as the K operand (see load_unit)
        const int o0 = K::MX ? 64 * s + 16 * hf : 64 * s + 32 * hf, o1 = K::MX ? o0 + 32 : o0 + 16;
        qreg[2 * s] = load16_or_zero(qp + o0, qi < lq);
        qreg[2 * s + 1] = load16_or_zero(qp + o1, qi < lq);
      }
#pragma unroll
      for (int t = 0; t < K::NK16; ++t) qreg8[t] = load8_or_zero(qp + 64 * K::NK64 + 16 * t + 8 * hf, qi < lq);
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow;
#pragma unroll
      for (int s = 0; s < KS; ++s) qreg[s] = load16_or_zero(qp + s * 16, qi < lq);
    }
  }

  // MXFP8: the E8M0 scales of this lane's query (byte b: head-dim block b)
  uint32_t qsc = 0;
  if constexpr (K::MX) qsc = load_scales<D / 32>(a.q_mx + ((long)(qs + min(qi, lq - 1)) * a.hq + h) * (D / 32));

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  const typename K::KOffs loffs = K::KOffs::make(lane);
  const typename K::VOffs voffs = K::VOffs::make(lane);

  const int esz2 = K::MX4 ? 1 : FP8 ? 2 : 4;  // bytes per two K elements
  const long kv_ld = (long)a.hkv * D, v_ld = (long)a.hkv * DV;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + ((long)ks * kv_ld + g * D) * esz2 / 2;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + ((long)ks * v_ld + g * DV) * 2;

  // Byte ranges of this sequence's K and V rows (all KV heads), addressed by
  // 32-bit offsets; the host keeps them below 2^31.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, lk * (int)kv_ld * esz2 / 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, lk * (int)v_ld * 2);
  auto stage = [&](int nb, uint8_t* kl, uint8_t* vl) {
    const int n0 = nb * BN;
    stage_tile_buf<BN, K::KROWB, NW, D * esz2 / 32>(krs, n0 * (int)kv_ld * esz2 / 2, (int)kv_ld * esz2 / 2,
                                                   lk - n0, kl, wave, lane);
    stage_tile_buf<BN, K::VROWB, NW, DV / 8>(vrs, n0 * (int)v_ld * 2, (int)v_ld * 2, lk - n0, vl, wave, lane);
  };
  // MX formats: the E8M0 scales of this lane's key in each 32-key block of a
  // tile, loaded with the tile's copy (one tile ahead), so the wait before the
  // tile's math covers them instead of a load inside it
  constexpr int NKS = K::MX ? NKB : 1;
  uint32_t ks_a[NKS], ks_b[NKS];
  auto load_ks = [&](int nb, uint32_t* kss) __attribute__((always_inline)) {
    if constexpr (K::MX) {
      const int n0 = nb * BN;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key = min(n0 + kb * 32 + (lane & 31), lk - 1);
        kss[kb] = load_scales<D / 32>(a.k_mx + ((long)(ks + key) * a.hkv + g) * (D / 32));
      }
    }
  };
  // One tile of math for this wave, two 32-key blocks at a time; the mask is
  // applied only where the window cuts a block (K and V rows past the last key
  // are staged as zeros and add nothing).
  auto compute = [&](int nb, const uint8_t* kl, const uint8_t* vl, const uint32_t* kss)
                     __attribute__((always_inline)) {
    if (!wave_active) return;
    const int n0 = nb * BN;
#pragma unroll
    for (int kb0 = 0; kb0 < NKB; kb0 += 2) {
      bool any = false, all_full = true;
      int mlo[2], mhi[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int b_lo = n0 + (kb0 + j) * 32, b_hi = b_lo + 31;  // keys of this 32-key block
        bool empty = b_lo >= lk, full = true;
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
      // MX formats: the E8M0 scales of this lane's key in each of the two blocks
      uint32_t ksc[2] = {0u, 0u};
      if constexpr (K::MX) {
        ksc[0] = kss[kb0];
        ksc[1] = kss[kb0 + 1];
      }
      if (all_full)
        K::template block_pair<false>(kl, vl, kb0, loffs, voffs, lane, qreg, qreg8, oacc, mlo, mhi, a.act, ksc, qsc);
      else
        K::template block_pair<true>(kl, vl, kb0, loffs, voffs, lane, qreg, qreg8, oacc, mlo, mhi, a.act, ksc, qsc);
    }
  };

  if (nb_begin < nb_end) {
    stage(nb_begin, k_lds0, v_lds0);
    load_ks(nb_begin, ks_a);
  }
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): tile copy landed
  __syncthreads();
  for (int nb = nb_begin; nb < nb_end; nb += 2) {
    if (nb + 1 < nb_end) {
      stage(nb + 1, k_lds1, v_lds1);
      load_ks(nb + 1, ks_b);
    }
    compute(nb, k_lds0, v_lds0, ks_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nb + 1 >= nb_end) break;
    if (nb + 2 < nb_end) {
      stage(nb + 2, k_lds0, v_lds0);
      load_ks(nb + 2, ks_a);
    }
    compute(nb + 1, k_lds1, v_lds1, ks_b);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: each wave stores its 32 rows of O through one of the (now
  // idle) tile buffers, rows in consecutive lanes; where a tile buffer is too
  // small (FP8 K), lanes store 4 consecutive head-dim values per register group
  if (!wave_active) return;
  if constexpr (NW == 4 && TileStore<NDB>::BYTES <= KBYTES && TileStore<NDB>::BYTES <= VBYTES) {
    uint8_t* sl = wave == 0 ? v_lds0 : wave == 1 ? v_lds1 : wave == 2 ? k_lds0 : k_lds1;
    TileStore<NDB>::store(oacc, a.act.pscale, sl, a.o, ((long)(qs + q0w) * a.hq + h) * DV, (long)a.hq * DV,
                          min(32, lq - q0w), a.out_kind, lane);
    return;
  }
  if (qi >= lq) return;
  const long orow = ((long)(qs + qi) * a.hq + h) * DV;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = db * 32 + hf * 4 + 8 * i4;
      const float ps = a.act.pscale;
      store4(a.o, orow + d, oacc[db][4 * i4] * ps, oacc[db][4 * i4 + 1] * ps, oacc[db][4 * i4 + 2] * ps,
             oacc[db][4 * i4 + 3] * ps, a.out_kind);
    }
  }
  };

  // Block -> work item: (sequence, KV head) pair on one XCD, costliest
  // sequences first; within a pair, query blocks run last-first.
  WorkItem w;
  if (!map_work(blockIdx.x, a.batch, a.hkv, a.group * a.mblocks, a.perm, w)) return;
  process(w.b, w.g, w.g * a.group + w.rest / a.mblocks, a.mblocks - 1 - w.rest % a.mblocks);
}

template <int D, int IN, int DV = D>
static hipError_t launch_fwd_d(const FwdArgs& a, int act_kind, hipStream_t stream) {
  // fp16 never splits P (the host keeps a single word within tolerance)
  if (IN == EL_F16 && a.psplit) return hipErrorInvalidValue;
  dim3 g((unsigned)fwd_grid(a)), blk(64 * kFwdNW);
  switch (act_kind) {
#define GDPA_FWD_CASE(K)                                                                          \
  case K:                                                                                         \
    if (IN == EL_F16 || !a.psplit)                                                                \
      hipLaunchKernelGGL((gdpa_fwd_kernel<D, K, IN, false, kFwdNW, DV>), g, blk, 0, stream, a);   \
    else                                                                                          \
      hipLaunchKernelGGL((gdpa_fwd_kernel<D, K, IN, true, kFwdNW, DV>), g, blk, 0, stream, a);    \
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

// Forward launches of one input element kind (each kind is instantiated in
// its own translation unit).  Head dims (Q/K, V): (64, 64), (96, 96),
// (128, 128), and (192, 128) for 16-bit inputs.
template <int IN>
static hipError_t launch_fwd_in(const FwdArgs& a, int head_dim, int head_dim_v, int act_kind, hipStream_t stream) {
  if constexpr (IN == EL_MX8 || IN == EL_MX4) {
    if (head_dim == head_dim_v && head_dim == 64) return launch_fwd_d<64, IN>(a, act_kind, stream);
    if (head_dim == head_dim_v && head_dim == 128) return launch_fwd_d<128, IN>(a, act_kind, stream);
    return hipErrorInvalidValue;
  } else {
    if (head_dim == head_dim_v) {
      if (head_dim == 64) return launch_fwd_d<64, IN>(a, act_kind, stream);
      if (head_dim == 96) return launch_fwd_d<96, IN>(a, act_kind, stream);
      if (head_dim == 128) return launch_fwd_d<128, IN>(a, act_kind, stream);
    }
    if constexpr (IN != EL_FP8)
      if (head_dim == 192 && head_dim_v == 128) return launch_fwd_d<192, IN, 128>(a, act_kind, stream);
    return hipErrorInvalidValue;
  }
}

}  // namespace gdpa
