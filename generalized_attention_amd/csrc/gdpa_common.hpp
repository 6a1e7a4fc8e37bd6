// Device-side building blocks shared by the GDPA kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_{bf16,fp8}):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l holds column l%32, the same k range
//   C (32 x 32): lane l holds column l%32, rows 4*(l/32) + 8*(r/4) + r%4 in
//                accumulator register r (0..15)
// A C tile therefore feeds the next product directly as a B operand that
// contracts over the C tile's rows: with S^T = K Q^T (keys x queries) in
// registers, O^T = V^T P^T takes P^T straight from the accumulators, provided
// the key order of the V^T operand follows the accumulator's row order.  The
// transposed LDS tiles below store their columns in exactly that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gdpa_kernels.hpp"

namespace gdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_fp8(const u32x2& a, const u32x2& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(__builtin_bit_cast(long, a),
                                                    __builtin_bit_cast(long, b), c, 0, 0, 0);
}

// FP8 E4M3 x E4M3 over 64 k-values per MFMA (gfx950's K = 64 form, twice the
// FP8 rate of the K = 16 form): each lane supplies 32 bytes of A (a0, a1) and of
// B (b0, b1).  The sum runs over every byte position, so any assignment of
// k-values to (lane half, byte) works if A and B use the same one.  No block
// scaling: the scale operands are 0, which selects the unscaled instruction.
__device__ __forceinline__ f32x16 mfma_fp8_k64(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                               const f32x16& c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same with E8M0 block scales (the OCP MX formats), sa and sb from byte 0
// of the scale operands.  The 64 k-values of a row form two blocks of 32: the
// first 16 bytes of lane halves 0 and 1 (scaled by 2^(s - 127) of the half-0
// lane: lane i for A row i, lane j for B column j) and their last 16 bytes
// (scaled by the half-1 lane's, i + 32 or j + 32); measured on gfx950.
__device__ __forceinline__ f32x16 mfma_fp8_k64_scaled(const u32x4& a0, const u32x4& a1, const u32x4& b0,
                                                      const u32x4& b1, const f32x16& c, uint32_t sa, uint32_t sb) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// FP4 E2M1 x E2M1 over 64 k-values with E8M0 block scales (the OCP MXFP4
// format): each lane supplies 16 bytes of A and of B, 32 elements, two per
// byte, element 2 i in the low nibble of byte i.  Measured on gfx950: the
// instruction reads 4 registers per operand, nibble i of lane l pairs with
// nibble i of the same lane of the other operand, and all 32 elements of a
// lane form one scale block, scaled by that lane's own scale byte (lane half
// h of a row therefore holds head-dim block 2 s + h of unit s).
__device__ __forceinline__ f32x16 mfma_fp4_k64_scaled(const u32x4& a, const u32x4& b, const f32x16& c, uint32_t sa,
                                                      uint32_t sb) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a8 = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 b8 = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// bf16 remainder of a packed pair: lo = bf16(x - float(hi)).
__device__ __forceinline__ uint32_t split_lo(float x0, float x1, uint32_t hi) {
  return pack_bf16x2(x0 - bf16_lo_to_f32(hi), x1 - bf16_hi_to_f32(hi));
}

// ------------------------------------------- 16-bit element types (bf16, fp16)
// Q, K, V, dO are bf16 or fp16 (or, forward only, FP8 Q/K with bf16 V); the
// probabilities P and the score gradients dS are rounded to the type of the
// operand they multiply, so every MFMA contracts two operands of one type.
template <int EL>
__device__ __forceinline__ f32x16 mfma16(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (EL == EL_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return mfma_bf16(a, b, c);
}
// Two fp32 -> two 16-bit values, round to nearest even (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32).
template <int EL>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (EL == EL_F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
  else
    return pack_bf16x2(lo, hi);
}
// Remainder of a packed pair in the same type: lo = round(x - float(hi)).
template <int EL>
__device__ __forceinline__ uint32_t split2(float x0, float x1, uint32_t hi) {
  if constexpr (EL == EL_F16) {
    const f16x2 h = __builtin_bit_cast(f16x2, hi);
    return pack2<EL_F16>(x0 - (float)h[0], x1 - (float)h[1]);
  } else {
    return split_lo(x0, x1, hi);
  }
}
// Four consecutive fp32 results -> output element idx.. of an fp32, bf16 or
// fp16 tensor (OUT_* kind).
__device__ __forceinline__ void store4(void* base, long idx, float x0, float x1, float x2, float x3, int kind) {
  if (kind == OUT_F32)
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = f32x4{x0, x1, x2, x3};
  else if (kind == OUT_BF16)
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = u32x2{pack2<EL_BF16>(x0, x1), pack2<EL_BF16>(x2, x3)};
  else
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = u32x2{pack2<EL_F16>(x0, x1), pack2<EL_F16>(x2, x3)};
}

// Calls f(std::integral_constant<int, i>) for i = I .. N-1 in order: a loop
// whose index is a compile-time constant in the body, with no reliance on the
// loop unroller (long unit streams exceed its default threshold, and a partly
// unrolled stream indexes its register arrays at run time, which moves them
// to scratch memory).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// The unit streams below spread the 8 activation pairs of a 32 x 32 block over
// the `span` MFMA units that follow the block: pair j rides under unit
// (j * span) / 8 (span is 6, 8 or 16 with head dims 96, 128, or a split).
__host__ __device__ constexpr bool pair_at(int j, int v, int span) { return (j * span) / 8 == v; }

// Head dim as laid out in LDS: 96- and 192-wide rows are padded to 128 and
// 256 so the chunk swizzle stays a bijection on whole 256-byte bank sweeps.
__host__ __device__ constexpr int lds_dim(int d) { return d == 96 ? 128 : d == 192 ? 256 : d; }

// ----------------------------------------------------------------- activations
// With c the score scale and s the raw dot product, y(s) satisfies
// act(c s) = pscale * y(s) and d(s) = act'(c s) (constants in ActConsts, set
// on the host from c).  Folding c into the constants removes the per-score
// multiply; pscale and the chain-rule c are applied once per output element.
// Exponentials use v_exp_f32 (2^x) and v_rcp_f32, both accurate to ~1 ulp,
// far below the bf16 rounding applied to P.  tanh-GELU is evaluated as
// x sigmoid(2u), u = sqrt(2/pi)(x + 0.044715 x^3), since 0.5(1 + tanh u) =
// sigmoid(2u).
//   IDENTITY   y = s                          pscale = c   d = 1
//   GELU       y = s (1 + erf(k0 s))          pscale = c/2 d = (1 + erf(k0 s))/2 + a0 s 2^(a1 s^2)
//   GELU_TANH  r = 1/(1 + 2^(s (k0 + k1 s^2))), y = s r, pscale = c,
//              d = r + r (1 - r) s (a0 + a1 s^2)
//   RELU       y = med3(s, a0, a1)            pscale = c   d = [k0 s > 0]
//              ((a0, a1) = (0, +inf) for c >= 0: y = max(s, 0); (-inf, 0) for
//              c < 0: y = min(s, 0), since relu(c s) = c min(s, 0) there)
//   RELU2      y = max(k0 s, 0)^2             pscale = 1   d = 2 max(k0 s, 0)
//   LEAKY      y = s + k1 med3(s, a0, a1)     pscale = p   d = k0 s > 0 ? 1 : alpha
//              (leaky(c s) = A max(s, 0) + B min(s, 0) with (A, B) = (c, alpha c)
//              for c > 0 and (alpha c, c) otherwise; p is the larger of A, B in
//              magnitude and k1 = (the other) / p - 1 on min(s, 0) = med3(s, -inf, 0)
//              or max(s, 0) = med3(s, 0, +inf), so |y| <= |s|; p = 0 when c = 0)
//   SILU       r = 1/(1 + 2^(k0 s)), y = s r, pscale = c, d = r + r (1 - r) a0 s
//   HARDSWISH  y = s clamp(k0 s + 3, 0, 6)    pscale = c/6 d = x < -3 ? 0 : x > 3 ? 1 : x/3 + 1/2 (x = k0 s)
template <int ACT>
struct Act;

template <>
struct Act<ACT_IDENTITY> {
  static __device__ __forceinline__ float f(float s, const ActConsts&) { return s; }
  static __device__ __forceinline__ float f_df(float s, const ActConsts&, float& d) { d = 1.0f; return s; }
};

template <>
struct Act<ACT_RELU> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    return __builtin_amdgcn_fmed3f(s, k.a0, k.a1);
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    d = k.k0 * s > 0.0f ? 1.0f : 0.0f;
    return __builtin_amdgcn_fmed3f(s, k.a0, k.a1);
  }
};

template <>
struct Act<ACT_RELU2> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    const float r = fmaxf(k.k0 * s, 0.0f);
    return r * r;
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    const float r = fmaxf(k.k0 * s, 0.0f);
    d = 2.0f * r;
    return r * r;
  }
};

template <>
struct Act<ACT_LEAKY> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    return __builtin_fmaf(k.k1, __builtin_amdgcn_fmed3f(s, k.a0, k.a1), s);
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    d = k.k0 * s > 0.0f ? 1.0f : k.alpha;
    return __builtin_fmaf(k.k1, __builtin_amdgcn_fmed3f(s, k.a0, k.a1), s);
  }
};

template <>
struct Act<ACT_SILU> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    return s * fast_rcp(1.0f + fast_exp2(k.k0 * s));
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    const float r = fast_rcp(1.0f + fast_exp2(k.k0 * s));
    const float y = s * r;
    d = __builtin_fmaf(k.a0 * y, 1.0f - r, r);  // r + r (1 - r) a0 s, reusing y = s r
    return y;
  }
};

template <>
struct Act<ACT_GELU_TANH> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    return s * fast_rcp(1.0f + fast_exp2(s * __builtin_fmaf(k.k1, s * s, k.k0)));
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    const float s2 = s * s;
    const float r = fast_rcp(1.0f + fast_exp2(s * __builtin_fmaf(k.k1, s2, k.k0)));
    const float y = s * r;
    d = __builtin_fmaf(y * __builtin_fmaf(k.a1, s2, k.a0), 1.0f - r, r);  // reusing y = s r
    return y;
  }
};

template <>
struct Act<ACT_GELU> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) { return s * (1.0f + erff(k.k0 * s)); }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    const float e = 1.0f + erff(k.k0 * s);
    d = __builtin_fmaf(k.a0 * s, fast_exp2(k.a1 * s * s), 0.5f * e);
    return s * e;
  }
};

template <>
struct Act<ACT_HARDSWISH> {
  static __device__ __forceinline__ float f(float s, const ActConsts& k) {
    return s * fminf(fmaxf(__builtin_fmaf(k.k0, s, 3.0f), 0.0f), 6.0f);
  }
  static __device__ __forceinline__ float f_df(float s, const ActConsts& k, float& d) {
    const float x = k.k0 * s;
    d = x < -3.0f ? 0.0f : (x > 3.0f ? 1.0f : __builtin_fmaf(x, 1.0f / 3.0f, 0.5f));
    // k0 s + 3 as one fused multiply-add, as in f: left to the compiler, the
    // contraction of x + 3 depends on the surrounding code, and kernels that
    // must agree bitwise (and the forward) would round P differently
    return s * fminf(fmaxf(__builtin_fmaf(k.k0, s, 3.0f), 0.0f), 6.0f);
  }
};

// Element-wise mask of a 32x32 accumulator block: element r sits at offset
// c_r = 8 (r/4) + r%4 (plus a lane-dependent base) along the accumulator rows;
// it is kept iff lo <= c_r <= hi, where lo/hi are the allowed range relative to
// that base (two compares and one select per element).
__device__ __forceinline__ bool in_range(int r, int lo, int hi) {
  const int c = 8 * (r >> 2) + (r & 3);
  return c >= lo && c <= hi;
}
// The same mask as a bit set, built once per block: bit c of range_bits(lo,
// hi) is set iff lo <= c <= hi (c in 0..31).  keep_bits clears a masked
// element with one sign-extending bit-field extract (0 or all ones) and one
// AND of its bits, which leaves +0 where the element is masked.
__device__ __forceinline__ uint32_t range_bits(int lo, int hi) {
  const int l = min(max(lo, 0), 32), h = min(max(hi, -1), 31) + 1;  // bits [l, h)
  const uint32_t below_h = h >= 32 ? ~0u : (1u << h) - 1u;
  const uint32_t below_l = l >= 32 ? ~0u : (1u << l) - 1u;
  return below_h & ~below_l;
}
__device__ __forceinline__ float keep_bits(float v, uint32_t bits, int r) {
  const int c = 8 * (r >> 2) + (r & 3);
  return __uint_as_float(__float_as_uint(v) & (uint32_t)__builtin_amdgcn_sbfe((int)bits, c, 1));
}

// ------------------------------------------------------------- global loads
// Loads below are branch-free: an out-of-range row is redirected to row
// nvalid-1 (callers guarantee nvalid >= 1) and its value replaced by zero with
// a select.  Keeping every load unconditional lets the compiler count
// outstanding loads exactly, so the prefetch of the next tile is not drained
// (s_waitcnt vmcnt(0)) before the current tile's MFMAs.
__device__ __forceinline__ u32x4 load16_or_zero(const void* p, bool valid) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return valid ? v : u32x4{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ u32x2 load8_or_zero(const void* p, bool valid) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  return valid ? v : u32x2{0u, 0u};
}

// ------------------------------------------------- direct HBM -> LDS row tiles
// Row-major [rows][ROWB bytes] tiles written by LDS-direct 16-byte loads: each
// lane's 16 bytes land at (LDS base of the instruction) + 16 * lane, so the
// chunk swizzle is chosen by picking which source chunk each lane fetches.
// Chunk swizzle f(row).  gfx950's LDS has 64 four-byte banks: a ds_read_b128
// serves 16 lanes per cycle and a ds_read_b64_tr_b16 32 lanes (4 rows x 64
// bytes).  f is a bijection on rows 16m..16m+15 modulo the 256-byte bank
// sweep (16 consecutive rows read row-wise at one chunk hit 16 distinct
// bank quads), and for rows of >= 128 bytes its upper bits put the 64-byte
// column blocks of 4 consecutive rows in distinct quarters of the sweep (a
// transposing read is conflict-free too).  f has period 16 in the row.
template <int ROWB>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (ROWB >= 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (ROWB == 128) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else if constexpr (ROWB == 64) return (row >> 2) & 3;
  // 32-byte rows (MXFP4 K at head dim 64): two chunks; eight rows fill one
  // 256-byte bank sweep, so rows r and r + 8 (read in the same 16-lane pass)
  // take different chunks
  else return (row >> 3) & 1;
}
template <int ROWB>
__device__ __forceinline__ int lds_off(int row, int chunk) {  // byte offset of a 16-byte chunk
  return row * ROWB + ((chunk ^ chunk_swz<ROWB>(row)) << 4);
}

// Issue the HBM -> LDS copy of a [NROW x ROWB-byte] row tile with
// buffer_load_dwordx4 ... lds.  rsrc covers the rows of one sequence (see
// make_rsrc); row0_off is the byte offset of the tile's first row in it, and
// nvalid (>= 1) the number of the sequence's rows from there on.  The resource
// spans exactly the sequence's rows, so tile rows at or past nvalid are read
// at row nvalid, the first row past the end: the range check turns those loads
// into zeros, written to LDS, and no memory is read (offsets are computed
// unsigned; the host keeps every span below 2^31 bytes).  Every activation maps
// 0 to 0 with a finite derivative, so a zero K, V, Q or dO row adds nothing to
// O, dV, dK or dQ, and tiles that run past a sequence's end need no mask.  (The FLAT form,
// global_load_lds, would also work, but the compiler then treats LDS counters
// as unordered and waits for lgkmcnt(0) before every later LDS read.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// GCH: 16-byte chunks per source row (ROWB / 16 unless the LDS row is padded,
// as for head dim 96 in 128-wide rows); lanes of padding chunks re-read a
// chunk of the same row (same cache lines, no extra traffic) and their LDS
// slots are never read.
template <int NROW, int ROWB, int NWAVES, int GCH = ROWB / 16>
__device__ __forceinline__ void stage_tile_buf(__amdgpu_buffer_rsrc_t rsrc, int row0_off, int ld_bytes, int nvalid,
                                               uint8_t* lds, int wave, int lane) {
  constexpr int U = ROWB / 16;
  static_assert(GCH <= U && 2 * GCH >= U, "padding chunks re-read chunks of the same row");
  constexpr int NI = NROW * U / (64 * NWAVES);
  static_assert(NROW * U % (64 * NWAVES) == 0, "tile must be a multiple of NWAVES KiB");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i * NWAVES + wave;
    const int p = blk * 64 + lane;
    const int row = p / U, pc = p % U;
    int c = pc ^ chunk_swz<ROWB>(row);
    if constexpr (GCH < U) c = c < GCH ? c : c - (U - GCH);
    const unsigned voff =
        (unsigned)row0_off + (unsigned)min(row, nvalid) * (unsigned)ld_bytes + (unsigned)(c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16,
                                             (int)voff, 0, 0, 0);
  }
}

// Transposed MFMA A operands come from a row-major 16-bit row tile via
// ds_read_b64_tr_b16.  Within each 16-lane group the instruction hands lane j
// element e of the 8-byte row that lane 4e + j/4 addressed, column j % 4.  So
// if lane r of group g addresses row (r0 + r/4), columns c0 + 4 (r%4) .. +3,
// lane j receives rows r0..r0+3 of column c0 + j.  Lane l thus obtains the A
// operand (row = column index c of the tile, l % 32 within a 32-block; k =
// 8 tile rows) whose k order matches the accumulator row order of a C tile:
// k position 4c' + e  <->  tile row 16 t + 8 c' + 4 (l / 32) + e.  Two such
// reads (c' = 0, 1: rows +0 and +8) make one 16-row operand (tr_at below).
// Row-major A operands: lane l reads row l % 32 of a 32-row block, 8
// consecutive columns at chunk 2 s + l / 32 (row_at below).

// Per-lane byte offsets of the MFMA operands inside a row-major swizzled
// [rows][ROWB bytes] LDS tile (the chunk swizzle has period 16 in the row, so
// one offset per k-step serves every 32-row block and one pair per head-dim
// block every 16-row group):
//   row[s]     : A operand of rows (lane % 32) + 32 j, k-step s     (+ 32 j ROWB)
//   tr[db][c]  : transposed A operand (ds_read_b64_tr_b16 pair, half c) of
//                head-dim block db, tile rows 16 t'                 (+ 16 t' ROWB)
// Keeping just these few registers live, and adding the tile's base and the
// constant parts per read, leaves the register file to the pipelines.
template <int ROWB>
struct TileOffs {
  static constexpr int KS = ROWB / 32;   // 16-element k-steps per row
  static constexpr int NDB = ROWB / 64;  // 32-column head-dim blocks per row
  int row[KS];
  int tr[NDB][2];
  // Transposed-read offsets of head-dim block db (db may be a run-time value:
  // computed, not looked up, so no register array is indexed at run time).
  static __device__ __forceinline__ void tr_of(int lane, int db, int (&o)[2]) {
    const int g = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 8 * c + 4 * (g >> 1) + (rr >> 2);
      const int col = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
      o[c] = row * ROWB + (((col >> 3) ^ chunk_swz<ROWB>(row)) << 4) + ((col & 4) << 1);
    }
  }
  static __device__ __forceinline__ TileOffs make(int lane) {
    TileOffs o;
    const int r = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int s = 0; s < KS; ++s) o.row[s] = r * ROWB + (((2 * s + hf) ^ chunk_swz<ROWB>(r)) << 4);
    const int g = lane >> 4, rr = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int row = 8 * c + 4 * (g >> 1) + (rr >> 2);
        const int col = 32 * db + 16 * (g & 1) + 4 * (rr & 3);
        o.tr[db][c] = row * ROWB + (((col >> 3) ^ chunk_swz<ROWB>(row)) << 4) + ((col & 4) << 1);
      }
    return o;
  }
};
__device__ __forceinline__ u32x4 row_at(const uint8_t* tile, int off) {
  return *reinterpret_cast<const u32x4*>(tile + off);
}
// Transposed operand of a 16-row group: base = byte offset of the group's
// first row, o = the lane's TileOffs pair of the head-dim block.
__device__ __forceinline__ u32x4 tr_at(const uint8_t* tile, const int (&o)[2], int base) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(tile + (o[0] + base)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(tile + (o[1] + base)));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------- coalesced tile store
// A wave's 32-row result tile in the accumulator layout the kernels end with
// (lane l owns output row l % 32; register 4 i + j of column block db holds
// column 32 db + 4 (l / 32) + 8 i + j), written so that consecutive lanes
// cover consecutive bytes of one row.  Stored straight from the accumulators,
// each 16-byte-per-lane store instruction would touch 32 rows with 32 bytes
// in each; the tile instead goes through a row-major LDS copy of itself, and
// every store covers whole rows (two rows of 512 bytes for fp32 at head dim
// 128).  LDS chunk c of row r sits at chunk position c ^ (r % 16) of a row
// padded to a multiple of 16 chunks, so the 16 lanes of each write (16 rows,
// one chunk) and of each read (one row, 16 chunks) hit 16 distinct bank
// quads.  The stores go through a buffer resource that ends at row nrows, so
// the hardware drops the rows past the end and no store needs a branch.  The
// LDS region (BYTES) is the wave's own and must be free: callers pass a tile
// buffer after the loop's last barrier.  A wave's LDS accesses complete in
// issue order, so no wait separates the write from the read-back.
template <int NDB>
struct TileStore {
  static constexpr int NC = NDB * 8;              // 16-byte chunks per fp32 row
  static constexpr int RS = (NC + 15) / 16 * 16;  // LDS row stride in chunks
  static constexpr int BYTES = 32 * RS * 16;      // LDS bytes per wave
  static constexpr int NR = NC / 2;               // 16-byte reads per lane
  static __device__ __forceinline__ int off(int r, int c) { return (r * RS + (c ^ (r & 15))) << 4; }
  // out + base: element (row 0, column 0) of the tile; ld: elements between
  // rows; rows at or past nrows are not written; kind: OUT_* element type.
  static __device__ __forceinline__ void store(const f32x16 (&acc)[NDB], float scale, uint8_t* lds, void* out,
                                               long base, long ld, int nrows, int kind, int lane) {
    // (an opaque copy of the lane id keeps the compiler from computing the
    // addresses below ahead of the kernel's main loop, where they would hold
    // registers through it)
    asm volatile("" : "+v"(lane));
    lane &= 63;
    const int r = lane & 31, hf = lane >> 5;
    // chunk 8 db + 2 i4 + hf of row r: the XOR only touches the low 4 bits,
    // so its position is 16 (db / 2) + ((8 (db % 2) + 2 i4) ^ (hf ^ r % 16))
    const int wbase = (r * RS) << 4, wy = hf ^ (r & 15);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(lds + wbase + ((16 * (db >> 1) + ((8 * (db & 1) + 2 * i4) ^ wy)) << 4)) =
            f32x4{acc[db][4 * i4] * scale, acc[db][4 * i4 + 1] * scale, acc[db][4 * i4 + 2] * scale,
                  acc[db][4 * i4 + 3] * scale};
    const int esz = kind == OUT_F32 ? 4 : 2;
    // base and nrows are the same in every lane of the wave: moved to scalar
    // registers, the resource needs no per-lane loop
    const uint64_t tile = reinterpret_cast<uint64_t>(static_cast<uint8_t*>(out) + base * esz);
    const uint64_t tile_s = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tile) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(tile >> 32)) << 32);
    const int nbytes = __builtin_amdgcn_readfirstlane(nrows > 0 ? nrows * (int)ld * esz : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const void*>(tile_s), nbytes);
    // (all row offsets go into the per-lane offset, which the range check
    // covers)
    f32x4 v[NR];
    int goff[NR];
    if constexpr (64 % NC == 0) {
      // read it covers rows RPI it + r0 (r0 = lane / NC), chunk c = lane % NC;
      // (RPI it) % 16 is a multiple of RPI > r0, so the row's swizzle is
      // (RPI it) % 16 + r0 and the chunk's position (c ^ r0) ^ ((RPI it) % 16)
      constexpr int RPI = 64 / NC;
      const int r0 = lane / NC, c = lane % NC, cx = c ^ r0;
      const int rb = (r0 * RS) << 4;
#pragma unroll
      for (int it = 0; it < NR; ++it)
        v[it] = *reinterpret_cast<const f32x4*>(lds + (it * RPI * RS * 16) + rb + ((cx ^ ((RPI * it) & 15)) << 4));
      const int g0 = (r0 * (int)ld + c * 4) * esz;
#pragma unroll
      for (int it = 0; it < NR; ++it) goff[it] = g0 + it * RPI * (int)ld * esz;
    } else {
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const unsigned idx = (unsigned)(it * 64 + lane);
        v[it] = *reinterpret_cast<const f32x4*>(lds + off((int)(idx / NC), (int)(idx % NC)));
        goff[it] = ((int)(idx / NC) * (int)ld + (int)(idx % NC) * 4) * esz;
      }
    }
    if (kind == OUT_F32) {
#pragma unroll
      for (int it = 0; it < NR; ++it)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[it]), rs, goff[it], 0, 0);
    } else if (kind == OUT_BF16) {
#pragma unroll
      for (int it = 0; it < NR; ++it)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2<EL_BF16>(v[it][0], v[it][1]), pack2<EL_BF16>(v[it][2], v[it][3])},
                                              rs, goff[it], 0, 0);
    } else {
#pragma unroll
      for (int it = 0; it < NR; ++it)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2<EL_F16>(v[it][0], v[it][1]), pack2<EL_F16>(v[it][2], v[it][3])},
                                              rs, goff[it], 0, 0);
    }
  }
};

}  // namespace gdpa
