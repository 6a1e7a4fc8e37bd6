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

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = static_cast<__bf16>(lo);
  __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ----------------------------------------------------------------- activations
// act(x) and act'(x) in fp32.  Exponentials use v_exp_f32 (2^x) and v_rcp_f32;
// both are accurate to about 1 ulp, far below the bf16 rounding applied to P.
// tanh-GELU uses 0.5 x (1 + tanh(u)) = x * sigmoid(2u), u = sqrt(2/pi)(x + 0.044715 x^3).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluC = 0.044715f;
constexpr float kInvSqrt2 = 0.7071067811865476f;
constexpr float kInvSqrt2Pi = 0.3989422804014327f;

template <int ACT>
struct Act;

template <>
struct Act<ACT_IDENTITY> {
  static __device__ __forceinline__ float f(float x, float) { return x; }
  static __device__ __forceinline__ float f_df(float x, float, float& df) { df = 1.0f; return x; }
};

template <>
struct Act<ACT_RELU> {
  static __device__ __forceinline__ float f(float x, float) { return fmaxf(x, 0.0f); }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    df = x > 0.0f ? 1.0f : 0.0f;
    return fmaxf(x, 0.0f);
  }
};

template <>
struct Act<ACT_RELU2> {
  static __device__ __forceinline__ float f(float x, float) { float r = fmaxf(x, 0.0f); return r * r; }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    float r = fmaxf(x, 0.0f);
    df = 2.0f * r;
    return r * r;
  }
};

template <>
struct Act<ACT_LEAKY> {
  static __device__ __forceinline__ float f(float x, float a) { return x >= 0.0f ? x : a * x; }
  static __device__ __forceinline__ float f_df(float x, float a, float& df) {
    df = x > 0.0f ? 1.0f : a;
    return x >= 0.0f ? x : a * x;
  }
};

template <>
struct Act<ACT_SILU> {
  static __device__ __forceinline__ float f(float x, float) {
    return x * fast_rcp(1.0f + fast_exp2(-kLog2e * x));
  }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    float s = fast_rcp(1.0f + fast_exp2(-kLog2e * x));
    df = s * (1.0f + x * (1.0f - s));
    return x * s;
  }
};

template <>
struct Act<ACT_GELU_TANH> {
  // sigmoid(2u) = 1 / (1 + 2^(x * (c0 + c1 x^2)))
  static constexpr float c0 = -2.0f * kSqrt2OverPi * kLog2e;
  static constexpr float c1 = c0 * kGeluC;
  static __device__ __forceinline__ float f(float x, float) {
    float t = x * __builtin_fmaf(c1, x * x, c0);
    return x * fast_rcp(1.0f + fast_exp2(t));
  }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    float x2 = x * x;
    float s = fast_rcp(1.0f + fast_exp2(x * __builtin_fmaf(c1, x2, c0)));
    // d/dx x s(2u) = s + x s (1 - s) 2 u',  2u' = 2 sqrt(2/pi) (1 + 3 c x^2)
    float du2 = 2.0f * kSqrt2OverPi * __builtin_fmaf(3.0f * kGeluC, x2, 1.0f);
    df = __builtin_fmaf(x * s * (1.0f - s), du2, s);
    return x * s;
  }
};

template <>
struct Act<ACT_GELU> {
  static __device__ __forceinline__ float f(float x, float) { return 0.5f * x * (1.0f + erff(x * kInvSqrt2)); }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    float cdf = 0.5f * (1.0f + erff(x * kInvSqrt2));
    df = __builtin_fmaf(x * kInvSqrt2Pi, fast_exp2(-0.5f * kLog2e * x * x), cdf);
    return x * cdf;
  }
};

template <>
struct Act<ACT_HARDSWISH> {
  static __device__ __forceinline__ float f(float x, float) {
    return x * fminf(fmaxf(x + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
  }
  static __device__ __forceinline__ float f_df(float x, float, float& df) {
    df = x < -3.0f ? 0.0f : (x > 3.0f ? 1.0f : __builtin_fmaf(x, 1.0f / 3.0f, 0.5f));
    return x * fminf(fmaxf(x + 3.0f, 0.0f), 6.0f) * (1.0f / 6.0f);
  }
};

// ------------------------------------------------------------- LDS tile layouts
// Row tile: [rows][D] bf16 (row = key or query), 16-byte chunks XOR-swizzled by
// (row & 7) so that 8 consecutive rows read at one chunk hit distinct banks.
template <int D>
__device__ __forceinline__ int row_tile_off(int row, int chunk) {  // in bf16 elements
  return row * D + ((chunk ^ (row & 7)) << 3);
}

// FP8 row tile: [rows][D] bytes, 8-byte units swizzled for conflict-free
// ds_read_b64 of 16 consecutive rows.
template <int D>
__device__ __forceinline__ int row_tile8_off(int row, int unit) {  // in bytes
  constexpr int kShift = (D == 64) ? 1 : 0;
  return row * D + ((unit ^ ((row >> kShift) & (D / 8 - 1))) << 3);
}

// Transposed tile: [D][NCOL] bf16, row = head-dim index d, columns = NCOL keys
// (or queries) in "accumulator order": within every 32-column block, logical
// 16-byte chunk 2*t + hf holds columns 16 t + 8 (p/4) + 4 hf + p%4, p = 0..7.
// Chunks are XOR-swizzled within their 128-byte bank sweep: by
// ((d ^ (d >> 3)) & 7) for rows of >= 64 columns, by (((d >> 1) ^ (d >> 3)) & 3)
// for 32-column rows (two rows per sweep).  Reads of 8 consecutive rows at one
// chunk are conflict-free; the transposing writes (rows 8c + e) are <= 4-way.
__device__ __forceinline__ int tr_chunk_of(int col) {  // logical chunk of column col
  int kk = col & 31;
  return ((col >> 5) << 2) + ((kk >> 4) << 1) + ((kk >> 2) & 1);
}
__device__ __forceinline__ int tr_pos_of(int col) {  // element position inside the chunk
  int kk = col & 31;
  return (((kk >> 3) & 1) << 2) + (kk & 3);
}
template <int NCOL>
__device__ __forceinline__ int tr_tile_off(int d, int chunk) {  // in bf16 elements
  static_assert(NCOL == 32 || NCOL == 64 || NCOL == 128, "transposed tile width");
  const int swz = (NCOL == 32) ? (((d >> 1) ^ (d >> 3)) & 3) : ((d ^ (d >> 3)) & 7);
  return d * NCOL + ((chunk ^ swz) << 3);
}

// Loads below are branch-free: an out-of-range row is redirected to row
// nvalid-1 (callers guarantee nvalid >= 1) and its value replaced by zero with
// a select.  Keeping every load unconditional lets the compiler count
// outstanding loads exactly, so the prefetch of the next tile is not drained
// (s_waitcnt vmcnt(0)) before the current tile's MFMAs.  The tile stagers
// apply the select only when they write LDS, after the current tile's math,
// so no instruction consumes the prefetched registers early.
__device__ __forceinline__ u32x4 load16_or_zero(const void* p, bool valid) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return valid ? v : u32x4{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ u32x2 load8_or_zero(const void* p, bool valid) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  return valid ? v : u32x2{0u, 0u};
}

// Stage a [NROW x D] bf16 tile from global memory (row stride `ld` elements,
// rows at or beyond `nvalid` >= 1 read as zero) into registers: thread t owns
// the 16-byte chunks t, t+256, ...
template <int NROW, int D>
struct RowTileRegs {
  static constexpr int CPR = D / 8;                    // chunks per row
  static constexpr int PER_THREAD = NROW * CPR / 256;
  u32x4 r[PER_THREAD];
  int nvalid;
  __device__ __forceinline__ void load(const __bf16* base, long ld, int nvalid_, int tid) {
    nvalid = nvalid_;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + 256 * i;
      int row = c / CPR, col = c % CPR;
      r[i] = *reinterpret_cast<const u32x4*>(base + (long)min(row, nvalid - 1) * ld + col * 8);
    }
  }
  __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + 256 * i;
      int row = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(lds + row_tile_off<D>(row, col)) = row < nvalid ? r[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
};

// Same for an FP8 tile ([NROW x D] bytes).
template <int NROW, int D>
struct RowTile8Regs {
  static constexpr int CPR = D / 16;
  static constexpr int PER_THREAD = NROW * CPR / 256;
  u32x4 r[PER_THREAD];
  int nvalid;
  __device__ __forceinline__ void load(const uint8_t* base, long ld, int nvalid_, int tid) {
    nvalid = nvalid_;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + 256 * i;
      int row = c / CPR, col = c % CPR;
      r[i] = *reinterpret_cast<const u32x4*>(base + (long)min(row, nvalid - 1) * ld + col * 16);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int c = tid + 256 * i;
      int row = c / CPR, col = c % CPR;
      const u32x4 v = row < nvalid ? r[i] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x2*>(lds + row_tile8_off<D>(row, 2 * col)) = u32x2{v[0], v[1]};
      *reinterpret_cast<u32x2*>(lds + row_tile8_off<D>(row, 2 * col + 1)) = u32x2{v[2], v[3]};
    }
  }
};

// Stage a [NROW x D] bf16 tile and store it transposed ([D][NROW], accumulator
// column order).  Thread t owns 4 consecutive rows (4a..4a+3) of one 8-wide
// column chunk cd; lanes with consecutive cd read one row contiguously.
template <int NROW, int D>
struct TrTileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int GROUPS = (NROW / 4) * CPR;      // (4-row group, chunk) pairs
  static constexpr int PER_THREAD = (GROUPS + 255) / 256;
  u32x4 r[PER_THREAD][4];
  int nvalid;
  __device__ __forceinline__ void load(const __bf16* base, long ld, int nvalid_, int tid) {
    nvalid = nvalid_;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int g = tid + 256 * i;
      int a = g / CPR, cd = g % CPR;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int row = 4 * a + rr;
        r[i][rr] = *reinterpret_cast<const u32x4*>(base + (long)min(row, nvalid - 1) * ld + cd * 8);
      }
    }
  }
  // zero the rows at or beyond nvalid (applied when writing LDS)
  __device__ __forceinline__ u32x4 val(int i, int rr, int tid) const {
    const int row = 4 * ((tid + 256 * i) / CPR) + rr;
    return row < nvalid ? r[i][rr] : u32x4{0u, 0u, 0u, 0u};
  }
  // The same registers written as a row tile (row_tile_off layout).
  __device__ __forceinline__ void store_rows(__bf16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int g = tid + 256 * i;
      if (GROUPS % 256 != 0 && g >= GROUPS) continue;
      int a = g / CPR, cd = g % CPR;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<u32x4*>(lds + row_tile_off<D>(4 * a + rr, cd)) = val(i, rr, tid);
    }
  }
  __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      int g = tid + 256 * i;
      if (GROUPS % 256 != 0 && g >= GROUPS) continue;
      int a = g / CPR, cd = g % CPR;
      int col = 4 * a;
      int chunk = tr_chunk_of(col);
      int pos = tr_pos_of(col);
      const u32x4 v0 = val(i, 0, tid), v1 = val(i, 1, tid), v2 = val(i, 2, tid), v3 = val(i, 3, tid);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int d = cd * 8 + e;
        int w = e >> 1;
        uint32_t x0 = v0[w], x1 = v1[w], x2 = v2[w], x3 = v3[w];
        uint32_t lo, hi;
        if (e & 1) {
          lo = (x0 >> 16) | (x1 & 0xffff0000u);
          hi = (x2 >> 16) | (x3 & 0xffff0000u);
        } else {
          lo = (x0 & 0xffffu) | (x1 << 16);
          hi = (x2 & 0xffffu) | (x3 << 16);
        }
        *reinterpret_cast<u32x2*>(lds + tr_tile_off<NROW>(d, chunk) + pos) = u32x2{lo, hi};
      }
    }
  }
};


// ------------------------------------------------- direct HBM -> LDS row tiles
// Row-major [rows][ROWB bytes] tiles written by global_load_lds_dwordx4: each
// lane's 16 bytes land at (LDS base of the instruction) + 16 * lane, so the
// chunk swizzle is chosen by picking which source chunk each lane fetches.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzle of a row-major LDS row tile.
template <int ROWB>
__device__ __forceinline__ int chunk_swz(int row) {
  return (ROWB >= 128) ? (row & 7) : ((row >> 1) & 3);  // 64-byte rows: two rows per bank sweep
}
template <int ROWB>
__device__ __forceinline__ int lds_off(int row, int chunk) {  // byte offset of a 16-byte chunk
  return row * ROWB + ((chunk ^ chunk_swz<ROWB>(row)) << 4);
}

// Issue the HBM -> LDS copy of a [NROW x ROWB-byte] row tile.  Rows at or
// beyond nvalid (>= 1) are redirected to row nvalid-1; the kernel masks the
// matching keys, so the duplicated rows never contribute.
template <int NROW, int ROWB>
__device__ __forceinline__ void stage_tile(const uint8_t* g, long ld_bytes, int nvalid, uint8_t* lds, int wave,
                                           int lane) {
  constexpr int U = ROWB / 16;                // 16-byte units per row
  constexpr int NI = NROW * U / 256;          // instructions per wave
  static_assert(NROW * U % 256 == 0, "tile must be a multiple of 4 KiB");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int blk = i * 4 + wave;             // 1 KiB block of LDS written by this instruction
    const int p = blk * 64 + lane;            // destination unit
    const int row = p / U, pc = p % U;
    const int c = pc ^ chunk_swz<ROWB>(row);  // logical chunk stored at physical chunk pc
    const uint8_t* src = g + (long)min(row, nvalid - 1) * ld_bytes + c * 16;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + blk * 1024), 16, 0, 0);
  }
}


// Transposed MFMA A operand from a row-major bf16 row tile via
// ds_read_b64_tr_b16.  Within each 16-lane group the instruction hands lane j
// element e of the 8-byte row that lane 4e + j/4 addressed, column j % 4.  So
// if lane r of group g addresses row (r0 + r/4), columns c0 + 4 (r%4) .. +3,
// lane j receives rows r0..r0+3 of column c0 + j.  Lane l thus obtains the A
// operand (row = column index c of the tile, l % 32 within a 32-block; k =
// 8 tile rows) whose k order matches the accumulator row order of a C tile:
// k position 4c' + e  <->  tile row 16 t + 8 c' + 4 (l / 32) + e.
template <int ROWB>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* tile, int row_base, int col_base, int lane) {
  const int g = lane >> 4, r = lane & 15;
  bf16x4 part[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = row_base + 8 * c + 4 * (g >> 1) + (r >> 2);
    const int col = col_base + 16 * (g & 1) + 4 * (r & 3);
    const uint8_t* p = tile + lds_off<ROWB>(row, col >> 3) + ((col & 4) << 1);
    part[c] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
  }
  return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-major MFMA A operand (row = tile row l % 32 of the 32-row block at
// row_base; k = 8 consecutive bf16 columns at chunk `chunk` + l / 32).
template <int ROWB>
__device__ __forceinline__ u32x4 row_operand(const uint8_t* tile, int row_base, int chunk, int lane) {
  return *reinterpret_cast<const u32x4*>(tile + lds_off<ROWB>(row_base + (lane & 31), chunk + (lane >> 5)));
}

}  // namespace gdpa
