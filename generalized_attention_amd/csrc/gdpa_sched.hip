// Longest-first processing order of a jagged batch, and the small utility
// kernels around the main ones (workspace clearing, decoding of 8- and 4-bit
// Q/K to bf16 for the backward).
//
// GDPA's jagged batches (the GDPA README's "Features": jagged sequences with
// load-balanced scheduling) mix short and long sequences.  The kernels take
// (sequence, KV head) pairs in the order of a permutation; processing the
// costliest sequences first is the longest-processing-time rule, which keeps
// long work items out of the tail of the launch.  A sequence's cost is the
// number of 64 x 64 (query, key) blocks its mask leaves any allowed pair in:
// every kernel's work per item is proportional to the blocks it visits, and a
// causal or windowed sequence visits far fewer than its lengths suggest.  One
// workgroup sorts the keys (cost, lq + lk, index) with a bitonic network;
// keys are unique, so the order is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdpa_kernels.hpp"

namespace gdpa {

__global__ __launch_bounds__(1024) void gdpa_schedule_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                             int wl, int wr, int32_t* perm, int32_t* counters) {
  __shared__ uint64_t key[kSortMax];
  if (threadIdx.x < kNumCounters) counters[threadIdx.x] = 0;
  auto make_key = [&](int i) { return schedule_key(cu_q[i + 1] - cu_q[i], cu_k[i + 1] - cu_k[i], wl, wr, i); };
  if (blockDim.x == 64) {
    // up to 64 sequences: the same network across the lanes of one wave
    const int i = threadIdx.x;
    uint64_t x = i < batch ? make_key(i) : ~0ull;
    for (int k = 2; k <= 64; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        const uint64_t y = __shfl_xor(x, j, 64);
        const bool take_min = ((i & j) == 0) == ((i & k) == 0);
        x = take_min ? (x < y ? x : y) : (x < y ? y : x);
      }
    }
    if (i < batch) perm[i] = schedule_key_index(x);
    return;
  }
  int n = 1;
  while (n < batch) n <<= 1;
  if ((int)blockDim.x >= n) {
    // up to 1024 sequences, one per thread: the same network with partners
    // less than 64 apart exchanged across the lanes of a wave, and only the
    // stages of wider partners through LDS (6 of 45 stages at 512 sequences)
    const int i = threadIdx.x;
    uint64_t x = i < batch ? make_key(i) : ~0ull;
    for (int k = 2; k <= (int)blockDim.x; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint64_t y;
        if (j >= 64) {
          key[i] = x;
          __syncthreads();
          y = key[i ^ j];
          __syncthreads();
        } else {
          y = __shfl_xor(x, j, 64);
        }
        const bool take_min = ((i & j) == 0) == ((i & k) == 0);
        x = take_min ? (x < y ? x : y) : (x < y ? y : x);
      }
    }
    if (i < batch) perm[i] = schedule_key_index(x);
    return;
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    if (i < batch) {
      key[i] = make_key(i);
    } else {
      key[i] = ~0ull;  // padding sorts last
    }
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = key[i], y = key[l];
          const bool ascending = (i & k) == 0;
          if ((x > y) == ascending) {
            key[i] = y;
            key[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < batch; i += blockDim.x) perm[i] = schedule_key_index(key[i]);
}

__global__ __launch_bounds__(256) void gdpa_zero_kernel(int32_t* p, long n) {
  // 16-byte stores over the 16-byte-aligned body, words before and after it singly
  const long head = (long)((16 - ((uintptr_t)p & 15)) & 15) / 4;
  const long h = head < n ? head : n;
  const long body = (n - h) / 4;
  const long stride = (long)gridDim.x * blockDim.x;
  const long t0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  for (long i = t0; i < h; i += stride) p[i] = 0;
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  i32x4* q = reinterpret_cast<i32x4*>(p + h);
  for (long i = t0; i < body; i += stride) q[i] = i32x4{0, 0, 0, 0};
  for (long i = h + 4 * body + t0; i < n; i += stride) p[i] = 0;
}

// E4M3 (OCP FP8: bias 7, 3 mantissa bits, S.1111.111 NaN, no infinities)
// and E2M1 (OCP MX FP4: bias 1, 1 mantissa bit) codes to fp32, built from
// the bit fields; every value is exact in fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, m = c & 0x7u;
  if ((c & 0x7Fu) == 0x7Fu) return __builtin_bit_cast(float, 0x7FC00000u | sign);
  if (e == 0) return __builtin_bit_cast(float, sign) + (sign ? -1.0f : 1.0f) * (float)m * 0x1p-9f;
  return __builtin_bit_cast(float, sign | ((e + 120u) << 23) | (m << 20));
}
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x8u) << 28, e = (c >> 1) & 0x3u, m = c & 0x1u;
  if (e == 0) return m ? __builtin_bit_cast(float, sign | 0x3F000000u) : __builtin_bit_cast(float, sign);
  return __builtin_bit_cast(float, sign | ((e + 126u) << 23) | (m << 22));
}
// fp32 -> bf16 bits, round to nearest even (the decoded values are exact in
// bf16 unless a block scale takes them outside its normal range)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One thread per 8 consecutive elements of a row (one 16-byte bf16 store): a
// block covers rpb = 256 / (d / 8) whole rows per pass, so each thread splits
// its index into (row, column) once and the loop over rows has no division.
__global__ __launch_bounds__(256) void gdpa_decode_kernel(const uint8_t* src, const uint8_t* scales, uint16_t* dst,
                                                          long rows, int d, int in_kind) {
  const int groups = d / 8, rpb = 256 / groups;
  const int tr = (int)threadIdx.x / groups;
  const int c0 = ((int)threadIdx.x - tr * groups) * 8;  // first element of the thread's group
  if (tr >= rpb) return;                                // 256 % groups spare threads
  for (long row = (long)blockIdx.x * rpb + tr; row < rows; row += (long)gridDim.x * rpb) {
    float v[8];
    if (in_kind == EL_MX4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + row * (d / 2) + c0 / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = e2m1_to_f32((w >> (4 * i)) & 0xFu);  // element 2i: low nibble
    } else {
      typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
      const u32x2v w = *reinterpret_cast<const u32x2v*>(src + row * d + c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = e4m3_to_f32((w[i / 4] >> (8 * (i % 4))) & 0xFFu);
    }
    if (in_kind != EL_FP8) {
      const uint32_t sc = scales[row * (d / 32) + c0 / 32];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = sc == 255u ? __builtin_nanf("") : __builtin_ldexpf(v[i], (int)sc - 127);
    }
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    u32x4v out;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4v*>(dst + row * d + c0) = out;
  }
}

hipError_t launch_decode_bf16(const uint8_t* src, const uint8_t* scales, uint16_t* dst, long rows, int d, int in_kind,
                              hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  // d / 8 groups of a row must fit one block of 256 threads
  if (d <= 0 || d % 32 != 0 || d > 2048 || (in_kind != EL_FP8 && in_kind != EL_MX8 && in_kind != EL_MX4))
    return hipErrorInvalidValue;
  const long rpb = 256 / (d / 8);
  long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gdpa_decode_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, scales, dst, rows, d,
                     in_kind);
  return hipGetLastError();
}

hipError_t launch_zero(int32_t* p, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long blocks = (n / 4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gdpa_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* cu_q, const int32_t* cu_k, int batch, int wl, int wr, int32_t* perm,
                           int32_t* counters, hipStream_t stream) {
  if (batch <= 0 || batch > kSortMax) return hipErrorInvalidValue;
  // up to 64 sequences sort in registers across one wave, up to 1024 with one
  // sequence per thread (wide partners through LDS), larger batches in LDS
  // with one compare-exchange per thread and stage
  int threads = 64;
  if (batch > 64) {
    threads = 128;
    while (threads < batch) threads <<= 1;
    if (threads > 1024) threads = 1024;
  }
  hipLaunchKernelGGL(gdpa_schedule_kernel, dim3(1), dim3(threads), 0, stream, cu_q, cu_k, batch, wl, wr, perm,
                     counters);
  return hipGetLastError();
}

}  // namespace gdpa
