// Longest-first processing order of a jagged batch.
//
// GDPA's jagged batches (the GDPA README's "Features": jagged sequences with
// load-balanced scheduling) mix short and long sequences.  The kernels take
// (sequence, KV head) pairs in the order of a permutation; processing the
// longest sequences first is the longest-processing-time rule, which keeps
// long work items out of the tail of the launch.  One workgroup sorts the
// keys (lq + lk, index) with a bitonic network in LDS; keys are unique, so
// the order is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdpa_kernels.hpp"

namespace gdpa {

__global__ __launch_bounds__(1024) void gdpa_schedule_kernel(const int32_t* cu_q, const int32_t* cu_k, int batch,
                                                             int32_t* perm, int32_t* counters) {
  __shared__ uint64_t key[kSortMax];
  if (threadIdx.x < kNumCounters) counters[threadIdx.x] = 0;
  auto make_key = [&](int i) {
    const int64_t len = (int64_t)(cu_q[i + 1] - cu_q[i]) + (cu_k[i + 1] - cu_k[i]);
    const uint64_t inv = (uint64_t)(0xffffffffLL - (len < 0xffffffffLL ? len : 0xffffffffLL));
    return (inv << 32) | (uint32_t)i;  // ascending key = descending length, then index
  };
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
    if (i < batch) perm[i] = (int32_t)(uint32_t)x;
    return;
  }
  int n = 1;
  while (n < batch) n <<= 1;
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
  for (int i = threadIdx.x; i < batch; i += blockDim.x) perm[i] = (int32_t)(uint32_t)key[i];
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

hipError_t launch_zero(int32_t* p, long n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long blocks = (n / 4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gdpa_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* cu_q, const int32_t* cu_k, int batch, int32_t* perm, int32_t* counters,
                           hipStream_t stream) {
  if (batch <= 0 || batch > kSortMax) return hipErrorInvalidValue;
  // up to 64 sequences sort in registers across one wave; larger batches in
  // LDS, one compare-exchange per thread and stage
  int threads = 64;
  if (batch > 64) {
    threads = 128;
    while (threads < 1024 && 2 * threads < batch) threads <<= 1;
  }
  hipLaunchKernelGGL(gdpa_schedule_kernel, dim3(1), dim3(threads), 0, stream, cu_q, cu_k, batch, perm, counters);
  return hipGetLastError();
}

}  // namespace gdpa
