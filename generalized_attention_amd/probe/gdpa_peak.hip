// Throughput probes for the roofline denominators: how many dense MFMA flops
// per second the chip sustains when nothing else runs (bf16 32x32x16 and the
// FP8 32x32x64 form the GDPA kernels use), at the clock it actually holds
// under that load, and how many v_exp_f32 per second (the activations'
// transcendental).  Each wave runs NCH independent accumulator chains so that
// the matrix core never waits on a dependency; the accumulators are summed
// into out[] at the end so that the compiler keeps the work.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int NCH = 4;

__global__ __launch_bounds__(256) void peak_bf16(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  f32x16 c[NCH] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void peak_fp8(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + lane + i;  // E4M3 codes near 1.0
    b[i] = 0x30303030 + lane - i;
  }
  f32x16 c[NCH] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < NCH; ++j)
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// v_exp_f32 issue rate: NEXP independent chains per lane, so only the
// transcendental unit's throughput limits the loop.
constexpr int NEXP = 16;
__global__ __launch_bounds__(256) void peak_exp(float* out, int iters) {
  float x[NEXP];
  for (int j = 0; j < NEXP; ++j) x[j] = -0.5f - 0.01f * (threadIdx.x + j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NEXP; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);  // converges; the negation is a free modifier
  }
  float s = 0.0f;
  for (int j = 0; j < NEXP; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Launches `blocks` workgroups of 256 threads; out must hold blocks * 256
// floats.  kind 0: bf16 32x32x16 MFMAs (32768 flops each), kind 1: FP8
// 32x32x64 MFMAs (131072 flops each), iters * NCH per wave; kind 2: v_exp_f32,
// iters * NEXP per lane.  Returns the flops (kinds 0, 1) or lane-exponentials
// (kind 2) one launch performs, or -1 for bad arguments or a launch error.
double gdpa_probe_mfma(int kind, float* out, int blocks, int iters, void* stream) {
  if (out == nullptr || blocks <= 0 || iters <= 0 || kind < 0 || kind > 2) return -1.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(peak_bf16, dim3(blocks), dim3(256), 0, s, out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL(peak_fp8, dim3(blocks), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(peak_exp, dim3(blocks), dim3(256), 0, s, out, iters);
  if (hipGetLastError() != hipSuccess) return -1.0;
  if (kind == 2) return (double)blocks * 256 * iters * NEXP;
  const double per = kind == 0 ? 32768.0 : 131072.0;
  return (double)blocks * 4 * iters * NCH * per;
}

}
