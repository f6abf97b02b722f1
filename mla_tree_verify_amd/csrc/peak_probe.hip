// Peak probe for the benchmark: a loop of independent bf16 MFMAs (the
// 32x32x16 instruction the verify kernels use), one wave per SIMD on every
// CU, timed with the shader clock. It gives the MFMA throughput this GPU
// sustains under a pure MFMA load (its clock drops below the 2.4 GHz peak
// under such a load), the yardstick beside the published dense bf16 peak.
// Not part of the verify path; the library is built beside libmla_verify.so.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_verify_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_loop(float* out, unsigned long long* cycles, int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)threadIdx.x + (float)i);
    b[i] = (__bf16)(0.5f * (float)i);
  }
  f32x16_t acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = (f32x16_t){};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int k = 0; k < kAcc; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kAcc; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
  if (threadIdx.x % 64 == 0) cycles[(int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

}  // namespace

extern "C" {

int32_t mlav_probe_mfma(int32_t grid, int32_t iters, float* out, unsigned long long* cycles, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 24) || !out || !cycles) return 2;
  hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, cycles, iters);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int32_t mlav_probe_mfma_per_wave(void) { return 16; }  // MFMAs per loop iteration per wave

}  // extern "C"
