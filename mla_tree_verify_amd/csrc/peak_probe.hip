// Probes for the benchmark, timed with the shader clock, one wave per SIMD on
// every CU: a loop of independent bf16 MFMAs (the 32x32x16 instruction the
// verify kernels use), which gives the MFMA throughput this GPU sustains under
// a pure MFMA load (its clock drops below the 2.4 GHz peak under such a load),
// the yardstick beside the published dense bf16 peak; and the split kernel's
// loop step as a bare data flow (step_mix below), which gives what that data
// flow costs on this GPU. Not part of the verify path; the library is built
// beside libmla_verify.so.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_verify_probe.h"

namespace {

#define LDS_AS __attribute__((address_space(3)))

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
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

// The split kernel's loop step as a data flow without its data dependencies:
// per 32-key step and wave, 18 MFMAs whose A operand is a 128-bit LDS read
// (the score product), 16 fragments of two transposing LDS reads each, each
// feeding two MFMAs into one accumulator (the value product with its hi and
// lo weights), nine 1 KB direct-to-LDS loads into the ring slot three steps
// ahead, and two workgroup barriers. Parts can be switched off to see what
// each adds to the 50-MFMA floor of a step. Operands are read a fixed number
// of MFMAs ahead, as in the kernel; the four ring slots are separate LDS
// objects, so a load into one slot orders no read of another.
constexpr int kSlot = 36864;  // one 32-key tile: 32 x (1024 + 128) bytes
constexpr int kAhead = 6;     // operand reads issued this many MFMAs ahead
constexpr uint32_t kSrcPieces = MLAV_MIX_SRC_BYTES / 1024;

__device__ inline void mix_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int kParts, int kS>
__device__ inline void mix_step(LDS_AS char* const (&ring)[4], __amdgpu_buffer_rsrc_t rs, int st, int wave,
                                int lane, const bf16x8_t (&q)[18], const bf16x8_t (&ph)[2],
                                const bf16x8_t (&pl)[2], f32x16_t& sc, f32x16_t (&o)[8]) {
  constexpr bool kLds = kParts & MLAV_MIX_LDS, kDma = kParts & MLAV_MIX_DMA, kBar = kParts & MLAV_MIX_BARRIERS;
  LDS_AS char* buf = ring[kS];
  LDS_AS char* next = ring[(kS + 3) & 3];
  // in-slot offsets: score reads below 32 KB, transposing reads below 24 KB
  auto kread = [&](int ks) -> bf16x8_t {
    if (!kLds) return q[ks];
    return *(const LDS_AS bf16x8_t*)(buf + ((lane * 16 + ks * 1024 + wave * 512) & 0x7FF0));
  };
  auto vread = [&](int f) -> bf16x8_t {
    if (!kLds) return q[f];
    const int off = (lane * 8 + f * 1024 + wave * 256) & 0x3FF8;
    const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(buf + off));
    const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(buf + off + 8192));
    return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  bf16x8_t op[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) op[j] = kread(j);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[ks % kAhead], q[ks], sc, 0, 0, 0);
    if (ks + kAhead < 18) op[ks % kAhead] = kread(ks + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kBar) mix_barrier();
#pragma unroll
  for (int j = 0; j < kAhead; ++j) op[j] = vread(j);
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    o[f & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[f % kAhead], ph[f >> 3], o[f & 7], 0, 0, 0);
    o[f & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[f % kAhead], pl[f >> 3], o[f & 7], 0, 0, 0);
    if (f + kAhead < 16) op[f % kAhead] = vread(f + kAhead);
    if (kDma && f < 9) {
      const uint32_t piece = (uint32_t)(st * 36 + wave * 9 + f) % kSrcPieces;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(next + (wave * 9 + f) * 1024), 16,
                                               (int)(piece * 1024u + 16u * (uint32_t)lane), 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kDma) __builtin_amdgcn_s_waitcnt(0x4F72);  // vmcnt(18): the loads of two steps back have landed
  if (kBar) mix_barrier();
}

template <int kParts>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void step_mix(const void* src, float* out, unsigned long long* cycles, int iters) {
  __shared__ __attribute__((aligned(16))) char r0[kSlot], r1[kSlot], r2[kSlot], r3[kSlot];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int i = threadIdx.x * 16; i < kSlot; i += 256 * 16) {
    *(uint4*)(r0 + i) = make_uint4(0, 0, 0, 0);
    *(uint4*)(r1 + i) = make_uint4(0, 0, 0, 0);
    *(uint4*)(r2 + i) = make_uint4(0, 0, 0, 0);
    *(uint4*)(r3 + i) = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, (int)MLAV_MIX_SRC_BYTES, 0x00020000);
  bf16x8_t q[18], ph[2], pl[2];
#pragma unroll
  for (int k = 0; k < 18; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) q[k][i] = (__bf16)(0.001f * (float)(lane + k) + (float)i);
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ph[k][i] = (__bf16)(0.5f * (float)(i + k));
      pl[k][i] = (__bf16)(0.001f * (float)(i + k));
    }
  // opaque: the operands stay in registers instead of being recomputed in the loop
#pragma unroll
  for (int k = 0; k < 18; ++k) asm volatile("" : "+v"(q[k]));
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    asm volatile("" : "+v"(ph[k]));
    asm volatile("" : "+v"(pl[k]));
  }
  f32x16_t sc = {}, o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = (f32x16_t){};
  LDS_AS char* const ring[4] = {(LDS_AS char*)r0, (LDS_AS char*)r1, (LDS_AS char*)r2, (LDS_AS char*)r3};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    mix_step<kParts, 0>(ring, rs, 4 * it + 0, wave, lane, q, ph, pl, sc, o);
    mix_step<kParts, 1>(ring, rs, 4 * it + 1, wave, lane, q, ph, pl, sc, o);
    mix_step<kParts, 2>(ring, rs, 4 * it + 2, wave, lane, q, ph, pl, sc, o);
    mix_step<kParts, 3>(ring, rs, 4 * it + 3, wave, lane, q, ph, pl, sc, o);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    s += sc[e];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += o[k][e];
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the MFMAs live
  if (lane == 0) cycles[(int64_t)blockIdx.x * 4 + wave] = t1 - t0;
}

}  // namespace

extern "C" {

int32_t mlav_probe_mfma(int32_t grid, int32_t iters, float* out, unsigned long long* cycles, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 24) || !out || !cycles) return 2;
  hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, cycles, iters);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int32_t mlav_probe_mfma_per_wave(void) { return 16; }  // MFMAs per loop iteration per wave

int32_t mlav_probe_step_mix(int32_t grid, int32_t iters, int32_t parts, const void* src, float* out,
                            unsigned long long* cycles, void* stream) {
  if (grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 20) || parts < 0 || parts > 7 || !src || !out ||
      !cycles)
    return 2;
  using K = void (*)(const void*, float*, unsigned long long*, int);
  static const K by_parts[8] = {step_mix<0>, step_mix<1>, step_mix<2>, step_mix<3>,
                                step_mix<4>, step_mix<5>, step_mix<6>, step_mix<7>};
  hipLaunchKernelGGL(by_parts[parts], dim3(grid), dim3(256), 0, (hipStream_t)stream, src, out, cycles, iters);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int32_t mlav_probe_steps_per_iteration(void) { return 4; }  // loop steps per iteration of step_mix

}  // extern "C"
