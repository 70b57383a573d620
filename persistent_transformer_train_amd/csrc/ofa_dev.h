// ofa_dev.h -- device helpers for gfx950: bf16 conversion, typed loads and
// stores, wavefront (64-lane) and workgroup reductions, scoped atomics for the
// release/acquire protocol, and the device status block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ofa_types.h"

namespace ofa {

constexpr int kThreads = 256;   // every task runs with 256 threads (4 wavefronts)
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even; NaN stays a (quiet) NaN
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float ldf(const void* p, int64_t i, int dt) {
  return dt == DT_BF16 ? bf2f(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

__device__ __forceinline__ void stf(void* p, int64_t i, int dt, float v) {
  if (dt == DT_BF16) ((uint16_t*)p)[i] = f2bf(v);
  else ((float*)p)[i] = v;
}

// ---------------------------------------------------------------- math

__device__ __forceinline__ float gelu_f(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}

__device__ __forceinline__ float gelu_grad_f(float u) {
  float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752f));
  float pdf = expf(-0.5f * u * u) * 0.39894228040143268f;
  return cdf + u * pdf;
}

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// workgroup sum, fixed order (deterministic); red must hold kWaves floats
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) s = fmaxf(s, red[i]);
  return s;
}

// ---------------------------------------------------------------- atomics

__device__ __forceinline__ uint64_t ld_acquire(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_release(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add_relaxed(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acq_rel_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
}
__device__ __forceinline__ void fence_acquire_agent() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void fence_release_agent() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Orders LDS accesses of one wavefront: the hardware executes a wave's LDS
// instructions in order; this keeps the compiler from moving them across.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// first error wins
__device__ __forceinline__ void raise_status(DevStatus* st, int code, int phase, int64_t step,
                                             int64_t info) {
  if (!st) return;
  int prev = atomicCAS(&st->code, 0, code);
  if (prev == 0) {
    st->phase = phase;
    st->step = step;
    st->info = info;
  }
}

// Context every task receives.
struct TaskCtx {
  const StepCtx* sc;
  DevStatus* status;
  int32_t phase;
  int64_t step;
};

}  // namespace ofa
