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

// fp32 -> bf16, rounding to nearest even (NaN stays a quiet NaN): gfx950's
// conversion instruction (v_cvt_pk_bf16_f32, two values per instruction)
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values packed into one word, a in the low half
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const bf16x2_v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float ldf(const void* p, int64_t i, int dt) {
  return dt == DT_BF16 ? bf2f(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

__device__ __forceinline__ void stf(void* p, int64_t i, int dt, float v) {
  if (dt == DT_BF16) ((uint16_t*)p)[i] = f2bf(v);
  else ((float*)p)[i] = v;
}

// ---------------------------------------------------------------- math

// GELU in its exact erf form, GELU(u) = u Phi(u), with erf from Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26 (absolute error
// at most 1.5e-7): erf(x) = 1 - t (a1 + t (a2 + ... + t a5)) exp(-x^2),
// t = 1 / (1 + p |x|), odd in x.  exp(-x^2) with x = u / sqrt(2) is also the
// Gaussian density's exponential, so GELU' = Phi(u) + u phi(u) takes one
// exponential.  One base-2 exponential and one reciprocal instruction each.
__device__ __forceinline__ float erf_as(float x, float e /* exp(-x*x) */) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, fabsf(x), 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f), 0.254829592f);
  return copysignf(1.0f - poly * e, x);
}

__device__ __forceinline__ float gelu_f(float u) {
  const float x = u * 0.70710678118654752f;
  const float e = __builtin_amdgcn_exp2f(-x * x * 1.44269504088896341f);
  return 0.5f * u * (1.0f + erf_as(x, e));
}

__device__ __forceinline__ float gelu_grad_f(float u) {
  const float x = u * 0.70710678118654752f;
  const float e = __builtin_amdgcn_exp2f(-x * x * 1.44269504088896341f);
  const float cdf = 0.5f * (1.0f + erf_as(x, e));
  return fmaf(u * 0.39894228040143268f, e, cdf);
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

// wavefront sum with DPP row shifts and broadcasts (no LDS round trips);
// every lane receives the total
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define OFA_DPP(x, ctrl, rmask, bc) \
  __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xf, bc))
  v += OFA_DPP(v, 0x111, 0xf, true);   // row_shr:1
  v += OFA_DPP(v, 0x112, 0xf, true);   // row_shr:2
  v += OFA_DPP(v, 0x114, 0xf, true);   // row_shr:4
  v += OFA_DPP(v, 0x118, 0xf, true);   // row_shr:8: lane 15 of each row holds the row sum
  v += OFA_DPP(v, 0x142, 0xa, false);  // row_bcast:15
  v += OFA_DPP(v, 0x143, 0xc, false);  // row_bcast:31: lane 63 holds the total
#undef OFA_DPP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// workgroup sum of a value and of a second one with one barrier pair, fixed
// order; red must hold 2 kWaves floats
__device__ __forceinline__ float2 block_sum2_dpp(float a, float b, float* red) {
  a = wave_sum_dpp(a);
  b = wave_sum_dpp(b);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    red[w] = a;
    red[kWaves + w] = b;
  }
  __syncthreads();
  float2 r = make_float2(0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    r.x += red[i];
    r.y += red[kWaves + i];
  }
  return r;
}

// workgroup sums of two values with one barrier pair, each in block_sum's
// order (so each equals block_sum of it); red must hold 2 kWaves floats
__device__ __forceinline__ float2 block_sum2(float a, float b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    red[w] = a;
    red[kWaves + w] = b;
  }
  __syncthreads();
  float2 r = make_float2(0.f, 0.f);
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    r.x += red[i];
    r.y += red[kWaves + i];
  }
  return r;
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

// ---------------------------------------------------------------- tile placement

// GEMM tile index -> (tile row, tile column).  tile_order 0 walks a row of
// tiles at a time, 1 a column of tiles; 2 walks bands of `group` tile rows,
// each band column by column, so a run of consecutive tiles covers a compact
// rectangle of C: the A panels of the band's rows and a few B panels.
__device__ __forceinline__ void gemm_tile_rc(const GemmArgs& g, int tile, int& tm, int& tn) {
  if (g.tile_order == 2) {
    const int r0 = tile / (g.group * g.tiles_n) * g.group;
    const int rows = min(g.group, g.tiles_m - r0);
    const int in = tile - r0 * g.tiles_n;
    tm = r0 + in % rows;
    tn = in / rows;
  } else if (g.tile_order == 1) {
    tm = tile % g.tiles_m;
    tn = tile / g.tiles_m;
  } else {
    tm = tile / g.tiles_n;
    tn = tile % g.tiles_n;
  }
}

// The hardware hands the workgroups of a launch to the eight accelerator
// dies (XCDs, each with its own L2) in turn: workgroup b runs on die b % 8.
// xcd_block maps b to a tile so that each die gets one contiguous run of the
// n tiles (die x: tiles [x q + min(x, r), ...) with q = n / 8, r = n % 8), and
// neighbouring tiles share that die's L2.  A bijection on [0, n).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_block(int b, int n) {
  const int x = b % kXcds, i = b / kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + min(x, r) + i;
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
// orders this workgroup's earlier stores (complete in its die's L2) before its later atomics
__device__ __forceinline__ void fence_release_workgroup() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
}
// the accelerator die (XCD) this wave runs on
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Orders LDS accesses of one wavefront: the hardware executes a wave's LDS
// instructions in order; this keeps the compiler from moving them across.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A wave-uniform copy of a 64-bit value held by the first active lane.  The
// builtin returns a signed int: each half is taken as unsigned before it is
// widened, so a low half with bit 31 set is not sign-extended into the high one.
__device__ __forceinline__ uint64_t readfirstlane_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// ---------------------------------------------------------------- direct-to-LDS copies

typedef __attribute__((address_space(3))) void lds_void_t;

// One wavefront-wide copy from global memory straight into LDS
// (global_load_lds_dwordx4): lane L's 16 bytes at src land at lds_block + 16 L.
// lds_block is wave-uniform.  The copy is inline assembly so that the
// compiler does not track it (it would otherwise wait for every outstanding
// copy before its own LDS accesses, gfx9 counting loads and copies on one
// counter); completion is awaited explicitly with vm_wait_barrier.  m0 is
// reserved to the compiler, which does not use it in these kernels; the
// clobber documents the write.
__device__ __forceinline__ void dma16_to_lds(const void* src, const void* lds_block) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds_block);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
#pragma clang diagnostic pop
}

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n wave-uniform, 0..47; larger values wait for all), then join
// the workgroup barrier.
#define OFA_VMW(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ")\n\ts_barrier" : : : "memory"); break;
__device__ __forceinline__ void vm_wait_barrier(int n) {
  switch (n) {
    OFA_VMW(1) OFA_VMW(2) OFA_VMW(3) OFA_VMW(4) OFA_VMW(5) OFA_VMW(6) OFA_VMW(7) OFA_VMW(8)
    OFA_VMW(9) OFA_VMW(10) OFA_VMW(11) OFA_VMW(12) OFA_VMW(13) OFA_VMW(14) OFA_VMW(15) OFA_VMW(16)
    OFA_VMW(17) OFA_VMW(18) OFA_VMW(19) OFA_VMW(20) OFA_VMW(21) OFA_VMW(22) OFA_VMW(23) OFA_VMW(24)
    OFA_VMW(25) OFA_VMW(26) OFA_VMW(27) OFA_VMW(28) OFA_VMW(29) OFA_VMW(30) OFA_VMW(31) OFA_VMW(32)
    OFA_VMW(33) OFA_VMW(34) OFA_VMW(35) OFA_VMW(36) OFA_VMW(37) OFA_VMW(38) OFA_VMW(39) OFA_VMW(40)
    OFA_VMW(41) OFA_VMW(42) OFA_VMW(43) OFA_VMW(44) OFA_VMW(45) OFA_VMW(46) OFA_VMW(47)
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory"); break;
  }
}
#undef OFA_VMW

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
  int64_t gen_base;   // decode: index of the first token of this instance's schedule period
};

}  // namespace ofa
