// k_mfma.h -- bf16 GEMM tile on the gfx950 matrix cores.
//
// The dense contractions of the step (QKV, attention output, MLP and LM-head
// products, forward and both backward products) run here: bf16 operands, fp32
// accumulation in v_mfma_f32_32x32x16_bf16.  The p4 page's profile ("Where a
// step's time goes", tiled products table) puts 40% of its step in these
// products.
//
// Tile: BM x 128 outputs per workgroup (BM = 128, or 256 for the LM-head
// products), four wavefronts in a 2 x 2 grid, each (BM/2) x 64 in MFMA blocks
// of 32 x 32.  K advances 64 at a time through a three-slice LDS ring filled
// by direct-to-LDS copies issued between the MFMAs; operands keep their memory
// layout in LDS (XOR-swizzled 16-byte chunks), and an operand whose
// contraction index is strided in memory (weight gradients, where k runs over
// tokens) is read with the transposing LDS read.  The epilogue parks the
// accumulators in LDS and applies bias / residual / GELU / GELU' / gated-GELU'
// / attention row sums on the way out (details below).
#pragma once
#include "k_simple.h"

namespace ofa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMBM = 128, kMBN = 128;   // output tile

// Epilogue through LDS: the waves park their accumulators in LDS (fp32,
// [rows][128]), then all 256 threads walk the tile: thread -> four adjacent
// columns (one 16-byte LDS read, one 8- or 16-byte global access per operand),
// eight rows at a time.  Rows go in batches of kEpiRows per thread whose global
// reads (residual, saved pre-activation) are issued before any store: the
// output never aliases those inputs, and without the batching every read
// would wait for the previous row's store.  N, ldc, ldaux, ldres and aux_off
// are multiples of 8 (checked on the host), so every access is aligned.  In
// bf16 mode every low-precision operand of an epilogue (C, aux) is bf16.
constexpr int kEpiRows = 4;
constexpr int kEpiPitch = 128 + 4;   // floats per parked row

typedef float epi_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t epi_u2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ epi_u2 pack_bf16x4(epi_f4 x) {
  return epi_u2{f2bf2(x.x, x.y), f2bf2(x.z, x.w)};
}
__device__ __forceinline__ epi_f4 unpack_bf16x4(epi_u2 p) {
  return epi_f4{__uint_as_float(p.x << 16), __uint_as_float(p.x & 0xffff0000u), __uint_as_float(p.y << 16),
                __uint_as_float(p.y & 0xffff0000u)};
}
__device__ __forceinline__ epi_f4 gelu4(epi_f4 x) { return epi_f4{gelu_f(x.x), gelu_f(x.y), gelu_f(x.z), gelu_f(x.w)}; }
__device__ __forceinline__ epi_f4 gelu_grad4(epi_f4 x) {
  return epi_f4{gelu_grad_f(x.x), gelu_grad_f(x.y), gelu_grad_f(x.z), gelu_grad_f(x.w)};
}

template <int EPI, bool CF32>
__device__ __forceinline__ void epi_tile(const GemmArgs& g, const float* cst, int rows, int row0, int n0) {
  const int c = (threadIdx.x & 31) * 4, col = n0 + c;
  if (col >= g.N) return;
  const epi_f4 bias = g.bias ? *(const epi_f4*)(g.bias + col) : epi_f4{0.f, 0.f, 0.f, 0.f};
  const int rend = min(rows, g.M - row0);
  float* Cf = (float*)g.C;
  uint16_t* Ch = (uint16_t*)g.C;
  const float* resid = g.resid;
  uint16_t* aux = (uint16_t*)g.aux;
  for (int rb = threadIdx.x >> 5; rb < rend; rb += 8 * kEpiRows) {
    epi_f4 v[kEpiRows], a0[kEpiRows], a1[kEpiRows];
#pragma unroll
    for (int u = 0; u < kEpiRows; ++u) {
      const int r = min(rb + 8 * u, rend - 1);   // rows past the end repeat the last row (not stored)
      const int64_t row = row0 + r;
      v[u] = *(const epi_f4*)(cst + r * kEpiPitch + c) + bias;
      if constexpr (EPI == EPI_RESID) a0[u] = *(const epi_f4*)(resid + row * g.ldres + col);
      if constexpr (EPI == EPI_DGELU || EPI == EPI_DGEGLU || EPI == EPI_DSUM)
        a0[u] = unpack_bf16x4(*(const epi_u2*)(aux + row * g.ldaux + col));
      if constexpr (EPI == EPI_DGEGLU) a1[u] = unpack_bf16x4(*(const epi_u2*)(aux + row * g.ldaux + col + g.aux_off));
    }
#pragma unroll
    for (int u = 0; u < kEpiRows; ++u) {
      const int r = rb + 8 * u;
      if (r < rend) {
        const int64_t row = row0 + r;
        const int64_t ci = row * g.ldc + col;
        const epi_f4 x = v[u];
        if constexpr (EPI == EPI_STORE) {
          if constexpr (CF32) *(epi_f4*)(Cf + ci) = x;
          else *(epi_u2*)(Ch + ci) = pack_bf16x4(x);
        } else if constexpr (EPI == EPI_RESID) {
          *(epi_f4*)(Cf + ci) = a0[u] + x;
        } else if constexpr (EPI == EPI_GELU) {
          *(epi_u2*)(Ch + ci) = pack_bf16x4(x);
          *(epi_u2*)(aux + row * g.ldaux + col) = pack_bf16x4(gelu4(x));
        } else if constexpr (EPI == EPI_DGELU) {
          *(epi_u2*)(Ch + ci) = pack_bf16x4(x * gelu_grad4(a0[u]));
        } else if constexpr (EPI == EPI_DGEGLU) {
          *(epi_u2*)(Ch + ci) = pack_bf16x4(x * a1[u] * gelu_grad4(a0[u]));
          *(epi_u2*)(Ch + ci + g.aux_off) = pack_bf16x4(x * gelu4(a0[u]));
        }
      }
      if constexpr (EPI == EPI_DSUM) {
        // dO rounded as stored, times O, summed over the head's 64 columns: the
        // 16 threads of a row's head (lanes 16k .. 16k+15, one row per 32 lanes)
        const epi_u2 pk = pack_bf16x4(v[u]);
        if (r < rend) *(epi_u2*)(Ch + (int64_t)(row0 + r) * g.ldc + col) = pk;
        const epi_f4 d = unpack_bf16x4(pk);
        float sm = d.x * a0[u].x + d.y * a0[u].y + d.z * a0[u].z + d.w * a0[u].w;
        sm += __shfl_xor(sm, 1);
        sm += __shfl_xor(sm, 2);
        sm += __shfl_xor(sm, 4);
        sm += __shfl_xor(sm, 8);
        if (r < rend && (threadIdx.x & 15) == 0) {
          const int64_t row = row0 + r;
          const int64_t bb = row / g.dsum_T, t = row % g.dsum_T;
          g.dsum[(bb * g.dsum_H + col / 64) * g.dsum_T + t] = sm;
        }
      }
    }
  }
}

// EPI_CE, the LM head fused with the softmax statistics: every row of the
// tile keeps its logits z only as p = exp(z - m) in bf16, with m the row's
// maximum over the tile's valid columns, and writes (m, sum of p) for the
// cross-entropy to combine over the row's tiles ("Coppelius training on the
// RTX 3090", "Where a step's time goes": the output product, cross-entropy and
// its backward).  The 32 threads of a 32-lane half hold one row (four columns
// each) and reduce with shuffles inside that half, in a fixed order.
// The value of the lane whose index differs from this one in bit log2(O) of
// its 32-lane group (what __shfl_xor(v, O) returns there): O = 16, 8, 4 by a
// swizzle (no address operand), O = 2, 1 by a DPP quad permutation (no LDS).
template <int O>
__device__ __forceinline__ float xor_peer32(float v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16, "a lane bit of the 32-lane group");
  if constexpr (O >= 4)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (O << 10)));
  else
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), O == 1 ? 0xb1 : 0x4e, 0xf, 0xf, false));
}

__device__ __forceinline__ void epi_ce_tile(const GemmArgs& g, const float* cst, int rows, int row0, int n0) {
  const int c = (threadIdx.x & 31) * 4, col = n0 + c;
  const bool valid = col < g.N;   // N % 8 == 0: a group of four columns is wholly in or out
  const int rend = min(rows, g.M - row0);
  uint16_t* Ch = (uint16_t*)g.C;
  const int tn = n0 / kMBN;
  constexpr float kLog2e = 1.44269504088896341f;
  // four rows per pass, so their shuffle chains overlap (each row's arithmetic
  // and reduction order as for one row at a time); rows past the end repeat
  // the last row and store nothing
  constexpr int U = 4;
  for (int rb = threadIdx.x >> 5; rb < rend; rb += 8 * U) {
    epi_f4 v[U];
    float m[U], sm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(rb + 8 * u, rend - 1);
      v[u] = valid ? *(const epi_f4*)(cst + r * kEpiPitch + c) : epi_f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      m[u] = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
    }
    // butterfly over the 32 lanes of the row, partners in bit 4, 3, 2, 1, 0
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], xor_peer32<16>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], xor_peer32<8>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], xor_peer32<4>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], xor_peer32<2>(m[u]));
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = fmaxf(m[u], xor_peer32<1>(m[u]));
    epi_f4 pz[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float ml2 = m[u] * kLog2e;
      pz[u] = epi_f4{__builtin_amdgcn_exp2f(fmaf(v[u].x, kLog2e, -ml2)), __builtin_amdgcn_exp2f(fmaf(v[u].y, kLog2e, -ml2)),
                     __builtin_amdgcn_exp2f(fmaf(v[u].z, kLog2e, -ml2)), __builtin_amdgcn_exp2f(fmaf(v[u].w, kLog2e, -ml2))};
      sm[u] = (pz[u].x + pz[u].y) + (pz[u].z + pz[u].w);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) sm[u] += xor_peer32<16>(sm[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) sm[u] += xor_peer32<8>(sm[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) sm[u] += xor_peer32<4>(sm[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) sm[u] += xor_peer32<2>(sm[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) sm[u] += xor_peer32<1>(sm[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + 8 * u;
      if (r >= rend) break;
      const int64_t row = row0 + r;
      if (valid) *(epi_u2*)(Ch + row * g.ldc + col) = pack_bf16x4(pz[u]);
      if ((threadIdx.x & 31) == 0) {
        g.stats[2 * (row * g.stats_ld + tn)] = m[u];
        g.stats[2 * (row * g.stats_ld + tn) + 1] = sm[u];
      }
    }
  }
}

// The waves park their accumulators in LDS as the fp32 tile [BM][kEpiPitch],
// then walk it with epi_tile.  The accumulators hold transposed 32 x 32 blocks
// (the MFMA takes the B fragment as its first operand): element e of lane l
// is C[l % 32][8 (e / 4) + 4 (l / 32) + e % 4] of the block, so each group of
// four is four adjacent columns of one row, parked with one 16-byte write.
// The pitch (128 + 4 floats) spreads the 32 rows a write touches over all
// banks.
template <int BM>
__device__ __forceinline__ void gemm_mfma_epilogue(const GemmArgs& g, const f32x16_t (&acc)[BM / 64][2], int m0,
                                                   int n0, int wm, int wn, int lane, float* cst) {
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BM / 64; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm + i * 32 + (lane & 31), cc = wn + j * 32 + 8 * q + 4 * (lane >> 5);
        *(epi_f4*)(cst + r * kEpiPitch + cc) =
            epi_f4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
  __syncthreads();
  switch (g.epi) {
    case EPI_STORE:
      if (g.c_dt == DT_F32) epi_tile<EPI_STORE, true>(g, cst, BM, m0, n0);
      else epi_tile<EPI_STORE, false>(g, cst, BM, m0, n0);
      break;
    case EPI_RESID: epi_tile<EPI_RESID, true>(g, cst, BM, m0, n0); break;
    case EPI_GELU: epi_tile<EPI_GELU, false>(g, cst, BM, m0, n0); break;
    case EPI_DGELU: epi_tile<EPI_DGELU, false>(g, cst, BM, m0, n0); break;
    case EPI_DSUM: epi_tile<EPI_DSUM, false>(g, cst, BM, m0, n0); break;
    case EPI_CE: epi_ce_tile(g, cst, BM, m0, n0); break;
    default: epi_tile<EPI_DGEGLU, false>(g, cst, BM, m0, n0); break;
  }
}

// ============================================================================
// GEMM tile, pipelined version (K a multiple of 8; every row-contiguous
// operand's contiguous dimension a multiple of 8).
//
// Tile: BM x 128 outputs (BM = 128 or 256), four waves in a 2 x 2 grid, each
// (BM/2) x 64 = (BM/64) x 2 MFMA blocks of 32 x 32.  The 256-row tile moves
// 1.5x the bytes of the 128-row tile per k slice for 2x the MFMAs: the copy
// rate of a CU, not the matrix cores, bounds the smaller tile.
//
// Operands stay in their memory layout in LDS: a k-contiguous operand as
// [rows][64 k], a row-contiguous operand as [64 k][rows], both with 16-byte
// chunks XOR-swizzled so that fragment reads avoid bank conflicts.  The LDS
// serves 64 banks of 4 bytes a cycle: 16 lanes of a 16-byte read, 32 lanes of
// an 8-byte one.  k-contiguous: chunk c of row r sits at c ^ ((r >> 1) & 7), so
// the 16 rows a 16-lane group reads (two per 128-byte row pair of bank
// offsets) land on 16 distinct chunk slots.  Row-contiguous: chunk c of k row k
// sits at c ^ 4 (k & 3), so the 4 chunks x 4 k rows of a 32-lane transposing
// read are 16 distinct slots.  (The counters showed 0.4-1.0 conflict cycles per
// access with swizzles built for 32 banks, none with these.)  Global ->
// LDS copies use the direct-to-LDS loads of gfx950 into a three-stage ring:
// the next two k slices are in flight while the current one is multiplied.
// Fragments of a k-contiguous operand are one 16-byte LDS read; fragments of
// a row-contiguous operand are two transposing 8-byte reads
// (ds_read_b64_tr_b16): within each group of 16 lanes, lane 4g+e receives
// element e of the 4-element pieces addressed by lanes g, g+4, g+8, g+12, so
// lane r addressing k row k0 + r/4 at columns c0 + 4*(r%4) makes every lane
// receive four consecutive k of one column.
// ============================================================================

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kP3BK = 64;

// LDS of a BM-row tile with a ring of `stages` k slices (it also holds the
// tile's fp32 epilogue staging).  One workgroup per CU: three stages (two
// slices in flight), 128 or 256 rows.  Two workgroups per CU (half the LDS
// each): two stages, 128 rows -- the other workgroup's MFMAs run while this
// one waits for its copies.
template <int BM, int STAGES>
__host__ __device__ constexpr size_t gemm_p3_lds_bytes_t() {
  const size_t ring = (size_t)STAGES * (BM + kMBN) * kP3BK * sizeof(uint16_t);
  const size_t park = (size_t)BM * kEpiPitch * sizeof(float);
  return ring > park ? ring : park;
}
__host__ __device__ constexpr size_t gemm_p3_lds_bytes() { return gemm_p3_lds_bytes_t<256, 3>(); }
__host__ __device__ constexpr size_t gemm_p3_lds_bytes_occ2() { return gemm_p3_lds_bytes_t<128, 2>(); }

// Issue part of the direct-to-LDS copy of one operand's (ROWS rows x 64 k)
// slice: copies q0 .. q0+NQ-1 of the ROWS/32 this wave issues.  Wave w's copy q
// is the 64-lane instruction w + 4q; lane L of instruction i fills physical
// 16-byte chunk p = 64 i + L.
template <bool KMAJOR, int ROWS, int NQ>
__device__ __forceinline__ void p3_issue(const uint16_t* base, int64_t ld, int r0, int R, int k0, uint16_t* stage,
                                         int wave, int lane, int q0) {
  constexpr int CPR = ROWS / 8;   // 16-byte chunks per k row
  const uint16_t* src[NQ];
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const int p = (wave + 4 * (q0 + qq)) * 64 + lane;
    if (KMAJOR) {
      // physical chunk p = 8 r + (c ^ ((r >> 1) & 7)): row r, logical k chunk c
      const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
      const int rr = min(r0 + r, R - 1);   // rows past the end: any valid row (their outputs are dropped)
      src[qq] = base + (int64_t)rr * ld + k0 + c * 8;
    } else {
      // physical chunk p = CPR k + (c ^ 4(k & 3)): k row k, logical row chunk c
      const int k = p / CPR, c = (p % CPR) ^ (4 * (k & 3));
      const int col = min(r0 + c * 8, R - 8);
      src[qq] = base + (int64_t)(k0 + k) * ld + col;
    }
  }
  // The copies are issued as inline assembly so that the compiler does not
  // track them: its own tracking would wait for every outstanding copy
  // (gfx9 counts loads and copies on one counter) before any LDS read.  The
  // waits are explicit (p3_wait_barrier).
  // m0 is reserved to the compiler, which does not use it in these kernels
  // (checked in the generated code); the clobber documents the write.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#pragma unroll
  for (int qq = 0; qq < NQ; ++qq) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)(stage + (wave + 4 * (q0 + qq)) * 64 * 8));   // wave-uniform
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src[qq]), "s"(lds) : "memory", "m0");
  }
#pragma clang diagnostic pop
}

// The last k slice when K is not a multiple of 64: ordinary loads with zero
// fill (K % 8 == 0, so a 16-byte chunk is either wholly inside or outside),
// written by ds_write to the same swizzled chunk the copy would have filled.
template <bool KMAJOR, int ROWS>
__device__ __forceinline__ void p3_fill_tail(const uint16_t* base, int64_t ld, int r0, int R, int k0, int K,
                                             uint16_t* stage, int wave, int lane) {
  constexpr int NQ = ROWS / 32, CPR = ROWS / 8;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int p = (wave + 4 * q) * 64 + lane;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (KMAJOR) {
      const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
      const int rr = min(r0 + r, R - 1), k = k0 + c * 8;
      if (k < K) v = *(const uint4*)(base + (int64_t)rr * ld + k);
    } else {
      const int k = p / CPR, c = (p % CPR) ^ (4 * (k & 3));
      const int col = min(r0 + c * 8, R - 8);
      if (k0 + k < K) v = *(const uint4*)(base + (int64_t)(k0 + k) * ld + col);
    }
    *(uint4*)(stage + p * 8) = v;
  }
}

// whole slice: the copies at once, or the zero-filled tail
template <bool KMAJOR, int ROWS>
__device__ __forceinline__ void p3_load(const uint16_t* base, int64_t ld, int r0, int R, int k0, int K, uint16_t* stage,
                                        int wave, int lane) {
  if (k0 + kP3BK <= K) p3_issue<KMAJOR, ROWS, ROWS / 32>(base, ld, r0, R, k0, stage, wave, lane, 0);
  else p3_fill_tail<KMAJOR, ROWS>(base, ld, r0, R, k0, K, stage, wave, lane);
}

// wait until at most N of this wave's vector-memory operations are
// outstanding, then join the workgroup barrier
template <int N>
__device__ __forceinline__ void p3_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

__device__ __forceinline__ bf16x8_t p3_frag_k(const uint16_t* stage, int row, int kc) {
  const int pc = kc ^ ((row >> 1) & 7);
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)(stage + row * kP3BK + pc * 8));
}

// fragment of rows rbase..rbase+31 (lane -> row rbase + lane%32), k16 chunk kk,
// from a [64 k][ROWS rows] stage
template <int ROWS>
__device__ __forceinline__ bf16x8_t p3_frag_t(const uint16_t* stage, int rbase, int kk, int lane) {
  const int G = lane >> 4, r = lane & 15;
  const int col = rbase + 16 * (G & 1) + 4 * (r & 3);
  const int c = col >> 3, sub = (col >> 2) & 1;
  i16x4_t v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kr = kk * 16 + 8 * (G >> 1) + 4 * t + (r >> 2);
    const int pc = c ^ (4 * (kr & 3));
    v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(stage + kr * ROWS + pc * 8 + sub * 4));
  }
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
  return __builtin_bit_cast(bf16x8_t, w);
}

template <bool AKM, bool BKM, int BM, int kP3Stages>
__device__ __forceinline__ void gemm_p3(const GemmArgs& g, int tile, char* smem) {
  static_assert(kP3Stages >= 2 && kP3Stages <= 4, "ring of two to four slices");
  constexpr int WMB = BM / 64;                         // 32-row MFMA blocks per wave
  constexpr int SA = BM * kP3BK, SB = kMBN * kP3BK;    // stage elements per operand
  constexpr int PER_SLICE = BM / 32 + kMBN / 32;       // copies per wave per k slice
  uint16_t* ring_a = (uint16_t*)smem;
  uint16_t* ring_b = ring_a + kP3Stages * SA;
  int tm, tn;
  gemm_tile_rc(g, tile, tm, tn);
  const int m0 = tm * BM, n0 = tn * kMBN;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = (w >> 1) * (BM / 2), wn = (w & 1) * 64;
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* B = (const uint16_t*)g.B;

  f32x16_t acc[WMB][2];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (g.K + kP3BK - 1) / kP3BK;
  __syncthreads();   // the previous tile's readers are done with the ring
  // prologue: slices 0 and 1 in flight
#pragma unroll
  for (int q = 0; q < kP3Stages - 1; ++q)
    if (q < nk) {
      p3_load<AKM, BM>(A, g.lda, m0, g.M, q * kP3BK, g.K, ring_a + q * SA, w, lane);
      p3_load<BKM, kMBN>(B, g.ldb, n0, g.N, q * kP3BK, g.K, ring_b + q * SB, w, lane);
    }
  // copy instructions per wave for one slice, and how many go between the
  // MFMAs of each 16-wide k step (all of them are issued within the slice)
  // The buffer being refilled is free from the slice's barrier on: every copy
  // of the slice ahead goes out at the start of the slice, so it has the whole
  // slice's MFMAs to land in (measured against spreading the copies over the k
  // steps: 9.37 against 10.09 ms per c3 step with a ring of two, 11.06 against
  // 11.22 with three).
  constexpr int NQA = BM / 32, NQB = kMBN / 32;
  int cur = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // Slice kt landed in every wave (the copies of the up to STAGES-2 slices
    // after it may stay in flight; a zero-filled tail slice is loaded
    // synchronously, which also retires every older copy).  Past this barrier
    // every wave has finished reading slice kt-1, so its buffer takes slice
    // kt+STAGES-1: one barrier per slice.
    if (kP3Stages > 3 && kt + 2 < nk) p3_wait_barrier<2 * PER_SLICE>();
    else if (kP3Stages > 2 && kt + 1 < nk) p3_wait_barrier<PER_SLICE>();
    else p3_wait_barrier<0>();
    const int ahead = kt + kP3Stages - 1;
    const int buf = cur == 0 ? kP3Stages - 1 : cur - 1;
    // a whole slice ahead is copied after the first fragment reads below; a partial one now
    const bool copy_ahead = ahead < nk && (ahead + 1) * kP3BK <= g.K;
    if (ahead < nk && !copy_ahead) {
      p3_fill_tail<AKM, BM>(A, g.lda, m0, g.M, ahead * kP3BK, g.K, ring_a + buf * SA, w, lane);
      p3_fill_tail<BKM, kMBN>(B, g.ldb, n0, g.N, ahead * kP3BK, g.K, ring_b + buf * SB, w, lane);
    }
    const uint16_t* sa = ring_a + cur * SA;
    const uint16_t* sb = ring_b + cur * SB;
    // fragments double-buffered: step kk+1's LDS reads go out before step kk's MFMAs
    bf16x8_t af[2][WMB], bfr[2][2];
    auto frags = [&](int kk, int slot) {
#pragma unroll
      for (int i = 0; i < WMB; ++i)
        af[slot][i] = AKM ? p3_frag_k(sa, wm + i * 32 + (lane & 31), 2 * kk + (lane >> 5))
                          : p3_frag_t<BM>(sa, wm + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[slot][j] = BKM ? p3_frag_k(sb, wn + j * 32 + (lane & 31), 2 * kk + (lane >> 5))
                           : p3_frag_t<kMBN>(sb, wn + j * 32, kk, lane);
    };
    frags(0, 0);
    if (copy_ahead) {
      p3_issue<AKM, BM, NQA>(A, g.lda, m0, g.M, ahead * kP3BK, ring_a + buf * SA, w, lane, 0);
      p3_issue<BKM, kMBN, NQB>(B, g.ldb, n0, g.N, ahead * kP3BK, ring_b + buf * SB, w, lane, 0);
    }
#pragma unroll
    for (int kk = 0; kk < kP3BK / 16; ++kk) {
      const int s0 = kk & 1;
      if (kk + 1 < kP3BK / 16) frags(kk + 1, s0 ^ 1);
#pragma unroll
      for (int m = 0; m < WMB * 2; ++m) {
        const int i = m >> 1, j = m & 1;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s0][j], af[s0][i], acc[i][j], 0, 0, 0);
      }
    }
    cur = cur + 1 == kP3Stages ? 0 : cur + 1;
  }
  gemm_mfma_epilogue<BM>(g, acc, m0, n0, wm, wn, lane, (float*)smem);
}

template <int BM, int STAGES>
__device__ __forceinline__ void task_gemm_p3_bm(const GemmArgs& g, int tile, char* smem) {
  if (g.a_kmajor) {
    if (g.b_kmajor) gemm_p3<true, true, BM, STAGES>(g, tile, smem); else gemm_p3<true, false, BM, STAGES>(g, tile, smem);
  } else {
    if (g.b_kmajor) gemm_p3<false, true, BM, STAGES>(g, tile, smem); else gemm_p3<false, false, BM, STAGES>(g, tile, smem);
  }
}

// one workgroup per CU (OCC 1) or two (OCC 2: 128-row tiles only, set by the host)
template <int OCC = 1>
__device__ __forceinline__ void task_gemm_p3(const GemmArgs& g, int tile, char* smem) {
  if constexpr (OCC == 2) {
    task_gemm_p3_bm<128, 2>(g, tile, smem);
  } else {
    if (g.bm == 256) task_gemm_p3_bm<256, 3>(g, tile, smem);
    else task_gemm_p3_bm<128, 3>(g, tile, smem);
  }
}

}  // namespace ofa
