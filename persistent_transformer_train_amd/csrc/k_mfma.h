// k_mfma.h -- bf16 GEMM tile on the gfx950 matrix cores.
//
// The dense contractions of the step (QKV, attention output, MLP and LM-head
// products, forward and both backward products) run here: bf16 operands, fp32
// accumulation in v_mfma_f32_32x32x16_bf16.  The p4 page's profile ("Where a
// step's time goes", tiled products table) puts 40% of its step in these
// products.
//
// Tile: 128 x 128 outputs per workgroup, 4 wavefronts in a 2 x 2 grid, each
// wavefront 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  K advances 32 at a time
// through two LDS buffers (the next tile's global loads are in flight while
// the current tile is multiplied).  Both operands are staged in LDS as
// [row][k] with k contiguous, so every MFMA operand fragment is one 16-byte
// LDS read.  An operand whose contraction index is strided in memory (the
// weight-gradient products, where k runs over tokens) is transposed while it
// is written to LDS.
#pragma once
#include "k_simple.h"

namespace ofa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMBM = 128, kMBN = 128, kMBK = 64;
constexpr int kMPitch = kMBK + 8;   // bf16 elements per LDS row: 144 bytes, conflict-free 16-byte row reads

struct GemmSmemMfma {
  uint16_t a[kMBM * kMPitch];
  uint16_t b[kMBN * kMPitch];
};

__host__ __device__ constexpr size_t gemm_mfma_lds_bytes() { return sizeof(GemmSmemMfma); }

// Registers holding one operand's next (128 rows x 64 k) slice: 4 x 16 bytes per thread.
struct OpStage {
  uint4 v[4];
};

__device__ __forceinline__ uint4 ld16_rows(const uint16_t* p, int r, int R) {
  // 8 consecutive rows-contiguous elements starting at row index r (bounds R)
  if (r + 8 <= R) return *(const uint4*)p;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (r + e < R) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Load rows r0..r0+127, k0..k0+63 of an operand.
// kmajor: element (r, k) at base[r*ld + k]: thread c reads row c/8, k chunk (c%8)*8.
// otherwise element (r, k) at base[k*ld + r]: thread c reads k rows k0+2*(c%32) and +1,
// row chunk (c/32)*8, so that the transposing LDS writes of a wavefront hit
// consecutive dwords.
__device__ __forceinline__ void mfma_load(OpStage& st, const uint16_t* base, int64_t ld, bool kmajor,
                                          int r0, int R, int k0, int K) {
  if (kmajor) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + i * kThreads;   // 1024 chunks
      const int r = r0 + (c >> 3), k = k0 + (c & 7) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < R && k < K) v = *(const uint4*)(base + (int64_t)r * ld + k);   // K % 8 == 0
      st.v[i] = v;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = threadIdx.x + i * kThreads;   // 512 (k pair, row chunk) items
      const int k = k0 + 2 * (c & 31), r = r0 + (c >> 5) * 8;
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (r < R) {
        if (k < K) v0 = ld16_rows(base + (int64_t)k * ld + r, r, R);
        if (k + 1 < K) v1 = ld16_rows(base + (int64_t)(k + 1) * ld + r, r, R);
      }
      st.v[2 * i] = v0;
      st.v[2 * i + 1] = v1;
    }
  }
}

__device__ __forceinline__ void mfma_store(const OpStage& st, uint16_t* lds, bool kmajor) {
  if (kmajor) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = threadIdx.x + i * kThreads;
      *(uint4*)(lds + (c >> 3) * kMPitch + (c & 7) * 8) = st.v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = threadIdx.x + i * kThreads;
      const int kp = c & 31, r = (c >> 5) * 8;
      const uint4 a = st.v[2 * i], b = st.v[2 * i + 1];
      const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (wa[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        const uint32_t hi = (wb[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        *(uint32_t*)(lds + (r + j) * kMPitch + 2 * kp) = lo | (hi << 16);
      }
    }
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* lds, int row, int k) {
  uint4 u = *(const uint4*)(lds + row * kMPitch + k);
  return __builtin_bit_cast(bf16x8_t, u);
}

// fast epilogues (plain store with optional bias, residual add) inline; the
// GELU family goes through the shared element-wise epilogue
__device__ __forceinline__ void gemm_mfma_epilogue(const GemmArgs& g, const f32x16_t (&acc)[2][2], int m0, int n0,
                                                   int wm, int wn, int lane) {
  const bool fast = g.epi == EPI_STORE || g.epi == EPI_RESID;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn + j * 32 + (lane & 31);
    const bool cok = col < g.N;
    const float bias = (g.bias && cok) ? g.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (!cok || row >= g.M) continue;
        if (fast) {
          float v = acc[i][j][e] + bias;
          const int64_t ci = (int64_t)row * g.ldc + col;
          if (g.epi == EPI_RESID) {
            ((float*)g.C)[ci] = g.resid[(int64_t)row * g.ldres + col] + v;
          } else if (g.c_dt == DT_BF16) {
            ((uint16_t*)g.C)[ci] = f2bf(v);
          } else {
            ((float*)g.C)[ci] = v;
          }
        } else {
          gemm_epilogue(g, row, col, acc[i][j][e]);
        }
      }
    }
  }
}

__device__ void task_gemm_mfma(const GemmArgs& g, int tile, char* smem) {
  GemmSmemMfma& s = *(GemmSmemMfma*)smem;
  const int tm = tile / g.tiles_n, tn = tile % g.tiles_n;
  const int m0 = tm * kMBM, n0 = tn * kMBN;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* B = (const uint16_t*)g.B;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  OpStage sa, sb;
  const int nk = (g.K + kMBK - 1) / kMBK;
  mfma_load(sa, A, g.lda, g.a_kmajor, m0, g.M, 0, g.K);
  mfma_load(sb, B, g.ldb, g.b_kmajor, n0, g.N, 0, g.K);
  __syncthreads();   // the previous tile's readers are done with the LDS
  mfma_store(sa, s.a, g.a_kmajor);
  mfma_store(sb, s.b, g.b_kmajor);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      mfma_load(sa, A, g.lda, g.a_kmajor, m0, g.M, (kt + 1) * kMBK, g.K);
      mfma_load(sb, B, g.ldb, g.b_kmajor, n0, g.N, (kt + 1) * kMBK, g.K);
    }
#pragma unroll
    for (int kk = 0; kk < kMBK; kk += 16) {
      const int kf = kk + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_frag(s.a, wm + i * 32 + (lane & 31), kf);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = lds_frag(s.b, wn + j * 32 + (lane & 31), kf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      __syncthreads();
      mfma_store(sa, s.a, g.a_kmajor);
      mfma_store(sb, s.b, g.b_kmajor);
      __syncthreads();
    }
  }
  gemm_mfma_epilogue(g, acc, m0, n0, wm, wn, lane);
}

}  // namespace ofa
