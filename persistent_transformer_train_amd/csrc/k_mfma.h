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

constexpr int kMBM = 128, kMBN = 128, kMBK = 32;
constexpr int kMPitch = kMBK + 8;   // bf16 elements per LDS row (16-byte pad)

struct GemmSmemMfma {
  uint16_t a[2][kMBM * kMPitch];
  uint16_t b[2][kMBN * kMPitch];
};

__host__ __device__ constexpr size_t gemm_mfma_lds_bytes() { return sizeof(GemmSmemMfma); }

// Stage registers for one operand tile: 2 x 16 bytes per thread.
struct OpStage {
  uint4 v[2];
};

// Load the (rows x 32) slice of an operand for rows r0.., k0.. into registers.
// kmajor: element (r, k) at base[r*ld + k]; else at base[k*ld + r].
__device__ __forceinline__ void mfma_load(OpStage& st, const uint16_t* base, int64_t ld, bool kmajor,
                                          int r0, int R, int k0, int K) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = threadIdx.x + i * kThreads;   // 0..511 chunks of 8 elements
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kmajor) {
      const int r = r0 + c / 4, k = k0 + (c % 4) * 8;
      if (r < R && k < K) val = *(const uint4*)(base + (int64_t)r * ld + k);   // K % 8 == 0
    } else {
      const int k = k0 + c / 16, r = r0 + (c % 16) * 8;
      if (k < K) {
        const uint16_t* p = base + (int64_t)k * ld + r;
        if (r + 8 <= R) {
          val = *(const uint4*)p;
        } else if (r < R) {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (r + e < R) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
          val = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    st.v[i] = val;
  }
}

__device__ __forceinline__ void mfma_store(const OpStage& st, uint16_t* lds, bool kmajor) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (kmajor) {
      const int r = c / 4, k = (c % 4) * 8;
      *(uint4*)(lds + r * kMPitch + k) = st.v[i];
    } else {
      const int k = c / 16, r = (c % 16) * 8;
      const uint32_t w[4] = {st.v[i].x, st.v[i].y, st.v[i].z, st.v[i].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) lds[(r + j) * kMPitch + k] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
    }
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* lds, int row, int k) {
  uint4 u = *(const uint4*)(lds + row * kMPitch + k);
  return __builtin_bit_cast(bf16x8_t, u);
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
  mfma_store(sa, s.a[0], g.a_kmajor);
  mfma_store(sb, s.b[0], g.b_kmajor);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      mfma_load(sa, A, g.lda, g.a_kmajor, m0, g.M, (kt + 1) * kMBK, g.K);
      mfma_load(sb, B, g.ldb, g.b_kmajor, n0, g.N, (kt + 1) * kMBK, g.K);
    }
#pragma unroll
    for (int kk = 0; kk < kMBK; kk += 16) {
      const int kf = kk + (lane >> 5) * 8;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_frag(s.a[cur], wm + i * 32 + (lane & 31), kf);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = lds_frag(s.b[cur], wn + j * 32 + (lane & 31), kf);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      mfma_store(sa, s.a[cur ^ 1], g.a_kmajor);
      mfma_store(sb, s.b[cur ^ 1], g.b_kmajor);
    }
    __syncthreads();
  }
  // accumulator element e of lane l: row (e/4)*8 + (l/32)*4 + e%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int col = n0 + wn + j * 32 + (lane & 31);
        gemm_epilogue(g, row, col, acc[i][j][e]);
      }
}

}  // namespace ofa
