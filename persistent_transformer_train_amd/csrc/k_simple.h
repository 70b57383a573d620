// k_simple.h -- the training-step task functions in their plain form: each
// one processes one tile with 256 threads.  These are the fp32 path and the
// fallback-free reference-quality versions of the bandwidth-bound steps; the
// dense contractions additionally have MFMA versions (k_mfma.h).
//
// What each step computes follows the kernel families of "Coppelius training
// on the RTX 3090" ("Where a step's time goes"): gather, layernorm-forward,
// layernorm-backward, layernorm-parameters, attention-forward, attention-key,
// attention-query, qk-rope, inverse-rope-qkv, gated-gelu-forward/-backward,
// cross-entropy(-backward), loss-target-gather, embedding-scatter, adamw.
#pragma once
#include "ofa_dev.h"

namespace ofa {

__device__ __forceinline__ int token_at(const StepCtx* sc, int b, int t, int T, int V,
                                        const TaskCtx& tc) {
  int tok = sc->tokens[(int64_t)b * (T + 1) + t];
  if (tok < 0 || tok >= V) {
    raise_status(tc.status, -1 /*OFA_E_ARG*/, tc.phase, tc.step, tok);
    tok = 0;
  }
  return tok;
}

// ---------------------------------------------------------------- embedding gather

__device__ void task_embed(const EmbedArgs& a, int tile, const TaskCtx& tc) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int BT = a.B * a.T;
  const int r0 = tile * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, BT);
  for (int r = r0 + w; r < r1; r += kWaves) {
    int b = r / a.T, t = r % a.T;
    int tok = token_at(tc.sc, b, t, a.T, a.V, tc);
    const float* e = a.wte + (int64_t)tok * a.d;
    const float* p = a.wpe ? a.wpe + (int64_t)t * a.d : nullptr;
    float* x = a.x + (int64_t)r * a.d;
    for (int j = l; j < a.d; j += kWave) x[j] = e[j] + (p ? p[j] : 0.f);
  }
}

// ---------------------------------------------------------------- LayerNorm
// Rows of d floats read as float4 (d is a multiple of 8 and at most 1024, so
// a lane holds at most four float4 of a row).  Each wave takes two rows at a
// time so that both rows' loads are in flight together.

constexpr int kMaxD4 = 4;   // float4 per lane: d <= 1024

__device__ __forceinline__ float4 f4_zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }

__device__ __forceinline__ void st_row4(void* y, int64_t e, int dt, float4 v) {
  if (dt == DT_BF16) {
    const uint32_t w0 = f2bf2(v.x, v.y);
    const uint32_t w1 = f2bf2(v.z, v.w);
    *(uint2*)((uint16_t*)y + e) = make_uint2(w0, w1);
  } else {
    *(float4*)((float*)y + e) = v;
  }
}

// kLnQ rows per wave in flight (a 16-row tile is one pass); COMB: the residual
// combine, whose extra operands leave room for two
template <int kLnQ, bool COMB>
__device__ void task_ln_fwd(const LnFwdArgs& a, int tile) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int r0 = tile * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, a.rows);
  const int n4 = a.d / 4;
  const float4* __restrict__ x4 = (const float4*)a.x;
  const float4* __restrict__ g4 = (const float4*)a.g;
  const float4* __restrict__ b4 = (const float4*)a.b;
  const float4* __restrict__ k4 = (const float4*)a.kp;
  const int64_t khalf = (int64_t)a.rows * n4;
  float4 gv[kMaxD4], bv[kMaxD4], kbv[kMaxD4];
#pragma unroll
  for (int c = 0; c < kMaxD4; ++c) {
    const int j = l + c * kWave;
    gv[c] = j < n4 ? g4[j] : f4_zero();
    bv[c] = j < n4 ? b4[j] : f4_zero();
    if constexpr (COMB) kbv[c] = (j < n4 && a.kb) ? ((const float4*)a.kb)[j] : f4_zero();
  }
  for (int r = r0 + w; r < r1; r += kLnQ * kWaves) {
    float4 v[kLnQ][kMaxD4];
    float mean[kLnQ], rstd[kLnQ];
#pragma unroll
    for (int q = 0; q < kLnQ; ++q) {
      const int rr = r + q * kWaves;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        const int j = l + c * kWave;
        const int64_t e = (int64_t)rr * n4 + j;
        v[q][c] = (rr < r1 && j < n4) ? x4[e] : f4_zero();
        if constexpr (COMB) {
          if (rr < r1 && j < n4) {
            const float4 p0 = k4[e], p1 = k4[khalf + e];
            // residual + (sum + bias), in the order of the product's own epilogue
            float4 t = make_float4(p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w);
            t = make_float4(t.x + kbv[c].x, t.y + kbv[c].y, t.z + kbv[c].z, t.w + kbv[c].w);
            v[q][c] = make_float4(v[q][c].x + t.x, v[q][c].y + t.y, v[q][c].z + t.z, v[q][c].w + t.w);
            ((float4*)a.x_out)[e] = v[q][c];
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kLnQ; ++q) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) s += (v[q][c].x + v[q][c].y) + (v[q][c].z + v[q][c].w);
      mean[q] = wave_sum(s) / a.d;
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        if (l + c * kWave < n4) {
          const float dx = v[q][c].x - mean[q], dy = v[q][c].y - mean[q];
          const float dz = v[q][c].z - mean[q], dw = v[q][c].w - mean[q];
          ss += (dx * dx + dy * dy) + (dz * dz + dw * dw);
        }
      }
      rstd[q] = 1.0f / sqrtf(wave_sum(ss) / a.d + 1e-5f);
    }
#pragma unroll
    for (int q = 0; q < kLnQ; ++q) {
      const int rr = r + q * kWaves;
      if (rr >= r1) break;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        const int j = l + c * kWave;
        if (j < n4) {
          const float m = mean[q], rs = rstd[q];
          float4 o;
          o.x = (v[q][c].x - m) * rs * gv[c].x + bv[c].x;
          o.y = (v[q][c].y - m) * rs * gv[c].y + bv[c].y;
          o.z = (v[q][c].z - m) * rs * gv[c].z + bv[c].z;
          o.w = (v[q][c].w - m) * rs * gv[c].w + bv[c].w;
          st_row4(a.y, (int64_t)rr * a.d + 4 * j, a.y_dt, o);
        }
      }
      if (l == 0) {
        a.mean[rr] = mean[q];
        a.rstd[rr] = rstd[q];
      }
    }
  }
}

// dx = rstd * (gy - mean(gy) - xhat * mean(gy*xhat)), gy = g*dy; dx_out = dx_in + dx.
// Column partial sums of the tile (fixed order): dy*xhat, dy, dx_out.
// kLnBwdQ: rows per wave in flight (four with the whole register file of one
// workgroup per CU; two where two workgroups share it)
template <int kLnBwdQ = 4>
__device__ void task_ln_bwd(const LnBwdArgs& a, int tile, char* smem) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int r0 = tile * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, a.rows);
  const int n4 = a.d / 4;
  const float4* __restrict__ x4 = (const float4*)a.x;
  const float4* __restrict__ dy4 = (const float4*)a.dy;
  const float4* __restrict__ in4 = (const float4*)a.dx_in;
  float4* __restrict__ out4 = (float4*)a.dx_out;
  float4 gv[kMaxD4], pg[kMaxD4], pb[kMaxD4], px[kMaxD4];
#pragma unroll
  for (int c = 0; c < kMaxD4; ++c) {
    const int j = l + c * kWave;
    gv[c] = j < n4 ? ((const float4*)a.g)[j] : f4_zero();
    pg[c] = pb[c] = px[c] = f4_zero();
  }
  // kLnBwdQ rows per wave in flight (a wave's rows are accumulated in the same
  // order whatever the count)
  for (int r = r0 + w; r < r1; r += kLnBwdQ * kWaves) {
    float4 xh[kLnBwdQ][kMaxD4], dyv[kLnBwdQ][kMaxD4], din[kLnBwdQ][kMaxD4];
    float rs[kLnBwdQ], m1[kLnBwdQ], m2[kLnBwdQ];
#pragma unroll
    for (int q = 0; q < kLnBwdQ; ++q) {
      const int rr = r + q * kWaves;
      const bool okr = rr < r1;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        const int j = l + c * kWave;
        const bool ok = okr && j < n4;
        const int64_t e = (int64_t)rr * n4 + j;
        xh[q][c] = ok ? x4[e] : f4_zero();
        dyv[q][c] = ok ? dy4[e] : f4_zero();
        din[q][c] = (ok && in4) ? in4[e] : f4_zero();
      }
    }
#pragma unroll
    for (int q = 0; q < kLnBwdQ; ++q) {
      const int rr = r + q * kWaves;
      const float mean = rr < r1 ? a.mean[rr] : 0.f;
      rs[q] = rr < r1 ? a.rstd[rr] : 0.f;
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        if (l + c * kWave < n4) {
          float4& h = xh[q][c];
          h.x = (h.x - mean) * rs[q];
          h.y = (h.y - mean) * rs[q];
          h.z = (h.z - mean) * rs[q];
          h.w = (h.w - mean) * rs[q];
          const float4 gy = make_float4(dyv[q][c].x * gv[c].x, dyv[q][c].y * gv[c].y, dyv[q][c].z * gv[c].z,
                                        dyv[q][c].w * gv[c].w);
          s1 += (gy.x + gy.y) + (gy.z + gy.w);
          s2 += (gy.x * h.x + gy.y * h.y) + (gy.z * h.z + gy.w * h.w);
        }
      }
      m1[q] = wave_sum(s1) / a.d;
      m2[q] = wave_sum(s2) / a.d;
    }
#pragma unroll
    for (int q = 0; q < kLnBwdQ; ++q) {
      const int rr = r + q * kWaves;
      if (rr >= r1) break;
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        const int j = l + c * kWave;
        if (j < n4) {
          const float4 h = xh[q][c], dv = dyv[q][c], g = gv[c];
          float4 o;
          o.x = din[q][c].x + rs[q] * (dv.x * g.x - m1[q] - h.x * m2[q]);
          o.y = din[q][c].y + rs[q] * (dv.y * g.y - m1[q] - h.y * m2[q]);
          o.z = din[q][c].z + rs[q] * (dv.z * g.z - m1[q] - h.z * m2[q]);
          o.w = din[q][c].w + rs[q] * (dv.w * g.w - m1[q] - h.w * m2[q]);
          const int64_t e = (int64_t)rr * n4 + j;
          out4[e] = o;
          if (a.dx_lp) st_row4(a.dx_lp, 4 * e, a.lp_dt, o);
          pg[c].x += dv.x * h.x; pg[c].y += dv.y * h.y; pg[c].z += dv.z * h.z; pg[c].w += dv.w * h.w;
          pb[c].x += dv.x; pb[c].y += dv.y; pb[c].z += dv.z; pb[c].w += dv.w;
          px[c].x += o.x; px[c].y += o.y; px[c].z += o.z; px[c].w += o.w;
        }
      }
    }
  }
  // combine the four waves in a fixed order
  float4* red = (float4*)smem;   // [kWaves][3][n4]
#pragma unroll
  for (int c = 0; c < kMaxD4; ++c) {
    const int j = l + c * kWave;
    if (j < n4) {
      red[(w * 3 + 0) * n4 + j] = pg[c];
      red[(w * 3 + 1) * n4 + j] = pb[c];
      red[(w * 3 + 2) * n4 + j] = px[c];
    }
  }
  __syncthreads();
  float4* out = (float4*)(a.partials + (int64_t)tile * 3 * a.d);
  for (int i = threadIdx.x; i < 3 * n4; i += kThreads) {
    float4 s = red[i];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) {
      const float4 t = red[ww * 3 * n4 + i];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    out[i] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- column sums

// tile = (row chunk, block of 512 columns).  Thread (g, c8): rows g, g+4, ...
// of the chunk at columns 8 c8 .. 8 c8 + 7, 16-byte loads, sixteen rows in
// flight; the four row groups are added in group order through LDS.
// partials[row chunk][col].  cols is a multiple of 8.
constexpr int kCsCols = 512;   // columns per column-sum tile

__device__ __forceinline__ void cs_load8(const ColsumArgs& a, int64_t e, float (&v)[8]) {
  if (a.dt == DT_BF16) {
    const uint4 p = *(const uint4*)((const uint16_t*)a.src + e);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  } else {
    const float4 p0 = *(const float4*)((const float*)a.src + e);
    const float4 p1 = *(const float4*)((const float*)a.src + e + 4);
    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
  }
}

__device__ void task_colsum(const ColsumArgs& a, int tile, char* smem) {
  float* red = (float*)smem;   // [kWaves][kCsCols]
  const int ncb = (a.cols + kCsCols - 1) / kCsCols;
  const int rc = tile / ncb, cb = tile % ncb;
  const int r0 = rc * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, a.rows);
  const int g = threadIdx.x / 64, c8 = threadIdx.x % 64;
  const int c = cb * kCsCols + 8 * c8;
  float s[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) s[q] = 0.f;
  if (c < a.cols) {
    constexpr int U = 16;
    for (int rb = r0 + g; rb < r1; rb += 4 * U) {
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = rb + 4 * u;
        if (r < r1) cs_load8(a, (int64_t)r * a.ld + c, v[u]);
        else
#pragma unroll
          for (int q = 0; q < 8; ++q) v[u][q] = 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) s[q] += v[u][q];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) red[g * kCsCols + 8 * c8 + q] = s[q];
  __syncthreads();
  for (int i = threadIdx.x; i < kCsCols; i += kThreads) {
    const int cc = cb * kCsCols + i;
    if (cc < a.cols)
      a.partials[(int64_t)rc * a.cols + cc] =
          ((red[i] + red[kCsCols + i]) + red[2 * kCsCols + i]) + red[3 * kCsCols + i];
  }
  __syncthreads();
}

// tile = (vector k, block of 16 columns).  Sixteen groups of 16 threads: group
// q sums partials q, q+16, q+32, ... of its column in that order (eight loads
// in flight); the sixteen group sums are then added in group order.
constexpr int kCrCols = 16;

__device__ void task_colred(const ColredArgs& a, int tile, char* smem) {
  float* red = (float*)smem;   // [16 groups][16 columns]
  const int ncb = (a.cols + kCrCols - 1) / kCrCols;
  const int k = tile / ncb, cb = tile % ncb;
  // select among values already in registers: a dynamic index would move the
  // argument copy to scratch memory
  float* o0 = (float*)readfirstlane_u64((uint64_t)a.out[0]);
  float* o1 = (float*)readfirstlane_u64((uint64_t)a.out[1]);
  float* o2 = (float*)readfirstlane_u64((uint64_t)a.out[2]);
  float* o = k == 0 ? o0 : (k == 1 ? o1 : o2);
  if (!o) return;   // uniform across the workgroup
  const int cl = threadIdx.x & (kCrCols - 1), grp = threadIdx.x / kCrCols;
  const int c = cb * kCrCols + cl;
  constexpr int G = kThreads / kCrCols, U = 8;
  float s = 0.f;
  if (c < a.cols) {
    const float* __restrict__ p0 = a.partials + (int64_t)k * a.cols + c;
    const int64_t stride = (int64_t)a.n_vec * a.cols;
    for (int p = grp; p < a.n_parts; p += G * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pp = p + G * u;
        v[u] = pp < a.n_parts ? p0[pp * stride] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) s += v[u];
    }
  }
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x < kCrCols && c < a.cols) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < G; ++q) t += red[q * kCrCols + cl];
    o[c] = t;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- plain GEMM
// 64x64 tile, BK = 16, each thread computes 4x4 outputs.  Operands of any
// layout / dtype; accumulation in fp32.

struct GemmSmemSimple {
  float As[16][64 + 4];
  float Bs[16][64 + 4];
};

__device__ __forceinline__ float gemm_a(const GemmArgs& g, int m, int k) {
  if (m >= g.M || k >= g.K) return 0.f;
  int64_t i = g.a_kmajor ? (int64_t)m * g.lda + k : (int64_t)k * g.lda + m;
  return ldf(g.A, i, g.a_dt);
}
__device__ __forceinline__ float gemm_b(const GemmArgs& g, int k, int n) {
  if (n >= g.N || k >= g.K) return 0.f;
  int64_t i = g.b_kmajor ? (int64_t)n * g.ldb + k : (int64_t)k * g.ldb + n;
  return ldf(g.B, i, g.b_dt);
}

__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, int m, int n, float acc) {
  if (m >= g.M || n >= g.N) return;
  float v = acc + (g.bias ? g.bias[n] : 0.f);
  int64_t ci = (int64_t)m * g.ldc + n;
  switch (g.epi) {
    case EPI_STORE:
      stf(g.C, ci, g.c_dt, v);
      break;
    case EPI_RESID:
      ((float*)g.C)[ci] = g.resid[(int64_t)m * g.ldres + n] + v;
      break;
    case EPI_GELU:
      stf(g.C, ci, g.c_dt, v);
      stf(g.aux, (int64_t)m * g.ldaux + n, g.aux_dt, gelu_f(v));
      break;
    case EPI_DGELU: {
      float u = ldf(g.aux, (int64_t)m * g.ldaux + n, g.aux_dt);
      stf(g.C, ci, g.c_dt, v * gelu_grad_f(u));
    } break;
    case EPI_DGEGLU: {
      int64_t ai = (int64_t)m * g.ldaux + n;
      float gt = ldf(g.aux, ai, g.aux_dt);
      float up = ldf(g.aux, ai + g.aux_off, g.aux_dt);
      stf(g.C, ci, g.c_dt, v * up * gelu_grad_f(gt));
      stf(g.C, ci + g.aux_off, g.c_dt, v * gelu_f(gt));
    } break;
  }
}

__device__ __forceinline__ void task_gemm_simple(const GemmArgs& g, int tile, char* smem) {
  GemmSmemSimple& s = *(GemmSmemSimple*)smem;
  int tm, tn;
  gemm_tile_rc(g, tile, tm, tn);
  const int m0 = tm * 64, n0 = tn * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    // each thread loads 4 elements of each operand
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      int idx = threadIdx.x + e * kThreads;   // 0..1023
      int kk, mm;
      if (g.a_kmajor) { mm = idx / 16; kk = idx % 16; } else { kk = idx / 64; mm = idx % 64; }
      s.As[kk][mm] = gemm_a(g, m0 + mm, k0 + kk);
      int nn;
      if (g.b_kmajor) { nn = idx / 16; kk = idx % 16; } else { kk = idx / 64; nn = idx % 64; }
      s.Bs[kk][nn] = gemm_b(g, k0 + kk, n0 + nn);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = s.As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = s.Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) gemm_epilogue(g, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j]);
}

// ---------------------------------------------------------------- RoPE (rotate-half)

__device__ void task_rope(const RopeArgs& a, int tile, bool inverse) {
  const int BT = a.B * a.T;
  const int half = a.dh / 2;
  const int r0 = tile * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, BT);
  const int per_row = 2 * a.H * half;   // q and k, every head, every pair
  for (int idx = threadIdx.x; idx < (r1 - r0) * per_row; idx += kThreads) {
    int r = r0 + idx / per_row;
    int rem = idx % per_row;
    int part = rem / (a.H * half);          // 0 = q, 1 = k
    int h = (rem / half) % a.H;
    int i = rem % half;
    int t = r % a.T + a.pos0;
    double theta = pow(10000.0, -2.0 * i / a.dh);
    double ang = (double)t * theta;
    float c = (float)cos(ang), sn = (float)sin(ang);
    if (inverse) sn = -sn;
    int64_t base = (int64_t)r * a.ld + part * a.d + h * a.dh;
    float x1 = ldf(a.qkv, base + i, a.dt), x2 = ldf(a.qkv, base + i + half, a.dt);
    stf(a.qkv, base + i, a.dt, x1 * c - x2 * sn);
    stf(a.qkv, base + i + half, a.dt, x1 * sn + x2 * c);
  }
}

// ---------------------------------------------------------------- gated GELU forward

__device__ void task_geglu_fwd(const GegluArgs& a, int tile) {
  const int r0 = tile * a.rows_per_tile;
  const int r1 = min(r0 + a.rows_per_tile, a.rows);
  for (int64_t idx = threadIdx.x; idx < (int64_t)(r1 - r0) * a.F; idx += kThreads) {
    int r = r0 + (int)(idx / a.F), f = (int)(idx % a.F);
    float g = ldf(a.gu, (int64_t)r * 2 * a.F + f, a.dt);
    float up = ldf(a.gu, (int64_t)r * 2 * a.F + a.F + f, a.dt);
    stf(a.a, (int64_t)r * a.F + f, a.dt, gelu_f(g) * up);
  }
}

// ---------------------------------------------------------------- attention (plain)
// One wavefront per query row (forward, dQ) or key row (dK, dV).  Rows of a
// tile share one (b, h).  Scores live in LDS, 4 bytes per key.

struct AttnIdx { int b, h, t; };

__device__ __forceinline__ AttnIdx attn_row(const AttnArgs& a, int tile, int i) {
  const int nblk = (a.T + a.block - 1) / a.block;
  int bh = tile / nblk, blk = tile % nblk;
  AttnIdx r;
  r.b = bh / a.H;
  r.h = bh % a.H;
  r.t = blk * a.block + i;
  return r;
}

__device__ void task_attn_fwd_simple(const AttnArgs& a, int tile, char* smem) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  float* qs = (float*)smem + w * (64 + a.T);   // q (64) then scores (T)
  float* sc = qs + 64;
  const float scale = 1.0f / sqrtf((float)a.dh);
  const int64_t ld = 3 * (int64_t)a.d;
  for (int i = w; i < a.block; i += kWaves) {
    AttnIdx r = attn_row(a, tile, i);
    if (r.t >= a.T) break;
    const int64_t row_q = ((int64_t)r.b * a.T + r.t) * ld + r.h * a.dh;
    if (l < a.dh) qs[l] = ldf(a.qkv, row_q + l, a.dt) * scale;
    wave_sync();
    float mx = -INFINITY;
    for (int s0 = 0; s0 <= r.t; s0 += kWave) {
      int s = s0 + l;
      float v = -INFINITY;
      if (s <= r.t) {
        const int64_t row_k = ((int64_t)r.b * a.T + s) * ld + a.d + r.h * a.dh;
        float acc = 0.f;
        for (int j = 0; j < a.dh; ++j) acc += qs[j] * ldf(a.qkv, row_k + j, a.dt);
        v = acc;
        sc[s] = v;
      }
      mx = fmaxf(mx, v);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int s = l; s <= r.t; s += kWave) {
      float p = expf(sc[s] - mx);
      sc[s] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    wave_sync();
    const float inv = 1.0f / sum;
    if (l < a.dh) {
      float acc = 0.f;
      for (int s = 0; s <= r.t; ++s) {
        const int64_t row_v = ((int64_t)r.b * a.T + s) * ld + 2 * a.d + r.h * a.dh;
        acc += sc[s] * ldf(a.qkv, row_v + l, a.dt);
      }
      stf(a.o, ((int64_t)r.b * a.T + r.t) * a.d + r.h * a.dh + l, a.dt, acc * inv);
    }
    if (l == 0) a.lse[((int64_t)r.b * a.H + r.h) * a.T + r.t] = mx + logf(sum);
    wave_sync();
  }
}

// D[b,h,t] = sum_j dO[b,t,h,j] * O[b,t,h,j].  bf16 with 64-wide heads: eight
// lanes per (row, head), one 16-byte load of each operand per lane, four
// items per lane in flight; otherwise one wave per (row, head).
__device__ void task_attn_prep(const AttnArgs& a, int tile) {
  const int BT = a.B * a.T;
  const int r0 = tile * a.block, r1 = min(r0 + a.block, BT);
  const int n_items = (r1 - r0) * a.H;
  if (a.dt == DT_BF16 && a.dh == 64) {
    const int sub = threadIdx.x & 7, slot = threadIdx.x >> 3;
    constexpr int S = kThreads / 8, U = 4;
    const uint16_t* __restrict__ dO = (const uint16_t*)a.dout;
    const uint16_t* __restrict__ O = (const uint16_t*)a.o;
    for (int i0 = 0; i0 < n_items; i0 += S * U) {
      uint4 x[U], y[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = i0 + slot + S * u;
        const int r = r0 + it / a.H, h = it % a.H;
        const int64_t e = (int64_t)r * a.d + h * 64 + sub * 8;
        x[u] = it < n_items ? *(const uint4*)(dO + e) : make_uint4(0, 0, 0, 0);
        y[u] = it < n_items ? *(const uint4*)(O + e) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t xa[4] = {x[u].x, x[u].y, x[u].z, x[u].w}, ya[4] = {y[u].x, y[u].y, y[u].z, y[u].w};
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          s += __uint_as_float(xa[q] << 16) * __uint_as_float(ya[q] << 16) +
               __uint_as_float(xa[q] & 0xffff0000u) * __uint_as_float(ya[q] & 0xffff0000u);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        const int it = i0 + slot + S * u;
        if (sub == 0 && it < n_items) {
          const int r = r0 + it / a.H, h = it % a.H;
          const int b = r / a.T, t = r % a.T;
          a.dsum[((int64_t)b * a.H + h) * a.T + t] = s;
        }
      }
    }
    return;
  }
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  for (int item = w; item < n_items; item += kWaves) {
    int r = r0 + item / a.H, h = item % a.H;
    float s = 0.f;
    for (int j = l; j < a.dh; j += kWave) {
      int64_t i = (int64_t)r * a.d + h * a.dh + j;
      s += ldf(a.dout, i, a.dt) * ldf(a.o, i, a.dt);
    }
    s = wave_sum(s);
    int b = r / a.T, t = r % a.T;
    if (l == 0) a.dsum[((int64_t)b * a.H + h) * a.T + t] = s;
  }
}

// key row s: dV_s = sum_{t>=s} P_ts dO_t;  dK_s = scale * sum_{t>=s} dS_ts q_t
__device__ void task_attn_bwd_kv_simple(const AttnArgs& a, int tile, char* smem) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  float* ks = (float*)smem + w * (2 * 64 + 2 * 64);
  float* vs = ks + 64;
  float* ps = vs + 64;
  float* dss = ps + 64;
  const float scale = 1.0f / sqrtf((float)a.dh);
  const int64_t ld = 3 * (int64_t)a.d;
  for (int i = w; i < a.block; i += kWaves) {
    AttnIdx r = attn_row(a, tile, i);
    if (r.t >= a.T) break;
    const int s = r.t;
    const int64_t rs = ((int64_t)r.b * a.T + s) * ld + r.h * a.dh;
    if (l < a.dh) {
      ks[l] = ldf(a.qkv, rs + a.d + l, a.dt);
      vs[l] = ldf(a.qkv, rs + 2 * a.d + l, a.dt);
    }
    wave_sync();
    float dk = 0.f, dv = 0.f;
    for (int t0 = s; t0 < a.T; t0 += kWave) {
      int t = t0 + l;
      float p = 0.f, ds = 0.f;
      if (t < a.T) {
        const int64_t rq = ((int64_t)r.b * a.T + t) * ld + r.h * a.dh;
        const int64_t ro = ((int64_t)r.b * a.T + t) * a.d + r.h * a.dh;
        float qk = 0.f, dpv = 0.f;
        for (int j = 0; j < a.dh; ++j) {
          qk += ldf(a.qkv, rq + j, a.dt) * ks[j];
          dpv += ldf(a.dout, ro + j, a.dt) * vs[j];
        }
        const int64_t st = ((int64_t)r.b * a.H + r.h) * a.T + t;
        p = expf(qk * scale - a.lse[st]);
        ds = p * (dpv - a.dsum[st]);
      }
      ps[l] = p;
      dss[l] = ds;
      wave_sync();
      if (l < a.dh) {
        const int n = min(kWave, a.T - t0);
        for (int u = 0; u < n; ++u) {
          const int64_t tt = (int64_t)r.b * a.T + t0 + u;
          dv += ps[u] * ldf(a.dout, tt * a.d + r.h * a.dh + l, a.dt);
          dk += dss[u] * ldf(a.qkv, tt * ld + r.h * a.dh + l, a.dt);
        }
      }
      wave_sync();
    }
    if (l < a.dh) {
      stf(a.dqkv, rs + a.d + l, a.dt, dk * scale);
      stf(a.dqkv, rs + 2 * a.d + l, a.dt, dv);
    }
    wave_sync();
  }
}

// query row t: dQ_t = scale * sum_{s<=t} dS_ts k_s
__device__ void task_attn_bwd_q_simple(const AttnArgs& a, int tile, char* smem) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  float* qs = (float*)smem + w * (3 * 64);
  float* dos = qs + 64;
  float* dss = dos + 64;
  const float scale = 1.0f / sqrtf((float)a.dh);
  const int64_t ld = 3 * (int64_t)a.d;
  for (int i = w; i < a.block; i += kWaves) {
    AttnIdx r = attn_row(a, tile, i);
    if (r.t >= a.T) break;
    const int t = r.t;
    const int64_t rq = ((int64_t)r.b * a.T + t) * ld + r.h * a.dh;
    const int64_t ro = ((int64_t)r.b * a.T + t) * a.d + r.h * a.dh;
    if (l < a.dh) {
      qs[l] = ldf(a.qkv, rq + l, a.dt);
      dos[l] = ldf(a.dout, ro + l, a.dt);
    }
    wave_sync();
    const int64_t st = ((int64_t)r.b * a.H + r.h) * a.T + t;
    const float lse = a.lse[st], D = a.dsum[st];
    float dq = 0.f;
    for (int s0 = 0; s0 <= t; s0 += kWave) {
      int s = s0 + l;
      float ds = 0.f;
      if (s <= t) {
        const int64_t rk = ((int64_t)r.b * a.T + s) * ld + r.h * a.dh;
        float qk = 0.f, dpv = 0.f;
        for (int j = 0; j < a.dh; ++j) {
          qk += qs[j] * ldf(a.qkv, rk + a.d + j, a.dt);
          dpv += dos[j] * ldf(a.qkv, rk + 2 * a.d + j, a.dt);
        }
        float p = expf(qk * scale - lse);
        ds = p * (dpv - D);
      }
      dss[l] = ds;
      wave_sync();
      if (l < a.dh) {
        const int n = min(kWave, t - s0 + 1);
        for (int u = 0; u < n; ++u) {
          const int64_t rk = ((int64_t)r.b * a.T + s0 + u) * ld + a.d + r.h * a.dh;
          dq += dss[u] * ldf(a.qkv, rk + l, a.dt);
        }
      }
      wave_sync();
    }
    if (l < a.dh) stf(a.dqkv, rq + l, a.dt, dq * scale);
    wave_sync();
  }
}

// ---------------------------------------------------------------- cross-entropy
// One row per tile.  loss_r = logsumexp(z) - z[y];  dz = (softmax(z) - onehot(y)) / rows.
// V % 8 == 0 and rows are 16-byte aligned, so the row is read as float4.  A
// row of up to 256 * NR float4 is read once into registers (all loads in
// flight together) and reduced from there; longer rows take three passes.

__device__ __forceinline__ void ce_store(const CeArgs& a, int r, int i, int y, float lse, float4 v) {
  float p[4] = {expf(v.x - lse), expf(v.y - lse), expf(v.z - lse), expf(v.w - lse)};
  const int v0 = 4 * i;
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = (p[e] - (v0 + e == y ? 1.f : 0.f)) * a.inv_rows;
  const int64_t o = (int64_t)r * a.V + v0;
  if (a.dt == DT_BF16) {
    const uint32_t w0 = f2bf2(p[0], p[1]);
    const uint32_t w1 = f2bf2(p[2], p[3]);
    *(uint2*)((uint16_t*)a.dz + o) = make_uint2(w0, w1);
  } else {
    *(float4*)((float*)a.dz + o) = make_float4(p[0], p[1], p[2], p[3]);
  }
}

// exp(x - m) as 2^(x log2(e) - m log2(e)) on the hardware base-2 exponential
// (one transcendental instruction); ml2 = m * log2(e)
__device__ __forceinline__ float exp_shift(float x, float ml2) {
  return __builtin_amdgcn_exp2f(fmaf(x, 1.44269504088896341f, -ml2));
}

// The row stays in registers: softmax numerators overwrite the logits, so each
// element takes one exponential.
// the logits are read once and d logits written once: non-temporal global accesses
typedef float ce_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t ce_u2 __attribute__((ext_vector_type(2)));
typedef uint32_t ce_u4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) ce_f4 ce_gf4;
typedef __attribute__((address_space(1))) ce_u2 ce_gu2;

template <int NR>
__device__ __forceinline__ void ce_row_regs(const CeArgs& a, int r, int y, float* red) {
  const ce_gf4* z4 = (const ce_gf4*)(a.logits + (int64_t)r * a.V);
  const int n4 = a.V / 4;
  ce_f4 v[NR];
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int i = threadIdx.x + u * kThreads;
    v[u] = i < n4 ? __builtin_nontemporal_load(z4 + i) : ce_f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < NR; ++u) mx = fmaxf(mx, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
  mx = block_max(mx, red);
  const float ml2 = mx * 1.44269504088896341f;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    v[u].x = exp_shift(v[u].x, ml2);
    v[u].y = exp_shift(v[u].y, ml2);
    v[u].z = exp_shift(v[u].z, ml2);
    v[u].w = exp_shift(v[u].w, ml2);
    s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  s = block_sum(s, red + kWaves);
  const float inv_s = 1.0f / s;
#pragma unroll
  for (int u = 0; u < NR; ++u) {
    const int i = threadIdx.x + u * kThreads;
    if (i >= n4 || !a.dz) continue;
    float p[4] = {v[u].x * inv_s, v[u].y * inv_s, v[u].z * inv_s, v[u].w * inv_s};
    const int v0 = 4 * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = (p[e] - (v0 + e == y ? 1.f : 0.f)) * a.inv_rows;
    const int64_t o = (int64_t)r * a.V + v0;
    if (a.dt == DT_BF16) {
      __builtin_nontemporal_store(ce_u2{f2bf2(p[0], p[1]), f2bf2(p[2], p[3])}, (ce_gu2*)((uint16_t*)a.dz + o));
    } else {
      __builtin_nontemporal_store(ce_f4{p[0], p[1], p[2], p[3]}, (ce_gf4*)((float*)a.dz + o));
    }
  }
  if (threadIdx.x == 0) a.loss_rows[r] = mx + logf(s) - a.logits[(int64_t)r * a.V + y];
}

__device__ __forceinline__ void ce_row_loop(const CeArgs& a, int r, int y, float* red) {
  const float4* z4 = (const float4*)(a.logits + (int64_t)r * a.V);
  const int n4 = a.V / 4;
  float mx = -INFINITY;
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const float4 v = z4[i];
    mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  mx = block_max(mx, red);
  float s = 0.f;
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const float4 v = z4[i];
    s += (expf(v.x - mx) + expf(v.y - mx)) + (expf(v.z - mx) + expf(v.w - mx));
  }
  s = block_sum(s, red + kWaves);
  const float lse = mx + logf(s);
  if (a.dz)
    for (int i = threadIdx.x; i < n4; i += kThreads) ce_store(a, r, i, y, lse, z4[i]);
  if (threadIdx.x == 0) a.loss_rows[r] = lse - a.logits[(int64_t)r * a.V + y];
}

// Two passes for rows too long to hold in registers: the maximum and the
// rescaled sum of exponentials in one pass (each thread keeps its own running
// pair, combined over the workgroup in thread order), then the gradient.
__device__ __forceinline__ void ce_row_online(const CeArgs& a, int r, int y, float* red) {
  const float4* __restrict__ z4 = (const float4*)(a.logits + (int64_t)r * a.V);
  const int n4 = a.V / 4;
  constexpr int U = 4;
  float m = -INFINITY, s = 0.f;
  for (int i0 = threadIdx.x; i0 < n4; i0 += U * kThreads) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      v[u] = i < n4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < U; ++u) cm = fmaxf(cm, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
    const float cl2 = cm * 1.44269504088896341f;
    float cs = m == -INFINITY ? 0.f : s * exp_shift(m, cl2);
#pragma unroll
    for (int u = 0; u < U; ++u)
      cs += (exp_shift(v[u].x, cl2) + exp_shift(v[u].y, cl2)) + (exp_shift(v[u].z, cl2) + exp_shift(v[u].w, cl2));
    m = cm;
    s = cs;
  }
  const float mx = block_max(m, red);
  const float ml2 = mx * 1.44269504088896341f;
  const float tot = block_sum(m == -INFINITY ? 0.f : s * exp_shift(m, ml2), red + kWaves);
  const float lse = mx + logf(tot);
  if (a.dz)
    for (int i = threadIdx.x; i < n4; i += kThreads) ce_store(a, r, i, y, lse, z4[i]);
  if (threadIdx.x == 0) a.loss_rows[r] = lse - a.logits[(int64_t)r * a.V + y];
}

// Cross-entropy of one row fused with the LM head (EPI_CE): the row's tiles
// left p = exp(z - m_t) in dz and (m_t, s_t) in stats.  Then
//   lse = M + log sum_t s_t exp(m_t - M),  M = max_t m_t,
//   loss = lse - z_y,  z_y = h[row] . w[y] (the target logit, recomputed),
//   dz = (p exp(m_t - lse) - [v == y]) / rows, written over p.
// Reductions run in a fixed order (per-thread strided sums, then the block).
__device__ __forceinline__ void ce_row_fused(const CeArgs& a, int r, int y, float* red) {
  constexpr float kLog2e = 1.44269504088896341f;
  float* cs = red + 16;   // [n_stats] per-tile scales
  const float* st = a.stats + (int64_t)r * a.n_stats * 2;
  // target logit: the final-LN row against the head row of the target; its
  // operands are requested first so that their round trip overlaps the
  // statistics (d <= 1024: at most one 8-element chunk per thread)
  const uint16_t* hr = (const uint16_t*)a.h + (int64_t)r * a.d;
  const uint16_t* wr = (const uint16_t*)a.w + (int64_t)y * a.d;
  const int j = threadIdx.x * 8;
  uint4 hv = make_uint4(0u, 0u, 0u, 0u), wv = hv;
  if (j < a.d) {
    hv = *(const uint4*)(hr + j);
    wv = *(const uint4*)(wr + j);
  }
  float m = -INFINITY;
  for (int t = threadIdx.x; t < a.n_stats; t += kThreads) m = fmaxf(m, st[2 * t]);
  m = block_max(m, red);
  float s = 0.f;
  for (int t = threadIdx.x; t < a.n_stats; t += kThreads) s += st[2 * t + 1] * __builtin_amdgcn_exp2f((st[2 * t] - m) * kLog2e);
  float zy = 0.f;
  if (j < a.d)
    zy += bf2f(hv.x & 0xffff) * bf2f(wv.x & 0xffff) + bf2f(hv.x >> 16) * bf2f(wv.x >> 16) +
          bf2f(hv.y & 0xffff) * bf2f(wv.y & 0xffff) + bf2f(hv.y >> 16) * bf2f(wv.y >> 16) +
          bf2f(hv.z & 0xffff) * bf2f(wv.z & 0xffff) + bf2f(hv.z >> 16) * bf2f(wv.z >> 16) +
          bf2f(hv.w & 0xffff) * bf2f(wv.w & 0xffff) + bf2f(hv.w >> 16) * bf2f(wv.w >> 16);
  const float2 sz = block_sum2(s, zy, red + kWaves);
  const float lse = m + logf(sz.x);
  if (threadIdx.x == 0) a.loss_rows[r] = lse - sz.y;
  for (int t = threadIdx.x; t < a.n_stats; t += kThreads)
    cs[t] = __builtin_amdgcn_exp2f((st[2 * t] - lse) * kLog2e) * a.inv_rows;
  __syncthreads();
  // every 8-column chunk lies in one 128-column tile (V % 8 == 0); eight
  // chunks per thread are requested before any is rewritten, so that enough
  // reads are in flight to cover the memory latency
  typedef __attribute__((address_space(1))) ce_u4 ce_gu4;
  ce_gu4* zp = (ce_gu4*)((uint16_t*)a.dz + (int64_t)r * a.V);
  const int n8 = a.V / 8;
  constexpr int U = 8;
  for (int i0 = threadIdx.x; i0 < n8; i0 += U * kThreads) {
    ce_u4 u[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int i = i0 + k * kThreads;
      u[k] = i < n8 ? __builtin_nontemporal_load(zp + i) : ce_u4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int i = i0 + k * kThreads;
      if (i >= n8) break;
      const float c = cs[(8 * i) >> 7];
      float p[8] = {bf2f(u[k].x & 0xffff), bf2f(u[k].x >> 16), bf2f(u[k].y & 0xffff), bf2f(u[k].y >> 16),
                    bf2f(u[k].z & 0xffff), bf2f(u[k].z >> 16), bf2f(u[k].w & 0xffff), bf2f(u[k].w >> 16)};
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = p[e] * c - (8 * i + e == y ? a.inv_rows : 0.f);
      __builtin_nontemporal_store(ce_u4{f2bf2(p[0], p[1]), f2bf2(p[2], p[3]), f2bf2(p[4], p[5]), f2bf2(p[6], p[7])},
                                  zp + i);
    }
  }
}

// OCC 2 (two workgroups per CU, half the registers): rows beyond 16 float4 per
// thread take the two-pass form
template <int OCC = 1>
__device__ __forceinline__ void task_ce(const CeArgs& a, int tile, const TaskCtx& tc, char* smem) {
  float* red = (float*)smem;
  const int r = tile;
  const int b = r / a.T, t = r % a.T;
  const int y = token_at(tc.sc, b, t + 1, a.T, a.V, tc);
  if (a.fused) {
    ce_row_fused(a, r, y, red);
    return;
  }
  const int n4 = a.V / 4;
  if (n4 <= 4 * kThreads) ce_row_regs<4>(a, r, y, red);
  else if (n4 <= 16 * kThreads) ce_row_regs<16>(a, r, y, red);
  else if (OCC == 1 && n4 <= 52 * kThreads) ce_row_regs<OCC == 1 ? 52 : 16>(a, r, y, red);
  else if (OCC == 2) ce_row_online(a, r, y, red);
  else ce_row_loop(a, r, y, red);
}

// mean of the per-row losses, fixed summation order; flags a non-finite loss
__device__ void task_loss(const LossArgs& a, const TaskCtx& tc, char* smem) {
  float* red = (float*)smem;
  double s = 0.0;
  for (int i = threadIdx.x; i < a.rows; i += kThreads) s += (double)a.loss_rows[i];
  s = wave_sum_d(s);
  int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  double* dred = (double*)red;
  __syncthreads();
  if (l == 0) dred[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < kWaves; ++i) tot += dred[i];
    float loss = (float)(tot / a.rows);
    if (tc.sc->loss_out) *tc.sc->loss_out = loss;
    if (!isfinite(loss)) raise_status(tc.status, -3 /*OFA_E_NONFINITE*/, tc.phase, tc.step, 0);
  }
  if (float* out = tc.sc->rows_out)
    for (int i = threadIdx.x; i < a.rows; i += kThreads) out[i] = a.loss_rows[i];
  __syncthreads();
}

// ---------------------------------------------------------------- embedding backward
// EMB_SORT (one tile): sort positions by (token, position) with a bitonic sort
// in LDS, so that every token's positions form one run in increasing position
// order.  For each token present, first[tok] = tag << 32 | start << 16 | count.

__device__ void task_emb_sort(const EmbSortArgs& a, const TaskCtx& tc, char* smem) {
  uint64_t* keys = (uint64_t*)smem;
  int n = 1;
  while (n < a.BT) n <<= 1;
  const int T1 = a.T + 1;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    uint64_t k = ~0ull;
    if (i < a.BT) {
      int tok = tc.sc->tokens[(int64_t)(i / a.T) * T1 + i % a.T];
      if (tok < 0 || tok >= a.V) tok = 0;   // reported by the embedding gather
      k = ((uint64_t)(uint32_t)tok << 32) | (uint32_t)i;
    }
    keys[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kThreads) {
        int ixj = i ^ j;
        if (ixj > i) {
          uint64_t x = keys[i], y = keys[ixj];
          bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < a.BT; i += kThreads) {
    uint64_t k = keys[i];
    uint32_t tok = (uint32_t)(k >> 32);
    a.sorted[i] = (int32_t)(k & 0xffffffffu);
    if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != tok) {
      int e = i + 1;
      while (e < a.BT && (uint32_t)(keys[e] >> 32) == tok) ++e;
      a.first[tok] = (tc.sc->tag << 32) | ((uint64_t)i << 16) | (uint64_t)(e - i);
    }
  }
  __syncthreads();
}

// rows of d wte: fixed-order sum over the token's positions (or zero); then rows of d wpe.
// Each wave owns consecutive vocabulary rows; one lane per row loads the row's
// run descriptor up front, rows are written as float4.
__device__ void task_emb_bwd(const EmbBwdArgs& a, int tile, const TaskCtx& tc) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int n4 = a.d / 4;
  if (tile < a.v_tiles) {
    const int v0 = tile * a.rows_per_tile, v1 = min(v0 + a.rows_per_tile, a.V);
    const int per_wave = (a.rows_per_tile + kWaves - 1) / kWaves;   // <= 64 (host)
    const int vw = v0 + w * per_wave;
    const uint32_t tag = (uint32_t)tc.sc->tag;
    const uint64_t f_l = (l < per_wave && vw + l < v1) ? a.first[vw + l] : 0;
    for (int i = 0; i < per_wave; ++i) {
      const int v = vw + i;
      if (v >= v1) break;
      const uint64_t f = __shfl(f_l, i);
      const bool present = (uint32_t)(f >> 32) == tag;
      if (!present && a.accumulate) continue;
      float4 acc[kMaxD4];
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) acc[c] = f4_zero();
      if (present) {
        // positions in increasing order, eight rows in flight: lane q < 8 fetches
        // the position index of the batch's q-th row
        const int start = (int)((f >> 16) & 0xffff), end = start + (int)(f & 0xffff);
        constexpr int U = 8;
        for (int k0 = start; k0 < end; k0 += U) {
          const int pos_l = (l < U && k0 + l < end) ? a.sorted[k0 + l] : -1;
          float4 x[U][kMaxD4];
#pragma unroll
          for (int q = 0; q < U; ++q) {
            const int pos = __shfl(pos_l, q);
            const float4* row = (const float4*)(a.dx0 + (int64_t)(pos < 0 ? 0 : pos) * a.d);
#pragma unroll
            for (int c = 0; c < kMaxD4; ++c) {
              const int j = l + c * kWave;
              x[q][c] = (pos >= 0 && j < n4) ? row[j] : f4_zero();
            }
          }
#pragma unroll
          for (int q = 0; q < U; ++q) {
            if (k0 + q >= end) break;
#pragma unroll
            for (int c = 0; c < kMaxD4; ++c) {
              acc[c].x += x[q][c].x; acc[c].y += x[q][c].y; acc[c].z += x[q][c].z; acc[c].w += x[q][c].w;
            }
          }
        }
      }
      float4* out = (float4*)(a.dwte + (int64_t)v * a.d);
#pragma unroll
      for (int c = 0; c < kMaxD4; ++c) {
        const int j = l + c * kWave;
        if (j < n4) {
          float4 o = acc[c];
          if (a.accumulate) {
            const float4 p = out[j];
            o = make_float4(p.x + o.x, p.y + o.y, p.z + o.z, p.w + o.w);
          }
          out[j] = o;
        }
      }
    }
  } else {
    // one position per wave: the sum over the batch in batch order, eight rows in flight
    const int t = (tile - a.v_tiles) * kWaves + w;
    if (t >= a.n_pos) return;
    float4 acc[kMaxD4];
#pragma unroll
    for (int c = 0; c < kMaxD4; ++c) acc[c] = f4_zero();
    constexpr int U = 8;
    for (int b0 = 0; t < a.T && b0 < a.B; b0 += U) {
      float4 x[U][kMaxD4];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int b = b0 + q;
        const float4* row = (const float4*)(a.dx0 + ((int64_t)(b < a.B ? b : 0) * a.T + t) * a.d);
#pragma unroll
        for (int c = 0; c < kMaxD4; ++c) {
          const int j = l + c * kWave;
          x[q][c] = (b < a.B && j < n4) ? row[j] : f4_zero();
        }
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        if (b0 + q >= a.B) break;
#pragma unroll
        for (int c = 0; c < kMaxD4; ++c) {
          acc[c].x += x[q][c].x; acc[c].y += x[q][c].y; acc[c].z += x[q][c].z; acc[c].w += x[q][c].w;
        }
      }
    }
    float4* out = (float4*)(a.dwpe + (int64_t)t * a.d);
#pragma unroll
    for (int c = 0; c < kMaxD4; ++c) {
      const int j = l + c * kWave;
      if (j < n4) out[j] = acc[c];
    }
  }
}

// ---------------------------------------------------------------- AdamW
// p <- p(1 - lr wd); m <- b1 m + (1-b1) g; v <- b2 v + (1-b2) g^2;
// p <- p - lr (m/bc1) / (sqrt(v/bc2) + eps); compute copy <- p.

// ibc1, ibc2: the reciprocals of the bias corrections (one per step)
__device__ __forceinline__ void adamw_one(float& p, float& m, float& v, float g, float decay, float lr, float ibc1,
                                          float ibc2, const AdamArgs& a) {
  p *= decay;
  m = a.beta1 * m + (1.0f - a.beta1) * g;
  v = a.beta2 * v + (1.0f - a.beta2) * g * g;
  p -= lr * (m * ibc1) / (sqrtf(v * ibc2) + a.eps);
}

// per_tile is a multiple of 1024 and n of 8 (checked on the host): float4
// access, kAdamU groups per thread with every load issued before the
// arithmetic (a streaming kernel needs many bytes in flight); the tail of the
// last tile element-wise
constexpr int kAdamU = 4;
__device__ void task_adamw(const AdamArgs& a, int tile, const TaskCtx& tc) {
  // An error raised earlier in this step (a token out of range, a non-finite
  // loss) or anywhere else in the launch leaves the weights, the moments and
  // the compute copy untouched.  Every earlier phase of the step completed
  // before this one (acquired through its dependency), so their status writes
  // are visible; one thread reads the word so the whole tile takes one decision.
  __shared__ int s_err;
  if (threadIdx.x == 0) s_err = __hip_atomic_load(&tc.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_err) return;
  const float lr = tc.sc->lr, ibc1 = 1.0f / tc.sc->bc1, ibc2 = 1.0f / tc.sc->bc2;
  const int64_t i0 = (int64_t)tile * a.per_tile;
  const int64_t i1 = min(i0 + (int64_t)a.per_tile, a.n);
  const float decay = 1.0f - lr * a.wd;
  const int64_t n4 = (i1 - i0) / 4;
  // co-resident mode: the serve slot of this step's version
  void* pub = a.pub ? (void*)((char*)a.pub + (int64_t)(tc.sc->tag & 1) * a.pub_slot_bytes) : nullptr;
  typedef float f4v __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(1))) f4v gf4v;   // global memory: plain global (not flat) accesses
  gf4v* P = (gf4v*)(a.p + i0);
  gf4v* M = (gf4v*)(a.m + i0);
  gf4v* Vv = (gf4v*)(a.v + i0);
  const gf4v* G = (const gf4v*)(a.g + i0);
  for (int64_t j0 = threadIdx.x; j0 < n4; j0 += kAdamU * kThreads) {
    f4v p[kAdamU], m[kAdamU], v[kAdamU], g[kAdamU];
#pragma unroll
    for (int u = 0; u < kAdamU; ++u) {
      const int64_t j = j0 + (int64_t)u * kThreads;
      if (j < n4) {
        // every byte is touched once per step: non-temporal (streaming) accesses
        p[u] = __builtin_nontemporal_load(P + j);
        m[u] = __builtin_nontemporal_load(M + j);
        v[u] = __builtin_nontemporal_load(Vv + j);
        g[u] = __builtin_nontemporal_load(G + j);
      }
    }
#pragma unroll
    for (int u = 0; u < kAdamU; ++u) {
      const int64_t j = j0 + (int64_t)u * kThreads;
      if (j >= n4) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float pc = p[u][c], mc = m[u][c], vc = v[u][c];
        adamw_one(pc, mc, vc, g[u][c], decay, lr, ibc1, ibc2, a);
        p[u][c] = pc;
        m[u][c] = mc;
        v[u][c] = vc;
      }
      __builtin_nontemporal_store(p[u], P + j);
      __builtin_nontemporal_store(m[u], M + j);
      __builtin_nontemporal_store(v[u], Vv + j);
      if (a.wc || pub) {
        const int64_t e = i0 + 4 * j;
        if (a.wc_dt == DT_BF16) {
          const uint2 w = make_uint2(f2bf2(p[u][0], p[u][1]), f2bf2(p[u][2], p[u][3]));
          if (a.wc) *(uint2*)((uint16_t*)a.wc + e) = w;
          if (pub) *(uint2*)((uint16_t*)pub + e) = w;
        } else {
          if (a.wc) *(f4v*)((float*)a.wc + e) = p[u];
          if (pub) *(f4v*)((float*)pub + e) = p[u];
        }
      }
    }
  }
  for (int64_t i = i0 + 4 * n4 + threadIdx.x; i < i1; i += kThreads) {
    float p = a.p[i], m = a.m[i], v = a.v[i];
    adamw_one(p, m, v, a.g[i], decay, lr, ibc1, ibc2, a);
    a.p[i] = p;
    a.m[i] = m;
    a.v[i] = v;
    if (a.wc) stf(a.wc, i, a.wc_dt, p);
    if (pub) stf(pub, i, a.wc_dt, p);
  }
}

__device__ void task_copy(const CopyArgs& a, int tile) {
  const int64_t i0 = (int64_t)tile * a.per_tile;
  const int64_t i1 = min(i0 + (int64_t)a.per_tile, a.n);
  for (int64_t i = i0 + threadIdx.x; i < i1; i += kThreads) stf(a.dst, i, a.dst_dt, ldf(a.src, i, a.src_dt));
}

}  // namespace ofa
