// k_decode.h -- batch-1 greedy decode tasks: embedding of the current token,
// matrix-vector products with fused LayerNorm / bias / residual / GELU / KV
// append epilogues, single-query attention over the bf16 (or fp32) KV cache,
// and argmax with the context-window rule.
//
// Serving generates autoregressively from the changing model ("Open Flapping
// Airplanes ... A100 reproduction", "What ran"); one token releases the next
// with no host launch in between ("How one persistent kernel runs three
// jobs").  Batch-1 decode reads every weight once per token, so these tasks
// are HBM-bound: weights are streamed with 16-byte loads, one wavefront per
// output row.
#pragma once
#include "k_simple.h"

namespace ofa {

template <typename T>
__device__ __forceinline__ const T* slot_ptr(const void* p, const DecState* st) {
  return (const T*)((const char*)p + st->w_delta);
}

// ---------------------------------------------------------------- embedding

__device__ void task_dec_embed(const DecEmbedArgs& a, int tile, const TaskCtx& tc) {
  __shared__ int s_tok;
  const int pos = tc.sc->pos;
  if (threadIdx.x == 0) {
    DecState* st = a.st;
    if (tc.sc->head & 2) {    // first position of a token: acquire the newest weights
      uint64_t ver = ld_acquire(a.published);
      st->version = ver;
      st->w_delta = a.slot_bytes ? (int64_t)(ver & 1) * a.slot_bytes : 0;
    }
    int tok = a.ctx_tok[pos];
    if (tok < 0 || tok >= a.V) {
      raise_status(tc.status, -1, tc.phase, tc.step, tok);
      tok = 0;
    }
    s_tok = tok;
  }
  __syncthreads();
  const int tok = s_tok;
  const DecState* st = a.st;
  for (int j = threadIdx.x; j < a.d; j += kThreads) {
    float v = ldf((const char*)a.wte + st->w_delta, (int64_t)tok * a.d + j, a.w_dt);
    if (a.wpe) v += ldf((const char*)a.wpe + st->w_delta, (int64_t)pos * a.d + j, a.w_dt);
    a.x[j] = v;
  }
}

// ---------------------------------------------------------------- GEMV

__host__ __device__ inline size_t dec_gemv_lds_bytes(const DecGemvArgs& a) {
  return (size_t)(a.K + 2 * a.rows_per_tile + 64) * sizeof(float);
}

// dot of one weight row (K elements, dtype w_dt) with the LDS vector xs
__device__ __forceinline__ float row_dot(const void* Wrow, int K, int w_dt, const float* xs, int lane) {
  float acc = 0.f;
  if (w_dt == DT_BF16) {
    const uint4* p = (const uint4*)Wrow;
    for (int c = lane; c < K / 8; c += kWave) {
      uint4 u = p[c];
      const uint16_t* e = (const uint16_t*)&u;
      const float* x = xs + c * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += bf2f(e[i]) * x[i];
    }
  } else {
    const float4* p = (const float4*)Wrow;
    for (int c = lane; c < K / 4; c += kWave) {
      float4 u = p[c];
      const float* x = xs + c * 4;
      acc += u.x * x[0] + u.y * x[1] + u.z * x[2] + u.w * x[3];
    }
  }
  return wave_sum(acc);
}

__device__ void task_dec_gemv(const DecGemvArgs& a, int tile, const TaskCtx& tc, char* smem) {
  if (a.epi == DEPI_LOGITS && !(tc.sc->head & 1)) return;   // prefill position: no logits needed
  float* xs = (float*)smem;                 // [K]
  float* ys = xs + a.K;                     // [rows_per_tile] (x2 for gated)
  float* red = ys + 2 * a.rows_per_tile;    // reduction scratch
  const DecState* st = a.st;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const size_t esz = a.w_dt == DT_BF16 ? 2 : 4;
  // input vector, LayerNorm'd when requested (every tile recomputes the statistics)
  float s = 0.f;
  for (int j = threadIdx.x; j < a.K; j += kThreads) {
    float v = a.xin[j];
    xs[j] = v;
    s += v;
  }
  if (a.ln_g) {
    const float mean = block_sum(s, red) / a.K;
    float q = 0.f;
    for (int j = threadIdx.x; j < a.K; j += kThreads) {
      float dv = xs[j] - mean;
      q += dv * dv;
    }
    const float rstd = 1.0f / sqrtf(block_sum(q, red + kWaves) / a.K + 1e-5f);
    const void* g = (const char*)a.ln_g + st->w_delta;
    const void* b = (const char*)a.ln_b + st->w_delta;
    for (int j = threadIdx.x; j < a.K; j += kThreads)
      xs[j] = (xs[j] - mean) * rstd * ldf(g, j, a.w_dt) + ldf(b, j, a.w_dt);
  }
  __syncthreads();
  const char* W = (const char*)a.W + st->w_delta;
  const void* bias = a.bias ? (const void*)((const char*)a.bias + st->w_delta) : nullptr;
  const int r0 = tile * a.rows_per_tile;
  const int nrows = min(a.rows_per_tile, (a.epi == DEPI_GEGLU ? a.F : a.N) - r0);
  for (int i = w; i < nrows; i += kWaves) {
    const int n = r0 + i;
    float v = row_dot(W + (size_t)n * a.K * esz, a.K, a.w_dt, xs, lane);
    if (bias) v += ldf(bias, n, a.w_dt);
    float v2 = 0.f;
    if (a.epi == DEPI_GEGLU) v2 = row_dot(W + (size_t)(n + a.F) * a.K * esz, a.K, a.w_dt, xs, lane);
    if (lane == 0) {
      ys[i] = v;
      ys[a.rows_per_tile + i] = v2;
    }
  }
  __syncthreads();
  const int pos = tc.sc->pos;
  for (int i = threadIdx.x; i < nrows; i += kThreads) {
    const int n = r0 + i;
    const float v = ys[i];
    switch (a.epi) {
      case DEPI_STORE: a.y[n] = v; break;
      case DEPI_RESID: a.y[n] = a.resid[n] + v; break;
      case DEPI_GELU: a.y[n] = gelu_f(v); break;
      case DEPI_GEGLU: a.y[n] = gelu_f(v) * ys[a.rows_per_tile + i]; break;
      case DEPI_LOGITS:
        a.y[n] = v;
        if (a.io->logits_out) a.io->logits_out[(int64_t)tc.sc->gen_idx * a.N + n] = v;
        break;
      case DEPI_QKV: {
        // a tile covers whole heads of one part (q, k or v): rows_per_tile % dh == 0
        const int part = n / a.d, h = (n % a.d) / a.dh, j = n % a.dh;
        float out = v;
        if (a.rope && part < 2) {
          const int half = a.dh / 2;
          const int jj = j < half ? j : j - half;
          const double ang = (double)pos * pow(10000.0, -2.0 * jj / a.dh);
          const float c = (float)cos(ang), sn = (float)sin(ang);
          const float other = ys[j < half ? i + half : i - half];
          out = j < half ? v * c - other * sn : other * sn + v * c;
        }
        if (part == 0) {
          a.y[n] = out;
        } else {
          const int64_t ci = (((int64_t)(part - 1) * a.H + h) * a.cap + pos) * a.dh + j;
          stf(a.kv, ci, a.kv_dt, out);
        }
      } break;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- attention (one head per tile)

__host__ __device__ inline size_t dec_attn_lds_bytes(const DecAttnArgs& a) {
  return (size_t)(a.cap + a.dh + kThreads + 16) * sizeof(float);
}

__device__ void task_dec_attn(const DecAttnArgs& a, int tile, const TaskCtx& tc, char* smem) {
  const int h = tile;
  const int pos = tc.sc->pos;
  float* sc = (float*)smem;          // [cap]
  float* qs = sc + a.cap;            // [dh]
  float* part = qs + a.dh;           // [kThreads]
  float* red = part + kThreads;      // [16]
  const float scale = 1.0f / sqrtf((float)a.dh);
  for (int j = threadIdx.x; j < a.dh; j += kThreads) qs[j] = a.q[h * a.dh + j] * scale;
  __syncthreads();
  const int64_t kbase = ((int64_t)0 * a.H + h) * a.cap * a.dh;
  const int64_t vbase = ((int64_t)1 * a.H + h) * a.cap * a.dh;
  float mx = -INFINITY;
  for (int s = threadIdx.x; s <= pos; s += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < a.dh; ++j) acc += qs[j] * ldf(a.kv, kbase + (int64_t)s * a.dh + j, a.kv_dt);
    sc[s] = acc;
    mx = fmaxf(mx, acc);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int s = threadIdx.x; s <= pos; s += kThreads) {
    float p = expf(sc[s] - mx);
    sc[s] = p;
    sum += p;
  }
  sum = block_sum(sum, red + kWaves);
  __syncthreads();
  const int groups = kThreads / a.dh;   // dh divides 256
  const int j = threadIdx.x % a.dh, g = threadIdx.x / a.dh;
  float acc = 0.f;
  for (int s = g; s <= pos; s += groups) acc += sc[s] * ldf(a.kv, vbase + (int64_t)s * a.dh + j, a.kv_dt);
  part[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < a.dh) {
    float o = 0.f;
    for (int gg = 0; gg < groups; ++gg) o += part[gg * a.dh + threadIdx.x];
    a.o[h * a.dh + threadIdx.x] = o / sum;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- argmax + context update

__device__ void task_dec_argmax(const DecArgmaxArgs& a, int tile, const TaskCtx& tc, char* smem) {
  if (!(tc.sc->head & 1)) return;
  float* bv = (float*)smem;             // [kThreads]
  int* bi = (int*)(bv + kThreads);      // [kThreads]
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int v = threadIdx.x; v < a.V; v += kThreads) {
    float z = a.logits[v];
    if (z > best) { best = z; idx = v; }   // strided ascending: first max per thread wins ties
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) {
      float ob = bv[threadIdx.x + off];
      int oi = bi[threadIdx.x + off];
      if (ob > bv[threadIdx.x] || (ob == bv[threadIdx.x] && oi < bi[threadIdx.x])) {
        bv[threadIdx.x] = ob;
        bi[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int y = bi[0];
    if (y < 0 || y >= a.V) {   // every logit was NaN
      raise_status(tc.status, -3 /*OFA_E_NONFINITE*/, tc.phase, tc.step, 0);
      y = 0;
    }
    DecState* st = a.st;
    const int gi = tc.sc->gen_idx;
    a.io->tokens_out[gi] = y;
    if (a.io->versions_out) a.io->versions_out[gi] = st->version;
    int L = st->ctx_len;
    if (L + 1 > a.cap) {
      // context full: keep the most recent `keep` tokens (the new one included) at 0..keep-1
      for (int i = 0; i < a.keep - 1; ++i) a.ctx_tok[i] = a.ctx_tok[L - a.keep + 1 + i];
      a.ctx_tok[a.keep - 1] = y;
      st->ctx_len = a.keep;
    } else {
      a.ctx_tok[L] = y;
      st->ctx_len = L + 1;
    }
    st->n_gen = gi + 1;
  }
  __syncthreads();
}

}  // namespace ofa
