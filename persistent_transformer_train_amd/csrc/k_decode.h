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
  __shared__ int s_tok[8];   // one per sequence (nseq <= 8)
  const int pos = tc.sc->pos;
  if (threadIdx.x == 0) {
    DecState* st = a.st;
    if (tc.sc->head & 4) {    // restart: the saved prompt becomes the context again
      const int n = st->prompt_len;
      for (int q = 0; q < a.nseq; ++q)
        for (int i = 0; i < n; ++i) a.ctx_tok[q * a.cap + i] = a.prompt[q * a.cap + i];
      st->ctx_len = n;
    }
    if ((tc.sc->head & 2) && a.io->doorbell) {
      // doorbell mode: the token starts once the host has rung for it (a bounded wait)
      const uint64_t g = (uint64_t)(tc.gen_base + tc.sc->gen_idx);
      const uint64_t start = now_ticks();
      for (int spins = 0; __hip_atomic_load(a.io->doorbell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) <= g; ++spins) {
        __builtin_amdgcn_s_sleep(1);
        if ((spins & 63) == 63 && now_ticks() - start > 500000000ull) {   // 5 s
          raise_status(tc.status, -4 /*OFA_E_TIMEOUT*/, tc.phase, tc.step, (int64_t)g);
          break;
        }
      }
      if (a.io->ticks && (int64_t)g < a.io->n_ticks) a.io->ticks[2 * g] = now_ticks();
    }
    if (tc.sc->head & 2) {    // first position of a token: acquire the newest weights
      uint64_t ver = ld_acquire(a.published);
      st->w_delta = a.slot_bytes ? (int64_t)(ver & 1) * a.slot_bytes : 0;
      // release: every read of the previous version's slot (earlier phases,
      // acquired through the dependency counters) happens before a trainer
      // that acquires this value overwrites that slot
      st_release(&st->version, ver);
    }
    for (int q = 0; q < a.nseq; ++q) {
      int tok = a.ctx_tok[q * a.cap + pos];
      if (tok < 0 || tok >= a.V) {
        raise_status(tc.status, -1, tc.phase, tc.step, tok);
        tok = 0;
      }
      s_tok[q] = tok;
    }
  }
  __syncthreads();
  const DecState* st = a.st;
  for (int q = 0; q < a.nseq; ++q) {
    const int tok = s_tok[q];
    for (int j = threadIdx.x; j < a.d; j += kThreads) {
      float v = ldf((const char*)a.wte + st->w_delta, (int64_t)tok * a.d + j, a.w_dt);
      if (a.wpe) v += ldf((const char*)a.wpe + st->w_delta, (int64_t)pos * a.d + j, a.w_dt);
      a.x[(int64_t)q * a.d + j] = v;
    }
  }
}

// ---------------------------------------------------------------- GEMV

// (value, index) maximum over the workgroup: larger value wins, equal values
// keep the lower index; the result is valid in every thread.  red holds 16
// words.
__device__ __forceinline__ void argmax_combine_block(float& bv, int& bi, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) {
    red[w] = bv;
    ((int*)red)[8 + w] = bi;
  }
  __syncthreads();
  bv = red[0];
  bi = ((int*)red)[8];
  for (int i = 1; i < kWaves; ++i) {
    const float ov = red[i];
    const int oi = ((int*)red)[8 + i];
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

// A ticket covers tiles [t0, t1) of a GEMV; tile t is rows [t R, t R + R) of W
// (for the gated MLP also rows F + t R ... of the up half, in the second half
// of the tile buffer).  The weights stream through an LDS ring of n_buf
// buffers of kDecTile bytes by direct-to-LDS copies; the persistent executor
// issues the first ones before the ticket's dependencies are met (weights do
// not depend on them), so weight streaming overlaps the previous phase.  Every
// tile takes the same number of copies per wave, so every wait count is a
// constant.  Rows are dot products of lpr lanes (16-byte chunks i, i + lpr, ...)
// against the LayerNorm'd input held in registers, each group of lpr lanes
// taking RPG rows per pass and reducing with DPP row operations.
// LDS: [ring n_buf x kDecTile][x: K fp32][ys: 2 ys_rows fp32][64 fp32 scratch].

constexpr int kDecTile = 32768;                    // bytes of one tile buffer
constexpr int kDecCopies = kDecTile / (1024 * kWaves);   // copies per wave per tile (8)
constexpr int kDecMaxChunks = 8;                   // 16-byte chunks of a row per lane

__host__ __device__ inline int dec_tile_rows_all(const DecGemvArgs& a) {
  return (a.epi == DEPI_GEGLU ? 2 : 1) * a.rows_per_tile;
}

// LDS: [ring n_buf x kDecTile][xs: nseq K fp32][ys: nseq ys_rows][ys2: nseq ys_rows][64 scratch]
__host__ __device__ inline int dec_nseq(const DecGemvArgs& a) { return a.nseq > 1 ? a.nseq : 1; }
__host__ __device__ inline size_t dec_gemv_lds_bytes(const DecGemvArgs& a) {
  return (size_t)a.n_buf * kDecTile + (size_t)(dec_nseq(a) * (a.K + 2 * a.ys_rows) + 64) * sizeof(float);
}

__device__ __forceinline__ int dec_row_bytes(const DecGemvArgs& a) { return a.K * (a.w_dt == DT_BF16 ? 2 : 4); }

// rows of W a tile of this GEMV covers (output rows; GEGLU: per half)
__device__ __forceinline__ int dec_tile_rows(const DecGemvArgs& a, int tile) {
  const int total = a.epi == DEPI_GEGLU ? a.F : a.N;
  return min(a.rows_per_tile, total - tile * a.rows_per_tile);
}

// N copies per wave of [src, src + 4 KB N) into dst; reads past `valid` bytes
// re-read the last valid chunk (nothing is read out of range)
template <int N>
__device__ __forceinline__ void dec_copy_n(const char* src, int valid, char* dst) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int blk = j * kWaves + w;
    dma16_to_lds(src + min(blk * 1024 + lane * 16, valid - 16), dst + blk * 1024);
  }
}

__device__ __forceinline__ void dec_tile_issue(const DecGemvArgs& a, const char* W, int tile, char* ring, int buf) {
  const int rb = dec_row_bytes(a);
  const int valid = dec_tile_rows(a, tile) * rb;
  const int64_t r0 = (int64_t)tile * a.rows_per_tile;
  char* dst = ring + buf * kDecTile;
  if (a.epi == DEPI_GEGLU) {
    dec_copy_n<kDecCopies / 2>(W + r0 * rb, valid, dst);
    dec_copy_n<kDecCopies / 2>(W + ((int64_t)a.F + r0) * rb, valid, dst + kDecTile / 2);
  } else {
    dec_copy_n<kDecCopies>(W + r0 * rb, valid, dst);
  }
}

// wait until tile i has landed while `later` (0..3) later tiles stay in flight,
// then join the workgroup barrier
__device__ __forceinline__ void dec_wait_tile(int later) {
  if (later >= 3) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" : : : "memory");
  else if (later == 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" : : : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" : : : "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
}
static_assert(kDecCopies == 8, "wait counts above assume 8 copies per wave per tile");

// Prefetch before the dependency wait: returns the number of tiles issued.
__device__ __forceinline__ int dec_gemv_prefetch(const DecGemvArgs& a, int t0, int t1, char* smem, bool allowed) {
  if (!allowed) return 0;
  const int64_t wd = a.pre_dep >= 0 ? a.st->w_delta : 0;
  const char* W = (const char*)a.W + wd;
  const int n = min(a.n_buf, t1 - t0);
  for (int i = 0; i < n; ++i) dec_tile_issue(a, W, t0 + i, smem, i);
  return n;
}

// sum over groups of lpr lanes (16, 32 or 64) with DPP; the sum lands in the
// group's last lane
__device__ __forceinline__ float dpp_group_sum(float v, int lpr) {
#define OFA_SHR(x, n) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + (n), 0xf, 0xf, true))
  v += OFA_SHR(v, 1);   // row_shr:1
  v += OFA_SHR(v, 2);   // row_shr:2
  v += OFA_SHR(v, 4);   // row_shr:4
  v += OFA_SHR(v, 8);   // row_shr:8 -> lane 15 of each row holds the row's sum
#undef OFA_SHR
  if (lpr >= 32)        // row_bcast:15 into rows 1 and 3
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  if (lpr >= 64)        // row_bcast:31 into rows 2 and 3
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}

// Dot products of one LDS tile's rows with the input chunks in xr; row rr of
// the tile (GEGLU: rows R.. are the up half) lands in ys[rr] or ys2[rr - R].
template <int RPG, bool BF16>
__device__ __forceinline__ void dec_dot_rows(const DecGemvArgs& a, const char* tilep, int rows,
                                             const float (&xr)[kDecMaxChunks][8], float* ys, float* ys2) {
  const int lpr = a.lpr, ng = kThreads / lpr;
  const int grp = threadIdx.x / lpr, li = threadIdx.x % lpr;
  const int R = a.rows_per_tile, TR = dec_tile_rows_all(a);
  const int rb = dec_row_bytes(a);
  const int nch = rb / 16;
  const int half = kDecTile / 2;
  int off[RPG];
#pragma unroll
  for (int k = 0; k < RPG; ++k) {
    const int rr = grp + k * ng;
    off[k] = (rr < TR && rr % R < rows) ? (rr / R) * half + (rr % R) * rb : 0;
  }
  float acc[RPG];
#pragma unroll
  for (int k = 0; k < RPG; ++k) acc[k] = 0.f;
#pragma unroll
  for (int j = 0; j < kDecMaxChunks; ++j) {
    const int c = li + j * lpr;
    if (j * lpr < nch && c < nch) {
      if constexpr (BF16) {
        uint4 u[RPG];
#pragma unroll
        for (int k = 0; k < RPG; ++k) u[k] = *(const uint4*)(tilep + off[k] + c * 16);
#pragma unroll
        for (int k = 0; k < RPG; ++k)
          acc[k] += bf2f(u[k].x & 0xffff) * xr[j][0] + bf2f(u[k].x >> 16) * xr[j][1] +
                    bf2f(u[k].y & 0xffff) * xr[j][2] + bf2f(u[k].y >> 16) * xr[j][3] +
                    bf2f(u[k].z & 0xffff) * xr[j][4] + bf2f(u[k].z >> 16) * xr[j][5] +
                    bf2f(u[k].w & 0xffff) * xr[j][6] + bf2f(u[k].w >> 16) * xr[j][7];
      } else {
        float4 u[RPG];
#pragma unroll
        for (int k = 0; k < RPG; ++k) u[k] = *(const float4*)(tilep + off[k] + c * 16);
#pragma unroll
        for (int k = 0; k < RPG; ++k)
          acc[k] += u[k].x * xr[j][0] + u[k].y * xr[j][1] + u[k].z * xr[j][2] + u[k].w * xr[j][3];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < RPG; ++k) {
    const float v = dpp_group_sum(acc[k], lpr);
    const int rr = grp + k * ng;
    if (li == lpr - 1 && rr < TR && rr % R < rows) {
      if (rr < R) ys[rr] = v;
      else ys2[rr - R] = v;
    }
  }
}

__device__ __forceinline__ void dec_tile_dot(const DecGemvArgs& a, const char* tilep, int rows,
                                             const float (&xr)[kDecMaxChunks][8], float* ys, float* ys2) {
  const bool bf = a.w_dt == DT_BF16;
  switch (a.rpg) {
    case 1: bf ? dec_dot_rows<1, true>(a, tilep, rows, xr, ys, ys2) : dec_dot_rows<1, false>(a, tilep, rows, xr, ys, ys2); break;
    case 2: bf ? dec_dot_rows<2, true>(a, tilep, rows, xr, ys, ys2) : dec_dot_rows<2, false>(a, tilep, rows, xr, ys, ys2); break;
    case 4: bf ? dec_dot_rows<4, true>(a, tilep, rows, xr, ys, ys2) : dec_dot_rows<4, false>(a, tilep, rows, xr, ys, ys2); break;
    default: bf ? dec_dot_rows<8, true>(a, tilep, rows, xr, ys, ys2) : dec_dot_rows<8, false>(a, tilep, rows, xr, ys, ys2); break;
  }
}

// Tiles [t0, t1) of one GEMV; tiles [t0, t0 + npre) were issued by the prefetch.
// Every sequence's rows are dot products against the same LDS tiles, in the
// same lane order as for one sequence.
// MULTI = false: one sequence, known at compile time (the loops over sequences
// fold away and the input chunks stay in registers for the whole ticket).
template <bool MULTI>
__device__ __forceinline__ void task_dec_gemv_range_t(const DecGemvArgs& a, int t0, int t1, const TaskCtx& tc,
                                                      char* smem, int npre) {
  if (a.epi == DEPI_LOGITS && !(tc.sc->head & 1)) {   // prefill position: no logits needed
    if (npre) vm_wait_barrier(0);                      // drain the prefetched copies
    return;
  }
  const int ns = MULTI ? dec_nseq(a) : 1;
  char* ring = smem;
  float* xs = (float*)(smem + (size_t)a.n_buf * kDecTile);   // [ns][K]
  float* ys = xs + (size_t)ns * a.K;                          // [ns][ys_rows]
  float* ys2 = ys + (size_t)ns * a.ys_rows;                   // [ns][ys_rows] (gated: up half)
  float* red = ys2 + (size_t)ns * a.ys_rows;                  // [64]
  const DecState* st = a.st;
  // with one weight slot the offset is always 0 (no dependent load)
  const int64_t wd = a.pre_dep >= 0 ? st->w_delta : 0;
  const char* W = (const char*)a.W + wd;
  const int nt = t1 - t0;
  for (int i = npre; i < min(a.n_buf, nt); ++i) dec_tile_issue(a, W, t0 + i, ring, i);
  int issued = min(a.n_buf, nt);
  // per-position values the epilogue needs, read now rather than after the tiles
  const int pos = tc.sc->pos;
  const int64_t gen_idx = tc.sc->gen_idx;
  float* const logits_out = a.epi == DEPI_LOGITS ? a.io->logits_out : nullptr;
  // Everything that does not come from the tiles is read in one batch of
  // loads: the input (and its first element, the LayerNorm shift), the
  // LayerNorm parameters, and the bias and residual of this thread's output
  // rows (sequence 0; further sequences read theirs in the epilogue).
  const void* bias = a.bias ? (const void*)((const char*)a.bias + wd) : nullptr;
  const int r0 = t0 * a.rows_per_tile;
  const int nrows = min(nt * a.rows_per_tile, (a.epi == DEPI_GEGLU ? a.F : a.N) - r0);
  constexpr int kPre = 4;   // rows per thread held in registers (the rest read in the epilogue)
  constexpr int kMaxK = 4;  // input elements per thread (K <= 1024)
  float pre_b[kPre], pre_r[kPre], gv[kMaxK], bv[kMaxK], xv[kMaxK];
#pragma unroll
  for (int m = 0; m < kPre; ++m) {
    const int i = threadIdx.x + m * kThreads;
    pre_b[m] = (bias && i < nrows) ? ldf(bias, r0 + i, a.w_dt) : 0.f;
    pre_r[m] = (a.epi == DEPI_RESID && i < nrows) ? a.resid[r0 + i] : 0.f;
  }
  if (a.ln_g) {
    const void* g = (const char*)a.ln_g + wd;
    const void* b = (const char*)a.ln_b + wd;
#pragma unroll
    for (int m = 0; m < kMaxK; ++m) {
      const int j = threadIdx.x + m * kThreads;
      gv[m] = j < a.K ? ldf(g, j, a.w_dt) : 0.f;
      bv[m] = j < a.K ? ldf(b, j, a.w_dt) : 0.f;
    }
  }
  for (int q = 0; q < ns; ++q) {
    float* xq = xs + (size_t)q * a.K;
    if (a.attn_part) {
      // the attention output: per head, the key-range partials rescaled to their
      // common maximum, summed, and divided by the summed weights
      const float* apq = a.attn_part + (int64_t)q * a.attn_ss;
      const int Wd = a.dh + 2;
      constexpr int kSplitMax = 8;
      for (int j = threadIdx.x; j < a.K; j += kThreads) {
        const float* ph = apq + (int64_t)(j / a.dh) * a.attn_split * Wd;
        float mc[kSplitMax], lc[kSplitMax], oc[kSplitMax];
#pragma unroll
        for (int c = 0; c < kSplitMax; ++c)   // all loads first: one round trip
          if (c < a.attn_split) {
            mc[c] = ph[c * Wd + a.dh];
            lc[c] = ph[c * Wd + a.dh + 1];
            oc[c] = ph[c * Wd + j % a.dh];
          }
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < kSplitMax; ++c)
          if (c < a.attn_split) m = fmaxf(m, mc[c]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int c = 0; c < kSplitMax; ++c)
          if (c < a.attn_split && mc[c] != -INFINITY) {   // an empty key range adds nothing
            const float e = expf(mc[c] - m);
            num += e * oc[c];
            den += e * lc[c];
          }
        xq[j] = num / den;
      }
    } else if (!a.ln_g) {
      const float* xin = a.xin + (int64_t)q * a.xin_ss;
      for (int j = threadIdx.x; j < a.K; j += kThreads) xq[j] = xin[j];   // any K (the MLP down product)
    } else {
      // LayerNorm'd input: K = d_model <= 1024, four elements per thread
      const float* xin = a.xin + (int64_t)q * a.xin_ss;
      const float x0 = xin[0];
#pragma unroll
      for (int m = 0; m < kMaxK; ++m) {
        const int j = threadIdx.x + m * kThreads;
        xv[m] = j < a.K ? xin[j] : 0.f;
      }
      {
        // one reduction for the sum and the sum of squares, both shifted by the
        // first element (the shift keeps the variance free of cancellation when
        // the mean is large against the spread)
        float s0 = 0.f, qq = 0.f;
#pragma unroll
        for (int m = 0; m < kMaxK; ++m)
          if (threadIdx.x + m * kThreads < a.K) {
            const float dv = xv[m] - x0;
            s0 += dv;
            qq += dv * dv;
          }
        const float2 sq = block_sum2_dpp(s0, qq, red);
        const float ms = sq.x / a.K;
        const float mean = x0 + ms;
        const float rstd = 1.0f / sqrtf(fmaxf(sq.y / a.K - ms * ms, 0.f) + 1e-5f);
#pragma unroll
        for (int m = 0; m < kMaxK; ++m) xv[m] = (xv[m] - mean) * rstd * gv[m] + bv[m];
      }
#pragma unroll
      for (int m = 0; m < kMaxK; ++m) {
        const int j = threadIdx.x + m * kThreads;
        if (j < a.K) xq[j] = xv[m];
      }
    }
  }
  __syncthreads();
  // this lane's input chunks of one sequence, in registers
  float xr[kDecMaxChunks][8];
  auto load_xr = [&](int q) {
    const float* xq = xs + (size_t)q * a.K;
    const int li = threadIdx.x % a.lpr;
    const bool bf = a.w_dt == DT_BF16;
    const int nch = dec_row_bytes(a) / 16;
#pragma unroll
    for (int j = 0; j < kDecMaxChunks; ++j) {
      const int c = li + j * a.lpr;
      float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
      if (c < nch) {
        if (bf) {
          lo = *(const float4*)(xq + c * 8);
          hi = *(const float4*)(xq + c * 8 + 4);
        } else {
          lo = *(const float4*)(xq + c * 4);
        }
      }
      xr[j][0] = lo.x; xr[j][1] = lo.y; xr[j][2] = lo.z; xr[j][3] = lo.w;
      xr[j][4] = hi.x; xr[j][5] = hi.y; xr[j][6] = hi.z; xr[j][7] = hi.w;
    }
  };
  if (ns == 1) load_xr(0);   // one sequence: loaded once for the whole ticket
  for (int i = 0; i < nt; ++i) {
    // tile i landed in every wave, and every wave is done with tile i - 1's buffer
    dec_wait_tile(issued - i - 1);
    if (a.n_buf > 1 && i >= 1 && issued < nt) {   // refill the buffer tile i - 1 used
      dec_tile_issue(a, W, t0 + issued, ring, issued % a.n_buf);
      ++issued;
    }
    for (int q = 0; q < ns; ++q) {
      if (ns > 1) load_xr(q);
      dec_tile_dot(a, ring + (size_t)(i % a.n_buf) * kDecTile, dec_tile_rows(a, t0 + i), xr,
                   ys + (size_t)q * a.ys_rows + i * a.rows_per_tile, ys2 + (size_t)q * a.ys_rows + i * a.rows_per_tile);
    }
    if (a.n_buf == 1 && issued < nt) {   // one buffer: refill once every wave has read it
      __syncthreads();
      dec_tile_issue(a, W, t0 + issued, ring, 0);
      ++issued;
    }
  }
  __syncthreads();
  // epilogue over the ticket's rows, sequence by sequence
  for (int q = 0; q < ns; ++q) {
    const float* ysq = ys + (size_t)q * a.ys_rows;
    const float* ys2q = ys2 + (size_t)q * a.ys_rows;
    float* yq = a.y + (int64_t)q * a.y_ss;
    const float* rq = a.resid ? a.resid + (int64_t)q * a.resid_ss : nullptr;
    void* kvq = a.kv ? (void*)((char*)a.kv + (size_t)q * a.kv_ss * (a.kv_dt == DT_BF16 ? 2 : 4)) : nullptr;
    for (int i = threadIdx.x, m = 0; i < nrows; i += kThreads, ++m) {
      const int n = r0 + i;
      float v = ysq[i];
      float rv = 0.f;
      if (m < kPre) {
#pragma unroll
        for (int u = 0; u < kPre; ++u)
          if (u == m) {
            v += pre_b[u];
            rv = pre_r[u];
          }
        if (q > 0 && a.epi == DEPI_RESID) rv = rq[n];
      } else {
        if (bias) v += ldf(bias, n, a.w_dt);
        if (a.epi == DEPI_RESID) rv = rq[n];
      }
      switch (a.epi) {
        case DEPI_STORE: yq[n] = v; break;
        case DEPI_RESID: yq[n] = rv + v; break;
        case DEPI_GELU: yq[n] = gelu_f(v); break;
        case DEPI_GEGLU: yq[n] = gelu_f(v) * ys2q[i]; break;
        case DEPI_LOGITS:
          yq[n] = v;
          if (logits_out) logits_out[(gen_idx * ns + q) * a.N + n] = v;
          break;
        case DEPI_QKV: {
          // a ticket covers whole heads when the rotation is on (host plan)
          const int part = n / a.d, h = (n % a.d) / a.dh, j = n % a.dh;
          float out = v;
          if (a.rope && part < 2) {
            const int hl = a.dh / 2;
            const int jj = j < hl ? j : j - hl;
            const double ang = (double)pos * pow(10000.0, -2.0 * jj / a.dh);
            const float c = (float)cos(ang), sn = (float)sin(ang);
            const int io = j < hl ? i + hl : i - hl;
            float other = ysq[io];
            if (bias) other += ldf(bias, r0 + io, a.w_dt);
            out = j < hl ? v * c - other * sn : other * sn + v * c;
          }
          if (part == 0) {
            yq[n] = out;
          } else {
            const int64_t ci = (((int64_t)(part - 1) * a.H + h) * a.cap + pos) * a.dh + j;
            stf(kvq, ci, a.kv_dt, out);
          }
        } break;
      }
    }
    if (a.epi == DEPI_LOGITS) {
      // this ticket's (max, first index): ascending per thread, then lowest index
      // among equal maxima; a NaN never wins
      float bvv = -INFINITY;
      int bi = 0x7fffffff;
      for (int i = threadIdx.x; i < nrows; i += kThreads)
        if (ysq[i] > bvv) {
          bvv = ysq[i];
          bi = r0 + i;
        }
      argmax_combine_block(bvv, bi, red);
      if (threadIdx.x == 0) {
        const int ticket = t0 / a.per_ticket;
        a.part_val[(int64_t)q * a.part_ss + ticket] = bvv;
        a.part_idx[(int64_t)q * a.part_ss + ticket] = bi;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void task_dec_gemv_range(const DecGemvArgs& a, int t0, int t1, const TaskCtx& tc, char* smem,
                                                    int npre) {
  if (a.nseq > 1) task_dec_gemv_range_t<true>(a, t0, t1, tc, smem, npre);
  else task_dec_gemv_range_t<false>(a, t0, t1, tc, smem, npre);
}

__device__ void task_dec_gemv(const DecGemvArgs& a, int tile, const TaskCtx& tc, char* smem) {
  task_dec_gemv_range(a, tile, tile + 1, tc, smem, 0);
}

// ---------------------------------------------------------------- attention
// Tile = (head h, key range c of `split`): scores of the query against the
// cached keys of the range, their maximum m, weights exp(score - m), their sum
// l and the weighted sum of the values o; the consumer (the output-projection
// GEMV) rescales the ranges to a common maximum and divides ("flash decoding":
// the softmax of the whole row, taken in pieces).

__host__ __device__ inline int dec_attn_ept(const DecAttnArgs& a) {
  return a.kv_dt == DT_BF16 ? 8 : (a.dh % 4 == 0 ? 4 : 2);
}

__host__ __device__ inline size_t dec_attn_lds_bytes(const DecAttnArgs& a) {
  const int ept = dec_attn_ept(a);
  return (size_t)(a.cap + a.dh + (kThreads / (a.dh / ept)) * a.dh + 16) * sizeof(float);
}

// elements [e0, e0 + ept) of a cache row, as fp32
__device__ __forceinline__ void kv_chunk(const void* kv, int64_t e0, int dt, int ept, float* out) {
  if (dt == DT_BF16) {
    const uint4 u = *(const uint4*)((const uint16_t*)kv + e0);
    out[0] = bf2f(u.x & 0xffff); out[1] = bf2f(u.x >> 16); out[2] = bf2f(u.y & 0xffff); out[3] = bf2f(u.y >> 16);
    out[4] = bf2f(u.z & 0xffff); out[5] = bf2f(u.z >> 16); out[6] = bf2f(u.w & 0xffff); out[7] = bf2f(u.w >> 16);
  } else if (ept == 4) {
    const float4 u = *(const float4*)((const float*)kv + e0);
    out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
  } else {
    const float2 u = *(const float2*)((const float*)kv + e0);
    out[0] = u.x; out[1] = u.y;
  }
}

template <int ept>
__device__ void dec_attn_tile(const DecAttnArgs& a, int tile, const TaskCtx& tc, char* smem) {
  constexpr int kKMax = 64 / ept;   // chunks of a key row (head size <= 64)
  constexpr int kVPre = 4;          // value rows per thread read ahead
  const int sq = tile / (a.H * a.split);
  const int h = (tile / a.split) % a.H, c = tile % a.split;
  const int pos = tc.sc->pos;
  const float* qv_base = a.q + (int64_t)sq * a.H * a.dh;
  const void* kvq = (const char*)a.kv + (size_t)sq * a.kv_ss * (a.kv_dt == DT_BF16 ? 2 : 4);
  const int n_keys = pos + 1;
  const int cl = (n_keys + a.split - 1) / a.split;
  const int s0 = min(c * cl, n_keys), s1 = min(s0 + cl, n_keys);
  float* sc = (float*)smem;                         // [cap]
  float* qs = sc + a.cap;                           // [dh]
  float* acc2 = qs + a.dh;                          // [row slots][dh]
  const int lpr = a.dh / ept, slots = kThreads / lpr;
  float* red = acc2 + slots * a.dh;                 // [16]
  float* out = a.part + (int64_t)sq * a.part_ss + (int64_t)(tile % (a.H * a.split)) * (a.dh + 2);
  const float scale = 1.0f / sqrtf((float)a.dh);
  const int64_t kbase = (int64_t)h * a.cap * a.dh;
  const int64_t vbase = ((int64_t)a.H + h) * a.cap * a.dh;
  const int nkc = a.dh / ept;
  const int slot = threadIdx.x / lpr, ci = threadIdx.x % lpr;
  // every load that does not depend on another is issued first: the query, this
  // thread's first key row and its first value chunks
  const float qv = threadIdx.x < a.dh ? qv_base[h * a.dh + threadIdx.x] : 0.f;
  const int s_k = s0 + threadIdx.x;
  float kr[kKMax][ept];
#pragma unroll
  for (int j = 0; j < kKMax; ++j)
    if (j < nkc && s_k < s1) kv_chunk(kvq, kbase + (int64_t)s_k * a.dh + j * ept, a.kv_dt, ept, kr[j]);
  float vr[kVPre][ept];
#pragma unroll
  for (int m = 0; m < kVPre; ++m) {
    const int s = s0 + slot + m * slots;
    if (s < s1) kv_chunk(kvq, vbase + (int64_t)s * a.dh + ci * ept, a.kv_dt, ept, vr[m]);
  }
  if (threadIdx.x < a.dh) qs[threadIdx.x] = qv * scale;
  __syncthreads();
  if (s0 >= s1) {   // empty range
    for (int j = threadIdx.x; j < a.dh; j += kThreads) out[j] = 0.f;
    if (threadIdx.x == 0) {
      out[a.dh] = -INFINITY;
      out[a.dh + 1] = 0.f;
    }
    __syncthreads();
    return;
  }
  // scores: one thread per key
  float mx = -INFINITY;
  if (s_k < s1) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kKMax; ++j)
      if (j < nkc)
#pragma unroll
        for (int e = 0; e < ept; ++e) acc += qs[j * ept + e] * kr[j][e];
    sc[s_k - s0] = acc;
    mx = acc;
  }
  for (int s = s_k + kThreads; s < s1; s += kThreads) {   // ranges longer than the workgroup
    float acc = 0.f;
    for (int j = 0; j < a.dh; j += ept) {
      float k[8];
      kv_chunk(kvq, kbase + (int64_t)s * a.dh + j, a.kv_dt, ept, k);
#pragma unroll
      for (int e = 0; e < ept; ++e) acc += qs[j + e] * k[e];
    }
    sc[s - s0] = acc;
    mx = fmaxf(mx, acc);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int s = s0 + threadIdx.x; s < s1; s += kThreads) {
    const float p = expf(sc[s - s0] - mx);
    sc[s - s0] = p;
    sum += p;
  }
  sum = block_sum(sum, red + kWaves);   // ends with a barrier: every weight is in LDS
  // weighted values: lpr lanes per value row, `slots` rows at a time
  float o[ept];
#pragma unroll
  for (int e = 0; e < ept; ++e) o[e] = 0.f;
#pragma unroll
  for (int m = 0; m < kVPre; ++m) {
    const int s = s0 + slot + m * slots;
    if (s < s1) {
      const float p = sc[s - s0];
#pragma unroll
      for (int e = 0; e < ept; ++e) o[e] += p * vr[m][e];
    }
  }
  for (int s = s0 + slot + kVPre * slots; s < s1; s += slots) {
    float v[8];
    kv_chunk(kvq, vbase + (int64_t)s * a.dh + ci * ept, a.kv_dt, ept, v);
    const float p = sc[s - s0];
#pragma unroll
    for (int e = 0; e < ept; ++e) o[e] += p * v[e];
  }
#pragma unroll
  for (int e = 0; e < ept; ++e) acc2[slot * a.dh + ci * ept + e] = o[e];
  __syncthreads();
  for (int j = threadIdx.x; j < a.dh; j += kThreads) {
    float t = 0.f;
    for (int q = 0; q < slots; ++q) t += acc2[q * a.dh + j];
    out[j] = t;
  }
  if (threadIdx.x == 0) {
    out[a.dh] = mx;
    out[a.dh + 1] = sum;
  }
  __syncthreads();
}

__device__ void task_dec_attn(const DecAttnArgs& a, int tile, const TaskCtx& tc, char* smem) {
  switch (dec_attn_ept(a)) {
    case 8: dec_attn_tile<8>(a, tile, tc, smem); break;
    case 4: dec_attn_tile<4>(a, tile, tc, smem); break;
    default: dec_attn_tile<2>(a, tile, tc, smem); break;
  }
}

// ---------------------------------------------------------------- argmax + context update

__device__ void task_dec_argmax(const DecArgmaxArgs& a, int tile, const TaskCtx& tc, char* smem) {
  if (!(tc.sc->head & 1)) return;
  float* red = (float*)smem;   // [16]
  int* ys = (int*)(red + 16);  // [nseq] chosen tokens
  for (int q = 0; q < a.nseq; ++q) {
    float best = -INFINITY;
    int idx = 0x7fffffff;
    for (int i = threadIdx.x; i < a.n_part; i += kThreads) {
      const float z = a.part_val[q * a.part_ss + i];
      const int zi = a.part_idx[q * a.part_ss + i];
      if (z > best || (z == best && zi < idx)) {
        best = z;
        idx = zi;
      }
    }
    argmax_combine_block(best, idx, red);
    if (threadIdx.x == 0) ys[q] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    DecState* st = a.st;
    const int gi = tc.sc->gen_idx;
    const int64_t g = tc.gen_base + gi;   // tokens emitted before this one
    const int64_t slot = g % a.io->ring_len;
    const int L = st->ctx_len;
    for (int q = 0; q < a.nseq; ++q) {
      int y = ys[q];
      if (y < 0 || y >= a.V) {   // every logit was NaN
        raise_status(tc.status, -3 /*OFA_E_NONFINITE*/, tc.phase, tc.step, 0);
        y = 0;
      }
      a.io->tokens_out[slot * a.nseq + q] = y;
      int32_t* ctx = a.ctx_tok + q * a.cap;
      if (L + 1 > a.cap) {
        // context full: keep the most recent `keep` tokens (the new one included) at 0..keep-1
        for (int i = 0; i < a.keep - 1; ++i) ctx[i] = ctx[L - a.keep + 1 + i];
        ctx[a.keep - 1] = y;
      } else {
        ctx[L] = y;
      }
    }
    if (a.io->versions_out) a.io->versions_out[slot] = st->version;
    if (a.io->ticks && g < a.io->n_ticks) a.io->ticks[2 * g + 1] = now_ticks();
    // system scope: the count may live in host memory the host polls
    if (a.io->n_generated) __hip_atomic_store(a.io->n_generated, (uint64_t)(g + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    st->ctx_len = L + 1 > a.cap ? a.keep : L + 1;
    st->n_gen = gi + 1;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- evaluation probe

// What the model predicts after row r of an evaluated context ("Coppelius
// training on the RTX 3090", "Prompt probe" and "Prediction entropy"): the
// most likely next token (lowest id on exact ties) and the entropy of the
// softmax of the logits, H = log(sum e^(z - m)) - sum e^(z - m) (z - m) / sum e^(z - m)
// with m the row maximum.  One probed row per tile.
__device__ void task_probe(const ProbeArgs& a, int tile, const TaskCtx& tc, char* smem) {
  const StepCtx* sc = tc.sc;
  if (tile >= sc->n_probe || !sc->probe_rows) return;
  float* red = (float*)smem;   // [32]
  const int r = sc->probe_rows[tile];
  if (r < 0 || r >= a.rows) {
    if (threadIdx.x == 0) raise_status(tc.status, -1 /*OFA_E_ARG*/, tc.phase, tc.step, r);
    return;
  }
  const float* z = a.logits + (int64_t)r * a.V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < a.V; i += kThreads) {
    const float v = z[i];
    if (v > bv) {   // ascending i: a thread keeps its first maximum
      bv = v;
      bi = i;
    }
  }
  argmax_combine_block(bv, bi, red);
  const float m = bv;
  float s = 0.f, t = 0.f;
  for (int i = threadIdx.x; i < a.V; i += kThreads) {
    const float d = z[i] - m;
    const float e = expf(d);
    s += e;
    t += e * d;
  }
  s = block_sum(s, red + 16);
  t = block_sum(t, red + 24);
  if (threadIdx.x == 0) {
    if (sc->probe_argmax) sc->probe_argmax[tile] = bi;
    if (sc->probe_entropy) sc->probe_entropy[tile] = logf(s) - t / s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- co-resident training

// The training step about to write serve slot (tag & 1) waits until the
// decoder has moved to version tag - 1 or later: the slot then holds no
// version the decoder still reads (version v lives in slot v & 1).  Waits only
// while co-resident decode runs; gives up on an error elsewhere or after ~10 s.
__device__ void task_slot_guard(const GuardArgs& a, const TaskCtx& tc) {
  if (threadIdx.x != 0) return;
  if (!__hip_atomic_load(&a.st->serving, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  const uint64_t need = tc.sc->tag - 1;
  const uint64_t start = now_ticks();
  for (int spins = 0; ld_acquire(&a.st->version) < need; ++spins) {
    if (__hip_atomic_load(&tc.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    __builtin_amdgcn_s_sleep(2);
    if ((spins & 63) == 63 && now_ticks() - start > 1000000000ull) {
      raise_status(tc.status, -4 /*OFA_E_TIMEOUT*/, tc.phase, tc.step, (int64_t)need);
      return;
    }
  }
}

// The step's weights (written to slot tag & 1 by AdamW, complete: this phase
// depends on it) become version tag.
// A step whose update was skipped after an error publishes nothing.
__device__ void task_publish(const PublishArgs& a, const TaskCtx& tc) {
  if (threadIdx.x == 0 && !__hip_atomic_load(&tc.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
    st_release(a.published, tc.sc->tag);
}

}  // namespace ofa
