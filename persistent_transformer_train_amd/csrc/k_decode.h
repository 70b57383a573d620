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
// not depend on them), so weight streaming overlaps the wait.
//
// Roles: waves 1..3 issue every weight copy; wave 0 issues none and reads
// everything else the ticket needs (the input vector, the LayerNorm
// parameters, bias and residual rows, the attention partials).  A wave's
// vector-memory counter completes in issue order, so a load issued behind a
// wave's copies would wait for all of them: with the copies out of wave 0 the
// input arrives while the weights are still streaming.  Every copy wave issues
// the same number of copies per tile, so every wait count is a constant.
//
// Rows are dot products of lpr lanes (16-byte chunks i, i + lpr, ...) against
// the LayerNorm'd input held in registers, each group of lpr lanes taking RPG
// rows per pass and reducing with DPP row operations.  The argument block and
// the instance's StepCtx are read through wave-uniform constant-address views
// (scalar loads: they are fixed for the whole launch and stay off the vector
// counter).

constexpr int kDecCopyWaves = kWaves - 1;                     // waves 1..3 stream the weights
constexpr int kDecCopies = 8;                                 // copies per copy wave per tile
constexpr int kDecTile = kDecCopyWaves * kDecCopies * 1024;   // bytes of one tile buffer (24 KB)
constexpr int kDecMaxChunks = 8;                              // 16-byte chunks of a row per lane

// constant address space on the device (the host pass of the same source,
// which emits none of this code, sees plain types)
#if defined(__HIP_DEVICE_COMPILE__)
#define OFA_CONST_AS __attribute__((address_space(4)))
#else
#define OFA_CONST_AS
#endif
typedef const OFA_CONST_AS DecGemvArgs DecGemvArgsC;
typedef const OFA_CONST_AS StepCtx StepCtxC;

// wave-uniform constant-address view of data that no wave writes during the launch
template <typename C, typename T>
__device__ __forceinline__ C* const_view(const T* p) {
  return (C*)(uintptr_t)readfirstlane_u64((uint64_t)(uintptr_t)p);
}

__host__ __device__ inline int dec_tile_rows_all(const DecGemvArgs& a) {
  return (a.epi == DEPI_GEGLU ? 2 : 1) * a.rows_per_tile;
}

__host__ __device__ inline int dec_nseq(const DecGemvArgs& a) { return a.nseq > 1 ? a.nseq : 1; }
// attention partials of one sequence, staged for the output projection
__host__ __device__ inline int dec_stage_floats(const DecGemvArgs& a) {
  return a.attn_part ? a.H * a.attn_split * (a.dh + 2) : 0;
}
// LDS: [ring n_buf x kDecTile][xs: nseq K][ys: nseq ys_rows][ys2: nseq ys_rows, gated MLP]
//      [eb: ys_rows bias][er: nseq ys_rows residual][stage: attention partials]
//      [scl: H split range weights][lnp: LayerNorm gain, shift][braw: bias as stored]
//      [xraw: LayerNorm input][64 scratch]
struct DecLds {
  int xs, ys, ys2, eb, er, stage, scl, lnp, braw, xraw, red, total;   // float offsets after the ring
};
// areas that wave 0 fills by direct-to-LDS copies are whole 1 KB blocks
__host__ __device__ inline int dec_pad1k(int nfloats) { return (nfloats + 255) & ~255; }
__host__ __device__ inline DecLds dec_lds_layout(const DecGemvArgs& a) {
  const int ns = dec_nseq(a);
  DecLds L;
  L.xs = 0;
  L.ys = L.xs + dec_pad1k(ns * a.K);
  L.ys2 = L.ys + ns * a.ys_rows;
  L.eb = L.ys2 + (a.epi == DEPI_GEGLU ? ns * a.ys_rows : 0);
  L.er = L.eb + (a.bias ? a.ys_rows : 0);
  L.stage = L.er + (a.epi == DEPI_RESID ? dec_pad1k(ns * a.ys_rows) : 0);
  L.scl = L.stage + (a.attn_part ? dec_pad1k(dec_stage_floats(a)) : 0);
  L.lnp = L.scl + (a.attn_part ? ((a.H * a.attn_split + 3) & ~3) : 0);
  L.braw = L.lnp + (a.ln_g ? 2 * dec_pad1k(a.K) : 0);
  L.xraw = L.braw + (a.bias ? dec_pad1k(a.ys_rows) : 0);
  L.red = L.xraw + (a.ln_g ? dec_pad1k(a.K) : 0);
  L.total = L.red + 64;
  return L;
}
__host__ __device__ inline size_t dec_gemv_lds_bytes(const DecGemvArgs& a) {
  return (size_t)a.n_buf * kDecTile + (size_t)dec_lds_layout(a).total * sizeof(float);
}

__device__ __forceinline__ int dec_row_bytes(const DecGemvArgs& a) { return a.K * (a.w_dt == DT_BF16 ? 2 : 4); }

// rows of W a tile of this GEMV covers (output rows; GEGLU: per half)
__device__ __forceinline__ int dec_tile_rows(const DecGemvArgs& a, int tile) {
  const int total = a.epi == DEPI_GEGLU ? a.F : a.N;
  return min(a.rows_per_tile, total - tile * a.rows_per_tile);
}

// N copies per copy wave of [src, src + 3 KB N) into dst; reads past `valid`
// bytes re-read the last valid chunk (nothing is read out of range).  Wave 0
// returns at once.
template <int N>
__device__ __forceinline__ void dec_copy_n(const char* src, int valid, char* dst) {
  const int w = threadIdx.x / kWave - 1, lane = threadIdx.x % kWave;
  if (w < 0) return;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int blk = j * kDecCopyWaves + w;
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
// then join the workgroup barrier (wave 0 has no copies: its waits pass)
__device__ __forceinline__ void dec_wait_tile(int later) {
  if (later >= 3) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" : : : "memory");
  else if (later == 2) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" : : : "memory");
  else if (later == 1) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" : : : "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
}
static_assert(kDecCopies == 8, "wait counts above assume 8 copies per copy wave per tile");

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

// Products of bf16 weights with an fp32 input: the input is carried as two
// bf16 terms, hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in fp32, so
// hi + lo matches x to about 2^-17 relative), and each 16-byte chunk of a row
// takes eight bf16 pair dot products with fp32 accumulation (v_dot2 on gfx950)
// instead of eight conversions and eight fused multiply-adds.
typedef __bf16 ofa_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t w2, uint32_t x2, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(ofa_bf16x2, w2), __builtin_bit_cast(ofa_bf16x2, x2), c, false);
}
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);   // round to nearest even
}
// 8 fp32 inputs -> 4 packed hi pairs in out[0..3], 4 packed lo pairs in out[4..7]
__device__ __forceinline__ void dec_split_x(const float4& a, const float4& b, float* out) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h0 = bf16_bits(v[2 * i]), h1 = bf16_bits(v[2 * i + 1]);
    const uint32_t l0 = bf16_bits(v[2 * i] - __uint_as_float(h0 << 16));
    const uint32_t l1 = bf16_bits(v[2 * i + 1] - __uint_as_float(h1 << 16));
    out[i] = __uint_as_float(h0 | (h1 << 16));
    out[4 + i] = __uint_as_float(l0 | (l1 << 16));
  }
}

// Dot products of one LDS tile's rows with the input chunks in xr; row rr of
// the tile (GEGLU: rows R.. are the up half) lands in ys[rr] or ys2[rr - R].
// A lane reads all chunks of a row before it uses one; cpl (whole chunks per
// lane) is wave-uniform, so only a ragged row's last chunk is lane-masked.
template <int RPG, bool BF16>
__device__ __forceinline__ void dec_dot_rows(const char* tilep, int lpr, int rb, int R, int TR, int rows,
                                             const float (&xr)[kDecMaxChunks][8], float* ys, float* ys2) {
  const int ng = kThreads / lpr;
  const int grp = threadIdx.x / lpr, li = threadIdx.x % lpr;
  const int nch = rb / 16;
  const int cpl = nch / lpr;
  const bool ragged = cpl * lpr != nch;
  const bool tail = li + cpl * lpr < nch;
  constexpr int half = kDecTile / 2;
#pragma unroll
  for (int k = 0; k < RPG; ++k) {
    const int rr = grp + k * ng;
    const bool ok = rr < TR && rr % R < rows;
    const char* rowp = tilep + (ok ? (rr / R) * half + (rr % R) * rb : 0) + li * 16;
    uint4 u[kDecMaxChunks];
#pragma unroll
    for (int j = 0; j < kDecMaxChunks; ++j) {
      u[j] = make_uint4(0u, 0u, 0u, 0u);
      if (j < cpl) u[j] = *(const uint4*)(rowp + j * lpr * 16);
    }
    if (ragged) {
#pragma unroll
      for (int j = 0; j < kDecMaxChunks; ++j)
        if (j == cpl && tail) u[j] = *(const uint4*)(rowp + j * lpr * 16);
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kDecMaxChunks; ++j) {
      if (j < cpl || (ragged && j == cpl)) {
        if constexpr (BF16) {
          float ah = 0.f, al = 0.f;
          ah = dot2_bf16(u[j].x, __float_as_uint(xr[j][0]), ah);
          al = dot2_bf16(u[j].x, __float_as_uint(xr[j][4]), al);
          ah = dot2_bf16(u[j].y, __float_as_uint(xr[j][1]), ah);
          al = dot2_bf16(u[j].y, __float_as_uint(xr[j][5]), al);
          ah = dot2_bf16(u[j].z, __float_as_uint(xr[j][2]), ah);
          al = dot2_bf16(u[j].z, __float_as_uint(xr[j][6]), al);
          ah = dot2_bf16(u[j].w, __float_as_uint(xr[j][3]), ah);
          al = dot2_bf16(u[j].w, __float_as_uint(xr[j][7]), al);
          acc += ah + al;
        } else {
          acc += __uint_as_float(u[j].x) * xr[j][0] + __uint_as_float(u[j].y) * xr[j][1] +
                 __uint_as_float(u[j].z) * xr[j][2] + __uint_as_float(u[j].w) * xr[j][3];
        }
      }
    }
    const float v = dpp_group_sum(acc, lpr);
    if (li == lpr - 1 && ok) {
      if (rr < R) ys[rr] = v;
      else ys2[rr - R] = v;
    }
  }
}

// The same with the chunk count fixed at compile time and no ragged chunk:
// straight-line loads, then the products (the shape of every large model's rows).
template <bool BF16, int CPL>
__device__ __forceinline__ void dec_dot_rows_fixed(const char* tilep, int lpr, int rb, int R, int TR, int rows,
                                                   const float (&xr)[kDecMaxChunks][8], float* ys, float* ys2) {
  const int lg = __builtin_ctz(lpr);
  const int grp = threadIdx.x >> lg, li = threadIdx.x & (lpr - 1);
  const int hsel = grp >= R ? 1 : 0;   // gated MLP: second half of the tile
  const int rw = grp - hsel * R;
  const bool ok = grp < TR && rw < rows;
  const char* rowp = tilep + (ok ? hsel * (kDecTile / 2) + rw * rb : 0) + li * 16;
  uint4 u[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) u[j] = *(const uint4*)(rowp + j * lpr * 16);
  float acc = 0.f;
  if constexpr (BF16) {
    // two-term bf16 input (high and low parts, see dec_split_x): bf16 pair dot
    // products with fp32 accumulation, one chain per part
    float ah[2] = {0.f, 0.f}, al[2] = {0.f, 0.f};   // four independent chains
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float& h = ah[j & 1];
      float& l = al[j & 1];
      h = dot2_bf16(u[j].x, __float_as_uint(xr[j][0]), h);
      l = dot2_bf16(u[j].x, __float_as_uint(xr[j][4]), l);
      h = dot2_bf16(u[j].y, __float_as_uint(xr[j][1]), h);
      l = dot2_bf16(u[j].y, __float_as_uint(xr[j][5]), l);
      h = dot2_bf16(u[j].z, __float_as_uint(xr[j][2]), h);
      l = dot2_bf16(u[j].z, __float_as_uint(xr[j][6]), l);
      h = dot2_bf16(u[j].w, __float_as_uint(xr[j][3]), h);
      l = dot2_bf16(u[j].w, __float_as_uint(xr[j][7]), l);
    }
    acc = (ah[0] + ah[1]) + (al[0] + al[1]);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      acc += __uint_as_float(u[j].x) * xr[j][0] + __uint_as_float(u[j].y) * xr[j][1] +
             __uint_as_float(u[j].z) * xr[j][2] + __uint_as_float(u[j].w) * xr[j][3];
  }
  const float v = dpp_group_sum(acc, lpr);
  if (li == lpr - 1 && ok) {
    if (hsel == 0) ys[rw] = v;
    else ys2[rw] = v;
  }
}

// CPL > 0: the fixed-count dot (chunks per lane known at compile time);
// CPL == 0: the general one
template <bool BF16, int CPL>
__device__ __forceinline__ void dec_tile_dot(int rpg, const char* tilep, int lpr, int rb, int R, int TR, int rows,
                                             const float (&xr)[kDecMaxChunks][8], float* ys, float* ys2) {
  if constexpr (CPL > 0) {
    dec_dot_rows_fixed<BF16, CPL>(tilep, lpr, rb, R, TR, rows, xr, ys, ys2);
  } else {
    switch (rpg) {
      case 1: dec_dot_rows<1, BF16>(tilep, lpr, rb, R, TR, rows, xr, ys, ys2); break;
      case 2: dec_dot_rows<2, BF16>(tilep, lpr, rb, R, TR, rows, xr, ys, ys2); break;
      case 4: dec_dot_rows<4, BF16>(tilep, lpr, rb, R, TR, rows, xr, ys, ys2); break;
      default: dec_dot_rows<8, BF16>(tilep, lpr, rb, R, TR, rows, xr, ys, ys2); break;
    }
  }
}

// this lane's input chunks of one sequence (xq: K values in LDS), in registers;
// for bf16 weights xq holds the split high / low bf16 pairs of dec_split_xs
template <bool BF16>
__device__ __forceinline__ void dec_load_xr(const float* xq, int lpr, int rb, float (&xr)[kDecMaxChunks][8]) {
  const int li = threadIdx.x % lpr;
  const int nch = rb / 16;
#pragma unroll
  for (int j = 0; j < kDecMaxChunks; ++j) {
    const int c = li + j * lpr;
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (c < nch) {
      if (BF16) {
        lo = *(const float4*)(xq + c * 8);
        hi = *(const float4*)(xq + c * 8 + 4);
      } else {
        lo = *(const float4*)(xq + c * 4);
      }
    }
    // bf16 weights: the chunk already holds its split pairs (dec_split_xs)
    xr[j][0] = lo.x; xr[j][1] = lo.y; xr[j][2] = lo.z; xr[j][3] = lo.w;
    xr[j][4] = hi.x; xr[j][5] = hi.y; xr[j][6] = hi.z; xr[j][7] = hi.w;
  }
}

// bf16 weights: every 8-element chunk of the inputs xs[0 .. n) (n a multiple of
// 8) replaced in place by its split form (four hi pairs, then four lo pairs),
// once per ticket, so the tile loop only reads it
__device__ __forceinline__ void dec_split_xs(float* xs, int n) {
  for (int c = threadIdx.x; c < n / 8; c += kThreads) {
    float4* p = (float4*)(xs + c * 8);
    float out[8];
    dec_split_x(p[0], p[1], out);
    p[0] = make_float4(out[0], out[1], out[2], out[3]);
    p[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

// The tiles of one ticket: wait for tile i, refill the ring, dot products of
// every sequence.  Returns nothing; ys / ys2 hold the ticket's row sums.
template <bool MULTI, bool BF16, int CPL>
__device__ __forceinline__ void dec_tiles(const DecGemvArgs& a, const char* W, char* ring, int t0, int nt, int issued,
                                          const float* xs, float* ys, float* ys2) {
  const int ns = MULTI ? dec_nseq(a) : 1;
  const int lpr = a.lpr, rb = dec_row_bytes(a), R = a.rows_per_tile, TR = dec_tile_rows_all(a), rpg = a.rpg;
  float xr[kDecMaxChunks][8];
  if (ns == 1) dec_load_xr<BF16>(xs, lpr, rb, xr);   // one sequence: loaded once for the whole ticket
  for (int i = 0; i < nt; ++i) {
    // tile i landed in every wave, and every wave is done with tile i - 1's buffer
    dec_wait_tile(issued - i - 1);
    if (a.n_buf > 1 && i >= 1 && issued < nt) {   // refill the buffer tile i - 1 used
      dec_tile_issue(a, W, t0 + issued, ring, issued % a.n_buf);
      ++issued;
    }
    const int rows = dec_tile_rows(a, t0 + i);
    for (int q = 0; q < ns; ++q) {
      if (ns > 1) dec_load_xr<BF16>(xs + (size_t)q * a.K, lpr, rb, xr);
      dec_tile_dot<BF16, CPL>(rpg, ring + (size_t)(i % a.n_buf) * kDecTile, lpr, rb, R, TR, rows, xr,
                              ys + (size_t)q * a.ys_rows + i * R, ys2 + (size_t)q * a.ys_rows + i * R);
    }
    if (a.n_buf == 1 && issued < nt) {   // one buffer: refill once every wave has read it
      __syncthreads();
      dec_tile_issue(a, W, t0 + issued, ring, 0);
      ++issued;
    }
  }
}

// Wave 0: n weights (bf16 or fp32) at src[0..n) into dst as fp32, 16 per lane per round.
template <bool BF16>
__device__ __forceinline__ void w0_load_w(const void* src, int n, float* dst) {
  const int lane = threadIdx.x;
  for (int b = 0; b < n; b += 16 * kWave) {
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {   // clamped index: every load is issued, one wait for all
      const int i = min(b + lane + m * kWave, n - 1);
      v[m] = BF16 ? bf2f(((const uint16_t*)src)[i]) : ((const float*)src)[i];
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = b + lane + m * kWave;
      if (i < n) dst[i] = v[m];
    }
  }
}

// Wave 0: n fp32 values at src into dst.  16-byte loads (16 per lane, 4096
// values per round) when src is 16-byte aligned and n a multiple of 4, else
// 16 single loads per lane per round.
__device__ __forceinline__ void w0_load_f(const float* src, int n, float* dst) {
  const int lane = threadIdx.x;
  if ((((uintptr_t)src | (uintptr_t)dst) & 15) == 0 && (n & 3) == 0) {
    const int n4 = n / 4;
    for (int b = 0; b < n4; b += 16 * kWave) {
      float4 v[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) v[m] = ((const float4*)src)[min(b + lane + m * kWave, n4 - 1)];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = b + lane + m * kWave;
        if (i < n4) ((float4*)dst)[i] = v[m];
      }
    }
    return;
  }
  for (int b = 0; b < n; b += 16 * kWave) {
    float v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = src[min(b + lane + m * kWave, n - 1)];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = b + lane + m * kWave;
      if (i < n) dst[i] = v[m];
    }
  }
}

// Wave 0: LayerNorm of x[0..K) (K <= 1024) with parameters g, b (fp32, in LDS) into dst.
// One reduction for the sum and the sum of squares, both shifted by the first
// element (the shift keeps the variance free of cancellation when the mean is
// large against the spread).
__device__ __forceinline__ void w0_layernorm(const float* x, const float* g, const float* b, int K, float* dst) {
  constexpr int kPer = 16;   // elements per lane (K <= 1024)
  const int lane = threadIdx.x;
  float xv[kPer], gv[kPer], bv[kPer];
  const float x0 = x[0];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {   // clamped index: every load is issued, one wait for all
    const int j = min(lane + m * kWave, K - 1);
    xv[m] = x[j];
    gv[m] = g[j];
    bv[m] = b[j];
  }
  float s0 = 0.f, qq = 0.f;
#pragma unroll
  for (int m = 0; m < kPer; ++m)
    if (lane + m * kWave < K) {
      const float dv = xv[m] - x0;
      s0 += dv;
      qq += dv * dv;
    }
  s0 = wave_sum_dpp(s0);
  qq = wave_sum_dpp(qq);
  const float ms = s0 / K;
  const float mean = x0 + ms;
  const float rstd = 1.0f / sqrtf(fmaxf(qq / K - ms * ms, 0.f) + 1e-5f);
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int j = lane + m * kWave;
    if (j < K) dst[j] = (xv[m] - mean) * rstd * gv[m] + bv[m];
  }
}

// Wave 0: the ticket's weights other than the matrix (bias rows, LayerNorm
// gain and shift) into their LDS areas, as fp32.
template <bool BF16>
__device__ __forceinline__ void dec_stage_params(const DecGemvArgs& a, int64_t wd, int r0, int nrows, float* fl) {
  const DecLds L = dec_lds_layout(a);
  if (a.bias) w0_load_w<BF16>((const char*)a.bias + wd + (size_t)r0 * (BF16 ? 2 : 4), nrows, fl + L.eb);
  if (a.ln_g) {
    w0_load_w<BF16>((const char*)a.ln_g + wd, a.K, fl + L.lnp);
    w0_load_w<BF16>((const char*)a.ln_b + wd, a.K, fl + L.lnp + dec_pad1k(a.K));
  }
}

// Prefetch before the dependency wait (the weights do not depend on the
// ticket's inputs): the copy waves issue the first tiles of the ring; wave 0
// issues nothing (it polls the dependencies).  Returns the number of tiles issued.
__device__ __forceinline__ int dec_gemv_prefetch(const DecGemvArgs* ap, int t0, int t1, char* smem, bool allowed) {
  if (!allowed) return 0;
  const DecGemvArgs a = *const_view<DecGemvArgsC>(ap);
  // the token's weight slot (written by this launch's embedding phase: a vector load)
  const int64_t wd = a.pre_dep >= 0 ? a.st->w_delta : 0;
  const char* W = (const char*)a.W + wd;
  const int n = min(a.n_buf, t1 - t0);
  for (int i = 0; i < n; ++i) dec_tile_issue(a, W, t0 + i, smem, i);
  return n;
}

// Wave 0: nbytes (a multiple of 16, at least 16) at src (16-byte aligned)
// into LDS at dst by direct-to-LDS copies, 1 KB per instruction; the last
// block's lanes past the end re-read the last 16 bytes (nothing is read out of
// range; dst has room for whole blocks).  Completion: s_waitcnt vmcnt(0).
__device__ __forceinline__ void w0_dma(const void* src, int nbytes, void* dst) {
  const int lane = threadIdx.x;
  for (int off = 0; off < nbytes; off += 1024)
    dma16_to_lds((const char*)src + min(off + lane * 16, nbytes - 16), (char*)dst + off);
}

// Wave 0: LayerNorm of x (K <= 1024 fp32, in LDS) with gain g and shift b as
// stored (bf16 or fp32, in LDS) into dst; the arithmetic of w0_layernorm.
template <bool BF16>
__device__ __forceinline__ void w0_layernorm_lds(const float* x, const float* g, const float* b, int K, float* dst) {
  const int lane = threadIdx.x;
  float xv[16];
  const float x0 = x[0];
#pragma unroll
  for (int m = 0; m < 16; ++m) xv[m] = x[min(lane + m * kWave, K - 1)];
  float s0 = 0.f, qq = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m)
    if (lane + m * kWave < K) {
      const float dv = xv[m] - x0;
      s0 += dv;
      qq += dv * dv;
    }
  s0 = wave_sum_dpp(s0);
  qq = wave_sum_dpp(qq);
  const float ms = s0 / K;
  const float mean = x0 + ms;
  const float rstd = 1.0f / sqrtf(fmaxf(qq / K - ms * ms, 0.f) + 1e-5f);
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int j = lane + m * kWave;
    if (j < K) {
      const float gj = BF16 ? bf2f(((const uint16_t*)g)[j]) : g[j];
      const float bj = BF16 ? bf2f(((const uint16_t*)b)[j]) : b[j];
      dst[j] = (xv[m] - mean) * rstd * gj + bj;
    }
  }
}

// Tiles [t0, t1) of one GEMV; tiles [t0, t0 + npre) were issued by the prefetch.
// Every sequence's rows are dot products against the same LDS tiles, in the
// same lane order as for one sequence.
// MULTI = false: one sequence, known at compile time (the loops over sequences
// fold away and the input chunks stay in registers for the whole ticket).
template <bool MULTI, bool BF16>
__device__ __forceinline__ void dec_gemv_body(const DecGemvArgs& a, int t0, int t1, const StepCtx* scp, char* smem,
                                              int npre) {
  StepCtxC* sc = const_view<StepCtxC>(scp);
  const int head = sc->head;
  if (a.epi == DEPI_LOGITS && !(head & 1)) {   // prefill position: no logits needed
    if (npre) vm_wait_barrier(0);               // drain the prefetched copies
    return;
  }
  const int ns = MULTI ? dec_nseq(a) : 1;
  const DecLds L = dec_lds_layout(a);
  char* ring = smem;
  float* fl = (float*)(smem + (size_t)a.n_buf * kDecTile);
  float* xs = fl + L.xs;     // [ns][K]
  float* ys = fl + L.ys;     // [ns][ys_rows]
  float* ys2 = fl + L.ys2;   // [ns][ys_rows] (gated: up half)
  float* eb = fl + L.eb;     // [ys_rows] bias of the ticket's rows
  float* er = fl + L.er;     // [ns][ys_rows] residual of the ticket's rows
  float* stage = fl + L.stage;
  float* red = fl + L.red;   // [64]
  const int pos = sc->pos;
  const int64_t gen_idx = sc->gen_idx;
  const int wave = threadIdx.x / kWave;
  // with one weight slot the offset is always 0 (no dependent load)
  const int64_t wd = a.pre_dep >= 0 ? a.st->w_delta : 0;
  const char* W = (const char*)a.W + wd;
  const int nt = t1 - t0;
  for (int i = npre; i < min(a.n_buf, nt); ++i) dec_tile_issue(a, W, t0 + i, ring, i);
  int issued = min(a.n_buf, nt);
  const int r0 = t0 * a.rows_per_tile;
  const int nrows = min(nt * a.rows_per_tile, (a.epi == DEPI_GEGLU ? a.F : a.N) - r0);
  const void* bias = a.bias ? (const void*)((const char*)a.bias + wd) : nullptr;
  // One sequence with 16-byte aligned pieces: wave 0 copies every input of the
  // ticket straight into LDS (no registers held, one wait for all of them),
  // then converts the bias and normalises.
  const int es = BF16 ? 2 : 4;
  auto al16 = [](const void* p, int64_t off) { return (((uintptr_t)p + off) & 15) == 0; };
  const bool dma_in = !MULTI && (a.ln_g ? a.K <= 16 * kWave && (a.K * es) % 16 == 0 && al16(a.ln_g, wd) && al16(a.ln_b, wd)
                                        : (a.K % 4) == 0) &&
                      al16(a.attn_part ? (const void*)a.attn_part : (const void*)a.xin, 0) &&
                      (!a.attn_part || dec_stage_floats(a) % 4 == 0) &&
                      (!bias || ((nrows * es) % 16 == 0 && al16(bias, (int64_t)r0 * es))) &&
                      (a.epi != DEPI_RESID || (nrows % 4 == 0 && al16(a.resid, (int64_t)r0 * 4)));
  if (wave == 0 && dma_in) {
    if (bias) w0_dma((const char*)bias + (size_t)r0 * es, nrows * es, fl + L.braw);
    if (a.epi == DEPI_RESID) w0_dma(a.resid + r0, nrows * 4, er);
    if (a.ln_g) {
      w0_dma((const char*)a.ln_g + wd, a.K * es, fl + L.lnp);
      w0_dma((const char*)a.ln_b + wd, a.K * es, fl + L.lnp + dec_pad1k(a.K));
      w0_dma(a.xin, a.K * 4, fl + L.xraw);
    } else if (a.attn_part) {
      w0_dma(a.attn_part, dec_stage_floats(a) * 4, stage);
    } else {
      w0_dma(a.xin, a.K * 4, xs);
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // every copy of this wave has landed
    if (bias)
      for (int i = threadIdx.x; i < nrows; i += kWave)
        eb[i] = BF16 ? bf2f(((const uint16_t*)(fl + L.braw))[i]) : fl[L.braw + i];
    if (a.ln_g) w0_layernorm_lds<BF16>(fl + L.xraw, fl + L.lnp, fl + L.lnp + dec_pad1k(a.K), a.K, xs);
  } else if (wave == 0) {
    // general shapes: the same in rounds
    dec_stage_params<BF16>(a, wd, r0, nrows, fl);
    const float* lg = fl + L.lnp;
    const float* lb = lg + dec_pad1k(a.K);
    for (int q = 0; q < ns; ++q) {
      if (a.attn_part) continue;
      const float* xin = a.xin + (int64_t)q * a.xin_ss;
      if (a.ln_g) w0_layernorm(xin, lg, lb, a.K, xs + (size_t)q * a.K);
      else w0_load_f(xin, a.K, xs + (size_t)q * a.K);
    }
    if (a.epi == DEPI_RESID)
      for (int q = 0; q < ns; ++q) w0_load_f(a.resid + (int64_t)q * a.resid_ss + r0, nrows, er + (size_t)q * a.ys_rows);
  }
  if (a.attn_part) {
    // the attention output: per head, the key-range partials rescaled to their
    // common maximum, summed, and divided by the summed weights; one sequence's
    // partials at a time pass through the staging area
    const int Wd = a.dh + 2;
    const int S = a.attn_split;
    constexpr int kSplitMax = 8;
    float* scl = fl + L.scl;   // [H][S] weights of the key ranges
    for (int q = 0; q < ns; ++q) {
      if (wave == 0 && !dma_in) w0_load_f(a.attn_part + (int64_t)q * a.attn_ss, dec_stage_floats(a), stage);
      __syncthreads();
      // range c of head h weighs exp(m_c - m) / sum_c' exp(m_c' - m) l_c', m the
      // largest range maximum; an empty range (m_c = -inf) weighs 0
      for (int t = threadIdx.x; t < a.H * S; t += kThreads) {
        const int h = t / S, c = t % S;
        const float* ph = stage + h * S * Wd;
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < kSplitMax; ++k)
          if (k < S) m = fmaxf(m, ph[k * Wd + a.dh]);
        float den = 0.f;
#pragma unroll
        for (int k = 0; k < kSplitMax; ++k)
          if (k < S) {
            const float mk = ph[k * Wd + a.dh];
            if (mk != -INFINITY) den += expf(mk - m) * ph[k * Wd + a.dh + 1];
          }
        const float mc = ph[c * Wd + a.dh];
        scl[t] = mc != -INFINITY ? expf(mc - m) / den : 0.f;
      }
      __syncthreads();
      float* xq = xs + (size_t)q * a.K;
      for (int j = threadIdx.x; j < a.K; j += kThreads) {
        const int h = j / a.dh;
        const float* ph = stage + h * S * Wd + j % a.dh;
        float v = 0.f;
#pragma unroll
        for (int c = 0; c < kSplitMax; ++c)
          if (c < S) v += scl[h * S + c] * ph[c * Wd];
        xq[j] = v;
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
  }
  if constexpr (BF16) {
    dec_split_xs(xs, ns * a.K);
    __syncthreads();
  }
  {
    // one dispatch per ticket on the row shape
    const int nch = dec_row_bytes(a) / 16;
    const int cpl = (BF16 && a.rpg == 1 && nch % a.lpr == 0 && nch / a.lpr <= kDecMaxChunks) ? nch / a.lpr : 0;
    switch (cpl) {
#define OFA_TILES(C) case C: dec_tiles<MULTI, BF16, C>(a, W, ring, t0, nt, issued, xs, ys, ys2); break;
      OFA_TILES(1) OFA_TILES(2) OFA_TILES(3) OFA_TILES(4) OFA_TILES(5) OFA_TILES(6) OFA_TILES(7) OFA_TILES(8)
#undef OFA_TILES
      default: dec_tiles<MULTI, BF16, 0>(a, W, ring, t0, nt, issued, xs, ys, ys2); break;
    }
  }
  __syncthreads();
  float* const logits_out = a.epi == DEPI_LOGITS ? a.io->logits_out : nullptr;
  // epilogue over the ticket's rows, sequence by sequence
  for (int q = 0; q < ns; ++q) {
    const float* ysq = ys + (size_t)q * a.ys_rows;
    const float* ys2q = ys2 + (size_t)q * a.ys_rows;
    const float* erq = er + (size_t)q * a.ys_rows;
    float* yq = a.y + (int64_t)q * a.y_ss;
    void* kvq = a.kv ? (void*)((char*)a.kv + (size_t)q * a.kv_ss * (a.kv_dt == DT_BF16 ? 2 : 4)) : nullptr;
    for (int i = threadIdx.x; i < nrows; i += kThreads) {
      const int n = r0 + i;
      float v = ysq[i];
      if (bias) v += eb[i];
      switch (a.epi) {
        case DEPI_STORE: yq[n] = v; break;
        case DEPI_RESID: yq[n] = erq[i] + v; break;
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
            if (bias) other += eb[io];
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

// ap points at the phase's argument block in the phase table (global memory)
template <bool MULTI>
__device__ __forceinline__ void task_dec_gemv_range_t(const DecGemvArgs* ap, int t0, int t1, const StepCtx* sc,
                                                      char* smem, int npre) {
  const DecGemvArgs a = *const_view<DecGemvArgsC>(ap);
  if (a.w_dt == DT_BF16) dec_gemv_body<MULTI, true>(a, t0, t1, sc, smem, npre);
  else dec_gemv_body<MULTI, false>(a, t0, t1, sc, smem, npre);
}

__device__ __forceinline__ void task_dec_gemv(const DecGemvArgs* ap, int tile, const StepCtx* sc, char* smem) {
  if (const_view<DecGemvArgsC>(ap)->nseq > 1) task_dec_gemv_range_t<true>(ap, tile, tile + 1, sc, smem, 0);
  else task_dec_gemv_range_t<false>(ap, tile, tile + 1, sc, smem, 0);
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

// elements [e0, e0 + ept) of a cache row, as fp32 (ept 8: bf16 cache; 4 or 2: fp32)
template <int ept>
__device__ __forceinline__ void kv_chunk(const void* kv, int64_t e0, float* out) {
  if constexpr (ept == 8) {
    const uint4 u = *(const uint4*)((const uint16_t*)kv + e0);
    out[0] = bf2f(u.x & 0xffff); out[1] = bf2f(u.x >> 16); out[2] = bf2f(u.y & 0xffff); out[3] = bf2f(u.y >> 16);
    out[4] = bf2f(u.z & 0xffff); out[5] = bf2f(u.z >> 16); out[6] = bf2f(u.w & 0xffff); out[7] = bf2f(u.w >> 16);
  } else if constexpr (ept == 4) {
    const float4 u = *(const float4*)((const float*)kv + e0);
    out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
  } else {
    const float2 u = *(const float2*)((const float*)kv + e0);
    out[0] = u.x; out[1] = u.y;
  }
}

typedef const OFA_CONST_AS DecAttnArgs DecAttnArgsC;

template <int ept>
__device__ __forceinline__ void dec_attn_tile(const DecAttnArgs* ap, int tile, const StepCtx* scp, char* smem) {
  const DecAttnArgs a = *const_view<DecAttnArgsC>(ap);
  constexpr int kKMax = 64 / ept;   // chunks of a key row (head size <= 64)
  constexpr int kVPre = 4;          // value rows per thread read ahead
  const int sq = tile / (a.H * a.split);
  const int h = (tile / a.split) % a.H, c = tile % a.split;
  const int pos = const_view<StepCtxC>(scp)->pos;
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
  // indices clamped into the range, so no load sits under a lane condition and
  // the batch costs one memory round trip (an empty range reads key 0: unused)
  const float qv = qv_base[h * a.dh + min((int)threadIdx.x, a.dh - 1)];
  const int s_k = s0 + threadIdx.x;
  const int s_kc = max(min(s_k, s1 - 1), 0);
  float kr[kKMax][ept];
#pragma unroll
  for (int j = 0; j < kKMax; ++j)
    if (j < nkc) kv_chunk<ept>(kvq, kbase + (int64_t)s_kc * a.dh + j * ept, kr[j]);
  float vr[kVPre][ept];
#pragma unroll
  for (int m = 0; m < kVPre; ++m) {
    const int s = max(min(s0 + slot + m * slots, s1 - 1), 0);
    kv_chunk<ept>(kvq, vbase + (int64_t)s * a.dh + ci * ept, vr[m]);
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
      kv_chunk<ept>(kvq, kbase + (int64_t)s * a.dh + j, k);
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
    kv_chunk<ept>(kvq, vbase + (int64_t)s * a.dh + ci * ept, v);
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

// ap points at the phase's argument block in the phase table (global memory)
__device__ __forceinline__ void task_dec_attn(const DecAttnArgs* ap, int tile, const StepCtx* sc, char* smem) {
  const DecAttnArgs a = *const_view<DecAttnArgsC>(ap);
  switch (dec_attn_ept(a)) {
    case 8: dec_attn_tile<8>(ap, tile, sc, smem); break;
    case 4: dec_attn_tile<4>(ap, tile, sc, smem); break;
    default: dec_attn_tile<2>(ap, tile, sc, smem); break;
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
