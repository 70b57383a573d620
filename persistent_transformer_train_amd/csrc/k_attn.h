// k_attn.h -- causal attention on the gfx950 matrix cores (bf16 operands,
// fp32 accumulation, head dim 64): forward with an online softmax that saves
// the row log-sum-exp, and the backward split the way the RTX 3090 page's
// profile splits it ("Where a step's time goes": attention-forward,
// attention-key, attention-query): a key-side pass producing dK and dV and a
// query-side pass producing dQ, both recomputing the probabilities from the
// saved log-sum-exp (no atomics, so results are deterministic).
//
// MFMA layout facts used throughout (v_mfma_f32_32x32x16_bf16, 64 lanes):
//  * operand A (M x K): lane l supplies row l%32, eight k values of its half
//    g = l/32; operand B (K x N): lane l supplies column l%32, same k slots.
//  * accumulator element r of lane l is C[row(r, l)][l%32] with
//    row(r, l) = 8*(r/4) + 4*(l/32) + r%4.
// A 32 x 32 accumulator fed back as a B operand over a 16-wide k chunk c
// holds, in slot i of half g, the k index 16c + 8*(i/4) + 4g + i%4 (the same
// formula as row()).  The partner A operand is then read with that same
// permutation ("kperm" fragments), so no register shuffle is needed.
#pragma once
#include "k_mfma.h"

namespace ofa {

// A 64-wide block row in LDS: 64 bf16 (128 bytes), its eight 16-byte chunks
// XOR-swizzled: chunk c of row r at c ^ s(r), s permuting the bits of
// (r >> 1) & 7 so that bit 0 moves to bit 2.  The LDS serves 64 banks of 4
// bytes a cycle (16 lanes of a 16-byte read, 32 lanes of an 8-byte one):
// * fragment reads, 16 consecutive rows at one chunk: rows of equal parity get
//   distinct chunk slots, the parity picks the bank half;
// * transposing reads, 4 consecutive keys x 4 aligned chunks x 2 halves: keys 2
//   apart differ in bit 2 of s, so their aligned groups of four chunk slots are
//   disjoint;
// * stash writes, two whole rows: any s.
// (A padded pitch of 72 elements measured 0.2 conflict cycles per access.)
constexpr int kAP = 64;   // LDS pitch (bf16 elements) of a 64-wide block
__device__ __forceinline__ int attn_swz(int r) {
  const int y = (r >> 1) & 7;
  return ((y & 1) << 2) | ((y >> 1) & 1) | (((y >> 2) & 1) << 1);
}
// element offset of chunk c (8 elements) of block row r
__device__ __forceinline__ int attn_off(int r, int c) { return r * kAP + ((c ^ attn_swz(r)) << 3); }

__device__ __forceinline__ int acc_row(int r, int lane) { return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3); }

// k: a multiple of 8 (one chunk)
__device__ __forceinline__ bf16x8_t frag16(const uint16_t* base, int row, int k) {
  return __builtin_bit_cast(bf16x8_t, *(const uint4*)(base + attn_off(row, k >> 3)));
}

// An A fragment over k chunk c (16 wide) with the accumulator's k permutation,
// read from an untransposed block [key][dh] (pitch kAP) with
// the transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane 4g+e receives element e of the 4-element pieces addressed by
// lanes g, g+4, g+8, g+12, so lane r addressing key k0 + r/4 at head dims
// c0 + 4(r%4) leaves lane L with keys k0..k0+3 of head dim c0 + L.  Two reads
// (keys 16c + 4g + 0..3 and 16c + 8 + 4g + 0..3) give the accumulator's k
// permutation.  dbase: first head dim of the 32-row block; kbase: 16c plus the
// block's first key.
__device__ __forceinline__ bf16x8_t frag_kperm_tr(const uint16_t* blk, int dbase, int kbase, int lane) {
  const int G = lane >> 4, r = lane & 15;
  const int col = dbase + 16 * (G & 1) + 4 * (r & 3);
  i16x4_t v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = kbase + 8 * t + 4 * (G >> 1) + (r >> 2);
    v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(blk + attn_off(key, col >> 3) + (col & 7)));
  }
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  i16x8_t w = {v[0][0], v[0][1], v[0][2], v[0][3], v[1][0], v[1][1], v[1][2], v[1][3]};
  return __builtin_bit_cast(bf16x8_t, w);
}

// eight fp32 values (accumulator elements 8c..8c+7) -> bf16 B operand
__device__ __forceinline__ bf16x8_t pack_bf16(const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f2bf2(v[2 * i], v[2 * i + 1]);
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

// A block of 64 rows x 64 head dims (bf16, row stride ld) moves to LDS in two
// steps so that the global reads of the next block overlap the current
// block's arithmetic: attn_fetch reads it into registers (two 16-byte chunks
// per thread), attn_stash writes them to LDS as [row][dh]; operands that need
// the block as [dh][row] read it back with the transposing LDS read.
struct AttnChunk { uint4 v[2]; };

__device__ __forceinline__ void attn_fetch(AttnChunk& c, const uint16_t* g, int64_t ld, int row0, int nvalid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + i * kThreads;   // 512 chunks of 8
    const int r = q >> 3, ch = (q & 7) * 8;
    c.v[i] = r < nvalid ? *(const uint4*)(g + (int64_t)(row0 + r) * ld + ch) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void attn_stash(const AttnChunk& c, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + i * kThreads;
    *(uint4*)(lds + attn_off(q >> 3, q & 7)) = c.v[i];
  }
}

// exp(x) as 2^(x log2 e) on the hardware base-2 exponential; callers fold
// log2(e) into their scale factors and offsets
constexpr float kLog2e = 1.44269504088896341f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// B-operand fragments of one wave's 32 rows (row stride ld) for the four 16-wide dh chunks
__device__ __forceinline__ void attn_row_frags(bf16x8_t f[4], const uint16_t* g, int64_t ld, int row, bool valid,
                                               int lane) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *(const uint4*)(g + (int64_t)row * ld + 16 * kk + 8 * (lane >> 5));
    f[kk] = __builtin_bit_cast(bf16x8_t, v);
  }
}

constexpr int kAttnFwdKeys = 128;   // keys (queries on the key side) per streamed block: one stash, two barriers
__host__ __device__ constexpr size_t attn_mfma_lds_bytes() { return 2 * kAttnFwdKeys * kAP * 2 + 2 * kAttnFwdKeys * 4; }

// ---------------------------------------------------------------- forward
// tile = (b, h, block of 128 queries), largest blocks first; wave w owns 32 queries.

__device__ void task_attn_fwd_mfma(const AttnArgs& a, int tile, char* smem) {
  constexpr int KB = kAttnFwdKeys;
  uint16_t* Ks = (uint16_t*)smem;        // [KB keys][dh]
  uint16_t* Vs = Ks + KB * kAP;          // [KB keys][dh]
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, g = lane >> 5;
  const int BH = a.B * a.H, nqb = (a.T + 127) / 128;
  const int qblk = nqb - 1 - tile / BH, bh = tile % BH, b = bh / a.H, h = bh % a.H;
  const int64_t ld = 3 * (int64_t)a.d;
  const uint16_t* base = (const uint16_t*)a.qkv + (int64_t)b * a.T * ld + h * a.dh;
  const int q0 = qblk * 128, qw = q0 + 32 * w, q = qw + (lane & 31);
  // scores are kept in the base-2 domain: s2 = (q.k) scale log2(e)
  const float scale2 = kLog2e / sqrtf((float)a.dh);
  bf16x8_t qf[4];
  attn_row_frags(qf, base, ld, q, q < a.T, lane);
  f32x16_t oacc[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) oacc[0][e] = oacc[1][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const int kend = min(q0 + 128, a.T);
  const int nkb = (kend + KB - 1) / KB;
  // a KB-key block in 64-row halves: attn_fetch / attn_stash move 64 rows
  AttnChunk kc[KB / 64], vc[KB / 64];
  auto fetch_block = [&](int kb) {
#pragma unroll
    for (int hh = 0; hh < KB / 64; ++hh) {
      const int r0 = kb * KB + hh * 64;
      attn_fetch(kc[hh], base + a.d, ld, r0, min(64, a.T - r0));
      attn_fetch(vc[hh], base + 2 * a.d, ld, r0, min(64, a.T - r0));
    }
  };
  fetch_block(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < KB / 64; ++hh) {
      attn_stash(kc[hh], Ks + hh * 64 * kAP);
      attn_stash(vc[hh], Vs + hh * 64 * kAP);
    }
    if (kb + 1 < nkb) fetch_block(kb + 1);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < KB / 32; ++sub) {
      const int kbase = kb * KB + sub * 32;
      if (kbase > qw + 31 || kbase >= a.T) continue;   // wave-uniform: causal / past the end
      f32x16_t s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag16(Ks, sub * 32 + (lane & 31), 16 * kk + 8 * g), qf[kk], s,
                                                    0, 0, 0);
      // s[r]: key kbase + acc_row(r), query q
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + acc_row(r, lane);
        const float v = (key <= q && key < a.T) ? s[r] * scale2 : -INFINITY;
        s[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx);
      const float alpha = (m == -INFINITY) ? 0.f : exp2_hw(m - mnew);
      float p[16], rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = (s[r] == -INFINITY) ? 0.f : exp2_hw(s[r] - mnew);
        rs += p[r];
      }
      rs += __shfl_xor(rs, 32, 64);
      lsum = lsum * alpha + rs;
      m = mnew;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        oacc[0][e] *= alpha;
        oacc[1][e] *= alpha;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t pb = pack_bf16(p + 8 * c);
#pragma unroll
        for (int db = 0; db < 2; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_kperm_tr(Vs, db * 32, sub * 32 + 16 * c, lane),
                                                             pb, oacc[db], 0, 0, 0);
      }
    }
  }
  if (q < a.T) {
    const float inv = 1.0f / lsum;
    uint16_t* o = (uint16_t*)a.o + ((int64_t)b * a.T + q) * a.d + h * a.dh;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = db * 32 + acc_row(4 * rg, lane);   // 4 consecutive head dims
        uint32_t w0 = f2bf2(oacc[db][4 * rg] * inv, oacc[db][4 * rg + 1] * inv);
        uint32_t w1 = f2bf2(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
        *(uint2*)(o + j) = make_uint2(w0, w1);
      }
    // natural-log LSE: m is in base-2 units
    if (g == 0) a.lse[((int64_t)b * a.H + h) * a.T + q] = m * 0.69314718055994531f + logf(lsum);
  }
}

// ---------------------------------------------------------------- backward, key side
// tile = (b, h, block of 128 keys), most work first; wave w owns 32 keys.
// S = Q K^T with lanes on keys: P, dP and dS come out as B operands for
// dV^T += dO^T P and dK^T += Q^T dS.

__device__ void task_attn_bwd_kv_mfma(const AttnArgs& a, int tile, char* smem) {
  constexpr int QB = kAttnFwdKeys;       // queries per streamed block
  uint16_t* Qs = (uint16_t*)smem;        // [QB q][dh]
  uint16_t* Ds = Qs + QB * kAP;          // dO [QB q][dh]
  float* lse_s = (float*)(Ds + QB * kAP);
  float* dd_s = lse_s + QB;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, g = lane >> 5;
  const int BH = a.B * a.H;
  const int kblk = tile / BH, bh = tile % BH, b = bh / a.H, h = bh % a.H;
  const int64_t ld = 3 * (int64_t)a.d;
  const uint16_t* base = (const uint16_t*)a.qkv + (int64_t)b * a.T * ld + h * a.dh;
  const uint16_t* dob = (const uint16_t*)a.dout + (int64_t)b * a.T * a.d + h * a.dh;
  const float* lse = a.lse + ((int64_t)b * a.H + h) * a.T;
  const float* dsum = a.dsum + ((int64_t)b * a.H + h) * a.T;
  const int k0 = kblk * 128, kw = k0 + 32 * w, key = kw + (lane & 31);
  const float scale = 1.0f / sqrtf((float)a.dh), scale2 = scale * kLog2e;
  bf16x8_t kf[4], vf[4];
  attn_row_frags(kf, base + a.d, ld, key, key < a.T, lane);
  attn_row_frags(vf, base + 2 * a.d, ld, key, key < a.T, lane);
  f32x16_t dk[2], dv[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) dk[0][e] = dk[1][e] = dv[0][e] = dv[1][e] = 0.f;
  const int nqb = (a.T + QB - 1) / QB;
  // query blocks stream through registers one block ahead (see attn_fetch),
  // in 64-row halves
  AttnChunk qc[QB / 64], dc[QB / 64];
  float lse_r = INFINITY, dd_r = 0.f;
  auto fetch = [&](int qb) {
    const int q0 = qb * QB;
#pragma unroll
    for (int hh = 0; hh < QB / 64; ++hh) {
      attn_fetch(qc[hh], base, ld, q0 + hh * 64, min(64, a.T - q0 - hh * 64));
      attn_fetch(dc[hh], dob, a.d, q0 + hh * 64, min(64, a.T - q0 - hh * 64));
    }
    if (threadIdx.x < QB) {
      const int qq = q0 + threadIdx.x;
      lse_r = qq < a.T ? lse[qq] * kLog2e : INFINITY;   // base-2 units
      dd_r = qq < a.T ? dsum[qq] : 0.f;
    }
  };
  if (k0 / QB < nqb) fetch(k0 / QB);
  for (int qb = k0 / QB; qb < nqb; ++qb) {
    const int q0 = qb * QB;
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < QB / 64; ++hh) {
      attn_stash(qc[hh], Qs + hh * 64 * kAP);
      attn_stash(dc[hh], Ds + hh * 64 * kAP);
    }
    if (threadIdx.x < QB) {
      lse_s[threadIdx.x] = lse_r;
      dd_s[threadIdx.x] = dd_r;
    }
    if (qb + 1 < nqb) fetch(qb + 1);
    __syncthreads();
    if (kw >= a.T) continue;
#pragma unroll
    for (int sub = 0; sub < QB / 32; ++sub) {
      const int qs0 = q0 + sub * 32;
      if (qs0 + 31 < kw || qs0 >= a.T) continue;   // every query of the chunk precedes the wave's keys
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag16(Qs, sub * 32 + (lane & 31), 16 * kk + 8 * g), kf[kk], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag16(Ds, sub * 32 + (lane & 31), 16 * kk + 8 * g), vf[kk],
                                                     dp, 0, 0, 0);
      }
      // s[r], dp[r]: query qs0 + acc_row(r), key `key`
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = sub * 32 + acc_row(r, lane);
        const int qq = q0 + ql;
        const float pv = (key <= qq && qq < a.T) ? exp2_hw(s[r] * scale2 - lse_s[ql]) : 0.f;
        p[r] = pv;
        ds[r] = pv * (dp[r] - dd_s[ql]);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t pb = pack_bf16(p + 8 * c), sb = pack_bf16(ds + 8 * c);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_kperm_tr(Ds, db * 32, sub * 32 + 16 * c, lane), pb,
                                                           dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_kperm_tr(Qs, db * 32, sub * 32 + 16 * c, lane), sb,
                                                           dk[db], 0, 0, 0);
        }
      }
    }
  }
  if (key < a.T) {
    uint16_t* out = (uint16_t*)a.dqkv + ((int64_t)b * a.T + key) * ld + h * a.dh;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = db * 32 + acc_row(4 * rg, lane);
        uint32_t k0w = f2bf2(dk[db][4 * rg] * scale, dk[db][4 * rg + 1] * scale);
        uint32_t k1w = f2bf2(dk[db][4 * rg + 2] * scale, dk[db][4 * rg + 3] * scale);
        *(uint2*)(out + a.d + j) = make_uint2(k0w, k1w);
        uint32_t v0w = f2bf2(dv[db][4 * rg], dv[db][4 * rg + 1]);
        uint32_t v1w = f2bf2(dv[db][4 * rg + 2], dv[db][4 * rg + 3]);
        *(uint2*)(out + 2 * a.d + j) = make_uint2(v0w, v1w);
      }
  }
}

// ---------------------------------------------------------------- backward, query side
// tile = (b, h, block of 128 queries), largest first; wave w owns 32 queries.
// S^T = K Q^T with lanes on queries: dS^T comes out as the B operand of dQ^T += K^T dS^T.

__device__ void task_attn_bwd_q_mfma(const AttnArgs& a, int tile, char* smem) {
  constexpr int KB = kAttnFwdKeys;       // keys per block, as in the forward
  uint16_t* Ks = (uint16_t*)smem;        // [KB keys][dh]
  uint16_t* Vs = Ks + KB * kAP;          // [KB keys][dh]
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave, g = lane >> 5;
  const int BH = a.B * a.H, nqb = (a.T + 127) / 128;
  const int qblk = nqb - 1 - tile / BH, bh = tile % BH, b = bh / a.H, h = bh % a.H;
  const int64_t ld = 3 * (int64_t)a.d;
  const uint16_t* base = (const uint16_t*)a.qkv + (int64_t)b * a.T * ld + h * a.dh;
  const uint16_t* dob = (const uint16_t*)a.dout + (int64_t)b * a.T * a.d + h * a.dh;
  const int q0 = qblk * 128, qw = q0 + 32 * w, q = qw + (lane & 31);
  const bool qv = q < a.T;
  const float scale = 1.0f / sqrtf((float)a.dh), scale2 = scale * kLog2e;
  bf16x8_t qf[4], df[4];
  attn_row_frags(qf, base, ld, q, qv, lane);
  attn_row_frags(df, dob, a.d, q, qv, lane);
  const int64_t st = ((int64_t)b * a.H + h) * a.T + (qv ? q : 0);
  const float lse_q = qv ? a.lse[st] * kLog2e : 0.f, d_q = qv ? a.dsum[st] : 0.f;
  f32x16_t dq[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) dq[0][e] = dq[1][e] = 0.f;
  const int kend = min(q0 + 128, a.T);
  const int nkb = (kend + KB - 1) / KB;
  // a KB-key block in 64-row halves: attn_fetch / attn_stash move 64 rows
  AttnChunk kc[KB / 64], vc[KB / 64];
  auto fetch_block = [&](int kb) {
#pragma unroll
    for (int hh = 0; hh < KB / 64; ++hh) {
      const int r0 = kb * KB + hh * 64;
      attn_fetch(kc[hh], base + a.d, ld, r0, min(64, a.T - r0));
      attn_fetch(vc[hh], base + 2 * a.d, ld, r0, min(64, a.T - r0));
    }
  };
  fetch_block(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < KB / 64; ++hh) {
      attn_stash(kc[hh], Ks + hh * 64 * kAP);
      attn_stash(vc[hh], Vs + hh * 64 * kAP);
    }
    if (kb + 1 < nkb) fetch_block(kb + 1);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < KB / 32; ++sub) {
      const int kbase = kb * KB + sub * 32;
      if (kbase > qw + 31 || kbase >= a.T) continue;
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = dp[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag16(Ks, sub * 32 + (lane & 31), 16 * kk + 8 * g), qf[kk], s,
                                                    0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag16(Vs, sub * 32 + (lane & 31), 16 * kk + 8 * g), df[kk],
                                                     dp, 0, 0, 0);
      }
      // s[r], dp[r]: key kbase + acc_row(r), query q
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + acc_row(r, lane);
        const float pv = (key <= q && key < a.T && qv) ? exp2_hw(s[r] * scale2 - lse_q) : 0.f;
        ds[r] = pv * (dp[r] - d_q);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t sb = pack_bf16(ds + 8 * c);
#pragma unroll
        for (int db = 0; db < 2; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_kperm_tr(Ks, db * 32, sub * 32 + 16 * c, lane), sb,
                                                           dq[db], 0, 0, 0);
      }
    }
  }
  if (qv) {
    uint16_t* out = (uint16_t*)a.dqkv + ((int64_t)b * a.T + q) * ld + h * a.dh;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = db * 32 + acc_row(4 * rg, lane);
        uint32_t w0 = f2bf2(dq[db][4 * rg] * scale, dq[db][4 * rg + 1] * scale);
        uint32_t w1 = f2bf2(dq[db][4 * rg + 2] * scale, dq[db][4 * rg + 3] * scale);
        *(uint2*)(out + j) = make_uint2(w0, w1);
      }
  }
}

}  // namespace ofa
