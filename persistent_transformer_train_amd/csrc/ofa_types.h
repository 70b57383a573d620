// ofa_types.h -- plain structs shared by the host library and the device code:
// the phase table (one entry per task family of a program), per-step context,
// the scheduler block and the device status block.
//
// A "program" (one training step, one decode token, ...) is a list of phases.
// Phase p has n_tiles independent tiles; a tile is the unit a workgroup claims.
// Dependencies name earlier phases whose tiles must all have finished.  The
// same table drives both executors: one kernel launch per phase (stream order
// provides the dependencies) and the persistent kernel (ticket counters and
// per-phase completion counters provide them), following the scheduling the
// review "How one persistent kernel runs three jobs" describes in its section
// of the same name: tickets claim work, completions are fenced then counted,
// dependents acquire-read the count.
#pragma once
#include <stdint.h>

namespace ofa {

enum Op : int32_t {
  OP_NOP = 0,
  OP_EMBED,        // x0 = wte[tok] (+ wpe[t])
  OP_LN_FWD,       // y = LN(x), saves mean / rstd
  OP_GEMM,         // C = epilogue(A B)
  OP_ROPE,         // rotate q, k in place (rotary configs)
  OP_ATTN_FWD,     // causal attention forward, saves log-sum-exp
  OP_GEGLU_FWD,    // a = GELU(g) * up
  OP_CE,           // softmax cross-entropy: per-row loss and d logits
  OP_LOSS,         // mean of per-row losses, non-finite check
  OP_LN_BWD,       // dx_out = dx_in + LN'(dy); column partial sums
  OP_COLSUM,       // column partial sums of a [rows][cols] matrix
  OP_COLRED,       // fixed-order reduction of column partials
  OP_ATTN_PREP,    // D = rowsum(dO * O)
  OP_ATTN_BWD_KV,  // dK, dV for one key block
  OP_ATTN_BWD_Q,   // dQ for one query block
  OP_ROPE_BWD,     // inverse rotation of dq, dk in place
  OP_EMB_SORT,     // positions sorted by token (one tile); run start/count per token
  OP_EMB_BWD,      // d wte rows (fixed-order sums), d wpe rows
  OP_ADAMW,        // fused AdamW + compute-copy write
  OP_COPY,         // plain copy / cast of a flat range
  OP_DEC_EMBED,    // decode: embedding of the current token
  OP_DEC_GEMV,     // decode: y = W x (+ epilogue)
  OP_DEC_ATTN,     // decode: one head's attention over the context
  OP_DEC_ARGMAX,   // decode: argmax over the logits, emit the token
  OP_SLOT_GUARD,   // co-resident training: wait until decode no longer reads the slot AdamW writes
  OP_PUBLISH,      // co-resident training: release the step's weights as a new version
  OP_PROBE,        // evaluation: argmax and prediction entropy of the logits at chosen rows
  OP_COUNT
};

enum DType : int32_t { DT_F32 = 0, DT_BF16 = 1 };

enum Epi : int32_t {
  EPI_STORE = 0,   // C = acc (+ bias)
  EPI_RESID = 1,   // C(f32) = resid + acc (+ bias)
  EPI_GELU = 2,    // u = acc (+ bias) -> C;  GELU(u) -> aux
  EPI_DGELU = 3,   // C = acc * GELU'(aux)
  EPI_DGEGLU = 4,  // aux = [g | up] (ld ldaux, up at +aux_off); C[:, n] = acc*up*GELU'(g), C[:, n+aux_off] = acc*GELU(g)
  EPI_DSUM = 5,    // attention output gradient: C = dO = acc (bf16), and with aux = O (bf16) the
                   // attention backward's row sums dsum[b][h][t] = sum over head h's 64 columns of dO O
                   // (matrix-core tile only; N a multiple of 128, 64-wide heads)
  EPI_CE = 6,      // LM head fused with the softmax statistics (matrix-core tile, bf16 C): for each
                   // row of the 128-column tile tn, m = max over its columns of the logits z,
                   // C = exp(z - m) (bf16), stats[row * stats_ld + tn] = (m, sum of exp(z - m))
};

enum GemmImpl : int32_t { GEMM_SIMPLE = 0, GEMM_P3 = 2 };

struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  const float* bias;
  const float* resid;
  void* aux;
  int64_t lda, ldb, ldc, ldaux, ldres;
  int32_t M, N, K;
  int32_t a_kmajor;   // 1: A(m,k) = A[m*lda + k];  0: A(m,k) = A[k*lda + m]
  int32_t b_kmajor;   // 1: B(k,n) = B[n*ldb + k];  0: B(k,n) = B[k*ldb + n]
  int32_t a_dt, b_dt, c_dt, aux_dt;
  int32_t epi;
  int32_t impl;
  int32_t tiles_m, tiles_n;
  int32_t aux_off;
  int32_t bm, bn;     // tile shape (rows of C, columns of C)
  int32_t tile_order; // 0: N index fastest; 1: M index fastest; 2: bands of `group` tile rows, M index fastest
  int32_t group;      // tile rows per band (tile_order 2)
  int32_t xcd;        // one-launch-per-phase executor: give each die a contiguous run of tiles
  float* dsum;        // EPI_DSUM: [B][H][T] row sums; T and H of its indexing
  int32_t dsum_T, dsum_H;
  float* stats;       // EPI_CE: [M][stats_ld] (max, sum) pairs
  int32_t stats_ld;
};

struct LnFwdArgs {
  const float* x; const float* g; const float* b;
  void* y; float* mean; float* rstd;
  // residual combine (kp non-null): the LN input is x + ((kp[e] + kp[rows d + e])
  // + kb[col]), a product's two k-half partial sums added to the residual as
  // its epilogue would (kb nullable), and is also written to x_out
  const float* kp; const float* kb; float* x_out;
  int32_t rows, d, y_dt, rows_per_tile;
};

struct LnBwdArgs {
  const float* dy;      // gradient w.r.t. the LN output, [rows][d]
  const float* x;       // LN input
  const float* mean; const float* rstd; const float* g;
  const float* dx_in;   // running residual gradient (nullable => zero)
  float* dx_out;        // dx_in + LN backward
  void* dx_lp;          // optional low-precision copy of dx_out (nullable)
  float* partials;      // [n_tiles][3][d]: sum(dy*xhat), sum(dy), sum(dx_out)
  int32_t rows, d, rows_per_tile, lp_dt;
};

struct ColsumArgs {
  const void* src; int64_t ld;
  float* partials;      // [n_tiles][cols]
  int32_t rows, cols, rows_per_tile, dt;
};

struct ColredArgs {
  const float* partials;  // [n_parts][n_vec][cols]
  float* out[3];          // nullable entries are skipped
  int32_t n_parts, n_vec, cols, cols_per_tile;
};

struct EmbedArgs {
  const float* wte; const float* wpe;  // wpe nullable
  float* x;
  int32_t B, T, d, V, rows_per_tile;
};

struct AttnArgs {
  const void* qkv;      // [B*T][3d]: q | k | v, head h at columns h*dh
  void* o;              // [B*T][d]
  float* lse;           // [B][H][T]
  const void* dout;     // dO [B*T][d]
  float* dsum;          // D = rowsum(dO*O) [B][H][T]
  void* dqkv;           // [B*T][3d]
  int32_t B, T, H, dh, d, dt;
  int32_t block;        // query / key rows per tile
  int32_t impl;
};

struct RopeArgs {
  void* qkv;            // q at column 0, k at column d; row stride ld
  int64_t ld;
  int32_t B, T, H, dh, d, dt, rows_per_tile, pos0;
};

struct GegluArgs {
  const void* gu;       // [rows][2F]
  void* a;              // [rows][F]
  int32_t rows, F, dt, rows_per_tile;
};

struct CeArgs {
  const float* logits;  // [rows][V]
  void* dz;             // [rows][V] (dt); null: loss only (evaluation)
  float* loss_rows;     // [rows]
  int32_t rows, V, T, dt;
  float inv_rows;
  // fused with the LM head (EPI_CE): dz holds exp(z - m_t) per 128-column tile t
  // (bf16) and stats the per-tile (m_t, s_t); the target logit is recomputed as
  // h[row] . w[y] (bf16 inputs, d wide); logits is unused
  int32_t fused, n_stats, d;
  const float* stats;
  const void* h;
  const void* w;
};

struct LossArgs {
  const float* loss_rows; int32_t rows;   // per-row losses also go to StepCtx::rows_out when set
};

struct ProbeArgs {
  const float* logits;  // [rows][V]; the rows probed come from StepCtx::probe_rows
  int32_t rows, V;
};

struct EmbSortArgs {
  int32_t* sorted;      // [BT]: positions ordered by (token, position)
  uint64_t* first;      // [V]: tag << 32 | start << 16 | count
  int32_t BT, T, V;
};

struct EmbBwdArgs {
  const float* dx0;     // [BT][d]
  const int32_t* sorted; const uint64_t* first;
  float* dwte; float* dwpe;   // dwpe nullable
  int32_t B, T, d, V, n_pos, accumulate, rows_per_tile, v_tiles;
};

struct AdamArgs {
  float* p; const float* g; float* m; float* v;
  void* wc;             // compute copy (nullable): bf16 or f32
  int64_t n; int32_t per_tile, wc_dt;
  float beta1, beta2, eps, wd;
  // co-resident mode: the updated weights also go to serve slot (step tag & 1)
  void* pub; int64_t pub_slot_bytes;
};

struct DecState;
struct GuardArgs {            // wait until the decoder reads version >= tag - 1
  const DecState* st;
};

struct PublishArgs {          // published = tag (release)
  uint64_t* published;
};

struct CopyArgs {
  const void* src; void* dst; int64_t n; int32_t src_dt, dst_dt, per_tile;
};

// ---- decode ----------------------------------------------------------------
// Weights are read from a flat "serve" copy (same canonical layout as the
// master parameters, dtype w_dt).  W and bias pointers below point into slot 0;
// the kernels add DecState::w_delta bytes to reach the slot holding the
// version the current token acquired.

struct DecState {
  uint64_t version;          // weight version read by the current token (release-stored)
  int64_t w_delta;           // byte offset from slot 0 to the slot being read
  int32_t ctx_len;           // tokens in the context list
  int32_t n_gen;             // tokens emitted in this call
  int32_t prompt_len;        // co-resident decode: tokens of the saved prompt a restart reloads
  int32_t serving;           // co-resident decode running (training then guards the slot it writes)
};

enum DecEpi : int32_t {
  DEPI_STORE = 0,    // y = W x + b
  DEPI_RESID = 1,    // y = resid + W x + b
  DEPI_GELU = 2,     // y = GELU(W x + b)
  DEPI_GEGLU = 3,    // rows f and F+f: y[f] = GELU(g) * up
  DEPI_QKV = 4,      // q -> y (rotated if rope); k, v -> cache at pos (rotated k)
  DEPI_LOGITS = 5,   // y = W x; optional copy to logits_out[gen_idx]
};

struct DecIO {               // per-call output pointers of a decode call
  int32_t* tokens_out;       // [ring_len]: token g goes to g % ring_len
  uint64_t* versions_out;    // [ring_len] (nullable)
  float* logits_out;         // [n_new][V] (nullable; step mode only)
  uint64_t* n_generated;     // tokens emitted so far (nullable; may be coherent host memory)
  int64_t ring_len;
  // doorbell mode (nullable): token g starts once *doorbell > g (a coherent host
  // word the host writes); ticks[2g] / ticks[2g + 1] = device time it woke / emitted
  const uint64_t* doorbell;
  uint64_t* ticks;
  int64_t n_ticks;
};

// Decode runs nseq sequences in lock-step (equal prompt lengths, one position
// per program instance for all of them); per-sequence data sit at fixed
// strides from sequence 0's.
struct DecEmbedArgs {
  const DecIO* io;                    // doorbell mode: the wait before each token
  const void* wte; const void* wpe;   // slot-0 pointers (wpe nullable)
  int32_t* ctx_tok;                   // [nseq][cap]
  const int32_t* prompt;              // saved prompt a restart reloads (co-resident decode)
  float* x;
  DecState* st;
  const uint64_t* published;          // published version (co-resident: slot = version & 1)
  int64_t slot_bytes;                 // distance between the two slots (0 = one slot)
  int32_t d, V, w_dt;
  int32_t nseq, cap;                  // sequences; context capacity (ctx_tok / prompt stride)
};

struct DecGemvArgs {
  const void* W;             // [N][K] row-major (out x in), slot 0
  const void* bias;          // [N] (slot 0, nullable)
  const float* xin;          // [K]
  const void* ln_g; const void* ln_b;   // LayerNorm applied to xin first (nullable)
  float* y;                  // output
  const float* resid;        // DEPI_RESID
  void* kv;                  // DEPI_QKV: cache [2][H][cap][dh] of this layer
  const DecIO* io;           // DEPI_LOGITS: optional logits copy
  DecState* st;
  int32_t N, K, w_dt, kv_dt, epi, rows_per_tile, d, H, dh, cap, rope, F;
  // LDS plan: weight tiles stream through a ring of n_buf buffers of tile_bytes
  // (a multiple of 4 KB) each; ys_rows = rows of the largest ticket
  int32_t tile_bytes, n_buf, ys_rows;
  // phase whose completion for the current instance must be seen before the
  // weights may be prefetched (the token's version acquire), -1 = any time
  int32_t pre_dep;
  // DEPI_LOGITS: per-ticket (max, first index) of the logits, for the argmax
  float* part_val; int32_t* part_idx;
  int32_t lpr;               // lanes that share one row's dot product (16, 32 or 64)
  int32_t rpg;               // rows per lane group in one pass over a tile (1, 2, 4 or 8)
  int32_t per_ticket;        // tiles per ticket (the ticket of tile t is t / per_ticket)
  // input = the attention partials [H][attn_split][dh + 2] combined (nullable; xin unused then)
  const float* attn_part; int32_t attn_split;
  // sequences and the strides between their data: input / output / residual
  // vectors (floats), KV cache (elements), attention partials (floats), argmax
  // partials (entries)
  int32_t nseq;
  int64_t xin_ss, y_ss, resid_ss, kv_ss, attn_ss, part_ss;
};

struct DecAttnArgs {
  const float* q;            // [nseq][d]
  const void* kv;            // this layer's cache [2][H][cap][dh] of sequence 0 (stride kv_ss elements)
  float* part;               // [nseq][H][split][dh + 2]: unnormalised output, running max, sum of weights
  int32_t H, dh, cap, kv_dt, split, nseq;
  int64_t kv_ss, part_ss;    // tile t: sequence t / (H split), head (t / split) % H, key range t % split
};

struct DecArgmaxArgs {
  const float* part_val; const int32_t* part_idx;   // per-ticket maxima of the LM-head GEMV, [nseq][part_ss]
  int32_t n_part;
  int32_t* ctx_tok;          // [nseq][cap]
  DecState* st;
  const DecIO* io;           // tokens_out[slot][nseq], logits_out[gen][nseq][V]
  int32_t V, cap, keep, nseq;
  int64_t part_ss;
};

union PhaseArgs {
  GemmArgs gemm; LnFwdArgs lnf; LnBwdArgs lnb; ColsumArgs cs; ColredArgs cr;
  EmbedArgs emb; AttnArgs attn; RopeArgs rope; GegluArgs geglu; CeArgs ce;
  LossArgs loss; EmbSortArgs esort; EmbBwdArgs ebwd; AdamArgs adam; CopyArgs copy;
  DecEmbedArgs dembed; DecGemvArgs dgemv; DecAttnArgs dattn; DecArgmaxArgs dargmax;
  GuardArgs guard; PublishArgs publish; ProbeArgs probe;
};

constexpr int kMaxDeps = 4;

struct Phase {
  int32_t op;
  int32_t n_tiles;
  int32_t tile_base;          // first tile of this phase inside one program instance
  int32_t dep[kMaxDeps];      // phases of the same instance that must be complete
                              // (-1 = none, -2 = every earlier phase)
  int32_t dep_prev;           // phase of the previous instance that must be complete (-1 = none)
  int32_t lds_bytes;
  int32_t per_ticket;         // persistent executor: tiles claimed by one ticket
  int32_t n_tickets;          // ceil(n_tiles / per_ticket)
  int32_t ticket_base;        // first ticket of this phase inside one program instance
  int32_t pad[4];
  PhaseArgs a;
};

// per-step (per program instance) values that change between steps
struct StepCtx {
  const int32_t* tokens;   // [B][T+1]
  float* loss_out;         // where the step's loss goes
  float lr, bc1, bc2;      // learning rate, 1 - beta1^t, 1 - beta2^t
  int32_t step_in_call;
  uint64_t tag;            // strictly increasing per step across calls
  int32_t pos;             // decode: position this instance processes
  int32_t head;            // decode: bit 0 = compute logits and emit a token afterwards,
                           // bit 1 = first position of a token (acquire the newest weights),
                           // bit 2 = restart: reload the saved prompt as the context
  int32_t gen_idx;         // decode: index of the emitted token in the call
  int32_t n_probe;         // evaluation: rows probed (entries of probe_rows)
  // evaluation outputs of this instance (each nullable): per-row losses [rows],
  // and at probe_rows[i]: the argmax token (lowest id on ties) and the entropy
  // of the predicted distribution in nats
  float* rows_out;
  const int32_t* probe_rows;
  int32_t* probe_argmax;
  float* probe_entropy;
};

constexpr int kMaxPhases = 512;

constexpr int kMaxParts = 8;        // ticket partitions of a job (one per die)
constexpr int kPartStride = 16;     // uint64 words between partition counters (one 128-byte line each)

struct Sched {                       // persistent-kernel scheduler block of one job (device)
  uint64_t ticket;                   // unused (each partition has its own counter below)
  uint64_t base;                     // debug counter base (added to every counter)
  uint64_t abort;                    // non-zero: every role stops (the first job's word is shared)
  uint64_t exited;                   // workgroups that left the loop
  uint64_t stop;                     // open-ended job: raised when the other job has finished
  uint64_t limit;                    // open-ended job: instances >= limit are not run (~0 = none yet)
  uint64_t pad[2];
  uint64_t done[kMaxPhases];         // completed tiles per phase, summed over instances
  uint64_t part_ticket[kMaxParts * kPartStride];   // next ticket of partition s at [s * kPartStride]
  uint64_t part_done[kMaxPhases * kMaxParts];      // tiles of phase i done by partition s at [i * kMaxParts + s]
};

struct DevStatus {
  int32_t code;            // 0 = ok, else an ofa_status value
  int32_t phase;
  int64_t step;
  int64_t info;
  uint64_t tickets;
  uint64_t pad[4];
};

struct PhaseTime { uint64_t t0, t1; };   // first tile start, last tile end (device ticks)

}  // namespace ofa
