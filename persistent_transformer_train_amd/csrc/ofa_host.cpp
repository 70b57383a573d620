// ofa_host.cpp -- libofa.so: the C ABI declared in include/ofa.h.
//
// Host responsibilities: validate the configuration, lay out the parameters
// and carve the caller's workspace, build the phase tables ("programs") of a
// training step and of a decode position, and run them with one of the two
// executors (one launch per phase, or the persistent kernel).  The host never
// touches model data: every step of the method runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <random>
#include <thread>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/ofa.h"
#include "ofa_launch.h"
#include "ofa_types.h"

using namespace ofa;

namespace {

constexpr int kMaxSteps = 8192;        // training steps per call
constexpr int kMaxDecInst = 1 << 16;   // decode positions per call
constexpr size_t kAlign = 256;
constexpr size_t kMiscBytes = 4096;    // one Phase (offset 0) and the DecIO block (offset 2048)
constexpr size_t kMiscDecIO = 2048;
constexpr int kMaxAttnSplit = 8;        // key ranges per head in decode attention
constexpr int kThreadsHost = 256;       // threads of every workgroup
constexpr int kMaxDecSeq = 8;           // sequences one decode call decodes together
// the device copies of the two programs' phase tables and their per-partition
// ticket tables live in the workspace (the library allocates no device memory)
constexpr size_t kTableBytes = 3 * (size_t)512 * 320 + 9 * (size_t)8 * 513 * 4 + 4096;
constexpr int kMaxProbe = 64;          // rows one evaluation call may probe
constexpr int kMaxBell = 4096;         // tokens of one doorbell decode call

// ---------------------------------------------------------------- parameter layout

struct TensorDesc {
  std::string name;
  int64_t off = 0, numel = 0;
  int kind = 0;   // 0 normal, 1 zeros, 2 ones
};

struct LayerOff {
  int64_t ln1_g = -1, ln1_b = -1, w_qkv = -1, b_qkv = -1, w_o = -1, b_o = -1, ln2_g = -1, ln2_b = -1;
  int64_t w_fc = -1, b_fc = -1, w_proj = -1, b_proj = -1, w_gate = -1, w_up = -1, w_down = -1;
};

struct Layout {
  std::vector<TensorDesc> t;
  int64_t total = 0;
  int64_t wte = -1, wpe = -1, lnf_g = -1, lnf_b = -1, w_lm = -1;
  std::vector<LayerOff> layer;
};

Layout make_layout(const ofa_config& c) {
  Layout L;
  const int64_t d = c.d_model, F = c.d_ff, V = c.vocab;
  auto add = [&](const std::string& n, int64_t numel, int kind) {
    TensorDesc td;
    td.name = n;
    td.off = L.total;
    td.numel = numel;
    td.kind = kind;
    L.t.push_back(td);
    L.total += numel;
    return td.off;
  };
  L.wte = add("wte", V * d, 0);
  if (c.n_pos) L.wpe = add("wpe", (int64_t)c.n_pos * d, 0);
  for (int l = 0; l < c.n_layer; ++l) {
    std::string p = "h" + std::to_string(l) + ".";
    LayerOff o;
    o.ln1_g = add(p + "ln1.g", d, 2);
    o.ln1_b = add(p + "ln1.b", d, 1);
    o.w_qkv = add(p + "w_qkv", 3 * d * d, 0);
    if (c.has_bias) o.b_qkv = add(p + "b_qkv", 3 * d, 1);
    o.w_o = add(p + "w_o", d * d, 0);
    if (c.has_bias) o.b_o = add(p + "b_o", d, 1);
    o.ln2_g = add(p + "ln2.g", d, 2);
    o.ln2_b = add(p + "ln2.b", d, 1);
    if (c.mlp_gated) {
      o.w_gate = add(p + "w_gate", F * d, 0);
      o.w_up = add(p + "w_up", F * d, 0);
      o.w_down = add(p + "w_down", d * F, 0);
    } else {
      o.w_fc = add(p + "w_fc", F * d, 0);
      if (c.has_bias) o.b_fc = add(p + "b_fc", F, 1);
      o.w_proj = add(p + "w_proj", d * F, 0);
      if (c.has_bias) o.b_proj = add(p + "b_proj", d, 1);
    }
    L.layer.push_back(o);
  }
  L.lnf_g = add("lnf.g", d, 2);
  L.lnf_b = add("lnf.b", d, 1);
  if (!c.tied_head) L.w_lm = add("w_lm", V * d, 0);
  return L;
}

std::string validate(const ofa_config& c) {
  char buf[256];
  auto bad = [&](const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return std::string(buf);
  };
  if (c.n_layer < 1 || c.n_layer > 64) return bad("n_layer %d out of [1, 64]", c.n_layer);
  if (c.n_head < 1 || c.d_model < 1 || c.d_model % c.n_head) return bad("d_model %d not divisible by n_head %d", c.d_model, c.n_head);
  const int dh = c.d_model / c.n_head;
  if (dh > 64 || dh % 2 || 256 % dh) return bad("head dim %d unsupported (even, divides 256, <= 64)", dh);
  if (c.d_model > 1024 || c.d_model % 8) return bad("d_model %d must be a multiple of 8 and <= 1024", c.d_model);
  if (c.d_ff < 8 || c.d_ff % 8) return bad("d_ff %d must be a positive multiple of 8", c.d_ff);
  if (c.vocab < 2 || c.vocab % 8) return bad("vocab %d must be a multiple of 8 (>= 8)", c.vocab);
  if (c.n_pos < 0) return bad("n_pos < 0");
  if (c.batch < 1 || c.seq < 1) return bad("batch/seq must be >= 1");
  if (c.n_pos && c.seq > c.n_pos) return bad("seq %d exceeds the position table (%d)", c.seq, c.n_pos);
  if (c.seq > 2048) return bad("seq %d > 2048", c.seq);
  if ((int64_t)c.batch * c.seq > 4096) return bad("batch*seq %d exceeds 4096 (embedding sort)", c.batch * c.seq);
  if ((int64_t)c.batch * c.seq % 8 && c.precision == OFA_BF16)
    return bad("batch*seq must be a multiple of 8 in bf16 mode");
  if (c.precision != OFA_FP32 && c.precision != OFA_BF16) return bad("precision %d unknown", c.precision);
  if (c.precision == OFA_BF16 && dh != 64) return bad("bf16 mode needs head dim 64 (got %d)", dh);
  if (c.mlp_gated && c.has_bias) return bad("gated MLP has no biases in this model family");
  if (c.n_pos == 0 && dh % 2) return bad("rotary positions need an even head dim");
  if (!(c.lr >= 0) || !(c.beta1 >= 0 && c.beta1 < 1) || !(c.beta2 >= 0 && c.beta2 < 1) || !(c.eps > 0))
    return bad("optimizer hyper-parameters out of range");
  if (c.lr_schedule != OFA_LR_CONSTANT && c.lr_schedule != OFA_LR_COSINE) return bad("lr_schedule unknown");
  if (c.lr_schedule == OFA_LR_COSINE && c.total_steps < 1) return bad("cosine schedule needs total_steps >= 1");
  if (c.exec_mode != OFA_EXEC_PERSISTENT && c.exec_mode != OFA_EXEC_LAUNCH_PER_PHASE) return bad("exec_mode unknown");
  const int win = c.decode_window ? c.decode_window : (c.n_pos ? c.n_pos : c.seq);
  if (win < 2 || (c.n_pos && win > c.n_pos)) return bad("decode_window %d invalid", win);
  if (win > 4096) return bad("decode_window %d > 4096", win);
  const int keep = c.prompt_len ? c.prompt_len : 1;
  if (keep < 1 || keep > win) return bad("prompt_len %d invalid for window %d", keep, win);
  if (c.train_cus < 0 || c.serve_cus < 0) return bad("negative CU count");
  if (c.decode_batch < 0 || c.decode_batch > kMaxDecSeq) return bad("decode_batch %d out of [0, %d]", c.decode_batch, kMaxDecSeq);
  if (c.decode_batch > 1 && c.train_cus > 0 && c.serve_cus > 0)
    return bad("co-resident decode runs one sequence (decode_batch %d)", c.decode_batch);
  for (int r : c.reserved)
    if (r) return bad("reserved fields must be zero");
  return "";
}

// ---------------------------------------------------------------- workspace carving

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    size_t o = off;
    off += bytes;
    return o;
  }
};

// One program's device tables: the phase table, its per-partition first
// tickets split into kMaxParts partitions and unsplit (PersistJob::part_tb),
// and tiles per partition and phase (PersistJob::part_tiles).
struct DevProg {
  Phase* ph = nullptr;
  int32_t* pt8 = nullptr;
  int32_t* pt1 = nullptr;
  int32_t* tiles8 = nullptr;
};

struct Carve {
  // offsets (bytes) into the workspace
  size_t p, g, m, v, wc, serve, xres, ln_mean, ln_rstd, h, qkv, o, lse, mlp1, mlp2, logits, dz, loss_rows, ce_stats;
  size_t dxres, dxlp, dln, dmlp, dout, dsum, dqkv, ln_part, cs_fc, cs_qkv, esorted, efirst, kpart;
  size_t sched, status, times, inst_end, steps, published, trace, tables, bell_ticks;
  size_t kv, ctx_tok, dstate, dx, dq, dapart, dmlp_v, dlogits, dsteps, dtimes, misc, dsched, dpart_v, dpart_i, dprompt;
  size_t total;
  int n_slots;
  int ln_tiles, cs_tiles;
};

struct Dims {
  int64_t B, T, BT, d, H, dh, F, V, L, P, win, keep, mlp1_cols, nseq;
  int lp_dt;
  size_t lp;   // bytes per low-precision element
};

Dims dims_of(const ofa_config& c, const Layout& lay) {
  Dims D;
  D.B = c.batch;
  D.T = c.seq;
  D.BT = D.B * D.T;
  D.d = c.d_model;
  D.H = c.n_head;
  D.dh = D.d / D.H;
  D.F = c.d_ff;
  D.V = c.vocab;
  D.L = c.n_layer;
  D.P = lay.total;
  D.win = c.decode_window ? c.decode_window : (c.n_pos ? c.n_pos : c.seq);
  D.keep = c.prompt_len ? c.prompt_len : 1;
  D.mlp1_cols = c.mlp_gated ? 2 * D.F : D.F;
  D.nseq = c.decode_batch > 1 ? c.decode_batch : 1;
  D.lp_dt = c.precision == OFA_BF16 ? DT_BF16 : DT_F32;
  D.lp = c.precision == OFA_BF16 ? 2 : 4;
  return D;
}

constexpr int kLnRows = 16;     // rows per LayerNorm tile
constexpr int kCsRows = 64;     // rows per column-sum tile

Carve carve(const ofa_config& c, const Layout& lay) {
  Dims D = dims_of(c, lay);
  Carve w;
  Bump b;
  const size_t f4 = 4, lp = D.lp;
  const bool bf = c.precision == OFA_BF16;
  const int64_t R = 2 * D.L + 1;   // residual points
  w.n_slots = (c.train_cus > 0 && c.serve_cus > 0) ? 2 : 1;
  w.ln_tiles = (int)((D.BT + kLnRows - 1) / kLnRows);
  w.cs_tiles = (int)((D.BT + kCsRows - 1) / kCsRows);
  w.p = b.take(D.P * f4);
  w.g = b.take(D.P * f4);
  w.m = b.take(D.P * f4);
  w.v = b.take(D.P * f4);
  w.wc = bf ? b.take(D.P * lp) : w.p;
  w.serve = b.take(D.P * lp * w.n_slots);
  w.xres = b.take(R * D.BT * D.d * f4);
  w.ln_mean = b.take(R * D.BT * f4);
  w.ln_rstd = b.take(R * D.BT * f4);
  w.h = b.take(R * D.BT * D.d * lp);
  w.qkv = b.take(D.L * D.BT * 3 * D.d * lp);
  w.o = b.take(D.L * D.BT * D.d * lp);
  w.lse = b.take(D.L * D.B * D.H * D.T * f4);
  w.mlp1 = b.take(D.L * D.BT * D.mlp1_cols * lp);
  w.mlp2 = b.take(D.L * D.BT * D.F * lp);
  w.logits = b.take(D.BT * D.V * f4);
  w.dz = b.take(D.BT * D.V * lp);
  w.loss_rows = b.take(D.BT * f4);
  w.ce_stats = b.take(D.BT * ((D.V + 127) / 128) * 2 * f4);   // per row and 128-column tile: (max, sum)
  w.dxres = b.take(R * D.BT * D.d * f4);
  w.dxlp = bf ? b.take(R * D.BT * D.d * lp) : w.dxres;
  w.dln = b.take(R * D.BT * D.d * f4);
  w.dmlp = b.take(D.L * D.BT * D.mlp1_cols * lp);
  w.dout = b.take(D.L * D.BT * D.d * lp);
  w.dsum = b.take(D.L * D.B * D.H * D.T * f4);
  w.dqkv = b.take(D.L * D.BT * 3 * D.d * lp);
  w.ln_part = b.take(R * w.ln_tiles * 3 * D.d * f4);
  w.cs_fc = b.take(D.L * w.cs_tiles * D.F * f4);
  w.cs_qkv = b.take(D.L * w.cs_tiles * 3 * D.d * f4);
  w.esorted = b.take(D.BT * 4);
  w.kpart = b.take(2 * D.BT * D.d * f4);   // two k-half partial sums of a residual product
  w.efirst = b.take(D.V * 8);
  w.sched = b.take(sizeof(Sched));
  w.status = b.take(sizeof(DevStatus));
  w.times = b.take(kMaxPhases * sizeof(PhaseTime));
  w.dtimes = b.take(kMaxPhases * sizeof(PhaseTime));
  w.inst_end = b.take(kMaxSteps * 8);
  w.steps = b.take(kMaxSteps * sizeof(StepCtx));
  w.published = b.take(64);
  // decode: per sequence s of nseq, [s][...] blocks (vectors: [point][s][d])
  w.kv = b.take(D.nseq * D.L * 2 * D.H * D.win * D.dh * lp);
  w.ctx_tok = b.take(D.nseq * D.win * 4);
  w.dstate = b.take(sizeof(DecState));
  w.dx = b.take(R * D.nseq * D.d * f4);
  w.dq = b.take(D.nseq * D.d * f4);
  w.dapart = b.take(D.L * D.nseq * D.H * kMaxAttnSplit * (D.dh + 2) * f4);
  w.dmlp_v = b.take(D.L * D.nseq * D.F * f4);
  w.dlogits = b.take(D.nseq * D.V * f4);
  w.dsteps = b.take((size_t)kMaxDecInst * sizeof(StepCtx));
  w.dsched = b.take(sizeof(Sched));
  w.dprompt = b.take(D.nseq * D.win * 4);
  w.dpart_v = b.take(D.nseq * D.V * f4);
  w.dpart_i = b.take(D.nseq * D.V * 4);
  w.misc = b.take(kMiscBytes);
  w.bell_ticks = b.take((size_t)kMaxBell * 16);
  w.tables = b.take(kTableBytes);
  w.trace = (c.debug_flags & OFA_DEBUG_TRACE) ? b.take((size_t)OFA_TRACE_INSTANCES * kMaxPhases * 32) : 0;
  w.total = (b.off + kAlign - 1) / kAlign * kAlign;
  return w;
}

template <typename T>
T* at(char* ws, size_t off) { return (T*)(ws + off); }

}  // namespace

// ---------------------------------------------------------------- the handle

struct ofa_handle {
  ofa_config cfg{};
  Layout lay;
  Dims D{};
  Carve cw{};
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  int n_cu = 0;
  int serve_wgs = 0;               // workgroups that run decode (one per serve CU)
  int train_occ = 1;               // workgroups per CU of step-mode persistent training (1 or 2)
  std::vector<Phase> train;        // one training step
  std::vector<Phase> dec;          // one decode position (with head)
  std::vector<Phase> eval;         // forward, loss and probe of one evaluated batch
  // device copies of the three programs (in the workspace) and their ticket tables
  DevProg dp_train, dp_dec, dp_eval;
  Phase* d_train = nullptr;
  Phase* d_dec = nullptr;
  uint8_t lineage[32] = {};        // SHA-256 of the checkpoint this state last came from or went to
  uint64_t* h_bell = nullptr;      // coherent pinned host words: doorbell at [0], progress at [8]
  std::vector<char> phase_names;   // for phase_times
  std::vector<std::string> train_names;
  std::vector<std::string> dec_names;
  StepCtx* h_steps = nullptr;      // pinned staging
  StepCtx* h_dsteps = nullptr;
  char* h_misc = nullptr;          // pinned staging for the misc block
  hipEvent_t ev_upload = nullptr, ev_t0 = nullptr, ev_t1 = nullptr;
  bool upload_pending = false;
  bool timed = false;              // ev_t0 / ev_t1 bracket a recorded call
  uint64_t steps_done = 0;
  uint64_t version = 0;
  int sticky = 0;
  int last_grid = 0;
  bool plan_ok = true;             // every decode GEMV found an LDS plan
  int trace_n_phases = 0;          // program length of the last traced launch (0 = none)
  int64_t trace_n_inst = 0;
  bool trace_dec = false;          // the last traced launch was a decode call
  uint64_t last_tickets = 0;
  double last_ms = 0;
  std::string err;
  int hip_err = 0;
  // decode host mirror of the context rule
  int64_t dec_ctx_len = 0, dec_processed = 0;
  bool dec_started = false;
  bool die_map = false;            // workgroup b of a launch runs on die b % 8 (probed at create)
  bool unpublished = false;        // compute weights set by ofa_set_params since the last publication
  bool host_model = false;         // built by ofa_sched_selftest: programs only, no device (the
                                   // matrix-core tiles are assumed available)
  bool is_static = false;          // made by ofa_create_static: workspace = the device's static array,
                                   // staging in static host arrays, no events
};

namespace {

ofa_status fail(ofa_handle* h, ofa_status s, const char* fmt, ...) {
  if (h) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    h->err = buf;
  }
  return s;
}

#define HIP_TRY(h, expr)                                                                   \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess) {                                                                \
      (void)hipGetLastError();                                                             \
      (h)->hip_err = (int)_e;                                                              \
      return fail((h), OFA_E_HIP, "%s failed: %s", #expr, hipGetErrorString(_e));          \
    }                                                                                      \
  } while (0)

// ---------------------------------------------------------------- program builders

struct Builder {
  std::vector<Phase>* out;
  std::vector<std::string>* names;
  int add(Op op, int n_tiles, const char* name, std::initializer_list<int> deps = {}) {
    Phase p;
    memset(&p, 0, sizeof p);
    p.op = op;
    p.n_tiles = n_tiles;
    for (int i = 0; i < kMaxDeps; ++i) p.dep[i] = -1;
    int i = 0;
    for (int d : deps)
      if (i < kMaxDeps) p.dep[i++] = d;
    p.dep_prev = -1;
    out->push_back(p);
    if (names) names->push_back(name);
    return (int)out->size() - 1;
  }
  Phase& operator[](int i) { return (*out)[i]; }
};

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

GemmArgs gemm(const ofa_handle* h, int M, int N, int K, const void* A, int64_t lda, int a_km, int a_dt,
              const void* B, int64_t ldb, int b_km, int b_dt, void* C, int64_t ldc, int c_dt, int epi) {
  GemmArgs g;
  memset(&g, 0, sizeof g);
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.a_kmajor = a_km;
  g.a_dt = a_dt;
  g.B = B;
  g.ldb = ldb;
  g.b_kmajor = b_km;
  g.b_dt = b_dt;
  g.C = C;
  g.ldc = ldc;
  g.c_dt = c_dt;
  g.epi = epi;
  // bf16 operands take the matrix-core tile; its shape limits (K, and the
  // contiguous dimension of a row-contiguous operand, multiples of 8) hold for
  // every bf16 configuration the validator accepts
  const bool mfma = h->cfg.precision == OFA_BF16 && a_dt == DT_BF16 && b_dt == DT_BF16 &&
                    (h->host_model || gemm_p3_available()) &&
                    K % 8 == 0 && (a_km || M % 8 == 0) && N % 8 == 0 && ldc % 8 == 0 && M >= 8 && N >= 8;
  g.impl = mfma ? GEMM_P3 : GEMM_SIMPLE;
  // 256-row tiles move fewer bytes per MFMA; they pay off where even they make
  // several waves of tiles over the whole GPU (the LM-head products)
  // (only with one workgroup per CU: two per CU leave each half the LDS)
  const bool big = h->train_occ == 1 &&
                   ((int64_t)cdiv(M, 256) * cdiv(N, 128) >= 1024 || (h->cfg.debug_flags & OFA_DEBUG_TILE256));
  g.bm = mfma ? (big ? 256 : 128) : 64;
  g.bn = mfma ? 128 : 64;
  g.tiles_m = cdiv(M, g.bm);
  g.tiles_n = cdiv(N, g.bn);
  if (h->cfg.debug_flags & OFA_DEBUG_PLAIN_TILES) {
    // walk the smaller operand fastest so the larger one is streamed about once
    g.tile_order = (int64_t)N > (int64_t)M ? 1 : 0;
  } else {
    // bands of eight tile rows: a die's run of tiles (or a window of tickets)
    // covers a compact block of C, whose operand panels its L2 can hold
    g.tile_order = 2;
    g.group = 8;
    g.xcd = 1;
  }
  return g;
}

// tile and ticket prefix sums; a ticket groups tiles so that a large phase
// hands out at most ~256 tickets, about one per workgroup of a whole-GPU launch
// (each ticket costs an atomic and a counter update, and a release fence per
// ticket or, with die partitions, per die and phase)
constexpr int kTicketsPerPhase = 256;

void finish_program(std::vector<Phase>& prog, int max_tickets = kTicketsPerPhase) {
  int tiles = 0, tickets = 0;
  for (auto& ph : prog) {
    ph.tile_base = tiles;
    tiles += ph.n_tiles;
    if (ph.per_ticket <= 0) ph.per_ticket = std::max(1, cdiv(ph.n_tiles, max_tickets));
    ph.n_tickets = cdiv(ph.n_tiles, ph.per_ticket);
    ph.ticket_base = tickets;
    tickets += ph.n_tickets;
    ph.lds_bytes = (int)phase_lds_bytes(ph);
  }
}

// tiles of each phase owned by each of P partitions (PersistJob::part_tiles)
std::vector<int32_t> part_tile_table(const std::vector<Phase>& prog, int P) {
  const size_t n = prog.size();
  std::vector<int32_t> t((size_t)P * n, 0);
  for (size_t i = 0; i < n; ++i)
    for (int j = 0; j < prog[i].n_tickets; ++j)
      t[(j % P) * n + i] += std::min(prog[i].per_ticket, prog[i].n_tiles - j * prog[i].per_ticket);
  return t;
}

// per-partition first tickets of each phase (PersistJob::part_tb): partition
// s of P owns a phase's tickets s, s + P, ...
std::vector<int32_t> part_table(const std::vector<Phase>& prog, int P) {
  const size_t n = prog.size();
  std::vector<int32_t> t((size_t)P * (n + 1));
  for (int s = 0; s < P; ++s) {
    int32_t acc = 0;
    for (size_t i = 0; i < n; ++i) {
      t[s * (n + 1) + i] = acc;
      const int T = prog[i].n_tickets;
      acc += T > s ? (T - s + P - 1) / P : 0;
    }
    t[s * (n + 1) + n] = acc;
  }
  return t;
}

void build_train(ofa_handle* h) {
  const ofa_config& c = h->cfg;
  const Dims& D = h->D;
  const Carve& w = h->cw;
  char* ws = h->ws;
  h->train.clear();
  h->train_names.clear();
  Builder b{&h->train, &h->train_names};
  const int lp = D.lp_dt;
  const int64_t BT = D.BT, d = D.d, F = D.F, V = D.V, L = D.L;
  float* P = at<float>(ws, w.p);
  float* G = at<float>(ws, w.g);
  char* WC = ws + w.wc;   // compute weights (lp)
  auto wc = [&](int64_t off) -> const void* { return WC + off * D.lp; };
  auto pf = [&](int64_t off) -> float* { return off < 0 ? nullptr : P + off; };
  auto gf = [&](int64_t off) -> float* { return off < 0 ? nullptr : G + off; };
  float* xres = at<float>(ws, w.xres);
  auto X = [&](int i) { return xres + (int64_t)i * BT * d; };
  auto Hh = [&](int i) -> void* { return ws + w.h + (size_t)i * BT * d * D.lp; };
  auto MEAN = [&](int i) { return at<float>(ws, w.ln_mean) + (int64_t)i * BT; };
  auto RSTD = [&](int i) { return at<float>(ws, w.ln_rstd) + (int64_t)i * BT; };
  auto QKV = [&](int l) -> void* { return ws + w.qkv + (size_t)l * BT * 3 * d * D.lp; };
  auto O = [&](int l) -> void* { return ws + w.o + (size_t)l * BT * d * D.lp; };
  auto LSE = [&](int l) { return at<float>(ws, w.lse) + (int64_t)l * D.B * D.H * D.T; };
  auto M1 = [&](int l) -> void* { return ws + w.mlp1 + (size_t)l * BT * D.mlp1_cols * D.lp; };
  auto M2 = [&](int l) -> void* { return ws + w.mlp2 + (size_t)l * BT * F * D.lp; };
  auto DX = [&](int i) { return at<float>(ws, w.dxres) + (int64_t)i * BT * d; };
  auto DXLP = [&](int i) -> void* { return ws + w.dxlp + (size_t)i * BT * d * D.lp; };
  auto DLN = [&](int i) { return at<float>(ws, w.dln) + (int64_t)i * BT * d; };
  auto DM = [&](int l) -> void* { return ws + w.dmlp + (size_t)l * BT * D.mlp1_cols * D.lp; };
  auto DOUT = [&](int l) -> void* { return ws + w.dout + (size_t)l * BT * d * D.lp; };
  auto DSUM = [&](int l) { return at<float>(ws, w.dsum) + (int64_t)l * D.B * D.H * D.T; };
  auto DQKV = [&](int l) -> void* { return ws + w.dqkv + (size_t)l * BT * 3 * d * D.lp; };
  auto LNP = [&](int i) { return at<float>(ws, w.ln_part) + (int64_t)i * w.ln_tiles * 3 * d; };
  auto CSF = [&](int l) { return at<float>(ws, w.cs_fc) + (int64_t)l * w.cs_tiles * F; };
  auto CSQ = [&](int l) { return at<float>(ws, w.cs_qkv) + (int64_t)l * w.cs_tiles * 3 * d; };
  const int lnt = w.ln_tiles;
  // bf16 with 64-wide heads runs the MFMA attention (128 rows per tile), else the plain one
  const int attn_impl = (c.precision == OFA_BF16 && D.dh == 64) ? 1 : 0;
  const int attn_block = attn_impl ? 128 : 16;
  const int attn_tiles = (int)(D.B * D.H * cdiv(D.T, attn_block));

  auto ln_fwd = [&](int i, int dep, const char* nm) {
    int p = b.add(OP_LN_FWD, lnt, nm, {dep});
    LnFwdArgs& a = b[p].a.lnf;
    a.x = X(i);
    a.g = nullptr;
    a.y = Hh(i);
    a.mean = MEAN(i);
    a.rstd = RSTD(i);
    a.rows = (int)BT;
    a.d = (int)d;
    a.y_dt = lp;
    a.rows_per_tile = kLnRows;
    return p;
  };
  auto set_ln_params = [&](int p, int64_t g_off, int64_t b_off) {
    b[p].a.lnf.g = pf(g_off);
    b[p].a.lnf.b = pf(b_off);
  };
  auto gemm_phase = [&](GemmArgs g, std::initializer_list<int> deps, const char* nm) {
    // the matrix-core epilogue accesses four columns at a time
    if (g.impl == GEMM_P3 && (g.ldaux % 8 || g.ldres % 8 || g.aux_off % 8)) {
      g.impl = GEMM_SIMPLE;
      g.bm = g.bn = 64;
      g.tiles_m = cdiv(g.M, 64);
      g.tiles_n = cdiv(g.N, 64);
    }
    int p = b.add(OP_GEMM, g.tiles_m * g.tiles_n, nm, deps);
    b[p].a.gemm = g;
    return p;
  };
  // A residual product with no more tiles than the device has CUs and a long k
  // (the MLP's second product) runs as two phases over the two k halves, each
  // writing fp32 partial sums; the LayerNorm that reads its output adds them to
  // the residual (and the bias) as the product's epilogue would, and writes the
  // sum.  Twice the tiles, each half as long.  Matrix-core bf16 path only, with
  // 16-byte aligned halves.  The test does not depend on the workgroups per CU,
  // so every occupancy runs the same program (and gets the same bits).
  float* KP = at<float>(ws, w.kpart);
  struct Pending { const float* resid; const float* bias; int p0, p1; } pend_comb{nullptr, nullptr, -1, -1};
  auto split_resid = [&](const GemmArgs& g, std::initializer_list<int> deps, const char* nm) -> bool {
    const int hk = g.K / 2;
    if (g.impl != GEMM_P3 || g.a_dt != DT_BF16 || g.b_dt != DT_BF16 || g.a_kmajor != 1 || g.b_kmajor != 1 ||
        g.K % 16 || hk < 256 || g.epi != EPI_RESID || g.tiles_m * g.tiles_n > h->n_cu)
      return false;
    GemmArgs g0 = gemm(h, g.M, g.N, hk, g.A, g.lda, 1, DT_BF16, g.B, g.ldb, 1, DT_BF16, KP, g.N, DT_F32, EPI_STORE);
    GemmArgs g1 = gemm(h, g.M, g.N, hk, (const char*)g.A + 2 * (int64_t)hk, g.lda, 1, DT_BF16,
                       (const char*)g.B + 2 * (int64_t)hk, g.ldb, 1, DT_BF16, KP + (int64_t)g.M * g.N, g.N, DT_F32,
                       EPI_STORE);
    const int p0 = gemm_phase(g0, deps, nm);
    const int p1 = gemm_phase(g1, deps, "k_half");
    pend_comb = {g.resid, g.bias, p0, p1};
    return true;
  };
  // the LayerNorm at residual point i takes a pending split product's sum
  auto take_comb = [&](int p, int i) {
    if (pend_comb.p0 < 0) return;
    LnFwdArgs& a = b[p].a.lnf;
    a.x = pend_comb.resid;
    a.kp = KP;
    a.kb = pend_comb.bias;
    a.x_out = X(i);
    b[p].dep[0] = pend_comb.p0;
    b[p].dep[1] = pend_comb.p1;
    pend_comb = {nullptr, nullptr, -1, -1};
  };
  auto attn_args = [&](int l) {
    AttnArgs a;
    memset(&a, 0, sizeof a);
    a.qkv = QKV(l);
    a.o = O(l);
    a.lse = LSE(l);
    a.dout = DOUT(l);
    a.dsum = DSUM(l);
    a.dqkv = DQKV(l);
    a.B = (int)D.B;
    a.T = (int)D.T;
    a.H = (int)D.H;
    a.dh = (int)D.dh;
    a.d = (int)d;
    a.dt = lp;
    a.block = attn_block;
    a.impl = attn_impl;
    return a;
  };
  auto rope_args = [&](void* buf) {
    RopeArgs r;
    memset(&r, 0, sizeof r);
    r.qkv = buf;
    r.ld = 3 * d;
    r.B = (int)D.B;
    r.T = (int)D.T;
    r.H = (int)D.H;
    r.dh = (int)D.dh;
    r.d = (int)d;
    r.dt = lp;
    r.rows_per_tile = 16;
    r.pos0 = 0;
    return r;
  };

  // ---- forward
  int p_emb = b.add(OP_EMBED, cdiv(BT, 16), "embed");
  {
    EmbedArgs& a = b[p_emb].a.emb;
    a.wte = pf(h->lay.wte);
    a.wpe = pf(h->lay.wpe);
    a.x = X(0);
    a.B = (int)D.B;
    a.T = (int)D.T;
    a.d = (int)d;
    a.V = (int)V;
    a.rows_per_tile = 16;
  }
  int p_sort = b.add(OP_EMB_SORT, 1, "emb_sort");
  {
    EmbSortArgs& a = b[p_sort].a.esort;
    a.sorted = at<int32_t>(ws, w.esorted);
    a.first = at<uint64_t>(ws, w.efirst);
    a.BT = (int)BT;
    a.T = (int)D.T;
    a.V = (int)V;
  }
  int last_x = p_emb;
  for (int l = 0; l < L; ++l) {
    const LayerOff& lo = h->lay.layer[l];
    int p_ln1 = ln_fwd(2 * l, last_x, "ln1");
    set_ln_params(p_ln1, lo.ln1_g, lo.ln1_b);
    if (pend_comb.p0 >= 0) {
      take_comb(p_ln1, 2 * l);
      last_x = p_ln1;   // the residual X(2l) is now written here
    }
    GemmArgs g = gemm(h, (int)BT, (int)(3 * d), (int)d, Hh(2 * l), d, 1, lp, wc(lo.w_qkv), d, 1, lp, QKV(l), 3 * d, lp,
                      EPI_STORE);
    g.bias = pf(lo.b_qkv);
    int p_qkv = gemm_phase(g, {p_ln1}, "qkv");
    int p_pre_attn = p_qkv;
    if (c.n_pos == 0) {
      int p = b.add(OP_ROPE, cdiv(BT, 16), "rope", {p_qkv});
      b[p].a.rope = rope_args(QKV(l));
      p_pre_attn = p;
    }
    int p_att = b.add(OP_ATTN_FWD, attn_tiles, "attn_fwd", {p_pre_attn});
    b[p_att].per_ticket = 1;   // causal tiles differ in work: one per ticket, largest first
    b[p_att].a.attn = attn_args(l);
    g = gemm(h, (int)BT, (int)d, (int)d, O(l), d, 1, lp, wc(lo.w_o), d, 1, lp, X(2 * l + 1), d, DT_F32, EPI_RESID);
    g.bias = pf(lo.b_o);
    g.resid = X(2 * l);
    g.ldres = d;
    int p_o = gemm_phase(g, {p_att, last_x}, "attn_out");
    int p_ln2 = ln_fwd(2 * l + 1, p_o, "ln2");
    set_ln_params(p_ln2, lo.ln2_g, lo.ln2_b);
    int p_down;
    if (c.mlp_gated) {
      g = gemm(h, (int)BT, (int)(2 * F), (int)d, Hh(2 * l + 1), d, 1, lp, wc(lo.w_gate), d, 1, lp, M1(l), 2 * F, lp,
               EPI_STORE);
      int p_gu = gemm_phase(g, {p_ln2}, "gate_up");
      int p_gg = b.add(OP_GEGLU_FWD, cdiv(BT, 16), "geglu", {p_gu});
      GegluArgs& ga = b[p_gg].a.geglu;
      ga.gu = M1(l);
      ga.a = M2(l);
      ga.rows = (int)BT;
      ga.F = (int)F;
      ga.dt = lp;
      ga.rows_per_tile = 16;
      g = gemm(h, (int)BT, (int)d, (int)F, M2(l), F, 1, lp, wc(lo.w_down), F, 1, lp, X(2 * l + 2), d, DT_F32,
               EPI_RESID);
      g.resid = X(2 * l + 1);
      g.ldres = d;
      p_down = split_resid(g, {p_gg, p_o}, "down") ? -1 : gemm_phase(g, {p_gg, p_o}, "down");
    } else {
      g = gemm(h, (int)BT, (int)F, (int)d, Hh(2 * l + 1), d, 1, lp, wc(lo.w_fc), d, 1, lp, M1(l), F, lp, EPI_GELU);
      g.bias = pf(lo.b_fc);
      g.aux = M2(l);
      g.ldaux = F;
      g.aux_dt = lp;
      int p_fc = gemm_phase(g, {p_ln2}, "fc");
      g = gemm(h, (int)BT, (int)d, (int)F, M2(l), F, 1, lp, wc(lo.w_proj), F, 1, lp, X(2 * l + 2), d, DT_F32,
               EPI_RESID);
      g.bias = pf(lo.b_proj);
      g.resid = X(2 * l + 1);
      g.ldres = d;
      p_down = split_resid(g, {p_fc, p_o}, "proj") ? -1 : gemm_phase(g, {p_fc, p_o}, "proj");
    }
    last_x = p_down;
  }
  int p_lnf = ln_fwd(2 * (int)L, last_x, "lnf");
  set_ln_params(p_lnf, h->lay.lnf_g, h->lay.lnf_b);
  take_comb(p_lnf, 2 * (int)L);
  const int64_t w_lm = c.tied_head ? h->lay.wte : h->lay.w_lm;
  GemmArgs g = gemm(h, (int)BT, (int)V, (int)d, Hh(2 * L), d, 1, lp, wc(w_lm), d, 1, lp, at<float>(ws, w.logits), V,
                    DT_F32, EPI_STORE);
  // bf16 with the matrix-core tile: the LM head is fused with the softmax
  // statistics (EPI_CE) and no fp32 logits are written; the cross-entropy then
  // combines the per-tile statistics and turns exp(z - m_t) into dz in place
  const bool fused_ce = g.impl == GEMM_P3 && lp == DT_BF16 && g.bn == 128 && !(c.debug_flags & OFA_DEBUG_CE_UNFUSED);
  if (fused_ce) {
    g.C = ws + w.dz;
    g.c_dt = lp;
    g.epi = EPI_CE;
    g.stats = at<float>(ws, w.ce_stats);
    g.stats_ld = g.tiles_n;
  }
  int p_head = gemm_phase(g, {p_lnf}, "lm_head");
  int p_ce = b.add(OP_CE, (int)BT, "cross_entropy", {p_head});
  {
    CeArgs& a = b[p_ce].a.ce;
    a.logits = at<float>(ws, w.logits);
    a.dz = ws + w.dz;
    a.loss_rows = at<float>(ws, w.loss_rows);
    a.rows = (int)BT;
    a.V = (int)V;
    a.T = (int)D.T;
    a.dt = lp;
    a.inv_rows = 1.0f / (float)BT;
    if (fused_ce && b[p_head].a.gemm.epi == EPI_CE) {
      a.fused = 1;
      a.n_stats = g.tiles_n;
      a.d = (int)d;
      a.stats = at<float>(ws, w.ce_stats);
      a.h = Hh(2 * L);
      a.w = wc(w_lm);
    }
  }
  int p_loss = b.add(OP_LOSS, 1, "loss", {p_ce});
  b[p_loss].a.loss.loss_rows = at<float>(ws, w.loss_rows);
  b[p_loss].a.loss.rows = (int)BT;

  // ---- backward
  void* dz = ws + w.dz;
  g = gemm(h, (int)BT, (int)d, (int)V, dz, V, 1, lp, wc(w_lm), d, 0, lp, DLN(2 * L), d, DT_F32, EPI_STORE);
  int p_head_dx = gemm_phase(g, {p_ce}, "lm_head_dx");
  g = gemm(h, (int)V, (int)d, (int)BT, dz, V, 0, lp, Hh(2 * L), d, 0, lp, gf(w_lm), d, DT_F32, EPI_STORE);
  int p_head_dw = gemm_phase(g, {p_ce}, "lm_head_dw");
  auto ln_bwd = [&](int i, int64_t g_off, int dx_in_idx, std::initializer_list<int> deps, const char* nm) {
    int p = b.add(OP_LN_BWD, lnt, nm, deps);
    LnBwdArgs& a = b[p].a.lnb;
    a.dy = DLN(i);
    a.x = X(i);
    a.mean = MEAN(i);
    a.rstd = RSTD(i);
    a.g = pf(g_off);
    a.dx_in = dx_in_idx >= 0 ? DX(dx_in_idx) : nullptr;
    a.dx_out = DX(i);
    a.dx_lp = c.precision == OFA_BF16 ? DXLP(i) : nullptr;
    a.lp_dt = lp;
    a.partials = LNP(i);
    a.rows = (int)BT;
    a.d = (int)d;
    a.rows_per_tile = kLnRows;
    return p;
  };
  auto ln_red = [&](int i, int dep, float* og, float* ob, float* ores, const char* nm) {
    int p = b.add(OP_COLRED, 3 * cdiv(d, 16), nm, {dep});
    ColredArgs& a = b[p].a.cr;
    a.partials = LNP(i);
    a.out[0] = og;
    a.out[1] = ob;
    a.out[2] = ores;
    a.n_parts = lnt;
    a.n_vec = 3;
    a.cols = (int)d;
    a.cols_per_tile = 16;
    return p;
  };
  auto colsum = [&](const void* src, int64_t ld, int cols, float* part, float* out, int dep, int dep2,
                    const char* nm) {
    int p = b.add(OP_COLSUM, w.cs_tiles * cdiv(cols, 512), nm, {dep, dep2});
    ColsumArgs& a = b[p].a.cs;
    a.src = src;
    a.ld = ld;
    a.partials = part;
    a.rows = (int)BT;
    a.cols = cols;
    a.rows_per_tile = kCsRows;
    a.dt = lp;
    int q = b.add(OP_COLRED, cdiv(cols, 16), "bias_grad", {p});
    ColredArgs& r = b[q].a.cr;
    r.partials = part;
    r.out[0] = out;
    r.n_parts = w.cs_tiles;
    r.n_vec = 1;
    r.cols = cols;
    r.cols_per_tile = 16;
    return q;
  };
  int p_lnf_b = ln_bwd(2 * (int)L, h->lay.lnf_g, -1, {p_head_dx}, "lnf_bwd");
  // colsum(dx at the last residual point) is the last MLP output bias gradient
  float* last_bias = c.has_bias ? gf(h->lay.layer[L - 1].b_proj) : nullptr;
  const int p_lnf_red = ln_red(2 * (int)L, p_lnf_b, gf(h->lay.lnf_g), gf(h->lay.lnf_b), last_bias, "lnf_params");
  int cur_dx = p_lnf_b;   // phase that produced dx at the current residual point

  // AdamW in parameter ranges, each started as soon as its gradients are final
  // (a layer's weight-gradient products, bias and LayerNorm-parameter sums, and
  // its input-gradient products, which read its compute copy), so most of the
  // update runs beside the rest of the backward instead of after it.  A range
  // is placed one layer later in ticket order than its last producer, so the
  // workgroups that claim its tickets seldom wait.  The embedding tables and
  // the first layer stay in a last range after every other phase.  Every range
  // also waits for the loss (a non-finite loss leaves the weights untouched)
  // and, co-resident, for the slot guard.
  const int adam_chunk = 16384;
  const bool coresident = w.n_slots > 1;
  int p_guard = -1;
  std::vector<std::vector<int>> grad_prod(L);   // per layer: the phases that write its gradients
  std::vector<int> ln1_red(L, -1);
  auto adam_range = [&](int64_t lo, int64_t hi, std::vector<int> deps, const char* nm) {
    int p = b.add(OP_ADAMW, (int)cdiv(hi - lo, adam_chunk), nm);
    AdamArgs& a = b[p].a.adam;
    a.p = P + lo;
    a.g = G + lo;
    a.m = at<float>(ws, w.m) + lo;
    a.v = at<float>(ws, w.v) + lo;
    a.wc = c.precision == OFA_BF16 ? (void*)(ws + w.wc + lo * D.lp) : nullptr;
    a.wc_dt = lp;
    a.n = hi - lo;
    a.per_tile = adam_chunk;
    a.beta1 = c.beta1;
    a.beta2 = c.beta2;
    a.eps = c.eps;
    a.wd = c.weight_decay;
    if (coresident) {
      a.pub = ws + w.serve + lo * D.lp;
      a.pub_slot_bytes = D.P * D.lp;
    }
    for (int i = 0; i < kMaxDeps; ++i) b[p].dep[i] = i < (int)deps.size() ? deps[i] : -1;
    return p;
  };
  // an early range: joins (one tile, no work) fold the producers into at most
  // three dependencies, the guard being the fourth
  auto adam_early = [&](int64_t lo, int64_t hi, std::vector<int> deps, const char* nm) {
    deps.push_back(p_loss);
    while (deps.size() > 3) {
      int j = b.add(OP_NOP, 1, "grad_join");
      for (int i = 0; i < kMaxDeps; ++i) b[j].dep[i] = deps[i];
      deps.erase(deps.begin(), deps.begin() + kMaxDeps);
      deps.insert(deps.begin(), j);
    }
    if (coresident) {
      if (p_guard < 0) {
        // before any range overwrites serve slot (tag & 1) the decoder must have left the version it holds
        p_guard = b.add(OP_SLOT_GUARD, 1, "slot_guard", {-2});
        b[p_guard].a.guard.st = at<DecState>(ws, w.dstate);
      }
      deps.push_back(p_guard);
    }
    // four tiles (65,536 parameters) per ticket: a ticket takes a workgroup
    // off the backward for a while, and ticket order is priority; measured per
    // c3 step with one, two, three, four, six, eight, sixteen and thirty-two
    // tiles per ticket: 9.37, 9.29, 9.23, 9.11, 9.14, 9.15, 9.30 and 9.63 ms
    // (9.30 with the update in one range at the end)
    const int pr = adam_range(lo, hi, deps, nm);
    b[pr].per_ticket = 4;
    return pr;
  };
  // ranges start on 16-byte boundaries (vector accesses); otherwise one range for everything
  auto layer_lo = [&](int l) { return l < (int)L ? h->lay.layer[l].ln1_g : h->lay.lnf_g; };
  bool split_adam = true;
  for (int l = 0; l <= (int)L; ++l) split_adam = split_adam && layer_lo(l) % 4 == 0;
  // ranges whose producers are all placed, waiting for their place in ticket
  // order (-1: the head, l >= 0: layer l).  They go in right after the next
  // layer's first input-gradient product, so that product's tickets are claimed
  // before them (c3 step: 9.02-9.04 ms; at the end of the block before it
  // 9.08-9.10, after the first weight-gradient product 9.08-9.10, after the
  // second input-gradient product 9.08-9.09).
  std::vector<int> pend;
  constexpr int kAdamPlace = 1;
  auto place = [&]() {
    for (int r : pend) {
      if (r < 0) {
        // final LayerNorm and LM head (untied): their gradients and the head's input gradient
        std::vector<int> deps = {p_head_dx, p_lnf_red};
        if (!c.tied_head) deps.push_back(p_head_dw);
        adam_early(h->lay.lnf_g, D.P, deps, "adamw_head");
      } else {
        // layer r: its producers, its own ln1_params (input gradients done) and
        // the phase that wrote its MLP output bias gradient
        std::vector<int> deps = grad_prod[r];
        deps.push_back(ln1_red[r]);
        deps.push_back(r + 1 < (int)L ? ln1_red[r + 1] : p_lnf_red);
        adam_early(layer_lo(r), layer_lo(r + 1), deps, "adamw_layer");
      }
    }
    pend.clear();
  };
  for (int l = (int)L - 1; l >= 0; --l) {
    const LayerOff& lo = h->lay.layer[l];
    const int ri = 2 * l + 2;   // residual point after the MLP
    void* dxo = DXLP(ri);
    int p_mdx, p_mdw2;
    if (c.mlp_gated) {
      g = gemm(h, (int)BT, (int)F, (int)d, dxo, d, 1, lp, wc(lo.w_down), F, 0, lp, DM(l), 2 * F, lp, EPI_DGEGLU);
      g.aux = M1(l);
      g.ldaux = 2 * F;
      g.aux_dt = lp;
      g.aux_off = (int)F;
      int p_ddx = gemm_phase(g, {cur_dx}, "down_dx");
      if (kAdamPlace == 1) place();
      g = gemm(h, (int)d, (int)F, (int)BT, dxo, d, 0, lp, M2(l), F, 0, lp, gf(lo.w_down), F, DT_F32, EPI_STORE);
      grad_prod[l].push_back(gemm_phase(g, {cur_dx}, "down_dw"));
      if (kAdamPlace == 2) place();
      g = gemm(h, (int)BT, (int)d, (int)(2 * F), DM(l), 2 * F, 1, lp, wc(lo.w_gate), d, 0, lp, DLN(2 * l + 1), d,
               DT_F32, EPI_STORE);
      p_mdx = gemm_phase(g, {p_ddx}, "gate_up_dx");
      if (kAdamPlace == 3) place();
      g = gemm(h, (int)(2 * F), (int)d, (int)BT, DM(l), 2 * F, 0, lp, Hh(2 * l + 1), d, 0, lp, gf(lo.w_gate), d,
               DT_F32, EPI_STORE);
      p_mdw2 = gemm_phase(g, {p_ddx}, "gate_up_dw");
      grad_prod[l].push_back(p_mdw2);
    } else {
      g = gemm(h, (int)BT, (int)F, (int)d, dxo, d, 1, lp, wc(lo.w_proj), F, 0, lp, DM(l), F, lp, EPI_DGELU);
      g.aux = M1(l);
      g.ldaux = F;
      g.aux_dt = lp;
      int p_pdx = gemm_phase(g, {cur_dx}, "proj_dx");
      if (kAdamPlace == 1) place();
      g = gemm(h, (int)d, (int)F, (int)BT, dxo, d, 0, lp, M2(l), F, 0, lp, gf(lo.w_proj), F, DT_F32, EPI_STORE);
      grad_prod[l].push_back(gemm_phase(g, {cur_dx}, "proj_dw"));
      if (kAdamPlace == 2) place();
      g = gemm(h, (int)BT, (int)d, (int)F, DM(l), F, 1, lp, wc(lo.w_fc), d, 0, lp, DLN(2 * l + 1), d, DT_F32,
               EPI_STORE);
      p_mdx = gemm_phase(g, {p_pdx}, "fc_dx");
      if (kAdamPlace == 3) place();
      g = gemm(h, (int)F, (int)d, (int)BT, DM(l), F, 0, lp, Hh(2 * l + 1), d, 0, lp, gf(lo.w_fc), d, DT_F32,
               EPI_STORE);
      p_mdw2 = gemm_phase(g, {p_pdx}, "fc_dw");
      grad_prod[l].push_back(p_mdw2);
      if (c.has_bias) grad_prod[l].push_back(colsum(DM(l), F, (int)F, CSF(l), gf(lo.b_fc), p_pdx, -1, "fc_bias_sum"));
    }
    (void)p_mdw2;
    int p_ln2b = ln_bwd(2 * l + 1, lo.ln2_g, ri, {p_mdx}, "ln2_bwd");
    grad_prod[l].push_back(ln_red(2 * l + 1, p_ln2b, gf(lo.ln2_g), gf(lo.ln2_b), c.has_bias ? gf(lo.b_o) : nullptr,
                                  "ln2_params"));
    void* dxm = DXLP(2 * l + 1);
    g = gemm(h, (int)BT, (int)d, (int)d, dxm, d, 1, lp, wc(lo.w_o), d, 0, lp, DOUT(l), d, lp, EPI_STORE);
    // With the matrix-core tile and 64-wide heads the attention backward's row
    // sums D = rowsum(dO * O) come out of this product's epilogue (a 128-column
    // tile holds two whole heads); otherwise a separate phase computes them.
    const bool fused_prep = attn_impl == 1 && g.impl == GEMM_P3 && d % 128 == 0;
    if (fused_prep) {
      g.epi = EPI_DSUM;
      g.aux = O(l);
      g.ldaux = d;
      g.aux_dt = lp;
      g.dsum = DSUM(l);
      g.dsum_T = (int)D.T;
      g.dsum_H = (int)D.H;
    }
    int p_odx = gemm_phase(g, {p_ln2b}, "attn_out_dx");
    g = gemm(h, (int)d, (int)d, (int)BT, dxm, d, 0, lp, O(l), d, 0, lp, gf(lo.w_o), d, DT_F32, EPI_STORE);
    grad_prod[l].push_back(gemm_phase(g, {p_ln2b}, "attn_out_dw"));
    int p_prep = p_odx;
    if (!fused_prep) {
      p_prep = b.add(OP_ATTN_PREP, cdiv(BT, 16), "attn_prep", {p_odx});
      b[p_prep].a.attn = attn_args(l);
      b[p_prep].a.attn.block = 16;
    }
    int p_kv = b.add(OP_ATTN_BWD_KV, attn_tiles, "attn_bwd_kv", {p_prep});
    b[p_kv].per_ticket = 1;
    b[p_kv].a.attn = attn_args(l);
    int p_q = b.add(OP_ATTN_BWD_Q, attn_tiles, "attn_bwd_q", {p_prep});
    b[p_q].per_ticket = 1;
    b[p_q].a.attn = attn_args(l);
    int p_dqkv = p_q;
    if (c.n_pos == 0) {
      int p = b.add(OP_ROPE_BWD, cdiv(BT, 16), "rope_bwd", {p_kv, p_q});
      b[p].a.rope = rope_args(DQKV(l));
      p_dqkv = p;
    }
      g = gemm(h, (int)BT, (int)d, (int)(3 * d), DQKV(l), 3 * d, 1, lp, wc(lo.w_qkv), d, 0, lp, DLN(2 * l), d, DT_F32,
             EPI_STORE);
    int p_qdx = gemm_phase(g, {p_dqkv, p_kv}, "qkv_dx");
    g = gemm(h, (int)(3 * d), (int)d, (int)BT, DQKV(l), 3 * d, 0, lp, Hh(2 * l), d, 0, lp, gf(lo.w_qkv), d, DT_F32,
             EPI_STORE);
    grad_prod[l].push_back(gemm_phase(g, {p_dqkv, p_kv}, "qkv_dw"));
    if (c.has_bias)
      grad_prod[l].push_back(colsum(DQKV(l), 3 * d, (int)(3 * d), CSQ(l), gf(lo.b_qkv), p_dqkv, p_kv, "qkv_bias_sum"));
    int p_ln1b = ln_bwd(2 * l, lo.ln1_g, 2 * l + 1, {p_qdx}, "ln1_bwd");
    float* prev_bias = (c.has_bias && l > 0) ? gf(h->lay.layer[l - 1].b_proj) : nullptr;
    // ln1_params also writes the previous layer's MLP output bias gradient; it
    // completes after every input-gradient product of this layer
    ln1_red[l] = ln_red(2 * l, p_ln1b, gf(lo.ln1_g), gf(lo.ln1_b), prev_bias, "ln1_params");
    cur_dx = p_ln1b;
    if (split_adam) {
      if (l == (int)L - 1) pend.push_back(-1);
      if (l + 1 < (int)L) pend.push_back(l + 1);
      if (kAdamPlace == 0) place();
    }
  }
  place();
  int v_rows = 64;
  int v_tiles = cdiv(V, v_rows);
  int pos_tiles = c.n_pos ? cdiv(c.n_pos, kThreadsHost / 64) : 0;   // one position per wavefront
  int p_eb = b.add(OP_EMB_BWD, v_tiles + pos_tiles, "emb_bwd", {cur_dx, p_sort, p_head_dw});
  {
    EmbBwdArgs& a = b[p_eb].a.ebwd;
    a.dx0 = DX(0);
    a.sorted = at<int32_t>(ws, w.esorted);
    a.first = at<uint64_t>(ws, w.efirst);
    a.dwte = gf(h->lay.wte);
    a.dwpe = gf(h->lay.wpe);
    a.B = (int)D.B;
    a.T = (int)D.T;
    a.d = (int)d;
    a.V = (int)V;
    a.n_pos = c.n_pos;
    a.accumulate = c.tied_head ? 1 : 0;
    a.rows_per_tile = v_rows;
    a.v_tiles = v_tiles;
  }
  // the last range: every earlier phase (the embedding tables' gradients come
  // last; co-resident, the slot guard is among the earlier phases)
  if (coresident && p_guard < 0) {
    p_guard = b.add(OP_SLOT_GUARD, 1, "slot_guard", {-2});
    b[p_guard].a.guard.st = at<DecState>(ws, w.dstate);
  }
  int p_adam = adam_range(0, split_adam ? layer_lo(1) : D.P, {-2}, "adamw");
  if (coresident) {
    int p_pub = b.add(OP_PUBLISH, 1, "publish", {p_adam});
    b[p_pub].a.publish.published = at<uint64_t>(ws, w.published);
  }
  // the next step's forward overwrites activations this step's backward reads
  b[p_emb].dep_prev = p_adam;
  b[p_sort].dep_prev = p_adam;
  // about one ticket per workgroup of a whole-GPU launch
  finish_program(h->train, std::max(kTicketsPerPhase, h->n_cu) * h->train_occ);
}

// Evaluation program of one batch: the training program's forward phases
// through the mean loss (no backward, no update) with the cross-entropy's
// gradient write left out, then the probe of chosen rows.  The embedding sort
// (needed by the backward only) becomes an empty phase, so phase indices and
// dependencies stay those of the training program.
void build_eval(ofa_handle* h) {
  h->eval.clear();
  int p_loss = -1, p_head = -1;
  for (size_t i = 0; i < h->train.size() && p_loss < 0; ++i) {
    Phase ph = h->train[i];
    if (ph.op == OP_EMB_SORT) {
      ph.op = OP_NOP;
      ph.n_tiles = 0;
      ph.per_ticket = 1;
    }
    if (ph.op == OP_CE) {
      // the LM head writes full fp32 logits here (the probe reads them) and the
      // cross-entropy only takes the loss
      p_head = ph.dep[0];
      ph.a.ce.dz = nullptr;
      ph.a.ce.fused = 0;
      GemmArgs& g = h->eval[p_head].a.gemm;
      g.epi = EPI_STORE;
      g.C = at<float>(h->ws, h->cw.logits);
      g.c_dt = DT_F32;
      g.ldc = h->D.V;
    }
    if (ph.op == OP_LOSS) p_loss = (int)i;
    h->eval.push_back(ph);
  }
  Builder b{&h->eval, nullptr};
  const int p_probe = b.add(OP_PROBE, kMaxProbe, "probe", {p_head, p_loss});
  b[p_probe].a.probe.logits = at<float>(h->ws, h->cw.logits);
  b[p_probe].a.probe.rows = (int)h->D.BT;
  b[p_probe].a.probe.V = (int)h->D.V;
  b[p_probe].per_ticket = 1;
  // the next batch's forward overwrites what this batch's loss and probe read
  h->eval[0].dep_prev = p_probe;
  h->eval[1].dep_prev = -1;
  finish_program(h->eval, std::max(kTicketsPerPhase, h->n_cu) * h->train_occ);
}

// Tile plan of a decode GEMV, whose task streams weight tiles through an LDS
// ring of fixed-size buffers: rows per tile chosen so that each of the G serve
// workgroups gets one ticket of whole tiles, up to four tiles in flight where
// the LDS allows.  With the rotation on, a ticket covers whole heads.
constexpr int kDecTileHost = 24576;   // bytes of one tile buffer (the task's kDecTile)

bool plan_gemv(Phase& ph, int G) {
  DecGemvArgs& a = ph.a.dgemv;
  const int64_t rb = (int64_t)a.K * (a.w_dt == DT_BF16 ? 2 : 4);
  const int halves = a.epi == DEPI_GEGLU ? 2 : 1;
  const int total = a.epi == DEPI_GEGLU ? a.F : a.N;
  const bool whole_heads = a.epi == DEPI_QKV && a.rope;
  const size_t avail = std::min(persistent_lds_bytes(1), lds_limit_bytes());
  const int nch = (int)(rb / 16);
  if (nch > 64 * 8) return false;                       // a row needs more than 8 chunks per lane
  const int lpr = nch <= 16 * 8 ? 16 : (nch <= 32 * 8 ? 32 : 64);
  const int r_max = (int)std::min<int64_t>({(int64_t)kDecTileHost / halves / rb, (int64_t)total,
                                            (int64_t)8 * (kThreadsHost / lpr) / halves});
  if (r_max < 1) return false;
  int R, per;
  if (whole_heads) {
    R = (int)a.dh;   // a power of two (the head size divides 256)
    while (R > r_max) R /= 2;
    const int rows_wg = cdiv(cdiv(total, G), a.dh) * (int)a.dh;
    per = cdiv(rows_wg, R);
  } else {
    const int rows_wg = cdiv(total, G);
    per = cdiv(rows_wg, r_max);
    R = cdiv(rows_wg, per);
  }
  a.rows_per_tile = R;
  a.lpr = lpr;
  const int per_group = cdiv(halves * R, kThreadsHost / lpr);
  a.rpg = per_group <= 1 ? 1 : per_group <= 2 ? 2 : per_group <= 4 ? 4 : 8;
  a.tile_bytes = kDecTileHost;
  a.ys_rows = (per * R + 3) / 4 * 4;   // keeps the LDS areas after it 16-byte aligned
  ph.n_tiles = cdiv(total, R);
  ph.per_ticket = per;
  a.per_ticket = per;
  for (a.n_buf = std::min(4, per); a.n_buf >= 1; --a.n_buf)
    if (phase_lds_bytes(ph) <= avail) return true;
  return false;
}

// decode program for one position (head phases skip themselves when the
// instance has no head)
void build_decode(ofa_handle* h) {
  const ofa_config& c = h->cfg;
  const Dims& D = h->D;
  const Carve& w = h->cw;
  char* ws = h->ws;
  h->dec.clear();
  h->dec_names.clear();
  Builder b{&h->dec, &h->dec_names};
  const int lp = D.lp_dt;
  const int64_t d = D.d, F = D.F, V = D.V;
  char* S = ws + w.serve;   // slot 0
  auto sw = [&](int64_t off) -> const void* { return off < 0 ? nullptr : S + off * D.lp; };
  float* dx = at<float>(ws, w.dx);
  const int64_t ns = D.nseq;
  auto XV = [&](int i) { return dx + (int64_t)i * ns * d; };   // [point][sequence][d]
  // per-sequence blocks: KV cache of all layers, attention partials of one layer
  const int64_t kv_ss = D.L * 2 * D.H * D.win * D.dh;
  const int64_t attn_ss = D.H * kMaxAttnSplit * (D.dh + 2);
  DecState* st = at<DecState>(ws, w.dstate);
  const int64_t slot_bytes = w.n_slots > 1 ? D.P * D.lp : 0;
  int p_emb = b.add(OP_DEC_EMBED, 1, "dec_embed");
  {
    DecEmbedArgs& a = b[p_emb].a.dembed;
    a.io = at<DecIO>(ws, w.misc + kMiscDecIO);
    a.wte = sw(h->lay.wte);
    a.wpe = sw(h->lay.wpe);
    a.ctx_tok = at<int32_t>(ws, w.ctx_tok);
    a.prompt = at<int32_t>(ws, w.dprompt);
    a.x = XV(0);
    a.nseq = (int)ns;
    a.cap = (int)D.win;
    a.st = st;
    a.published = at<uint64_t>(ws, w.published);
    a.slot_bytes = slot_bytes;
    a.d = (int)d;
    a.V = (int)V;
    a.w_dt = lp;
  }
  auto gemv = [&](const char* nm, int dep, const void* W, const void* bias, const float* xin, const void* lg, const void* lb, float* y,
                  int N, int K, int epi, int rpt, int64_t xin_ss, int64_t y_ss) {
    (void)rpt;
    int p = b.add(OP_DEC_GEMV, 1, nm, {dep});
    DecGemvArgs& a = b[p].a.dgemv;
    a.nseq = (int)ns;
    a.xin_ss = xin_ss;
    a.y_ss = y_ss;
    a.resid_ss = d;
    a.kv_ss = kv_ss;
    a.attn_ss = attn_ss;
    a.part_ss = V;
    a.W = W;
    a.bias = bias;
    a.xin = xin;
    a.ln_g = lg;
    a.ln_b = lb;
    a.y = y;
    a.st = st;
    a.N = N;
    a.K = K;
    a.w_dt = lp;
    a.kv_dt = lp;
    a.epi = epi;
    a.rows_per_tile = rpt;
    a.d = (int)d;
    a.H = (int)D.H;
    a.dh = (int)D.dh;
    a.cap = (int)D.win;
    a.rope = c.n_pos == 0;
    a.F = (int)F;
    a.io = at<DecIO>(ws, w.misc + kMiscDecIO);
    a.pre_dep = slot_bytes ? p_emb : -1;
    if (!plan_gemv(b[p], h->serve_wgs)) h->plan_ok = false;
    return p;
  };
  int last = p_emb;
  for (int l = 0; l < D.L; ++l) {
    const LayerOff& lo = h->lay.layer[l];
    void* kv = ws + w.kv + (size_t)l * 2 * D.H * D.win * D.dh * D.lp;
    int p_qkv = gemv("dec_qkv", last, sw(lo.w_qkv), sw(lo.b_qkv), XV(2 * l), sw(lo.ln1_g), sw(lo.ln1_b), at<float>(ws, w.dq),
                     (int)(3 * d), (int)d, DEPI_QKV, (int)D.dh, d, d);
    b[p_qkv].a.dgemv.kv = kv;
    const int split = std::max(1, std::min(kMaxAttnSplit, h->serve_wgs / (int)D.H));
    float* apart = at<float>(ws, w.dapart) + (int64_t)l * ns * attn_ss;
    int p_att = b.add(OP_DEC_ATTN, (int)(ns * D.H * split), "dec_attn", {p_qkv});
    {
      DecAttnArgs& a = b[p_att].a.dattn;
      a.q = at<float>(ws, w.dq);
      a.kv = kv;
      a.part = apart;
      a.nseq = (int)ns;
      a.kv_ss = kv_ss;
      a.part_ss = attn_ss;
      a.H = (int)D.H;
      a.dh = (int)D.dh;
      a.cap = (int)D.win;
      a.kv_dt = lp;
      a.split = split;
    }
    int p_o = gemv("dec_attn_out", p_att, sw(lo.w_o), sw(lo.b_o), nullptr, nullptr, nullptr, XV(2 * l + 1),
                   (int)d, (int)d, DEPI_RESID, 16, 0, d);
    b[p_o].a.dgemv.attn_part = apart;
    b[p_o].a.dgemv.attn_split = split;
    b[p_o].a.dgemv.resid = XV(2 * l);
    float* act = at<float>(ws, w.dmlp_v) + l * ns * F;
    int p_fc;
    if (c.mlp_gated)
      p_fc = gemv("dec_fc", p_o, sw(lo.w_gate), nullptr, XV(2 * l + 1), sw(lo.ln2_g), sw(lo.ln2_b), act, (int)(2 * F), (int)d,
                  DEPI_GEGLU, 16, d, F);
    else
      p_fc = gemv("dec_fc", p_o, sw(lo.w_fc), sw(lo.b_fc), XV(2 * l + 1), sw(lo.ln2_g), sw(lo.ln2_b), act, (int)F, (int)d,
                  DEPI_GELU, 16, d, F);
    int p_pr = gemv("dec_proj", p_fc, sw(c.mlp_gated ? lo.w_down : lo.w_proj), sw(lo.b_proj), act, nullptr, nullptr,
                    XV(2 * l + 2), (int)d, (int)F, DEPI_RESID, 16, F, d);
    b[p_pr].a.dgemv.resid = XV(2 * l + 1);
    last = p_pr;
  }
  const int64_t w_lm = c.tied_head ? h->lay.wte : h->lay.w_lm;
  int p_lm = gemv("dec_lm_head", last, sw(w_lm), nullptr, XV(2 * (int)D.L), sw(h->lay.lnf_g), sw(h->lay.lnf_b),
                  at<float>(ws, w.dlogits), (int)V, (int)d, DEPI_LOGITS, 16, d, V);
  b[p_lm].a.dgemv.part_val = at<float>(ws, w.dpart_v);
  b[p_lm].a.dgemv.part_idx = at<int32_t>(ws, w.dpart_i);
  int p_am = b.add(OP_DEC_ARGMAX, 1, "dec_argmax", {p_lm});
  {
    DecArgmaxArgs& a = b[p_am].a.dargmax;
    a.part_val = at<float>(ws, w.dpart_v);
    a.part_idx = at<int32_t>(ws, w.dpart_i);
    a.n_part = cdiv(b[p_lm].n_tiles, b[p_lm].per_ticket);
    a.ctx_tok = at<int32_t>(ws, w.ctx_tok);
    a.st = st;
    a.io = at<DecIO>(ws, w.misc + kMiscDecIO);
    a.V = (int)V;
    a.cap = (int)D.win;
    a.keep = (int)D.keep;
    a.nseq = (int)ns;
    a.part_ss = V;
  }
  b[p_emb].dep_prev = p_am;
  finish_program(h->dec);
}

double lr_at(const ofa_config& c, uint64_t step) {
  if (c.lr_schedule == OFA_LR_COSINE)
    return c.lr * 0.5 * (1.0 + std::cos(M_PI * (double)step / (double)c.total_steps));
  return c.lr;
}

ofa_status check_sticky(ofa_handle* h) {
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  if (h->sticky) return fail(h, (ofa_status)h->sticky, "an earlier call left device status %d", h->sticky);
  return OFA_OK;
}

// device-time stamp of a call (handles without events record nothing)
ofa_status record(ofa_handle* h, hipEvent_t ev) {
  if (ev) HIP_TRY(h, hipEventRecord(ev, h->stream));
  return OFA_OK;
}

ofa_status upload(ofa_handle* h, void* dst, const void* src, size_t bytes) {
  HIP_TRY(h, hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, h->stream));
  return OFA_OK;
}

// waits until the previous upload from the pinned staging area has been consumed
ofa_status staging_ready(ofa_handle* h) {
  if (h->upload_pending) {
    HIP_TRY(h, hipEventSynchronize(h->ev_upload));
    h->upload_pending = false;
  }
  return OFA_OK;
}

ofa_status mark_upload(ofa_handle* h) {
  if (!h->ev_upload) {   // static handle: the staging area is reused once the stream has consumed it
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    return OFA_OK;
  }
  HIP_TRY(h, hipEventRecord(h->ev_upload, h->stream));
  h->upload_pending = true;
  return OFA_OK;
}

ofa_status run_launch_per_phase(ofa_handle* h, const std::vector<Phase>& prog, const Phase* d_prog,
                                const StepCtx* d_ctx, int64_t n_inst, int64_t step0, bool dec_head_gate,
                                PhaseTime* tm) {
  DevStatus* st = at<DevStatus>(h->ws, h->cw.status);
  for (int64_t s = 0; s < n_inst; ++s) {
    const bool head = dec_head_gate ? (h->h_dsteps[s].head & 1) != 0 : true;
    for (size_t i = 0; i < prog.size(); ++i) {
      if (dec_head_gate && !head && (prog[i].op == OP_DEC_ARGMAX || (prog[i].op == OP_DEC_GEMV &&
                                                                     prog[i].a.dgemv.epi == DEPI_LOGITS)))
        continue;
      HIP_TRY(h, launch_phase(prog[i], d_prog, (int)i, d_ctx + s, st, tm, step0 + s, h->stream));
    }
  }
  return OFA_OK;
}

// Decode schedule (host mirror of the device's context rule): the positions
// processed before each of n_new emitted tokens, appended to h_dsteps from
// index *n_inst on; the first position of each token acquires the newest
// weights, the last one emits.  Advances the handle's context mirror.
bool dec_schedule(ofa_handle* h, int n_new, int head_extra_first, int64_t* n_inst) {
  const Dims& D = h->D;
  for (int i = 0; i < n_new; ++i) {
    for (int64_t p = h->dec_processed; p < h->dec_ctx_len; ++p) {
      if (*n_inst >= kMaxDecInst - 64) return false;
      StepCtx& sc = h->h_dsteps[(*n_inst)++];
      memset(&sc, 0, sizeof sc);
      sc.pos = (int)p;
      sc.head = (p == h->dec_ctx_len - 1 ? 1 : 0) | (p == h->dec_processed ? 2 : 0);
      if (i == 0 && p == h->dec_processed) sc.head |= head_extra_first;
      sc.gen_idx = i;
    }
    h->dec_processed = h->dec_ctx_len;
    if (h->dec_ctx_len + 1 > D.win) {
      h->dec_ctx_len = D.keep;
      h->dec_processed = 0;
    } else {
      h->dec_ctx_len += 1;
    }
  }
  return true;
}

// Scheduler block reset for one launch: ticket and counters start at the
// debug base, stop/limit cleared.
ofa_status reset_sched(ofa_handle* h, size_t sched_off, int n_phases) {
  Sched* sc = at<Sched>(h->ws, sched_off);
  const uint64_t base = h->cfg.debug_counter_base;
  HIP_TRY(h, launch_fill_u64(&sc->ticket, base, 1, h->stream));
  HIP_TRY(h, launch_fill_u64(&sc->base, base, 1, h->stream));
  HIP_TRY(h, launch_fill_u64(&sc->abort, 0, 3, h->stream));   // abort, exited, stop
  HIP_TRY(h, launch_fill_u64(&sc->limit, ~0ull, 1, h->stream));
  HIP_TRY(h, launch_fill_u64(sc->part_ticket, base, kMaxParts * kPartStride, h->stream));
  HIP_TRY(h, launch_fill_u64(sc->part_done, base, (int64_t)n_phases * kMaxParts, h->stream));
  HIP_TRY(h, launch_fill_u64(sc->done, base, n_phases, h->stream));
  return OFA_OK;
}

PersistJob make_job(ofa_handle* h, const std::vector<Phase>& prog, const Phase* d_prog, const StepCtx* d_ctx,
                    int64_t n_inst, size_t sched_off, PhaseTime* times, uint64_t* inst_end, int n_wg,
                    bool open_ended = false) {
  PersistJob j;
  memset(&j, 0, sizeof j);
  j.phases = d_prog;
  j.n_phases = (int)prog.size();
  j.tickets_per_inst = prog.back().ticket_base + prog.back().n_tickets;
  // tickets are claimed per die (eight partitions: 32 workgroups per counter
  // instead of 256 for training); an open-ended job (co-resident decode, whose
  // stopping rule needs one counter) or a grid under eight keeps one, and so
  // does decode, with a release per ticket: its phases have few tickets each
  // and follow one another, and the workgroup finishing a phase then makes one
  // counter round trip instead of two (its die's share, then the phase)
  const DevProg& dp = &prog == &h->train ? h->dp_train : &prog == &h->eval ? h->dp_eval : h->dp_dec;
  if (n_wg >= kMaxParts && !open_ended && &prog != &h->dec) {
    j.n_parts = kMaxParts;
    j.part_tb = dp.pt8;
    // the hardware hands workgroup b to die b % 8, so partition s is die s
    // (each workgroup checks this on the device)
    j.die_release = (h->die_map && !(h->cfg.debug_flags & OFA_DEBUG_WG_RELEASE)) ? 1 : 0;
    j.part_tiles = dp.tiles8;
  } else {
    j.n_parts = 1;
    j.part_tb = dp.pt1;
  }
  j.n_inst = n_inst;
  j.steps = d_ctx;
  j.period = n_inst;
  j.sched = at<Sched>(h->ws, sched_off);
  j.times = times;
  j.inst_end = inst_end;
  j.n_wg = n_wg;
  return j;
}

// One persistent launch of one or two jobs.
ofa_status launch_jobs(ofa_handle* h, PersistJob* jobs, int n_jobs, int occ = 1) {
  const ofa_config& c = h->cfg;
  PersistParams pp;
  memset(&pp, 0, sizeof pp);
  int grid = 0;
  h->trace_n_phases = 0;
  for (int i = 0; i < n_jobs; ++i) {
    pp.job[i] = jobs[i];
    grid += jobs[i].n_wg;
  }
  pp.n_jobs = n_jobs;
  pp.status = at<DevStatus>(h->ws, h->cw.status);
  pp.abort = &pp.job[0].sched->abort;
  pp.watchdog_ticks = (c.debug_flags & OFA_DEBUG_SHORT_WATCHDOG) ? 100000ull : 1000000000ull;
  pp.shuffle = (c.debug_flags & OFA_DEBUG_SHUFFLE_TICKETS) ? 1 : 0;
  if (n_jobs == 1 && (c.debug_flags & OFA_DEBUG_TRACE)) {
    PersistJob& j = pp.job[0];
    j.trace = at<uint64_t>(h->ws, h->cw.trace);
    j.trace_inst = std::min<int64_t>(j.n_inst, OFA_TRACE_INSTANCES);
    HIP_TRY(h, launch_fill_u64(j.trace, 0, j.trace_inst * j.n_phases * 4, h->stream));
    h->trace_n_phases = j.n_phases;
    h->trace_n_inst = j.trace_inst;
    h->trace_dec = j.phases == h->d_dec;
  }
  h->last_grid = grid;
  HIP_TRY(h, launch_persistent(pp, grid, h->stream, occ));
  return OFA_OK;
}

// One persistent launch of n_inst instances of a program on `cus` CUs, with
// the kernel built for `kocc` workgroups per CU.
ofa_status run_persistent(ofa_handle* h, const std::vector<Phase>& prog, const Phase* d_prog, const StepCtx* d_ctx,
                          int64_t n_inst, size_t sched_off, PhaseTime* times, uint64_t* inst_end, int cus,
                          int kocc = 1) {
  const int occ = persistent_occupancy(kocc);
  if (occ < 1) return fail(h, OFA_E_HIP, "persistent kernel does not fit a CU");
  ofa_status s = reset_sched(h, sched_off, (int)prog.size());
  if (s != OFA_OK) return s;
  if (inst_end) HIP_TRY(h, launch_fill_u64(inst_end, 0, n_inst, h->stream));
  PersistJob j = make_job(h, prog, d_prog, d_ctx, n_inst, sched_off, times, inst_end, cus * occ);
  return launch_jobs(h, &j, 1, kocc);
}

}  // namespace

// =====================================================================  C ABI

static ofa_status publish(ofa_handle* h);
static ofa_status copy_flat(ofa_handle* h, const void* src, int sdt, void* dst, int ddt, int64_t n);

extern "C" {

ofa_status ofa_validate_config(const ofa_config* cfg, char* msg, size_t msg_len) {
  if (!cfg) return OFA_E_ARG;
  std::string e = validate(*cfg);
  if (e.empty()) return OFA_OK;
  if (msg && msg_len) {
    strncpy(msg, e.c_str(), msg_len - 1);
    msg[msg_len - 1] = 0;
  }
  return OFA_E_ARG;
}

size_t ofa_workspace_bytes(const ofa_config* cfg) {
  if (!cfg || !validate(*cfg).empty()) return 0;
  Layout L = make_layout(*cfg);
  return carve(*cfg, L).total;
}

int64_t ofa_param_count(const ofa_config* cfg) {
  if (!cfg || !validate(*cfg).empty()) return -1;
  return make_layout(*cfg).total;
}

int32_t ofa_param_tensor_count(const ofa_config* cfg) {
  if (!cfg || !validate(*cfg).empty()) return -1;
  return (int32_t)make_layout(*cfg).t.size();
}

ofa_status ofa_param_tensor(const ofa_config* cfg, int32_t i, int64_t* offset, int64_t* numel, int32_t* kind,
                            char* name, size_t name_len) {
  if (!cfg || !validate(*cfg).empty()) return OFA_E_ARG;
  Layout L = make_layout(*cfg);
  if (i < 0 || i >= (int32_t)L.t.size()) return OFA_E_ARG;
  const TensorDesc& t = L.t[i];
  if (offset) *offset = t.off;
  if (numel) *numel = t.numel;
  if (kind) *kind = t.kind;
  if (name && name_len) {
    strncpy(name, t.name.c_str(), name_len - 1);
    name[name_len - 1] = 0;
  }
  return OFA_OK;
}

ofa_status ofa_task_budget(uint64_t iterations, uint64_t tasks_per_unit, uint64_t* out) {
  if (!out) return OFA_E_ARG;
  if (tasks_per_unit && iterations > (uint64_t)INT64_MAX / tasks_per_unit) return OFA_E_OVERFLOW;
  *out = iterations * tasks_per_unit;
  return OFA_OK;
}

const char* ofa_status_string(ofa_status s) {
  switch (s) {
    case OFA_OK: return "ok";
    case OFA_E_ARG: return "invalid argument";
    case OFA_E_HIP: return "HIP runtime error";
    case OFA_E_NONFINITE: return "non-finite value";
    case OFA_E_TIMEOUT: return "device wait timed out";
    case OFA_E_OVERFLOW: return "budget overflow";
    case OFA_E_STATE: return "invalid state";
  }
  return "unknown";
}

const char* ofa_last_error(const ofa_handle* h) { return h ? h->err.c_str() : "null handle"; }

}  // extern "C"

namespace {

// Everything ofa_create and ofa_create_static share, on a handle whose config,
// layout, dims, carve, workspace and stream are set (and, for a static handle,
// whose staging pointers point at the static host arrays).
ofa_status init_handle(ofa_handle* h, const float* dev_init_params);

}  // namespace

extern "C" {

ofa_status ofa_create(const ofa_config* cfg, void* dev_workspace, size_t ws_bytes, const float* dev_init_params,
                      void* hip_stream, ofa_handle** out) {
  if (!cfg || !out || !dev_workspace || !dev_init_params) return OFA_E_ARG;
  *out = nullptr;
  if (!validate(*cfg).empty()) return OFA_E_ARG;
  if ((uintptr_t)dev_workspace % kAlign) return OFA_E_ARG;
  ofa_handle* h = new ofa_handle();
  h->cfg = *cfg;
  h->lay = make_layout(*cfg);
  h->D = dims_of(*cfg, h->lay);
  h->cw = carve(*cfg, h->lay);
  if (ws_bytes < h->cw.total) {
    delete h;
    return OFA_E_ARG;
  }
  h->ws = (char*)dev_workspace;
  h->stream = (hipStream_t)hip_stream;
  *out = h;
  return init_handle(h, dev_init_params);
}

}  // extern "C"

namespace {

// One handle per device for ofa_create_static, with its host staging arrays.
struct StaticSlot {
  ofa_handle h;
  StepCtx steps[kMaxSteps];
  StepCtx dsteps[kMaxDecInst];
  alignas(64) char misc[kMiscBytes];
};
StaticSlot g_static_slot[kStaticMaxDevices];

ofa_status init_handle(ofa_handle* h, const float* dev_init_params) {
  static bool kernels_ready = false;
  if (!kernels_ready) {
    HIP_TRY(h, init_kernels());
    kernels_ready = true;
  }
  // the sort of the embedding backward keeps batch*seq 64-bit keys in LDS
  if ((size_t)h->D.BT * 8 + 64 > persistent_lds_bytes(1))
    return fail(h, OFA_E_ARG, "batch*seq %lld needs more LDS than the device allows", (long long)h->D.BT);
  int dev = 0;
  HIP_TRY(h, hipGetDevice(&dev));
  HIP_TRY(h, hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, dev));
  if (h->cfg.train_cus > h->n_cu || h->cfg.serve_cus > h->n_cu || h->cfg.train_cus + h->cfg.serve_cus > h->n_cu)
    return fail(h, OFA_E_ARG, "CU partition %d + %d exceeds the device's %d CUs", h->cfg.train_cus,
                h->cfg.serve_cus, h->n_cu);
  if (!h->is_static) {
    HIP_TRY(h, hipHostMalloc((void**)&h->h_steps, sizeof(StepCtx) * kMaxSteps, hipHostMallocDefault));
    HIP_TRY(h, hipHostMalloc((void**)&h->h_dsteps, sizeof(StepCtx) * kMaxDecInst, hipHostMallocDefault));
    HIP_TRY(h, hipHostMalloc((void**)&h->h_misc, kMiscBytes, hipHostMallocDefault));
    HIP_TRY(h, hipEventCreateWithFlags(&h->ev_upload, hipEventDisableTiming));
    HIP_TRY(h, hipEventCreate(&h->ev_t0));
    HIP_TRY(h, hipEventCreate(&h->ev_t1));
    HIP_TRY(h, hipHostMalloc((void**)&h->h_bell, 128, hipHostMallocCoherent));
  }
  {
    const int occ = std::max(1, persistent_occupancy(1));
    h->serve_wgs = (h->cfg.serve_cus > 0 ? h->cfg.serve_cus : h->n_cu) * occ;
  }
  // Step-mode training runs two workgroups per CU where the kernel fits twice
  // (co-resident launches keep one: both jobs share one kernel): one workgroup's
  // matrix-core work then overlaps the other's epilogue, copies and waits.  At c3
  // this measured 10.24 against 10.71 ms a step (OFA_DEBUG_OCC1 keeps one).
  const bool coresident_cfg = h->cfg.train_cus > 0 && h->cfg.serve_cus > 0;
  h->train_occ = (!coresident_cfg && !(h->cfg.debug_flags & OFA_DEBUG_OCC1) && persistent_occupancy(2) >= 2) ? 2 : 1;
  build_train(h);
  build_eval(h);
  build_decode(h);
  if (!h->plan_ok) return fail(h, OFA_E_ARG, "a decode matrix-vector product does not fit the LDS");
  if (h->train.size() > (size_t)kMaxPhases || h->dec.size() > (size_t)kMaxPhases || h->eval.size() > (size_t)kMaxPhases)
    return fail(h, OFA_E_ARG, "program too long");
  for (const auto* prog : {&h->train, &h->dec})
    for (const Phase& ph : *prog)
      if ((size_t)ph.lds_bytes > persistent_lds_bytes(1) || (size_t)ph.lds_bytes > lds_limit_bytes())
        return fail(h, OFA_E_ARG, "phase op %d needs %d bytes of LDS (> %zu)", ph.op, ph.lds_bytes,
                    persistent_lds_bytes(1));
  if (h->train_occ == 2)
    for (const Phase& ph : h->train)
      if (phase_lds_bytes_occ(ph, 2) > persistent_lds_bytes(2)) h->train_occ = 1;   // one per CU after all
  // phase tables: uploaded into their slot of the caller's workspace
  // (pageable host sources: the stream is synchronised before they go out of scope)
  std::vector<std::vector<int32_t>> keep;
  size_t toff = h->cw.tables;
  auto put = [&](size_t bytes) -> void* {
    toff = (toff + 15) / 16 * 16;
    void* dst = h->ws + toff;
    toff += bytes;
    return toff - h->cw.tables <= kTableBytes ? dst : nullptr;
  };
  for (auto [prog, dp] : {std::pair<std::vector<Phase>*, DevProg*>{&h->train, &h->dp_train}, {&h->dec, &h->dp_dec},
                          {&h->eval, &h->dp_eval}}) {
    keep.push_back(part_table(*prog, kMaxParts));
    keep.push_back(part_table(*prog, 1));
    keep.push_back(part_tile_table(*prog, kMaxParts));
    const size_t k = keep.size();
    dp->ph = (Phase*)put(prog->size() * sizeof(Phase));
    dp->pt8 = (int32_t*)put(keep[k - 3].size() * 4);
    dp->pt1 = (int32_t*)put(keep[k - 2].size() * 4);
    dp->tiles8 = (int32_t*)put(keep[k - 1].size() * 4);
    if (!dp->ph || !dp->pt8 || !dp->pt1 || !dp->tiles8) return fail(h, OFA_E_ARG, "phase tables exceed their slot");
    HIP_TRY(h, hipMemcpyAsync(dp->ph, prog->data(), prog->size() * sizeof(Phase), hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipMemcpyAsync(dp->pt8, keep[k - 3].data(), keep[k - 3].size() * 4, hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipMemcpyAsync(dp->pt1, keep[k - 2].data(), keep[k - 2].size() * 4, hipMemcpyHostToDevice, h->stream));
    HIP_TRY(h, hipMemcpyAsync(dp->tiles8, keep[k - 1].data(), keep[k - 1].size() * 4, hipMemcpyHostToDevice,
                              h->stream));
  }
  static_assert(sizeof(Phase) <= 320, "phase table slot");
  h->d_train = h->dp_train.ph;
  h->d_dec = h->dp_dec.ph;
  char* ws = h->ws;
  const Carve& w = h->cw;
  // Once per device: does workgroup b of a launch run on die b % 8?  The
  // persistent executor's once-per-die release needs it; without it every
  // ticket is released on its own (the probe writes into the misc block).
  static int die_map_of[64];   // 0 = not probed, 1 = b % 8, 2 = another mapping
  if (dev < 0 || dev >= 64 || die_map_of[dev] == 0) {
    const int occ = std::max({1, persistent_occupancy(1), persistent_occupancy(2)});
    const int n = std::min<int>((int)(kMiscBytes / 4), std::max(kMaxParts, h->n_cu * occ));
    uint32_t* probe = at<uint32_t>(ws, w.misc);
    std::vector<uint32_t> ids(n);
    HIP_TRY(h, launch_xcc_probe(probe, n, h->stream));
    HIP_TRY(h, hipMemcpyAsync(ids.data(), probe, (size_t)n * 4, hipMemcpyDeviceToHost, h->stream));
    HIP_TRY(h, hipStreamSynchronize(h->stream));
    bool ok = true;
    for (int i = 0; i < n; ++i) ok = ok && ids[i] == (uint32_t)(i % kMaxParts);
    if (dev >= 0 && dev < 64) die_map_of[dev] = ok ? 1 : 2;
    h->die_map = ok;
  } else {
    h->die_map = die_map_of[dev] == 1;
  }
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  // state
  const size_t P = h->D.P;
  HIP_TRY(h, hipMemcpyAsync(ws + w.p, dev_init_params, P * 4, hipMemcpyDeviceToDevice, h->stream));
  HIP_TRY(h, launch_fill_u32(at<uint32_t>(ws, w.m), 0, (int64_t)P, h->stream));
  HIP_TRY(h, launch_fill_u32(at<uint32_t>(ws, w.v), 0, (int64_t)P, h->stream));
  HIP_TRY(h, launch_fill_u32(at<uint32_t>(ws, w.g), 0, (int64_t)P, h->stream));
  HIP_TRY(h, launch_fill_u64(at<uint64_t>(ws, w.efirst), 0, h->D.V, h->stream));
  HIP_TRY(h, launch_fill_u32((uint32_t*)at<DevStatus>(ws, w.status), 0, sizeof(DevStatus) / 4, h->stream));
  HIP_TRY(h, launch_fill_u64(at<uint64_t>(ws, w.published), 0, 8, h->stream));
  HIP_TRY(h, launch_fill_u32((uint32_t*)at<DecState>(ws, w.dstate), 0, sizeof(DecState) / 4, h->stream));
  ofa_status s = ofa_set_params(h, at<float>(ws, w.p));
  if (s != OFA_OK) return s;
  h->version = 0;   // the initial weights are version 0
  s = publish(h);
  if (s != OFA_OK) return s;
  h->unpublished = false;
  return OFA_OK;
}

}  // namespace

extern "C" {

ofa_status ofa_create_static(const ofa_config* cfg, const float* dev_init_params, void* hip_stream,
                             ofa_handle** out) {
  if (!cfg || !out || !dev_init_params) return OFA_E_ARG;
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) {
    (void)hipGetLastError();
    return OFA_E_HIP;
  }
  StaticSlot& slot = g_static_slot[dev];
  ofa_handle* h = &slot.h;
  if (h->ws) (void)hipStreamSynchronize(h->stream);   // the earlier model's work is done with the array
  *h = ofa_handle();
  h->is_static = true;
  h->h_steps = slot.steps;
  h->h_dsteps = slot.dsteps;
  h->h_misc = slot.misc;
  *out = h;
  std::string e = validate(*cfg);
  if (!e.empty()) return fail(h, OFA_E_ARG, "%s", e.c_str());
  h->cfg = *cfg;
  h->lay = make_layout(*cfg);
  h->D = dims_of(*cfg, h->lay);
  h->cw = carve(*cfg, h->lay);
  if (h->cw.total > kStaticScratchBytes)
    return fail(h, OFA_E_ARG, "this model needs a %zu-byte workspace; the static one holds %zu bytes", h->cw.total,
                kStaticScratchBytes);
  void* ws = nullptr;
  HIP_TRY(h, static_scratch(&ws));
  h->ws = (char*)ws;
  h->stream = (hipStream_t)hip_stream;
  return init_handle(h, dev_init_params);
}


ofa_status ofa_destroy(ofa_handle* h) {
  if (!h) return OFA_E_ARG;
  (void)hipStreamSynchronize(h->stream);
  if (h->is_static) {   // the device's static handle stays; it only stops working
    h->ws = nullptr;
    return OFA_OK;
  }
  if (h->h_steps) (void)hipHostFree(h->h_steps);
  if (h->h_dsteps) (void)hipHostFree(h->h_dsteps);
  if (h->h_misc) (void)hipHostFree(h->h_misc);
  if (h->ev_upload) (void)hipEventDestroy(h->ev_upload);
  if (h->ev_t0) (void)hipEventDestroy(h->ev_t0);
  if (h->ev_t1) (void)hipEventDestroy(h->ev_t1);
  if (h->h_bell) (void)hipHostFree(h->h_bell);
  delete h;
  return OFA_OK;
}

// copy / cast a flat range with one COPY phase launched on its own
static ofa_status copy_flat(ofa_handle* h, const void* src, int sdt, void* dst, int ddt, int64_t n) {
  // small helper program: built on the fly into the staging slot after the phase tables
  Phase p;
  memset(&p, 0, sizeof p);
  p.op = OP_COPY;
  const int per = 65536;
  p.n_tiles = cdiv(n, per);
  p.a.copy.src = src;
  p.a.copy.dst = dst;
  p.a.copy.n = n;
  p.a.copy.src_dt = sdt;
  p.a.copy.dst_dt = ddt;
  p.a.copy.per_tile = per;
  for (int i = 0; i < kMaxDeps; ++i) p.dep[i] = -1;
  p.dep_prev = -1;
  static_assert(sizeof(Phase) <= kMiscDecIO, "misc block too small");
  Phase* d_p = (Phase*)(h->ws + h->cw.misc);
  ofa_status s = staging_ready(h);
  if (s != OFA_OK) return s;
  memcpy(h->h_misc, &p, sizeof p);
  s = upload(h, d_p, h->h_misc, sizeof p);
  if (s != OFA_OK) return s;
  HIP_TRY(h, launch_phase(p, d_p, 0, nullptr, at<DevStatus>(h->ws, h->cw.status), nullptr, 0, h->stream));
  return mark_upload(h);
}

ofa_status ofa_set_params(ofa_handle* h, const float* dev_params) {
  if (!h || !dev_params) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  char* ws = h->ws;
  const int64_t P = h->D.P;
  if ((const char*)dev_params != ws + h->cw.p)
    HIP_TRY(h, hipMemcpyAsync(ws + h->cw.p, dev_params, P * 4, hipMemcpyDeviceToDevice, h->stream));
  h->unpublished = true;
  if (h->cfg.precision == OFA_BF16) return copy_flat(h, ws + h->cw.p, DT_F32, ws + h->cw.wc, DT_BF16, P);
  return OFA_OK;
}

ofa_status ofa_get_params(ofa_handle* h, float* dev_params) {
  if (!h || !dev_params) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  HIP_TRY(h, hipMemcpyAsync(dev_params, h->ws + h->cw.p, h->D.P * 4, hipMemcpyDeviceToDevice, h->stream));
  return OFA_OK;
}

ofa_status ofa_get_grads(ofa_handle* h, float* dev_grads) {
  if (!h || !dev_grads) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  HIP_TRY(h, hipMemcpyAsync(dev_grads, h->ws + h->cw.g, h->D.P * 4, hipMemcpyDeviceToDevice, h->stream));
  return OFA_OK;
}

// serve copy <- compute weights, then the published version number
// (two slots: version v lives in slot v & 1)
static ofa_status publish(ofa_handle* h) {
  char* ws = h->ws;
  const size_t slot = h->cw.n_slots > 1 ? (size_t)(h->version & 1) * (size_t)h->D.P * h->D.lp : 0;
  ofa_status s = copy_flat(h, ws + h->cw.wc, h->D.lp_dt, ws + h->cw.serve + slot, h->D.lp_dt, h->D.P);
  if (s != OFA_OK) return s;
  HIP_TRY(h, launch_fill_u64(at<uint64_t>(ws, h->cw.published), h->version, 1, h->stream));
  return OFA_OK;
}

ofa_status ofa_publish_weights(ofa_handle* h, uint64_t* version_out) {
  if (!h) return OFA_E_ARG;
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  if (h->cw.n_slots > 1 && !h->unpublished) {
    // co-resident configuration: every training step has published its weights already
    if (version_out) *version_out = h->version;
    return OFA_OK;
  }
  h->version += 1;
  s = publish(h);
  if (s != OFA_OK) return s;
  h->unpublished = false;
  if (version_out) *version_out = h->version;
  return OFA_OK;
}

ofa_status ofa_train_step(ofa_handle* h, const int32_t* dev_tokens, int32_t n_steps, float* dev_losses) {
  if (!h || !dev_tokens || !dev_losses || n_steps < 1) return fail(h, OFA_E_ARG, "bad arguments");
  if (n_steps > kMaxSteps) return fail(h, OFA_E_ARG, "n_steps %d > %d", n_steps, kMaxSteps);
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  const ofa_config& c = h->cfg;
  s = staging_ready(h);
  if (s != OFA_OK) return s;
  const int64_t per = h->D.B * (h->D.T + 1);
  for (int i = 0; i < n_steps; ++i) {
    StepCtx& sc = h->h_steps[i];
    memset(&sc, 0, sizeof sc);
    const uint64_t t = h->steps_done + i + 1;
    sc.tokens = dev_tokens + per * i;
    sc.loss_out = dev_losses + i;
    sc.lr = (float)lr_at(c, t - 1);
    sc.bc1 = (float)(1.0 - std::pow((double)c.beta1, (double)t));
    sc.bc2 = (float)(1.0 - std::pow((double)c.beta2, (double)t));
    sc.step_in_call = i;
    // co-resident configurations: the tag is the weight version the step publishes
    sc.tag = h->cw.n_slots > 1 ? h->version + i + 1 : t;
  }
  StepCtx* d_steps = at<StepCtx>(h->ws, h->cw.steps);
  s = upload(h, d_steps, h->h_steps, sizeof(StepCtx) * n_steps);
  if (s != OFA_OK) return s;
  s = mark_upload(h);
  if (s != OFA_OK) return s;
  const int np = (int)h->train.size();
  // phase times: t0 <- max, t1 <- 0
  PhaseTime* tm = at<PhaseTime>(h->ws, h->cw.times);
  HIP_TRY(h, launch_fill_pairs((uint64_t*)tm, ~0ull, 0ull, np, h->stream));
  { ofa_status rs = record(h, h->ev_t0); if (rs != OFA_OK) return rs; }
  if (c.exec_mode == OFA_EXEC_LAUNCH_PER_PHASE) {
    s = run_launch_per_phase(h, h->train, h->d_train, d_steps, n_steps, (int64_t)h->steps_done, false, tm);
    if (s != OFA_OK) return s;
  } else {
    int cus = c.train_cus > 0 ? c.train_cus : h->n_cu;
    s = run_persistent(h, h->train, h->d_train, d_steps, n_steps, h->cw.sched, tm,
                       at<uint64_t>(h->ws, h->cw.inst_end), cus, h->train_occ);
    if (s != OFA_OK) return s;
  }
  { ofa_status rs = record(h, h->ev_t1); if (rs != OFA_OK) return rs; }
  h->timed = h->ev_t0 != nullptr;
  h->steps_done += n_steps;
  if (h->cw.n_slots > 1) {   // co-resident configuration: each step published
    h->version += n_steps;
    h->unpublished = false;
  }
  return OFA_OK;
}

}  // extern "C"

namespace {

// One decode call (ofa_decode_token; with a doorbell, ofa_decode_doorbell).
ofa_status decode_call(ofa_handle* h, const int32_t* dev_prompt, int32_t n_prompt, int32_t n_new,
                       int32_t* dev_tokens_out, float* dev_logits_out, uint64_t* dev_versions_out,
                       const uint64_t* doorbell, uint64_t* progress, uint64_t* ticks, int64_t n_ticks) {
  if (!h || n_new < 1 || !dev_tokens_out || n_prompt < 0) return fail(h, OFA_E_ARG, "bad arguments");
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  const Dims& D = h->D;
  if (n_prompt > D.win) return fail(h, OFA_E_ARG, "prompt %d longer than the window %d", n_prompt, (int)D.win);
  if (n_prompt == 0 && !h->dec_started) return fail(h, OFA_E_STATE, "no context to continue");
  char* ws = h->ws;
  DecState* st = at<DecState>(ws, h->cw.dstate);
  if (n_prompt > 0) {
    if (!dev_prompt) return fail(h, OFA_E_ARG, "null prompt");
    // sequence q's prompt dev_prompt[q][0..n_prompt) -> its context ctx_tok[q][0..)
    HIP_TRY(h, hipMemcpy2DAsync(ws + h->cw.ctx_tok, (size_t)D.win * 4, dev_prompt, (size_t)n_prompt * 4,
                                (size_t)n_prompt * 4, (size_t)D.nseq, hipMemcpyDeviceToDevice, h->stream));
    // ctx_len = n_prompt, n_gen = 0 (DecState: version, w_delta, ctx_len, n_gen)
    HIP_TRY(h, launch_fill_u32((uint32_t*)&st->ctx_len, (uint32_t)n_prompt, 1, h->stream));
    HIP_TRY(h, launch_fill_u32((uint32_t*)&st->n_gen, 0, 1, h->stream));
    h->dec_ctx_len = n_prompt;
    h->dec_processed = 0;
    h->dec_started = true;
  }
  s = staging_ready(h);
  if (s != OFA_OK) return s;
  int64_t n_inst = 0;
  if (!dec_schedule(h, n_new, 0, &n_inst)) return fail(h, OFA_E_ARG, "decode call too long");
  StepCtx* d_dsteps = at<StepCtx>(ws, h->cw.dsteps);
  s = upload(h, d_dsteps, h->h_dsteps, sizeof(StepCtx) * n_inst);
  if (s != OFA_OK) return s;
  // outputs of this call
  DecIO io{dev_tokens_out, dev_versions_out, dev_logits_out, progress, (int64_t)n_new, doorbell, ticks, n_ticks};
  memcpy(h->h_misc + kMiscDecIO, &io, sizeof io);
  s = upload(h, h->ws + h->cw.misc + kMiscDecIO, h->h_misc + kMiscDecIO, sizeof io);
  if (s != OFA_OK) return s;
  s = mark_upload(h);
  if (s != OFA_OK) return s;
  PhaseTime* dtm = at<PhaseTime>(ws, h->cw.dtimes);
  HIP_TRY(h, launch_fill_pairs((uint64_t*)dtm, ~0ull, 0ull, (int64_t)h->dec.size(), h->stream));
  { ofa_status rs = record(h, h->ev_t0); if (rs != OFA_OK) return rs; }
  if (h->cfg.exec_mode == OFA_EXEC_LAUNCH_PER_PHASE)
    s = run_launch_per_phase(h, h->dec, h->d_dec, d_dsteps, n_inst, 0, true, dtm);
  else
    s = run_persistent(h, h->dec, h->d_dec, d_dsteps, n_inst, h->cw.dsched, dtm, nullptr,
                       h->serve_wgs / std::max(1, persistent_occupancy(1)));
  if (s != OFA_OK) return s;
  { ofa_status rs = record(h, h->ev_t1); if (rs != OFA_OK) return rs; }
  h->timed = h->ev_t0 != nullptr;
  return OFA_OK;
}

}  // namespace

extern "C" {

ofa_status ofa_decode_token(ofa_handle* h, const int32_t* dev_prompt, int32_t n_prompt, int32_t n_new,
                            int32_t* dev_tokens_out, float* dev_logits_out, uint64_t* dev_versions_out) {
  return decode_call(h, dev_prompt, n_prompt, n_new, dev_tokens_out, dev_logits_out, dev_versions_out, nullptr,
                     nullptr, nullptr, 0);
}

ofa_status ofa_decode_doorbell(ofa_handle* h, const int32_t* dev_prompt, int32_t n_prompt, int32_t n_new,
                               int32_t* dev_tokens_out, double* host_ring_to_token_us, double* dev_wake_to_token_us) {
  if (!h) return OFA_E_ARG;
  if (!h->h_bell) return fail(h, OFA_E_STATE, "this handle has no doorbell (made by ofa_create_static)");
  if (h->cfg.exec_mode != OFA_EXEC_PERSISTENT) return fail(h, OFA_E_STATE, "the doorbell needs the persistent executor");
  if (n_new < 1 || n_new > kMaxBell) return fail(h, OFA_E_ARG, "n_new %d out of [1, %d]", n_new, kMaxBell);
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  HIP_TRY(h, hipStreamSynchronize(h->stream));   // the previous call no longer reads the words
  volatile uint64_t* bell = h->h_bell;
  volatile uint64_t* prog = h->h_bell + 8;        // its own 64-byte line
  *bell = 0;
  *prog = 0;
  std::atomic_thread_fence(std::memory_order_seq_cst);
  uint64_t* ticks = at<uint64_t>(h->ws, h->cw.bell_ticks);
  HIP_TRY(h, launch_fill_u64(ticks, 0, 2 * (int64_t)n_new, h->stream));
  s = decode_call(h, dev_prompt, n_prompt, n_new, dev_tokens_out, nullptr, nullptr, h->h_bell, h->h_bell + 8, ticks,
                  n_new);
  if (s != OFA_OK) return s;
  // ring for each token and wait until it is out (each wait bounded)
  using clk = std::chrono::steady_clock;
  bool timed_out = false;
  for (int k = 0; k < n_new && !timed_out; ++k) {
    const auto t0 = clk::now();
    std::atomic_thread_fence(std::memory_order_seq_cst);
    *bell = (uint64_t)(k + 1);
    std::atomic_thread_fence(std::memory_order_seq_cst);
    while (*prog < (uint64_t)(k + 1)) {
      if (clk::now() - t0 > std::chrono::seconds(10)) {
        timed_out = true;
        break;
      }
    }
    if (host_ring_to_token_us) host_ring_to_token_us[k] = std::chrono::duration<double, std::micro>(clk::now() - t0).count();
  }
  if (timed_out) *bell = (uint64_t)n_new;   // release every remaining wait
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  if (timed_out) return fail(h, OFA_E_TIMEOUT, "a doorbell token did not come back within 10 s");
  if (dev_wake_to_token_us) {
    std::vector<uint64_t> t(2 * (size_t)n_new);
    HIP_TRY(h, hipMemcpy(t.data(), ticks, t.size() * 8, hipMemcpyDeviceToHost));
    for (int k = 0; k < n_new; ++k) dev_wake_to_token_us[k] = (double)(t[2 * k + 1] - t[2 * k]) * 0.01;   // 100 MHz
  }
  return OFA_OK;
}

ofa_status ofa_train_and_serve(ofa_handle* h, const int32_t* dev_tokens, int32_t n_steps, float* dev_losses,
                               const int32_t* dev_prompt, int32_t n_prompt, int32_t* dev_tokens_out,
                               uint64_t* dev_versions_out, int32_t ring_len, uint64_t* dev_n_generated) {
  if (!h || !dev_tokens || !dev_losses || n_steps < 1 || !dev_prompt || !dev_tokens_out || ring_len < 1)
    return fail(h, OFA_E_ARG, "bad arguments");
  const ofa_config& c = h->cfg;
  if (c.train_cus <= 0 || c.serve_cus <= 0) return fail(h, OFA_E_STATE, "configuration has no CU partition");
  if (c.exec_mode != OFA_EXEC_PERSISTENT) return fail(h, OFA_E_STATE, "co-resident mode needs the persistent executor");
  if (n_steps > kMaxSteps) return fail(h, OFA_E_ARG, "n_steps %d > %d", n_steps, kMaxSteps);
  const Dims& D = h->D;
  if (n_prompt < 1 || n_prompt > D.win) return fail(h, OFA_E_ARG, "prompt length %d invalid", n_prompt);
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  s = staging_ready(h);
  if (s != OFA_OK) return s;
  char* ws = h->ws;
  const Carve& w = h->cw;
  // training schedule
  const int64_t per = D.B * (D.T + 1);
  for (int i = 0; i < n_steps; ++i) {
    StepCtx& sc = h->h_steps[i];
    memset(&sc, 0, sizeof sc);
    const uint64_t t = h->steps_done + i + 1;
    sc.tokens = dev_tokens + per * i;
    sc.loss_out = dev_losses + i;
    sc.lr = (float)lr_at(c, t - 1);
    sc.bc1 = (float)(1.0 - std::pow((double)c.beta1, (double)t));
    sc.bc2 = (float)(1.0 - std::pow((double)c.beta2, (double)t));
    sc.step_in_call = i;
    // co-resident configurations: the tag is the weight version the step publishes
    sc.tag = h->cw.n_slots > 1 ? h->version + i + 1 : t;
  }
  // decode: one restart period = the prompt reloaded, then restart_every tokens
  const int per_gen = c.restart_every > 0 ? c.restart_every : 512;
  h->dec_ctx_len = n_prompt;
  h->dec_processed = 0;
  int64_t period = 0;
  if (!dec_schedule(h, per_gen, 4, &period)) return fail(h, OFA_E_ARG, "restart period too long");
  h->dec_started = false;   // the co-resident context is not continued by later decode calls
  StepCtx* d_steps = at<StepCtx>(ws, w.steps);
  StepCtx* d_dsteps = at<StepCtx>(ws, w.dsteps);
  s = upload(h, d_steps, h->h_steps, sizeof(StepCtx) * n_steps);
  if (s != OFA_OK) return s;
  s = upload(h, d_dsteps, h->h_dsteps, sizeof(StepCtx) * period);
  if (s != OFA_OK) return s;
  DecIO io{dev_tokens_out, dev_versions_out, nullptr, dev_n_generated, (int64_t)ring_len};
  memcpy(h->h_misc + kMiscDecIO, &io, sizeof io);
  s = upload(h, ws + w.misc + kMiscDecIO, h->h_misc + kMiscDecIO, sizeof io);
  if (s != OFA_OK) return s;
  s = mark_upload(h);
  if (s != OFA_OK) return s;
  HIP_TRY(h, hipMemcpyAsync(ws + w.dprompt, dev_prompt, (size_t)n_prompt * 4, hipMemcpyDeviceToDevice, h->stream));
  // decoder state: prompt length, serving on, version = the newest published
  DecState* st = at<DecState>(ws, w.dstate);
  HIP_TRY(h, launch_fill_u32((uint32_t*)&st->prompt_len, (uint32_t)n_prompt, 1, h->stream));
  HIP_TRY(h, launch_fill_u32((uint32_t*)&st->serving, 1, 1, h->stream));
  HIP_TRY(h, launch_fill_u64(&st->version, h->version, 1, h->stream));
  if (dev_n_generated) HIP_TRY(h, launch_fill_u64(dev_n_generated, 0, 1, h->stream));
  const int occ = persistent_occupancy(1);
  if (occ < 1) return fail(h, OFA_E_HIP, "persistent kernel does not fit a CU");
  PhaseTime* tm = at<PhaseTime>(ws, w.times);
  PhaseTime* dtm = at<PhaseTime>(ws, w.dtimes);
  HIP_TRY(h, launch_fill_pairs((uint64_t*)tm, ~0ull, 0ull, (int64_t)h->train.size(), h->stream));
  HIP_TRY(h, launch_fill_pairs((uint64_t*)dtm, ~0ull, 0ull, (int64_t)h->dec.size(), h->stream));
  s = reset_sched(h, w.sched, (int)h->train.size());
  if (s != OFA_OK) return s;
  s = reset_sched(h, w.dsched, (int)h->dec.size());
  if (s != OFA_OK) return s;
  PersistJob jobs[2];
  // job 0: decode on the serve workgroups, open-ended, stopped by training's end
  jobs[0] = make_job(h, h->dec, h->d_dec, d_dsteps, (int64_t)1 << 40, w.dsched, dtm, nullptr, c.serve_cus * occ,
                     true);
  jobs[0].period = period;
  jobs[0].gen_per_period = per_gen;
  jobs[0].open_ended = 1;
  // job 1: the n_steps training steps on the train workgroups
  jobs[1] = make_job(h, h->train, h->d_train, d_steps, n_steps, w.sched, tm, at<uint64_t>(ws, w.inst_end),
                     c.train_cus * occ);
  jobs[1].raise_stop = &at<Sched>(ws, w.dsched)->stop;
  HIP_TRY(h, launch_fill_u64(jobs[1].inst_end, 0, n_steps, h->stream));
  { ofa_status rs = record(h, h->ev_t0); if (rs != OFA_OK) return rs; }
  s = launch_jobs(h, jobs, 2);
  if (s != OFA_OK) return s;
  { ofa_status rs = record(h, h->ev_t1); if (rs != OFA_OK) return rs; }
  HIP_TRY(h, launch_fill_u32((uint32_t*)&st->serving, 0, 1, h->stream));
  h->timed = h->ev_t0 != nullptr;
  h->steps_done += n_steps;
  h->version += n_steps;   // every step published its weights
  h->unpublished = false;
  return OFA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- SHA-256 (FIPS 180-4)

namespace {

// The hash's constants are the first 32 bits of the fractional parts of the
// square roots (initial state, first 8 primes) and cube roots (round
// constants, first 64 primes) of the primes, FIPS 180-4 sections 4.2.2 and
// 5.3.3; they are derived here rather than tabulated.
struct Sha256Consts {
  uint32_t k[64], h0[8];
  Sha256Consts() {
    int primes[64], n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d) prime = prime && c % d;
      if (prime) primes[n++] = c;
    }
    auto frac32 = [](long double x) { return (uint32_t)((x - std::floor(x)) * 4294967296.0L); };
    for (int i = 0; i < 64; ++i) k[i] = frac32(std::cbrt((long double)primes[i]));
    for (int i = 0; i < 8; ++i) h0[i] = frac32(std::sqrt((long double)primes[i]));
  }
};

struct Sha256 {
  uint32_t st[8];
  uint8_t buf[64];
  size_t fill = 0;
  uint64_t total = 0;
  static const Sha256Consts& K() {
    static const Sha256Consts c;
    return c;
  }
  Sha256() { memcpy(st, K().h0, sizeof st); }
  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
  void block(const uint8_t* p) {
    uint32_t w[64];
    for (int i = 0; i < 16; ++i) w[i] = (uint32_t)p[4 * i] << 24 | (uint32_t)p[4 * i + 1] << 16 | (uint32_t)p[4 * i + 2] << 8 | p[4 * i + 3];
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = st[0], b = st[1], c = st[2], d = st[3], e = st[4], f = st[5], g = st[6], hh = st[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t t1 = hh + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + K().k[i] + w[i];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
    }
    st[0] += a; st[1] += b; st[2] += c; st[3] += d; st[4] += e; st[5] += f; st[6] += g; st[7] += hh;
  }
  void update(const void* data, size_t n) {
    const uint8_t* p = (const uint8_t*)data;
    total += n;
    while (n) {
      if (fill == 0 && n >= 64) {   // whole blocks straight from the input
        block(p);
        p += 64;
        n -= 64;
        continue;
      }
      const size_t take = std::min(n, 64 - fill);
      memcpy(buf + fill, p, take);
      fill += take;
      p += take;
      n -= take;
      if (fill == 64) {
        block(buf);
        fill = 0;
      }
    }
  }
  void final(uint8_t out[32]) {
    const uint64_t bits = total * 8;
    const uint8_t one = 0x80, zero = 0;
    update(&one, 1);
    while (fill != 56) update(&zero, 1);
    uint8_t len[8];
    for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(bits >> (56 - 8 * i));
    update(len, 8);
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(st[i] >> (24 - 8 * j));
  }
};

// Checkpoint blob: this header, then the fp32 master weights, the AdamW first
// and second moments (ofa_param_count scalars each).
constexpr char kCkptMagic[8] = {'O', 'F', 'A', 'C', 'K', 'P', 'T', '1'};
static_assert(sizeof(ofa_checkpoint_header) == 256, "checkpoint header size");

// SHA-256 over the values that define the model and its optimizer (the state
// a checkpoint holds is only meaningful for these)
void model_fingerprint(const ofa_config& c, uint8_t out[32]) {
  const int32_t iv[] = {c.n_layer, c.d_model, c.n_head, c.d_ff, c.vocab, c.n_pos, c.mlp_gated, c.tied_head,
                        c.has_bias, c.precision, c.lr_schedule, c.total_steps};
  const float fv[] = {c.lr, c.beta1, c.beta2, c.eps, c.weight_decay};
  Sha256 sh;
  sh.update(iv, sizeof iv);
  sh.update(fv, sizeof fv);
  sh.final(out);
}

// SHA-256 of n bytes of device memory (the stream is synchronised first)
ofa_status sha256_device(ofa_handle* h, const void* dev, size_t n, uint8_t out[32]) {
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  std::vector<uint8_t> host(std::min<size_t>(n, (size_t)64 << 20));
  Sha256 sh;
  for (size_t off = 0; off < n; off += host.size()) {
    const size_t len = std::min(host.size(), n - off);
    HIP_TRY(h, hipMemcpy(host.data(), (const char*)dev + off, len, hipMemcpyDeviceToHost));
    sh.update(host.data(), len);
  }
  sh.final(out);
  return OFA_OK;
}

}  // namespace

extern "C" {

constexpr int kCeilingPasses = 8;   // passes over the buffer per timed launch

ofa_status ofa_read_ceiling(int32_t n_wg, const void* dev_buf, int64_t bytes, uint32_t* dev_sink, int32_t reps,
                            double* gbps_out, double* best_us_out) {
  if (n_wg <= 0 || !dev_buf || !dev_sink || bytes <= 0 || reps <= 0 || !gbps_out) return OFA_E_ARG;
  const int64_t per = bytes / n_wg / kDecTileHost * kDecTileHost;   // whole tiles per workgroup
  if (per < kDecTileHost) return OFA_E_ARG;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return OFA_E_HIP;
  }
  ofa_status st = OFA_OK;
  float best = -1.f;
  for (int r = 0; r <= reps && st == OFA_OK; ++r) {   // the first launch warms up
    if (hipEventRecord(e0, 0) != hipSuccess || launch_read_ceiling(dev_buf, per, kCeilingPasses, n_wg, dev_sink, 0) != hipSuccess ||
        hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
      st = OFA_E_HIP;
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) st = OFA_E_HIP;
    else if (r > 0 && (best < 0.f || ms < best)) best = ms;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != OFA_OK) return st;
  *gbps_out = (double)per * n_wg * kCeilingPasses / (best * 1e-3) / 1e9;
  if (best_us_out) *best_us_out = best * 1e3;
  return OFA_OK;
}

ofa_status ofa_sha256(const void* host_data, size_t n, uint8_t* out32) {
  if ((!host_data && n) || !out32) return OFA_E_ARG;
  Sha256 sh;
  sh.update(host_data, n);
  sh.final(out32);
  return OFA_OK;
}

size_t ofa_checkpoint_bytes(const ofa_config* cfg) {
  const int64_t P = ofa_param_count(cfg);
  return P < 0 ? 0 : sizeof(ofa_checkpoint_header) + 3 * (size_t)P * 4;
}

ofa_status ofa_checkpoint_save(ofa_handle* h, void* dev_ckpt, const uint8_t* note32, uint8_t* sha256_out) {
  if (!h || !dev_ckpt) return fail(h, OFA_E_ARG, "bad arguments");
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  // allowed after a device error too: the state can be read back for inspection
  ofa_status s = staging_ready(h);
  if (s != OFA_OK) return s;
  ofa_checkpoint_header hd;
  memset(&hd, 0, sizeof hd);
  memcpy(hd.magic, kCkptMagic, 8);
  hd.n_params = (uint64_t)h->D.P;
  hd.steps_done = h->steps_done;
  hd.version = h->version;
  model_fingerprint(h->cfg, hd.model_sha256);
  memcpy(hd.parent_sha256, h->lineage, 32);
  if (note32) memcpy(hd.note, note32, 32);
  static_assert(sizeof hd <= kMiscDecIO, "staging");
  memcpy(h->h_misc, &hd, sizeof hd);
  char* dst = (char*)dev_ckpt;
  s = upload(h, dst, h->h_misc, sizeof hd);
  if (s != OFA_OK) return s;
  s = mark_upload(h);
  if (s != OFA_OK) return s;
  const size_t pb = (size_t)h->D.P * 4;
  const size_t src[3] = {h->cw.p, h->cw.m, h->cw.v};
  for (int i = 0; i < 3; ++i)
    HIP_TRY(h, hipMemcpyAsync(dst + sizeof hd + i * pb, h->ws + src[i], pb, hipMemcpyDeviceToDevice, h->stream));
  uint8_t sha[32];
  s = sha256_device(h, dst, sizeof hd + 3 * pb, sha);
  if (s != OFA_OK) return s;
  memcpy(h->lineage, sha, 32);
  if (sha256_out) memcpy(sha256_out, sha, 32);
  return OFA_OK;
}

ofa_status ofa_checkpoint_load(ofa_handle* h, const void* dev_ckpt, uint8_t* sha256_out) {
  if (!h || !dev_ckpt) return fail(h, OFA_E_ARG, "bad arguments");
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  ofa_checkpoint_header hd;
  HIP_TRY(h, hipMemcpy(&hd, dev_ckpt, sizeof hd, hipMemcpyDeviceToHost));
  uint8_t fp[32];
  model_fingerprint(h->cfg, fp);
  if (memcmp(hd.magic, kCkptMagic, 8)) return fail(h, OFA_E_ARG, "not a checkpoint of this library");
  if (hd.n_params != (uint64_t)h->D.P) return fail(h, OFA_E_ARG, "checkpoint holds %llu parameters, model has %lld",
                                                   (unsigned long long)hd.n_params, (long long)h->D.P);
  if (memcmp(hd.model_sha256, fp, 32)) return fail(h, OFA_E_ARG, "checkpoint of another model or optimizer configuration");
  const size_t pb = (size_t)h->D.P * 4;
  uint8_t sha[32];
  s = sha256_device(h, dev_ckpt, sizeof hd + 3 * pb, sha);
  if (s != OFA_OK) return s;
  const char* src = (const char*)dev_ckpt + sizeof hd;
  const size_t dst[3] = {h->cw.p, h->cw.m, h->cw.v};
  for (int i = 0; i < 3; ++i)
    HIP_TRY(h, hipMemcpyAsync(h->ws + dst[i], src + i * pb, pb, hipMemcpyDeviceToDevice, h->stream));
  h->steps_done = hd.steps_done;
  s = ofa_set_params(h, at<float>(h->ws, h->cw.p));   // the compute copy
  if (s != OFA_OK) return s;
  h->version = hd.version;
  s = publish(h);
  if (s != OFA_OK) return s;
  h->unpublished = false;
  memcpy(h->lineage, sha, 32);
  if (sha256_out) memcpy(sha256_out, sha, 32);
  return OFA_OK;
}

ofa_status ofa_evaluate(ofa_handle* h, const int32_t* dev_tokens, int32_t n_batches, float* dev_losses,
                        float* dev_row_losses, const int32_t* dev_probe_rows, int32_t n_probe,
                        int32_t* dev_probe_argmax, float* dev_probe_entropy) {
  if (!h || !dev_tokens || !dev_losses || n_batches < 1 || n_probe < 0 || (n_probe && !dev_probe_rows))
    return fail(h, OFA_E_ARG, "bad arguments");
  if (n_batches > kMaxSteps) return fail(h, OFA_E_ARG, "n_batches %d > %d", n_batches, kMaxSteps);
  if (n_probe > kMaxProbe) return fail(h, OFA_E_ARG, "n_probe %d > %d", n_probe, kMaxProbe);
  ofa_status s = check_sticky(h);
  if (s != OFA_OK) return s;
  s = staging_ready(h);
  if (s != OFA_OK) return s;
  const int64_t per = h->D.B * (h->D.T + 1), BT = h->D.BT;
  for (int i = 0; i < n_batches; ++i) {
    StepCtx& sc = h->h_steps[i];
    memset(&sc, 0, sizeof sc);
    sc.tokens = dev_tokens + per * i;
    sc.loss_out = dev_losses + i;
    sc.step_in_call = i;
    sc.rows_out = dev_row_losses ? dev_row_losses + BT * i : nullptr;
    sc.n_probe = n_probe;
    sc.probe_rows = n_probe ? dev_probe_rows : nullptr;
    sc.probe_argmax = dev_probe_argmax ? dev_probe_argmax + (int64_t)n_probe * i : nullptr;
    sc.probe_entropy = dev_probe_entropy ? dev_probe_entropy + (int64_t)n_probe * i : nullptr;
  }
  StepCtx* d_steps = at<StepCtx>(h->ws, h->cw.steps);
  s = upload(h, d_steps, h->h_steps, sizeof(StepCtx) * n_batches);
  if (s != OFA_OK) return s;
  s = mark_upload(h);
  if (s != OFA_OK) return s;
  { ofa_status rs = record(h, h->ev_t0); if (rs != OFA_OK) return rs; }
  if (h->cfg.exec_mode == OFA_EXEC_LAUNCH_PER_PHASE) {
    s = run_launch_per_phase(h, h->eval, h->dp_eval.ph, d_steps, n_batches, 0, false, nullptr);
  } else {
    const int cus = h->cfg.train_cus > 0 ? h->cfg.train_cus : h->n_cu;
    s = run_persistent(h, h->eval, h->dp_eval.ph, d_steps, n_batches, h->cw.sched, nullptr, nullptr, cus,
                       h->train_occ);
  }
  if (s != OFA_OK) return s;
  { ofa_status rs = record(h, h->ev_t1); if (rs != OFA_OK) return rs; }
  h->timed = h->ev_t0 != nullptr;
  return OFA_OK;
}

// The AdamW ranges of the training program cover every parameter once, and
// each runs after every phase of its step that writes its gradients or reads
// its master weights or compute copy (through the dependencies, transitively).
// Phases touch parameters through the pointer fields listed here; a pointer
// into a buffer names the element it starts at, and a tensor never straddles
// two ranges.  Empty string when it holds.
static std::string audit_adam(const ofa_handle* h) {
  const std::vector<Phase>& prog = h->train;
  const int np = (int)prog.size();
  const int64_t P = h->D.P;
  const char* pb = h->ws + h->cw.p;
  const char* gb = h->ws + h->cw.g;
  const char* wb = h->ws + h->cw.wc;
  const int64_t wes = h->cw.wc == h->cw.p ? 4 : h->D.lp;   // compute-copy element size
  // ancestors through the dependencies of the same instance
  std::vector<std::vector<char>> anc(np, std::vector<char>(np, 0));
  for (int i = 0; i < np; ++i)
    for (int d = 0; d < kMaxDeps; ++d) {
      const int q = prog[i].dep[d];
      if (q == -2) {
        for (int j = 0; j < i; ++j) anc[i][j] = 1;
      } else if (q >= 0) {
        anc[i][q] = 1;
        for (int j = 0; j < np; ++j) anc[i][j] |= anc[q][j];
      }
    }
  // parameter element a pointer starts at (-1: none)
  auto elem = [&](const void* ptr) -> int64_t {
    const char* c = (const char*)ptr;
    if (!c) return -1;
    if (c >= pb && c < pb + P * 4) return (c - pb) / 4;
    if (c >= gb && c < gb + P * 4) return (c - gb) / 4;
    if (c >= wb && c < wb + P * wes) return (c - wb) / wes;
    return -1;
  };
  auto touched = [&](const Phase& ph) {
    std::vector<int64_t> e;
    auto add = [&](const void* q) {
      const int64_t x = elem(q);
      if (x >= 0) e.push_back(x);
    };
    switch (ph.op) {
      case OP_GEMM: add(ph.a.gemm.A); add(ph.a.gemm.B); add(ph.a.gemm.C); add(ph.a.gemm.bias); break;
      case OP_LN_FWD: add(ph.a.lnf.g); add(ph.a.lnf.b); add(ph.a.lnf.kb); break;
      case OP_LN_BWD: add(ph.a.lnb.g); break;
      case OP_COLRED: for (int k = 0; k < 3; ++k) add(ph.a.cr.out[k]); break;
      case OP_EMBED: add(ph.a.emb.wte); add(ph.a.emb.wpe); break;
      case OP_EMB_BWD: add(ph.a.ebwd.dwte); add(ph.a.ebwd.dwpe); break;
      case OP_CE: add(ph.a.ce.w); break;
      default: break;
    }
    return e;
  };
  std::vector<std::pair<int64_t, int64_t>> cover;
  for (int r = 0; r < np; ++r) {
    if (prog[r].op != OP_ADAMW) continue;
    const int64_t lo = elem(prog[r].a.adam.p), hi = lo + prog[r].a.adam.n;
    if (lo < 0) return "an AdamW range starts outside the parameters (phase " + std::to_string(r) + ")";
    cover.push_back({lo, hi});
    for (int q = 0; q < np; ++q) {
      if (q == r || prog[q].op == OP_ADAMW) continue;
      for (int64_t x : touched(prog[q]))
        if (x >= lo && x < hi && !anc[r][q])
          return "AdamW phase " + std::to_string(r) + " [" + std::to_string(lo) + ", " + std::to_string(hi) +
                 ") does not wait for phase " + std::to_string(q) + ", which touches element " + std::to_string(x);
    }
  }
  std::sort(cover.begin(), cover.end());
  int64_t at_ = 0;
  for (auto& rg : cover) {
    if (rg.first != at_) return "the AdamW ranges leave a gap or overlap at element " + std::to_string(at_);
    at_ = rg.second;
  }
  if (at_ != P) return "the AdamW ranges end at " + std::to_string(at_) + " of " + std::to_string(P);
  return "";
}

ofa_status ofa_sched_selftest(const ofa_config* cfg, int32_t program, int32_t n_workers, int32_t n_cu, int64_t n_inst,
                              uint64_t counter_base, int32_t per_die, uint64_t seed, char* msg, size_t msg_len) {
  auto say = [&](const std::string& m) {
    if (msg && msg_len) {
      strncpy(msg, m.c_str(), msg_len - 1);
      msg[msg_len - 1] = 0;
    }
  };
  if (!cfg || n_workers < kMaxParts || n_cu < 1 || n_inst < 1 || program < 0 || program > 1) {
    say("bad arguments");
    return OFA_E_ARG;
  }
  std::string e = validate(*cfg);
  if (!e.empty()) {
    say(e);
    return OFA_E_ARG;
  }
  // the programs of a handle over a workspace that is never touched
  ofa_handle hh;
  ofa_handle* h = &hh;
  h->host_model = true;
  h->cfg = *cfg;
  h->lay = make_layout(*cfg);
  h->D = dims_of(*cfg, h->lay);
  h->cw = carve(*cfg, h->lay);
  h->ws = (char*)(uintptr_t)0x100000000ull;   // addresses only: nothing dereferences them
  h->n_cu = n_cu;
  h->serve_wgs = n_cu;
  build_train(h);
  build_eval(h);
  if (program == 0) {
    const std::string a = audit_adam(h);
    if (!a.empty()) {
      say(a);
      return OFA_E_STATE;
    }
  }
  const std::vector<Phase>& prog = program == 0 ? h->train : h->eval;
  const int np = (int)prog.size();
  const int P = kMaxParts;
  const std::vector<int32_t> ptb = part_table(prog, P), ptiles = part_tile_table(prog, P);
  // the scheduler block, as on the device: 64-bit counters starting at the base
  std::vector<std::atomic<uint64_t>> part_ticket(P), done(np), part_done((size_t)np * P);
  for (auto& c : part_ticket) c = counter_base;
  for (auto& c : done) c = counter_base;
  for (auto& c : part_done) c = counter_base;
  // shadow state: tiles of (instance, phase) finished, tickets claimed
  std::vector<std::atomic<int32_t>> finished((size_t)n_inst * np), claimed((size_t)n_inst * (prog.back().ticket_base + prog.back().n_tickets));
  for (auto& c : finished) c = 0;
  for (auto& c : claimed) c = 0;
  std::atomic<int> failed{0};
  std::string fail_msg;
  std::atomic<bool> msg_taken{false};
  auto bad = [&](const std::string& m) {
    if (!msg_taken.exchange(true)) fail_msg = m;
    failed = 1;
  };
  const auto deadline = std::chrono::steady_clock::now() + std::chrono::seconds(120);
  auto worker = [&](int b) {
    std::mt19937_64 rng(seed * 1000003u + (uint64_t)b);
    const int part = b % P;
    const int32_t* tb = ptb.data() + part * (np + 1);
    const int tpi = tb[np];
    const uint64_t total = (uint64_t)n_inst * (uint64_t)tpi;
    int pi = 0;
    for (;;) {
      if (failed) return;
      const uint64_t t = part_ticket[part].fetch_add(1) - counter_base;
      if (t >= total) return;
      const int64_t inst = (int64_t)(t / (uint64_t)tpi);
      const int r = (int)(t % (uint64_t)tpi);
      if (tb[pi] > r) pi = 0;
      while (pi + 1 < np && tb[pi + 1] <= r) ++pi;
      const Phase& ph = prog[pi];
      const int j = (r - tb[pi]) * P + part;
      const int tile0 = j * ph.per_ticket, tile1 = std::min(tile0 + ph.per_ticket, ph.n_tiles);
      if (j >= ph.n_tickets || tile0 >= tile1) {
        bad("ticket maps outside its phase: phase " + std::to_string(pi) + " ticket " + std::to_string(j));
        return;
      }
      claimed[(size_t)inst * (prog.back().ticket_base + prog.back().n_tickets) + ph.ticket_base + j]++;
      // dependencies: completion counters reach base + (instance + 1) * tiles
      auto need = [&](int q, int64_t i) {
        const uint64_t want = counter_base + (uint64_t)(i + 1) * (uint64_t)prog[q].n_tiles;
        while (done[q].load(std::memory_order_acquire) < want) {
          if (failed) return false;
          if (std::chrono::steady_clock::now() > deadline) {
            bad("wait timed out: phase " + std::to_string(pi) + " waits on " + std::to_string(q));
            return false;
          }
          std::this_thread::yield();
        }
        if (finished[(size_t)i * np + q].load() != prog[q].n_tiles) {
          bad("counter complete before every tile finished: phase " + std::to_string(q));
          return false;
        }
        return true;
      };
      bool ok = true;
      for (int d = 0; d < kMaxDeps && ok; ++d) {
        const int q = ph.dep[d];
        if (q == -2)
          for (int qq = 0; qq < pi && ok; ++qq) ok = need(qq, inst);
        else if (q >= 0)
          ok = need(q, inst);
      }
      if (ok && ph.dep_prev >= 0 && inst > 0) ok = need(ph.dep_prev, inst - 1);
      if (!ok) return;
      const uint64_t n = (uint64_t)(tile1 - tile0);
      if (per_die == 2) done[pi].fetch_add(n, std::memory_order_release);   // injected error: count, then work
      if (rng() % 4 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
      finished[(size_t)inst * np + pi] += tile1 - tile0;   // the work
      if (per_die == 2) continue;
      if (per_die) {
        const uint64_t share = (uint64_t)ptiles[part * np + pi];
        const uint64_t prev = part_done[(size_t)pi * P + part].fetch_add(n);
        if (prev + n - counter_base == (uint64_t)(inst + 1) * share) done[pi].fetch_add(share, std::memory_order_release);
      } else {
        done[pi].fetch_add(n, std::memory_order_release);
      }
    }
  };
  std::vector<std::thread> th;
  for (int b = 0; b < n_workers; ++b) th.emplace_back(worker, b);
  for (auto& x : th) x.join();
  if (failed) {
    say(fail_msg);
    return OFA_E_STATE;
  }
  const int tps = prog.back().ticket_base + prog.back().n_tickets;
  for (int64_t i = 0; i < n_inst; ++i) {
    for (int q = 0; q < np; ++q)
      if (finished[(size_t)i * np + q] != prog[q].n_tiles) {
        say("instance " + std::to_string(i) + " phase " + std::to_string(q) + " ran " +
            std::to_string(finished[(size_t)i * np + q].load()) + " of " + std::to_string(prog[q].n_tiles) + " tiles");
        return OFA_E_STATE;
      }
    for (int k = 0; k < tps; ++k)
      if (claimed[(size_t)i * tps + k] != 1) {
        say("ticket " + std::to_string(k) + " of instance " + std::to_string(i) + " claimed " +
            std::to_string(claimed[(size_t)i * tps + k].load()) + " times");
        return OFA_E_STATE;
      }
  }
  for (int q = 0; q < np; ++q)
    if (done[q] != counter_base + (uint64_t)n_inst * prog[q].n_tiles) {
      say("phase " + std::to_string(q) + " counter ends at the wrong value");
      return OFA_E_STATE;
    }
  say("ok: " + std::to_string(np) + " phases, " + std::to_string(tps) + " tickets per instance");
  return OFA_OK;
}

ofa_status ofa_status_sync(ofa_handle* h, ofa_stats* out) {
  if (!h) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  DevStatus ds;
  HIP_TRY(h, hipMemcpy(&ds, h->ws + h->cw.status, sizeof ds, hipMemcpyDeviceToHost));
  float ms = 0.f;
  if (h->timed) {
    if (hipEventElapsedTime(&ms, h->ev_t0, h->ev_t1) == hipSuccess) h->last_ms = ms;
    (void)hipGetLastError();
  }
  if (ds.code && !h->sticky) {
    h->sticky = ds.code;
    h->err = std::string("device status: ") + ofa_status_string((ofa_status)ds.code) +
             " (phase " + std::to_string(ds.phase) + ", step " + std::to_string(ds.step) + ", info " +
             std::to_string(ds.info) + ")";
  }
  if (out) {
    memset(out, 0, sizeof *out);
    out->status = ds.code;
    out->err_phase = ds.code ? ds.phase : -1;
    out->err_step = ds.step;
    out->err_info = ds.info;
    uint64_t pt[kMaxParts * kPartStride];
    HIP_TRY(h, hipMemcpy(pt, h->ws + h->cw.sched + offsetof(Sched, part_ticket), sizeof pt, hipMemcpyDeviceToHost));
    out->tickets_claimed = 0;
    for (int i = 0; i < kMaxParts; ++i) out->tickets_claimed += pt[i * kPartStride] - h->cfg.debug_counter_base;
    out->steps_done = h->steps_done;
    out->version = h->version;
    out->last_call_ms = h->last_ms;
    out->n_phases = (int32_t)h->train.size();
    out->n_tiles_step = h->train.back().tile_base + h->train.back().n_tiles;
    out->grid = h->last_grid;
    out->n_tickets_step = h->train.back().ticket_base + h->train.back().n_tickets;
  }
  return ds.code ? (ofa_status)ds.code : OFA_OK;
}

static ofa_status phase_times_of(ofa_handle* h, const std::vector<std::string>& nm, size_t off, uint64_t* host_t,
                                 int32_t n, int32_t* n_out, char* names, size_t name_stride) {
  if (!h || !host_t || !n_out) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  int np = std::min<int>(n, (int)nm.size());
  HIP_TRY(h, hipMemcpy(host_t, h->ws + off, np * sizeof(PhaseTime), hipMemcpyDeviceToHost));
  if (names && name_stride)
    for (int i = 0; i < np; ++i) {
      strncpy(names + i * name_stride, nm[i].c_str(), name_stride - 1);
      names[i * name_stride + name_stride - 1] = 0;
    }
  *n_out = np;
  return OFA_OK;
}

ofa_status ofa_phase_times(ofa_handle* h, uint64_t* host_t, int32_t n, int32_t* n_out, char* names,
                           size_t name_stride) {
  if (!h) return OFA_E_ARG;
  return phase_times_of(h, h->train_names, h->cw.times, host_t, n, n_out, names, name_stride);
}

ofa_status ofa_trace(ofa_handle* h, int32_t decode, uint64_t* host_t, int64_t n, int64_t* n_out, int32_t* n_phases) {
  if (!h || !host_t || !n_out || !n_phases) return OFA_E_ARG;
  if (!h->ws) return fail(h, OFA_E_STATE, "the handle was destroyed");
  if (!(h->cfg.debug_flags & OFA_DEBUG_TRACE)) return fail(h, OFA_E_STATE, "tracing is off in this configuration");
  if (!h->trace_n_phases || h->trace_dec != (decode != 0)) return fail(h, OFA_E_STATE, "no traced call of that kind");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  const int64_t quads = std::min<int64_t>(n / 2, h->trace_n_inst * h->trace_n_phases);
  HIP_TRY(h, hipMemcpy(host_t, h->ws + h->cw.trace, quads * 32, hipMemcpyDeviceToHost));
  for (int64_t i = 0; i < quads; ++i) host_t[4 * i] = ~host_t[4 * i];   // stored complemented
  *n_out = quads;
  *n_phases = h->trace_n_phases;
  return OFA_OK;
}

ofa_status ofa_decode_phase_times(ofa_handle* h, uint64_t* host_t, int32_t n, int32_t* n_out, char* names,
                                  size_t name_stride) {
  if (!h) return OFA_E_ARG;
  return phase_times_of(h, h->dec_names, h->cw.dtimes, host_t, n, n_out, names, name_stride);
}

}  // extern "C"
