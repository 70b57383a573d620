// ofa_kernels.hip -- the two executors of a phase table.
//
// 1. launch per phase: phase_kernel<OP> runs every tile of one phase; stream
//    order supplies the dependencies.  Used for debugging and per-kernel
//    profiles.
// 2. persistent: one cooperative launch; every workgroup loops claiming 64-bit
//    tickets from its partition's counter (one partition per die when the job
//    has eight or more workgroups; partition s owns every eighth ticket of a
//    phase).  Tickets name (instance, phase, tiles) in program order, and a
//    partition's tickets are claimed in order, so the lowest unfinished phase
//    always has its tickets held by running workgroups or claimable: the loop
//    cannot deadlock.  A finished tile is published with a release, then an
//    increment of its phase's completion counter (with partitions, the last
//    workgroup of a die to finish its share writes that die's L2 back once and
//    adds the share); a dependent tile acquire-reads the counters it needs.
//    This is the claim / fence-then-count / acquire-wait scheme of "How one
//    persistent kernel runs three jobs" (review page, section of the same
//    name), with every counter 64-bit after the 32-bit budget overflow
//    described on the A100 reproduction page ("A longer run exposed a
//    scheduler overflow").
#include <hip/hip_runtime.h>

#include "k_simple.h"
#include "k_mfma.h"
#include "k_attn.h"
#include "k_decode.h"
#include "ofa_launch.h"

namespace ofa {

// ---------------------------------------------------------------- dispatch

// decode attention reached through the generic dispatch (launch-per-phase
// executor, or the training kernel's switch): out of line, so its registers
// stay out of the callers' allocation
__device__ __noinline__ void task_dec_attn_call(const DecAttnArgs* ap, int tile, const StepCtx* sc, char* smem) {
  task_dec_attn(ap, tile, sc, smem);
}

// Each task receives a by-value copy of its argument block, read once when the
// task starts: arguments read through the phase-table reference inside the
// tasks' loops would be reloaded on every iteration (the compiler cannot rule
// out that the loop's stores change them), and every such reload waits for all
// outstanding memory operations, the streaming copies included.
#define OFA_ARGS(FIELD) const auto a = ph.a.FIELD
template <int OP, int OCC = 1>
__device__ __forceinline__ void run_task(const Phase& ph, int tile, const TaskCtx& tc, char* smem) {
  if constexpr (OP == OP_EMBED) { OFA_ARGS(emb); task_embed(a, tile, tc); }
  else if constexpr (OP == OP_LN_FWD) {
    OFA_ARGS(lnf);
    if (a.kp) task_ln_fwd<2, true>(a, tile);
    else task_ln_fwd<4, false>(a, tile);
  }
  else if constexpr (OP == OP_GEMM) {
    OFA_ARGS(gemm);
    if (a.impl == GEMM_P3) task_gemm_p3<OCC>(a, tile, smem);
    else task_gemm_simple(a, tile, smem);
  }
  else if constexpr (OP == OP_ROPE) { OFA_ARGS(rope); task_rope(a, tile, false); }
  else if constexpr (OP == OP_ATTN_FWD) {
    OFA_ARGS(attn);
    if (a.impl == 1) task_attn_fwd_mfma(a, tile, smem);
    else task_attn_fwd_simple(a, tile, smem);
  }
  else if constexpr (OP == OP_GEGLU_FWD) { OFA_ARGS(geglu); task_geglu_fwd(a, tile); }
  else if constexpr (OP == OP_CE) { OFA_ARGS(ce); task_ce<OCC>(a, tile, tc, smem); }
  else if constexpr (OP == OP_LOSS) { OFA_ARGS(loss); task_loss(a, tc, smem); }
  else if constexpr (OP == OP_LN_BWD) { OFA_ARGS(lnb); task_ln_bwd<OCC == 1 ? 4 : 2>(a, tile, smem); }
  else if constexpr (OP == OP_COLSUM) { OFA_ARGS(cs); task_colsum(a, tile, smem); }
  else if constexpr (OP == OP_COLRED) { OFA_ARGS(cr); task_colred(a, tile, smem); }
  else if constexpr (OP == OP_ATTN_PREP) { OFA_ARGS(attn); task_attn_prep(a, tile); }
  else if constexpr (OP == OP_ATTN_BWD_KV) {
    OFA_ARGS(attn);
    if (a.impl == 1) task_attn_bwd_kv_mfma(a, tile, smem);
    else task_attn_bwd_kv_simple(a, tile, smem);
  }
  else if constexpr (OP == OP_ATTN_BWD_Q) {
    OFA_ARGS(attn);
    if (a.impl == 1) task_attn_bwd_q_mfma(a, tile, smem);
    else task_attn_bwd_q_simple(a, tile, smem);
  }
  else if constexpr (OP == OP_ROPE_BWD) { OFA_ARGS(rope); task_rope(a, tile, true); }
  else if constexpr (OP == OP_EMB_SORT) { OFA_ARGS(esort); task_emb_sort(a, tc, smem); }
  else if constexpr (OP == OP_EMB_BWD) { OFA_ARGS(ebwd); task_emb_bwd(a, tile, tc); }
  else if constexpr (OP == OP_ADAMW) { OFA_ARGS(adam); task_adamw(a, tile, tc); }
  else if constexpr (OP == OP_COPY) { OFA_ARGS(copy); task_copy(a, tile); }
  else if constexpr (OP == OP_DEC_EMBED) { OFA_ARGS(dembed); task_dec_embed(a, tile, tc); }
  // the decode GEMV and attention read their arguments through a scalar view of the phase table
  else if constexpr (OP == OP_DEC_GEMV) { task_dec_gemv(&ph.a.dgemv, tile, tc.sc, smem); }
  else if constexpr (OP == OP_DEC_ATTN) { task_dec_attn_call(&ph.a.dattn, tile, tc.sc, smem); }
  else if constexpr (OP == OP_DEC_ARGMAX) { OFA_ARGS(dargmax); task_dec_argmax(a, tile, tc, smem); }
  else if constexpr (OP == OP_SLOT_GUARD) { OFA_ARGS(guard); task_slot_guard(a, tc); }
  else if constexpr (OP == OP_PUBLISH) { OFA_ARGS(publish); task_publish(a, tc); }
  else if constexpr (OP == OP_PROBE) { OFA_ARGS(probe); task_probe(a, tile, tc, smem); }
}
#undef OFA_ARGS

template <int OCC>
__device__ __noinline__ void run_any(const Phase& ph, int tile, const TaskCtx& tc, char* smem) {
  switch (ph.op) {
#define OFA_CASE(X) case X: run_task<X, OCC>(ph, tile, tc, smem); break;
    OFA_CASE(OP_EMBED) OFA_CASE(OP_LN_FWD) OFA_CASE(OP_GEMM) OFA_CASE(OP_ROPE)
    OFA_CASE(OP_ATTN_FWD) OFA_CASE(OP_GEGLU_FWD) OFA_CASE(OP_CE) OFA_CASE(OP_LOSS)
    OFA_CASE(OP_LN_BWD) OFA_CASE(OP_COLSUM) OFA_CASE(OP_COLRED) OFA_CASE(OP_ATTN_PREP)
    OFA_CASE(OP_ATTN_BWD_KV) OFA_CASE(OP_ATTN_BWD_Q) OFA_CASE(OP_ROPE_BWD) OFA_CASE(OP_EMB_SORT)
    OFA_CASE(OP_EMB_BWD) OFA_CASE(OP_ADAMW) OFA_CASE(OP_COPY) OFA_CASE(OP_DEC_EMBED)
    OFA_CASE(OP_DEC_ATTN) OFA_CASE(OP_DEC_ARGMAX) OFA_CASE(OP_SLOT_GUARD) OFA_CASE(OP_PUBLISH)
    OFA_CASE(OP_PROBE)
    // OP_DEC_GEMV runs through run_dec_gemv (whole tickets, prefetched); keeping it
    // out of this switch keeps its registers out of every other task's call
#undef OFA_CASE
    default: break;
  }
}

// one non-inlined function per form, so the one-sequence form keeps its own
// register allocation
// ap and sc are addresses in the phase and step tables (read through scalar
// views).  The one-sequence GEMV and the attention are inlined into the
// decode kernel: a call saves and restores the callee-saved registers through
// scratch memory on every ticket, stores that the per-phase L2 write-back
// then carries to HBM.  The batch GEMV stays a call (about 150 MB of such
// writes per position at eight sequences): inlined as well, its registers
// slow the one-sequence path by 7% and the batch path by 3%.
__device__ __forceinline__ void run_dec_gemv1(const DecGemvArgs* ap, int t0, int t1, const StepCtx* sc, char* smem,
                                              int npre) {
  task_dec_gemv_range_t<false>(ap, t0, t1, sc, smem, npre);
}
__device__ __noinline__ void run_dec_gemvN(const DecGemvArgs* ap, int t0, int t1, const StepCtx* sc, char* smem,
                                           int npre) {
  task_dec_gemv_range_t<true>(ap, t0, t1, sc, smem, npre);
}
__device__ __forceinline__ void run_dec_attn(const DecAttnArgs* ap, int tile, const StepCtx* sc, char* smem) {
  task_dec_attn(ap, tile, sc, smem);
}

__device__ __noinline__ int prefetch_dec_gemv(const DecGemvArgs* ap, int t0, int t1, char* smem, bool allowed) {
  return dec_gemv_prefetch(ap, t0, t1, smem, allowed);
}

// ---------------------------------------------------------------- executor 1: one launch per phase

template <int OP>
__global__ __launch_bounds__(kThreads) void phase_kernel(const Phase* phases, int idx, const StepCtx* sc,
                                                         DevStatus* status, PhaseTime* times, int64_t step) {
  extern __shared__ __align__(16) char smem[];
  const Phase& ph = phases[idx];
  TaskCtx tc{sc, status, idx, step, 0};
  const uint64_t t0 = now_ticks();
  if constexpr (OP == OP_DEC_GEMV) {
    // one workgroup per ticket, as the persistent executor hands them out
    for (int t = blockIdx.x; t < ph.n_tickets; t += gridDim.x) {
      if (ph.a.dgemv.nseq > 1) task_dec_gemv_range_t<true>(&ph.a.dgemv, t * ph.per_ticket, min((t + 1) * ph.per_ticket, ph.n_tiles), sc, smem, 0);
      else task_dec_gemv_range_t<false>(&ph.a.dgemv, t * ph.per_ticket, min((t + 1) * ph.per_ticket, ph.n_tiles), sc, smem, 0);
    }
  } else {
    for (int tile = blockIdx.x; tile < ph.n_tiles; tile += gridDim.x) run_task<OP>(ph, tile, tc, smem);
  }
  if (times && threadIdx.x == 0) {
    atomicMin((unsigned long long*)&times[idx].t0, (unsigned long long)t0);
    atomicMax((unsigned long long*)&times[idx].t1, (unsigned long long)now_ticks());
  }
}

// one kernel per GEMM implementation, so each gets its own register budget
template <int IMPL>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const Phase* phases, int idx, PhaseTime* times) {
  extern __shared__ __align__(16) char smem[];
  const Phase& ph = phases[idx];
  const uint64_t t0 = now_ticks();
  const GemmArgs g = ph.a.gemm;   // by value: see OFA_ARGS
  // one tile per workgroup (the grid is the tile count): a loop around the
  // tile lets the compiler hoist every layout variant's addressing out of it,
  // which spills
  const int tile = g.xcd ? xcd_block(blockIdx.x, ph.n_tiles) : (int)blockIdx.x;
  if (tile < ph.n_tiles) {
    if constexpr (IMPL == GEMM_P3) task_gemm_p3(g, tile, smem);
    else task_gemm_simple(g, tile, smem);
  }
  if (times && threadIdx.x == 0) {
    atomicMin((unsigned long long*)&times[idx].t0, (unsigned long long)t0);
    atomicMax((unsigned long long*)&times[idx].t1, (unsigned long long)now_ticks());
  }
}

// ---------------------------------------------------------------- executor 2: persistent

// Polls a completion counter with relaxed loads (the caller issues one
// acquire fence once every wait has succeeded).  Gives up when the scheduler
// aborts, when the watchdog deadline passes (an error) or, in an open-ended
// job, when the instance lies past the job's stopping point (not an error).
__device__ __forceinline__ bool wait_count(const uint64_t* ctr, uint64_t need, const PersistParams& p,
                                           const PersistJob& J, const TaskCtx& tc) {
  if (ld_relaxed(ctr) >= need) return true;
  const uint64_t start = now_ticks();
  for (int spins = 0;; ++spins) {
    // the counter and the stop words are read together: one memory round trip per poll
    const uint64_t c = ld_relaxed(ctr);
    const uint64_t ab = ld_relaxed(p.abort);
    const uint64_t lim = J.open_ended ? ld_relaxed(&J.sched->limit) : ~0ull;
    if (c >= need) return true;
    if (ab) return false;
    if (lim <= (uint64_t)tc.step) return false;
    __builtin_amdgcn_s_sleep(1);
    if ((spins & 63) == 63 && now_ticks() - start > p.watchdog_ticks) {
      raise_status(p.status, -4 /*OFA_E_TIMEOUT*/, tc.phase, tc.step, (int64_t)need);
      st_release(p.abort, 1);
      return false;
    }
  }
}

// OCC: workgroups per CU the launch is built for.  OCC 2 (training only: two
// workgroups share a CU's LDS and registers, so one's MFMAs run while the
// other waits on memory) leaves out the decode tasks.
template <int OCC>
__global__ __launch_bounds__(kThreads, OCC) void persistent_kernel(PersistParams p) {
  extern __shared__ __align__(16) char smem[];
  __shared__ uint64_t s_ticket;
  __shared__ int s_ok;
  __shared__ int s_pre;
  __shared__ int s_stop;              // this workgroup saw the stop word of its open-ended job
  // instance s_all_inst: phases [0, s_all_upto) this workgroup saw complete
  __shared__ int64_t s_all_inst;
  __shared__ int32_t s_all_upto;
  // The phases' first tickets, and per phase the latest instance this
  // workgroup has seen complete (with an acquire at the time): a ticket whose
  // dependencies are all known complete neither polls the counters nor
  // repeats the acquire.
  __shared__ int32_t s_tb[kMaxPhases];
  __shared__ int64_t s_known[kMaxPhases];
  const int ji = (p.n_jobs > 1 && (int)blockIdx.x >= p.job[0].n_wg) ? 1 : 0;
  const PersistJob& J = p.job[ji];
  const uint64_t base = J.sched->base;
  // this workgroup's ticket partition: its counter, and its first ticket of each phase
  const int part = (int)(blockIdx.x % (unsigned)J.n_parts);
  uint64_t* part_ctr = &J.sched->part_ticket[part * kPartStride];
  const int32_t* ptb = J.part_tb + part * (J.n_phases + 1);
  const int tpi = ptb[J.n_phases];   // this partition's tickets per instance
  const uint64_t total = (uint64_t)J.n_inst * (uint64_t)tpi;
  if (threadIdx.x == 0) {
    s_all_inst = -1;
    s_all_upto = 0;
    s_stop = 0;
    // the once-per-die release relies on partition == die; a workgroup elsewhere stops the run
    if (J.die_release && xcc_id() != (uint32_t)part) {
      raise_status(p.status, -2 /*OFA_E_HIP*/, -1, 0, (int64_t)xcc_id());
      st_release(p.abort, 1);
    }
  }
  for (int i = threadIdx.x; i < J.n_phases; i += kThreads) {
    s_tb[i] = ptb[i];
    s_known[i] = -1;
  }
  __syncthreads();
  int pi = 0;   // phase of the previous ticket (tickets only grow, so the search starts there)
  for (;;) {
    if (threadIdx.x == 0) s_ticket = add_relaxed(part_ctr, 1) - base;
    __syncthreads();
    // wave-uniform copy, so the phase table is read with scalar loads
    const uint64_t t = readfirstlane_u64(s_ticket);
    if (t >= total) break;
    const int64_t inst = (int64_t)(t / (uint64_t)tpi);
    const int r = (int)(t % (uint64_t)tpi);
    // phase owning the partition's ticket r: last phase whose first ticket
    // <= r (a phase with fewer tickets than partitions may have none here)
    if (s_tb[pi] > r) pi = 0;   // a later instance starts over
    while (pi + 1 < J.n_phases && s_tb[pi + 1] <= r) ++pi;
    const Phase& ph = J.phases[pi];
    const int j = (r - s_tb[pi]) * J.n_parts + part;   // the phase's ticket
    int tile0 = j * ph.per_ticket;
    const int tile1 = min(tile0 + ph.per_ticket, ph.n_tiles);
    const int64_t period_idx = inst / J.period;
    TaskCtx tc{J.steps + (inst - period_idx * J.period), p.status, pi, inst, period_idx * J.gen_per_period};
    // a decode GEMV starts streaming its weights before its dependencies are
    // met; with two weight slots only once this token's version is known
    int npre = 0;
    if (OCC == 1 && ph.op == OP_DEC_GEMV) {
      const DecGemvArgs& a = ph.a.dgemv;
      bool allow = !(a.epi == DEPI_LOGITS && !(tc.sc->head & 1));
      if (allow && a.pre_dep >= 0) {
        if (threadIdx.x == 0) {
          const bool seen = ld_relaxed(&J.sched->done[a.pre_dep]) >=
                            base + (uint64_t)(inst + 1) * J.phases[a.pre_dep].n_tiles;
          if (seen) fence_acquire_agent();
          s_pre = seen ? 1 : 0;
        }
        __syncthreads();
        allow = __builtin_amdgcn_readfirstlane(s_pre) != 0;
      }
      if constexpr (OCC == 1) npre = prefetch_dec_gemv(&ph.a.dgemv, tile0, tile1, smem, allow);
    }
    // An open-ended job stops at an instance boundary once the other job has
    // finished: the workgroup holding an instance's first ticket checks the
    // stop word (in the second wave, beside thread 0's dependency wait); if it
    // is raised the instance becomes the limit (a minimum over such holders) and
    // is not started.  Every instance below the final limit runs whole: the
    // limit only decreases and its holders saw no stop.  Tickets of instances at
    // or past it find their dependencies unmet and leave their wait on the limit.
    if (J.open_ended && r == 0 && threadIdx.x == kWave && ld_relaxed(&J.sched->stop)) {
      atomicMin((unsigned long long*)&J.sched->limit, (unsigned long long)inst);
      s_stop = 1;
    }
    // An "every earlier phase" dependency: wave 0 first reads the counters of
    // 64 phases per round trip and records those already complete (each lane
    // that saw one then takes the acquire itself), so that thread 0 waits only
    // for the rest instead of polling every phase in turn.
    // (Training launches only: in the one-workgroup-per-CU kernel, which runs
    // decode, the extra code on every ticket cost batch-1 decode 1.7%.)
    bool all_dep = false;
    if constexpr (OCC == 2)
      for (int d = 0; d < kMaxDeps; ++d) all_dep |= ph.dep[d] == -2;
    if (all_dep && threadIdx.x < kWave) {
      const int from = s_all_inst == inst ? s_all_upto : 0;
      bool seen = false;
      for (int q0 = from; q0 < pi; q0 += kWave) {
        const int q = q0 + (int)threadIdx.x;
        if (q < pi && s_known[q] < inst &&
            ld_relaxed(&J.sched->done[q]) >= base + (uint64_t)(inst + 1) * J.phases[q].n_tiles) {
          s_known[q] = inst;
          seen = true;
        }
      }
      if (seen) fence_acquire_agent();
    }
    // wait for the dependencies (thread 0), then one acquire for the workgroup
    if (threadIdx.x == 0) {
      bool ok = true, fresh = false;
      // phase q complete for instance i (i >= 0)
      auto need = [&](int q, int64_t i) {
        if (s_known[q] >= i) return true;
        fresh = true;
        const bool done = wait_count(&J.sched->done[q], base + (uint64_t)(i + 1) * J.phases[q].n_tiles, p, J, tc);
        if (done) s_known[q] = i;
        return done;
      };
      for (int d = 0; d < kMaxDeps && ok; ++d) {
        const int q = ph.dep[d];
        if (q == -2) {
          if (s_all_inst != inst) {
            s_all_inst = inst;
            s_all_upto = 0;
          }
          for (int qq = s_all_upto; qq < pi && ok; ++qq) ok = need(qq, inst);
          if (ok && s_all_upto < pi) s_all_upto = pi;
        } else if (q >= 0) {
          ok = need(q, inst);
        }
      }
      if (ok && ph.dep_prev >= 0 && inst > 0) ok = need(ph.dep_prev, inst - 1);
      if (ok && fresh) fence_acquire_agent();
      s_ok = ok ? 1 : 0;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_ok) || __builtin_amdgcn_readfirstlane(s_stop)) {
      if (npre) vm_wait_barrier(0);   // no copy may land in LDS after the exit
      break;
    }
    const uint64_t t0 = now_ticks();
    if (J.trace && inst < J.trace_inst && threadIdx.x == 0) {
      // word 0 keeps the complement of the earliest start, so every word starts at 0 and takes a maximum
      atomicMax((unsigned long long*)&J.trace[4 * (inst * J.n_phases + pi)], ~(unsigned long long)t0);
      atomicMax((unsigned long long*)&J.trace[4 * (inst * J.n_phases + pi) + 1], (unsigned long long)t0);
    }
    bool gemv = false;
    if constexpr (OCC == 1) {
      if (ph.op == OP_DEC_GEMV) {
        if (ph.a.dgemv.nseq > 1) run_dec_gemvN(&ph.a.dgemv, tile0, tile1, tc.sc, smem, npre);
        else run_dec_gemv1(&ph.a.dgemv, tile0, tile1, tc.sc, smem, npre);
        gemv = true;
      }
    }
    if (!gemv) for (int tile = tile0; tile < tile1; ++tile) {
      int tl = tile;
      if (p.shuffle && ph.n_tiles > 1) {
        // reversal after a rotation: a permutation of the phase's tiles
        const int rot = (int)(((uint64_t)inst * 977u + 31u) % (uint64_t)ph.n_tiles);
        tl = ph.n_tiles - 1 - (tile + rot) % ph.n_tiles;
      }
      if constexpr (OCC == 1) {
        if (ph.op == OP_DEC_ATTN) {
          run_dec_attn(&ph.a.dattn, tl, tc.sc, smem);
        } else {
          // run_any takes the context by reference, so it lives in scratch
          // memory for the call; built here, the decode tickets that make no
          // call (the GEMVs and attention) write none
          const TaskCtx tcc = tc;
          run_any<OCC>(ph, tl, tcc, smem);
        }
      } else {
        run_any<OCC>(ph, tl, tc, smem);
      }
    }
    // publish: an agent-scope release fence (per ticket, or once per die and
    // phase) makes the tile's stores visible before the counter moves.  With
    // the once-per-die release every wave first waits until its own stores are
    // complete in the die's L2 (vmcnt counts a store until the L2 has taken
    // it); the barrier then puts all of them before thread 0's counter add.
    if (J.die_release) asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      if (J.trace && inst < J.trace_inst)
        atomicMax((unsigned long long*)&J.trace[4 * (inst * J.n_phases + pi) + 2], (unsigned long long)now_ticks());
      if (J.die_release) {
        // Every workgroup of the die had its stores in the die's L2 before its
        // add; the add that completes the die's share of the phase comes after
        // all of them, so one write-back of that L2 (the agent-scope release)
        // by that workgroup covers the whole share.
        fence_release_workgroup();
        const uint64_t share = (uint64_t)J.part_tiles[part * J.n_phases + pi];
        const uint64_t prev = add_relaxed(&J.sched->part_done[pi * kMaxParts + part], (uint64_t)(tile1 - tile0));
        if (prev + (uint64_t)(tile1 - tile0) - base == (uint64_t)(inst + 1) * share) {
          fence_release_agent();
          add_relaxed(&J.sched->done[pi], share);
        }
      } else {
        fence_release_agent();
        add_relaxed(&J.sched->done[pi], (uint64_t)(tile1 - tile0));
      }
      if (J.times) {
        atomicMin((unsigned long long*)&J.times[pi].t0, (unsigned long long)t0);
        atomicMax((unsigned long long*)&J.times[pi].t1, (unsigned long long)now_ticks());
      }
      if (J.inst_end) atomicMax((unsigned long long*)&J.inst_end[inst], (unsigned long long)now_ticks());
      if (J.trace && inst < J.trace_inst)
        atomicMax((unsigned long long*)&J.trace[4 * (inst * J.n_phases + pi) + 3], (unsigned long long)now_ticks());
    }
  }
  if (threadIdx.x == 0) {
    // the last workgroup of a job to leave raises the other job's stop word
    if (add_relaxed(&J.sched->exited, 1) + 1 == (uint64_t)J.n_wg && J.raise_stop) st_release(J.raise_stop, 1);
  }
}

// ---------------------------------------------------------------- static workspace

// The workspace of handles made by ofa_create_static: one array per device,
// held until the process ends.  Host code never uses the array's name as an
// address (on the host it is a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept here.
static __device__ __align__(256) char scratch[kStaticScratchBytes];
static void* g_scratch_ptr[kStaticMaxDevices];

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kStaticMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------- small utility kernels

// out[b] = the die (XCD) workgroup b runs on
__global__ void xcc_probe_kernel(uint32_t* out, int n) {
  if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = xcc_id();
}

__global__ void fill_u64_kernel(uint64_t* p, uint64_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void fill_pairs_kernel(uint64_t* p, uint64_t a, uint64_t b, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    p[2 * i] = a;
    p[2 * i + 1] = b;
  }
}

// ---------------------------------------------------------------- streaming-read ceiling

// The read ceiling of the decode GEMV's weight stream: workgroup b copies its
// share of the buffer (`per_wg` bytes, whole 24 KB tiles, from b * per_wg)
// `passes` times into a four-tile LDS ring exactly as the GEMV streams a
// ticket's weights (waves 1..3 issue eight 1 KB direct-to-LDS copies per tile,
// a tile's buffer refilled once every wave is past it); repeated passes over
// the same bytes are what decode does token after token, and they make the
// launch long against its own start-up.  Wave 0 folds one word of every tile
// into `sink` so the copies cannot be dropped.
__global__ __launch_bounds__(kThreads) void read_ceiling_kernel(const char* buf, int64_t per_wg, int passes,
                                                                uint32_t* sink) {
  extern __shared__ __align__(16) char ring[];
  const char* src = buf + (int64_t)blockIdx.x * per_wg;
  const int per = (int)(per_wg / kDecTile);
  const int nt = per * passes;   // tile t is tile t % per of the share
  const int nb = min(4, nt);
  uint32_t acc = 0;
  for (int i = 0; i < nb; ++i) dec_copy_n<kDecCopies>(src + (int64_t)(i % per) * kDecTile, kDecTile, ring + i * kDecTile);
  int issued = nb;
  for (int i = 0; i < nt; ++i) {
    dec_wait_tile(issued - i - 1);
    if (threadIdx.x == 0) acc += *(const uint32_t*)(ring + (i % 4) * kDecTile + (i & 255) * 16);
    if (i >= 1 && issued < nt) {   // refill the buffer tile i - 1 used (every wave is past it)
      dec_copy_n<kDecCopies>(src + (int64_t)(issued % per) * kDecTile, kDecTile, ring + (issued % 4) * kDecTile);
      ++issued;
    }
  }
  vm_wait_barrier(0);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

hipError_t launch_read_ceiling(const void* buf, int64_t per_wg, int passes, int n_wg, uint32_t* sink, hipStream_t s) {
  const int lds = 4 * kDecTile;
  hipError_t e = hipFuncSetAttribute((const void*)read_ceiling_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(n_wg), dim3(kThreads), lds, s, (const char*)buf, per_wg, passes, sink);
  return hipGetLastError();
}

// ---------------------------------------------------------------- host side

static size_t lds_for(const Phase& ph) {
  switch (ph.op) {
    case OP_GEMM:
      return ph.a.gemm.impl == GEMM_P3 ? gemm_p3_lds_bytes() : sizeof(GemmSmemSimple);
    case OP_LN_BWD: return (size_t)kWaves * 3 * ph.a.lnb.d * sizeof(float);
    case OP_ATTN_FWD:
      return ph.a.attn.impl == 1 ? attn_mfma_lds_bytes() : (size_t)kWaves * (64 + ph.a.attn.T) * sizeof(float);
    case OP_ATTN_BWD_KV:
      return ph.a.attn.impl == 1 ? attn_mfma_lds_bytes() : (size_t)kWaves * 256 * sizeof(float);
    case OP_ATTN_BWD_Q:
      return ph.a.attn.impl == 1 ? attn_mfma_lds_bytes() : (size_t)kWaves * 192 * sizeof(float);
    case OP_CE: return ph.a.ce.fused ? (size_t)(16 + ph.a.ce.n_stats) * sizeof(float) : 64;
    case OP_LOSS: return 64;
    case OP_COLRED: return 16 * 16 * sizeof(float);
    case OP_COLSUM: return (size_t)kWaves * kCsCols * sizeof(float);
    case OP_EMB_SORT: {
      int n = 1;
      while (n < ph.a.esort.BT) n <<= 1;
      return (size_t)n * sizeof(uint64_t);
    }
    case OP_DEC_GEMV: return dec_gemv_lds_bytes(ph.a.dgemv);
    case OP_DEC_ATTN: return dec_attn_lds_bytes(ph.a.dattn);
    case OP_DEC_ARGMAX: return 2048;
    case OP_PROBE: return 256;
    default: return 0;
  }
}

size_t phase_lds_bytes(const Phase& ph) { return lds_for(ph); }

// LDS a phase needs in the persistent kernel built for occ workgroups per CU
// (the matrix-core GEMM tile keeps a two-slice ring there)
size_t phase_lds_bytes_occ(const Phase& ph, int occ) {
  if (occ == 2 && ph.op == OP_GEMM && ph.a.gemm.impl == GEMM_P3) return gemm_p3_lds_bytes_occ2();
  return lds_for(ph);
}

// Dynamic LDS: every phase fits 64 KB.  The pipelined GEMM uses exactly
// 64 KB, which together with the kernels' own static LDS needs the raised
// per-kernel limit; without it that GEMM is not used.
static size_t g_lds_limit = 60 * 1024;
static size_t g_persist_lds = 60 * 1024;
static size_t g_persist_lds2 = 0;   // OCC 2 kernel: half of a CU's LDS (0: not available)
static bool g_p3_ok = false;
size_t persistent_lds_bytes(int occ) { return occ == 2 ? g_persist_lds2 : g_persist_lds; }
bool gemm_p3_available() { return g_p3_ok; }

// Dynamic LDS of the persistent kernel (and of the kernels whose phases need
// more than the default): as much of the CU's LDS as one workgroup may hold,
// at least the pipelined GEMM's ring.  The persistent kernel runs one
// workgroup per CU in any case (registers), so the LDS is otherwise idle.
hipError_t init_kernels() {
  int dev = 0, max_blk = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    max_blk = 64 * 1024;
  (void)hipGetLastError();
  hipFuncAttributes fa;
  size_t stat = 2048;
  if (hipFuncGetAttributes(&fa, (const void*)persistent_kernel<1>) == hipSuccess) stat = fa.sharedSizeBytes;
  (void)hipGetLastError();
  size_t want = max_blk > (int)stat ? ((size_t)max_blk - stat) / 1024 * 1024 : 0;
  if (want < gemm_p3_lds_bytes()) return hipSuccess;   // pipelined GEMM unavailable; small tiles only
  const void* big[] = {(const void*)gemm_kernel<GEMM_P3>, (const void*)persistent_kernel<1>,
                       (const void*)phase_kernel<OP_DEC_GEMV>};
  bool ok = true;
  for (const void* f : big)
    ok = ok && hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)want) == hipSuccess;
  (void)hipGetLastError();
  if (ok) {
    g_p3_ok = true;
    g_lds_limit = want;
    g_persist_lds = want;
  }
  // the two-per-CU kernel: half of the CU's LDS, less its own static LDS
  size_t stat2 = stat;
  if (hipFuncGetAttributes(&fa, (const void*)persistent_kernel<2>) == hipSuccess) stat2 = fa.sharedSizeBytes;
  (void)hipGetLastError();
  const size_t half = (size_t)max_blk / 2;
  const size_t want2 = half > stat2 ? (half - stat2) / 1024 * 1024 : 0;
  if (ok && want2 >= gemm_p3_lds_bytes_occ2() &&
      hipFuncSetAttribute((const void*)persistent_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)want2) ==
          hipSuccess)
    g_persist_lds2 = want2;
  (void)hipGetLastError();
  return hipSuccess;
}

size_t lds_limit_bytes() { return g_lds_limit; }

int persistent_occupancy(int occ) {
  int n = 0;
  if (occ == 2 && g_persist_lds2 == 0) return 0;
  const hipError_t e = occ == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, persistent_kernel<2>, kThreads,
                                                                              g_persist_lds2)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, persistent_kernel<1>, kThreads,
                                                                              g_persist_lds);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

hipError_t launch_phase(const Phase& h, const Phase* d_phases, int idx, const StepCtx* d_sc, DevStatus* st,
                        PhaseTime* tm, int64_t step, hipStream_t s) {
  // a join phase has no work: in stream order its dependencies already hold
  if (h.n_tiles <= 0 || h.op == OP_NOP) return hipSuccess;
  (void)hipGetLastError();   // report this launch's error, not a stale one
  const int grid = h.op == OP_DEC_GEMV ? h.n_tickets : h.n_tiles;
  const size_t lds = lds_for(h);
  if (h.op == OP_GEMM) {
    if (h.a.gemm.impl == GEMM_P3)
      hipLaunchKernelGGL(gemm_kernel<GEMM_P3>, dim3(grid), dim3(kThreads), lds, s, d_phases, idx, tm);
    else
      hipLaunchKernelGGL(gemm_kernel<GEMM_SIMPLE>, dim3(grid), dim3(kThreads), lds, s, d_phases, idx, tm);
    return hipGetLastError();
  }
  switch (h.op) {
#define OFA_LAUNCH(X) \
  case X: hipLaunchKernelGGL(phase_kernel<X>, dim3(grid), dim3(kThreads), lds, s, d_phases, idx, d_sc, st, tm, step); break;
    OFA_LAUNCH(OP_EMBED) OFA_LAUNCH(OP_LN_FWD) OFA_LAUNCH(OP_GEMM) OFA_LAUNCH(OP_ROPE)
    OFA_LAUNCH(OP_ATTN_FWD) OFA_LAUNCH(OP_GEGLU_FWD) OFA_LAUNCH(OP_CE) OFA_LAUNCH(OP_LOSS)
    OFA_LAUNCH(OP_LN_BWD) OFA_LAUNCH(OP_COLSUM) OFA_LAUNCH(OP_COLRED) OFA_LAUNCH(OP_ATTN_PREP)
    OFA_LAUNCH(OP_ATTN_BWD_KV) OFA_LAUNCH(OP_ATTN_BWD_Q) OFA_LAUNCH(OP_ROPE_BWD) OFA_LAUNCH(OP_EMB_SORT)
    OFA_LAUNCH(OP_EMB_BWD) OFA_LAUNCH(OP_ADAMW) OFA_LAUNCH(OP_COPY) OFA_LAUNCH(OP_DEC_EMBED)
    OFA_LAUNCH(OP_DEC_GEMV) OFA_LAUNCH(OP_DEC_ATTN) OFA_LAUNCH(OP_DEC_ARGMAX) OFA_LAUNCH(OP_SLOT_GUARD)
    OFA_LAUNCH(OP_PUBLISH) OFA_LAUNCH(OP_PROBE)
#undef OFA_LAUNCH
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Cooperative launches: every workgroup is resident at once, and (measured)
// workgroup b runs on die b % 8.  A plain launch of the same kernel did not keep
// that placement (a 32-workgroup launch put a workgroup on another die), and the
// once-per-die release depends on it.
hipError_t launch_persistent(const PersistParams& p, int grid, hipStream_t s, int occ) {
  (void)hipGetLastError();
  void* args[] = {(void*)&p};
  const void* fn = occ == 2 ? (const void*)persistent_kernel<2> : (const void*)persistent_kernel<1>;
  const size_t lds = occ == 2 ? g_persist_lds2 : g_persist_lds;
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, lds, s);
}

// the same kind of launch as the persistent kernel's
hipError_t launch_xcc_probe(uint32_t* out, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  (void)hipGetLastError();
  void* args[] = {(void*)&out, (void*)&n};
  return hipLaunchCooperativeKernel((const void*)xcc_probe_kernel, dim3(n), dim3(kThreads), args, 0, s);
}

hipError_t launch_fill_u64(uint64_t* p, uint64_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
  (void)hipGetLastError();
  hipLaunchKernelGGL(fill_u64_kernel, dim3(grid), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
  (void)hipGetLastError();
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_fill_pairs(uint64_t* p, uint64_t a, uint64_t b, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int grid = (int)std::min<int64_t>((n + 255) / 256, 1024);
  (void)hipGetLastError();
  hipLaunchKernelGGL(fill_pairs_kernel, dim3(grid), dim3(256), 0, s, p, a, b, n);
  return hipGetLastError();
}

}  // namespace ofa
