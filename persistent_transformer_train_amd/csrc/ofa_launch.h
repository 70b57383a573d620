// ofa_launch.h -- host-side entry points of the device code (ofa_kernels.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "ofa_types.h"

namespace ofa {

// One job of the persistent kernel: a program run instance after instance by
// its own workgroups, with its own scheduler block.
struct PersistJob {
  const Phase* phases;       // one program instance's phase table
  int32_t n_phases;
  int32_t tickets_per_inst;  // sum of n_tickets over the phases
  // Tickets are claimed per partition: workgroup b belongs to partition
  // b % n_parts (its die when n_parts is 8) and claims from that partition's
  // counter.  Partition s owns tickets s, s + n_parts, s + 2 n_parts, ... of
  // every phase; part_tb[s (n_phases + 1) + i] is the partition's first ticket
  // of phase i inside one instance, and [s (n_phases + 1) + n_phases] its
  // tickets per instance.  Every partition has at least one workgroup.
  const int32_t* part_tb;
  int32_t n_parts;
  // Release once per die and phase (n_parts == 8, partition s = die s): each
  // workgroup's stores reach its die's L2, it counts its tiles in
  // sched->part_done, and the workgroup completing the die's share
  // (part_tiles[s n_phases + i] tiles of phase i per instance) writes that
  // L2 back and moves the phase counter by the whole share.
  int32_t die_release;
  const int32_t* part_tiles;
  int64_t n_inst;            // instances to run (open-ended jobs: a bound no run reaches)
  const StepCtx* steps;      // instance i runs steps[i % period]
  int64_t period;
  int64_t gen_per_period;    // decode: tokens emitted per period
  Sched* sched;
  PhaseTime* times;          // [n_phases] (nullable)
  uint64_t* inst_end;        // [n_inst] device time each instance finished (nullable)
  uint64_t* trace;           // debug: [trace_inst][n_phases][4] (nullable)
  int64_t trace_inst;
  int32_t n_wg;              // workgroups that run this job
  int32_t open_ended;        // stops at sched->limit once sched->stop is raised
  uint64_t* raise_stop;      // when this job's last workgroup leaves, this word is raised (nullable)
};

// Everything the persistent kernel reads; passed by value.  With two jobs,
// workgroups [0, job[0].n_wg) run job 0 and the rest job 1.
struct PersistParams {
  PersistJob job[2];
  int32_t n_jobs;
  DevStatus* status;
  uint64_t* abort;           // shared stop word: any error stops every job
  uint64_t watchdog_ticks;   // a wait longer than this raises OFA_E_TIMEOUT
  int32_t shuffle;           // debug: permute tiles inside a phase
};

// The static workspace of ofa_create_static: kStaticScratchBytes of device
// memory per device, whose address static_scratch returns for the current device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;   // OFA_STATIC_WORKSPACE_BYTES
constexpr int kStaticMaxDevices = 8;
hipError_t static_scratch(void** ptr);

hipError_t init_kernels();
size_t phase_lds_bytes(const Phase& ph);   // dynamic LDS a phase needs
size_t phase_lds_bytes_occ(const Phase& ph, int occ);   // the same in the persistent kernel built for occ
size_t persistent_lds_bytes(int occ);      // dynamic LDS of the persistent kernel built for occ workgroups per CU (0: none)
size_t lds_limit_bytes();                  // dynamic LDS a per-phase kernel may use
bool gemm_p3_available();                  // the pipelined GEMM tile can be launched
int persistent_occupancy(int occ);         // workgroups per CU of the persistent kernel built for occ (1 or 2)

hipError_t launch_phase(const Phase& host_ph, const Phase* dev_phases, int idx, const StepCtx* dev_sc,
                        DevStatus* status, PhaseTime* times, int64_t step, hipStream_t s);
// one cooperative launch (every workgroup resident at once; workgroup b on die b % 8)
hipError_t launch_persistent(const PersistParams& p, int grid, hipStream_t s, int occ);
// out[b] (device, n words) = the die workgroup b of an n-workgroup launch runs on
hipError_t launch_xcc_probe(uint32_t* out, int n, hipStream_t s);
// n_wg workgroups each stream per_wg bytes (whole decode tiles) of buf through LDS, passes times
hipError_t launch_read_ceiling(const void* buf, int64_t per_wg, int passes, int n_wg, uint32_t* sink, hipStream_t s);
hipError_t launch_fill_u64(uint64_t* p, uint64_t v, int64_t n, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
// p[2i] = a, p[2i+1] = b for i < n_pairs
hipError_t launch_fill_pairs(uint64_t* p, uint64_t a, uint64_t b, int64_t n_pairs, hipStream_t s);

}  // namespace ofa
