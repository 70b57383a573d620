/*
 * ofa.h -- C ABI of libofa.so: one GPT training step (embedding, causal
 * multi-head attention, MLP, LayerNorm, softmax cross-entropy forward and
 * backward, fused AdamW) and batch-1 greedy decode that reads the live,
 * changing weights, on one AMD Instinct MI355X (gfx950).
 *
 * Pages cited below, by title:
 *  [A100]   "Open Flapping Airplanes ... A100 reproduction"
 *  [Review] "How one persistent kernel runs three jobs"
 *  [News]   "Magni engineers open-source a reproduction ...", section "What happened"
 *  [3090]   "Coppelius training on the RTX 3090"
 *
 * Memory ownership.  All device memory is the caller's.  The caller passes one
 * device workspace of ofa_workspace_bytes() bytes to ofa_create(); the library
 * carves it (model state, activations, scheduler counters, phase tables) and
 * never allocates or frees device memory.  The handle owns only host-side state
 * (the configuration, host copies of the phase tables, the error string and a
 * small pinned staging area).  The caller frees the workspace after
 * ofa_destroy().
 *
 * Synchronisation.  Every call enqueues work on the HIP stream given to
 * ofa_create() and returns without waiting, except where stated.  Device
 * results are valid once the caller has synchronised that stream.  The device
 * status block is read back by ofa_status_sync(); a non-zero device status
 * makes every later call return that status ([3090] "Channel health": every
 * invocation reports an error notifier and a status block).
 *
 * Errors.  No call throws.  Each returns an ofa_status; on failure
 * ofa_last_error(h) returns a message owned by the handle (valid until the
 * next call on that handle).  Thread safety: one handle must not be used by
 * two host threads at once.
 */
#ifndef OFA_H
#define OFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ofa_handle ofa_handle;   /* opaque, owned by the library */

/* Status codes.  [3090] "Channel health" (error notifier, status block, finite
 * loss); [A100] "A longer run exposed a scheduler overflow" (a budget that did
 * not fit its counter). */
typedef enum {
  OFA_OK = 0,
  OFA_E_ARG = -1,        /* invalid argument, configuration or input token */
  OFA_E_HIP = -2,        /* a HIP runtime call failed (code kept in the handle), or a persistent
                            workgroup ran on another die than its ticket partition assumes */
  OFA_E_NONFINITE = -3,  /* a step produced a non-finite loss */
  OFA_E_TIMEOUT = -4,    /* a device-side wait exceeded its watchdog deadline */
  OFA_E_OVERFLOW = -5,   /* a requested budget does not fit its counters */
  OFA_E_STATE = -6       /* call not valid in the handle's current state */
} ofa_status;

typedef enum { OFA_FP32 = 0, OFA_BF16 = 1 } ofa_precision;
typedef enum { OFA_LR_CONSTANT = 0, OFA_LR_COSINE = 1 } ofa_lr_schedule;
typedef enum { OFA_EXEC_PERSISTENT = 0, OFA_EXEC_LAUNCH_PER_PHASE = 1 } ofa_exec_mode;

/* Model, optimizer and execution configuration (plain values, no pointers).
 * Model shapes: [A100] "What ran" (12 layers, width 768, 12 heads, 8 x 512
 * tokens a step, AdamW) and [3090] "Run" (16 blocks, width 512, 8 heads,
 * context 1024, FFN 1408, vocabulary 12288).  CU partition: [Review] (static
 * partitions of the compute units between training and serving). */
typedef struct {
  int32_t n_layer, d_model, n_head, d_ff, vocab;
  int32_t n_pos;          /* learned position-table length; 0 = rotary positions */
  int32_t mlp_gated;      /* 1 = GELU(h Wg^T) * (h Wu^T); 0 = GELU(h W1^T + b1) */
  int32_t tied_head;      /* 1 = logits use the token-embedding table */
  int32_t has_bias;       /* 1 = every linear layer has a bias */
  int32_t batch, seq;     /* one step trains on batch x seq positions */
  int32_t precision;      /* ofa_precision */
  float lr, beta1, beta2, eps, weight_decay;
  int32_t lr_schedule;    /* ofa_lr_schedule; cosine decays to 0 at total_steps */
  int32_t total_steps;
  int32_t train_cus;      /* persistent mode: compute units given to training */
  int32_t serve_cus;      /* compute units given to decode (0 = no serve role) */
  int32_t decode_window;  /* positions held by the decode context (<= n_pos if n_pos) */
  int32_t prompt_len;     /* tokens kept when the decode context restarts */
  int32_t restart_every;  /* co-resident decode: restart from the prompt every N tokens */
  int32_t exec_mode;      /* ofa_exec_mode */
  uint64_t debug_counter_base;  /* start value of every ticket/phase counter (tests) */
  int32_t debug_flags;          /* OFA_DEBUG_* bits (tests only) */
  int32_t decode_batch;   /* sequences ofa_decode_token decodes together (0 or 1: one; at most 8) */
  int32_t reserved[6];          /* must be zero */
} ofa_config;

#define OFA_DEBUG_SHUFFLE_TICKETS 1  /* persistent mode: permute tile order inside a phase */
#define OFA_DEBUG_SHORT_WATCHDOG  2  /* device waits give up after ~1 ms instead of ~10 s */
#define OFA_DEBUG_TRACE           4  /* persistent mode: per (instance, phase) timestamps, see ofa_trace */
#define OFA_DEBUG_TILE256         8  /* every matrix-core GEMM takes the 256-row tile (normally only large ones) */
#define OFA_DEBUG_OCC1           16  /* step-mode persistent training with one workgroup per CU (default: two where they fit) */
#define OFA_DEBUG_PLAIN_TILES    32  /* GEMM tiles in plain row / column order, not placed by die (for comparison) */
#define OFA_DEBUG_WG_RELEASE     64  /* persistent launches: every workgroup writes its die's L2 back after each ticket */
#define OFA_DEBUG_CE_UNFUSED    128  /* bf16: LM head writes fp32 logits and a separate cross-entropy reads them */

/* Size in bytes of the device workspace ofa_create() needs for cfg; 0 if cfg is
 * invalid (ofa_validate_config() says why).  Host only. */
size_t ofa_workspace_bytes(const ofa_config *cfg);

/* Checks cfg without touching the GPU.  On OFA_E_ARG, writes a message into
 * msg (NUL-terminated, at most msg_len bytes) when msg is not NULL. */
ofa_status ofa_validate_config(const ofa_config *cfg, char *msg, size_t msg_len);

/* Number of parameters (fp32 scalars) of the model cfg describes, -1 if cfg is
 * invalid.  [A100] "What ran" quotes 162,417,408 for its model; this layout of
 * the same shapes (biases, gains, learned positions, untied head) has
 * 162,716,160. */
int64_t ofa_param_count(const ofa_config *cfg);

/* Canonical parameter layout: tensor i (0 <= i < ofa_param_tensor_count) starts
 * at flat offset *offset, has *numel scalars and init kind *kind
 * (0 = N(0, 0.02), 1 = zeros, 2 = ones).  name receives a NUL-terminated
 * tensor name (at most name_len bytes).  Host only. */
int32_t ofa_param_tensor_count(const ofa_config *cfg);
ofa_status ofa_param_tensor(const ofa_config *cfg, int32_t i, int64_t *offset, int64_t *numel,
                            int32_t *kind, char *name, size_t name_len);

/* Creates a handle.  [A100] "Reproduce the run": the initial weights are made
 * on the host and handed over.  dev_workspace: device pointer to ws_bytes >=
 * ofa_workspace_bytes(cfg) bytes, 256-byte aligned.  dev_init_params: device
 * pointer to ofa_param_count(cfg) fp32 scalars in canonical order; they are
 * copied (the caller may free them after the stream synchronises).
 * hip_stream: the hipStream_t all work of this handle is ordered on (NULL =
 * the default stream).  Publishes the initial weights as version 0.  Waits for
 * the stream once (phase-table upload).  OFA_E_ARG for an invalid
 * configuration, a short or misaligned workspace, or a CU split larger than
 * the device. */
ofa_status ofa_create(const ofa_config *cfg, void *dev_workspace, size_t ws_bytes,
                      const float *dev_init_params, void *hip_stream, ofa_handle **out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): ofa_create
 * with the library's own static workspace instead of the caller's.  Every
 * device the library runs on holds one static array of 64 MiB
 * (OFA_STATIC_WORKSPACE_BYTES) until the process ends, and one handle that uses
 * it: this call (re)creates that handle for the current device and returns it
 * (every call on a device returns the same handle, which then holds the new
 * model; the previous model's state is gone).  Calls on one device that
 * overlap race on the array.  A model whose ofa_workspace_bytes exceeds the
 * array is rejected with OFA_E_ARG (ofa_last_error(*out) says why).  The call
 * allocates no device memory and no pinned host memory and creates no events:
 * its staging areas are static host arrays, uploads wait for the stream, and
 * last_call_ms stays 0.  Every other call works on the handle as on one from
 * ofa_create; ofa_destroy waits for the stream and retires the handle until the
 * next ofa_create_static on its device.  The caller still owns dev_init_params
 * and every buffer it passes to later calls. */
#define OFA_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
ofa_status ofa_create_static(const ofa_config *cfg, const float *dev_init_params, void *hip_stream,
                             ofa_handle **out);

/* Runs n_steps >= 1 training steps: forward, backward and the AdamW update
 * ([A100] "What ran"), each step one pass over one batch; persistent mode runs
 * all n_steps in one kernel launch with no host launch between forward,
 * backward and update ([Review]).  dev_tokens: device int32 [n_steps][batch][seq+1];
 * step s trains inputs tokens[s][:, :seq] on targets tokens[s][:, 1:].
 * dev_losses: device fp32 [n_steps], receives each step's mean cross-entropy
 * (taken before that step's update).  Every token must lie in [0, vocab):
 * checked on the device; a bad token, or a non-finite loss, sets OFA_E_ARG /
 * OFA_E_NONFINITE in the status block, and the update of that step and of
 * every later step of the call is skipped (weights, moments and compute copy
 * keep their values).  The learning rate and bias corrections of each step
 * follow the step count kept in the handle ([A100] "Reproducibility needs
 * inputs...": the schedule is a function of the step index and the planned
 * total, not of the run length). */
ofa_status ofa_train_step(ofa_handle *h, const int32_t *dev_tokens, int32_t n_steps,
                          float *dev_losses);

/* Publication of the weights decode reads ([News] "What happened": decode
 * from live weights; [Review]: a finished phase fences its writes, then
 * releases a counter that readers acquire).  Step-mode configuration (one
 * weight slot): copies the current compute weights to the serve copy and
 * makes them version v+1; *version_out (host, may be NULL) receives it.
 * Co-resident configuration (train_cus > 0 and serve_cus > 0, two slots):
 * every training step already published its weights, so the latest version is
 * returned unchanged -- unless ofa_set_params or ofa_checkpoint_load changed the
 * weights since, in which case they are copied into slot (v+1) & 1 and become
 * version v+1. */
ofa_status ofa_publish_weights(ofa_handle *h, uint64_t *version_out);

/* Batch-1 greedy decode with the latest published weights ([A100] "What ran":
 * autoregressive generation from the changing model; [Review]: one token
 * releases the next with no host launch in between).
 * dev_prompt: device int32 [n_prompt]; n_prompt > 0 starts a new context from
 * this prompt (n_prompt <= decode_window); n_prompt == 0 continues the previous
 * context (OFA_E_STATE if there is none).  Generates n_new tokens into
 * dev_tokens_out (device int32 [n_new]).  dev_logits_out (device fp32
 * [n_new][vocab], may be NULL) receives the logits each token was chosen from.
 * dev_versions_out (device uint64 [n_new], may be NULL) receives the weight
 * version each token read (one version for all layers of a token).  Greedy:
 * the lowest token id wins exact ties.  When the context would exceed
 * decode_window positions it restarts from its most recent prompt_len tokens at
 * positions 0..prompt_len-1 (the pages give no window rule; this is the reading
 * taken). */
ofa_status ofa_decode_token(ofa_handle *h, const int32_t *dev_prompt, int32_t n_prompt,
                            int32_t n_new, int32_t *dev_tokens_out, float *dev_logits_out,
                            uint64_t *dev_versions_out);

/* Host doorbell to wake-up ([3090] "Host doorbell to wake-up": per
 * invocation, over the host-stamped submissions).  A batch-1 decode of n_new
 * (<= 4096) tokens from dev_prompt (as ofa_decode_token starts a context) in
 * which every token waits, on the device, until the host rings for it: the
 * library launches the decode, then for token k writes k + 1 into a coherent
 * pinned host word, spins until the decode's progress word (also pinned host
 * memory, written by the device at system scope) reaches k + 1, and moves on.
 * host_ring_to_token_us[k] (host, may be NULL): ring to token k seen by the host,
 * host clock; dev_wake_to_token_us[k] (host, may be NULL): the device saw the
 * ring to token k emitted, device clock.  Their difference is the doorbell's
 * trip to the device plus the progress word's trip back.  Synchronous.  Needs
 * the persistent executor and a handle from ofa_create (OFA_E_STATE
 * otherwise); a token not back within 10 s gives OFA_E_TIMEOUT (the device
 * side stops waiting after 5 s). */
ofa_status ofa_decode_doorbell(ofa_handle *h, const int32_t *dev_prompt, int32_t n_prompt, int32_t n_new,
                               int32_t *dev_tokens_out, double *host_ring_to_token_us,
                               double *dev_wake_to_token_us);

/* Co-resident mode ([A100] "What ran": training and serving share one
 * persistent kernel on static SM partitions; [Review]).  Needs train_cus > 0,
 * serve_cus > 0 and the persistent executor (else OFA_E_STATE).  One persistent
 * launch trains n_steps steps on the train partition while the serve partition
 * decodes continuously from dev_prompt (device int32 [n_prompt]), restarting
 * from it every restart_every tokens and acquiring the newest published
 * version at every token.  Generated tokens go round-robin into
 * dev_tokens_out[ring_len], their versions into dev_versions_out[ring_len]
 * (may be NULL); *dev_n_generated (device uint64, may be NULL) receives the
 * count.  Training publishes after every AdamW update; a step waits before
 * overwriting a slot the decoder still reads. */
ofa_status ofa_train_and_serve(ofa_handle *h, const int32_t *dev_tokens, int32_t n_steps,
                               float *dev_losses, const int32_t *dev_prompt, int32_t n_prompt,
                               int32_t *dev_tokens_out, uint64_t *dev_versions_out,
                               int32_t ring_len, uint64_t *dev_n_generated);

/* Forward-only evaluation on the current weights, no backward and no update
 * ([3090] "Loss": the first step of an invocation is scored on a context the
 * model has not trained on; "Per-row spread" and "Sampled rows": per-row
 * cross-entropy; "Prompt probe": the most likely next token at chosen rows;
 * "Prediction entropy": the entropy of the next-token distribution, in nats).
 * dev_tokens: device int32 [n_batches][batch][seq+1] (targets = inputs shifted
 * by one, as in training).  dev_losses: device fp32 [n_batches], the mean
 * cross-entropy of each batch.  dev_row_losses (device fp32
 * [n_batches][batch*seq], may be NULL): each row's cross-entropy.
 * dev_probe_rows: device int32 [n_probe] flat row indices b*seq + t (0 <= n_probe
 * <= 64; a row outside [0, batch*seq) sets OFA_E_ARG); for each batch and probed
 * row, dev_probe_argmax (device int32 [n_batches][n_probe], may be NULL)
 * receives the argmax token (lowest id on exact ties) and dev_probe_entropy
 * (device fp32 [n_batches][n_probe], may be NULL) the entropy of the softmax. */
ofa_status ofa_evaluate(ofa_handle *h, const int32_t *dev_tokens, int32_t n_batches, float *dev_losses,
                        float *dev_row_losses, const int32_t *dev_probe_rows, int32_t n_probe,
                        int32_t *dev_probe_argmax, float *dev_probe_entropy);

/* Checkpoint of the training state ([3090] "Checkpoint lineage": each
 * invocation resumes the checkpoint the one before wrote, and each checkpoint
 * is identified by its SHA-256; [A100] "Reproducibility needs inputs and an
 * environment record": input SHA-256 fingerprints).  A checkpoint is this
 * 256-byte header followed by the fp32 master weights, the AdamW first moments
 * and the AdamW second moments, ofa_param_count scalars each. */
typedef struct {
  char magic[8];             /* "OFACKPT1" */
  uint64_t n_params;
  uint64_t steps_done;       /* training steps taken (sets the next step's rate and bias corrections) */
  uint64_t version;          /* weight version published when the state was saved */
  uint8_t model_sha256[32];  /* SHA-256 of the model and optimizer settings the state belongs to */
  uint8_t parent_sha256[32]; /* SHA-256 of the checkpoint this state was loaded from or last saved as (zeros: none) */
  uint8_t note[32];          /* caller's 32 bytes, e.g. the SHA-256 of the inputs trained on since the parent */
  uint8_t reserved[128];
} ofa_checkpoint_header;

/* Bytes of a checkpoint of cfg's model (header + 3 * 4 * ofa_param_count); 0 if
 * cfg is invalid.  Host only. */
size_t ofa_checkpoint_bytes(const ofa_config *cfg);

/* Writes the training state into dev_ckpt (device, ofa_checkpoint_bytes bytes;
 * the caller owns it); also after a device error, to read the state back.  note32 (host, 32 bytes, may be NULL) goes into the
 * header.  Synchronises the stream and hashes the checkpoint on the host:
 * sha256_out (host, 32 bytes, may be NULL) receives its SHA-256, which also
 * becomes the parent of the next checkpoint saved from this handle. */
ofa_status ofa_checkpoint_save(ofa_handle *h, void *dev_ckpt, const uint8_t *note32, uint8_t *sha256_out);

/* Replaces the training state (weights, moments, step count, version) by the
 * checkpoint at dev_ckpt, refreshes the compute copy and publishes the loaded
 * weights under the checkpoint's version.  OFA_E_ARG if the header's magic,
 * parameter count or model fingerprint does not match this handle.
 * Synchronises the stream; sha256_out (host, may be NULL) receives the
 * checkpoint's SHA-256.  Training resumed from a checkpoint gives losses and
 * weights bit-identical to an uninterrupted run. */
ofa_status ofa_checkpoint_load(ofa_handle *h, const void *dev_ckpt, uint8_t *sha256_out);

/* Measurement helper: the streaming-read ceiling of the decode weight stream
 * on n_wg workgroups (one per CU; the pages' serving share, "Open Flapping
 * Airplanes ... A100 reproduction", "What ran", is 48 of the GPU's compute
 * units).  Workgroup b copies bytes [b s, (b + 1) s) of dev_buf through LDS
 * eight times over, exactly as a decode GEMV ticket streams its weights (decode
 * re-reads the same weights every token), s the largest whole number of 24 KB
 * tiles with n_wg s <= bytes; one word per workgroup goes to dev_sink (device,
 * n_wg uint32).  Runs on the null stream: one warm-up launch, then reps timed
 * launches; *gbps_out = 8 n_wg s / (fastest launch), and *best_us_out (may be
 * NULL) that launch's duration.  dev_buf is only read.  OFA_E_ARG for a null
 * pointer, n_wg or reps <= 0, or less than one tile per workgroup. */
ofa_status ofa_read_ceiling(int32_t n_wg, const void *dev_buf, int64_t bytes, uint32_t *dev_sink, int32_t reps,
                            double *gbps_out, double *best_us_out);

/* SHA-256 (FIPS 180-4) of n bytes of host memory into out32 (host, 32 bytes).
 * Host only; for input fingerprints and checkpoint lineage. */
ofa_status ofa_sha256(const void *host_data, size_t n, uint8_t *out32);

/* Copies the fp32 master weights to / from dev_params (device fp32
 * [ofa_param_count]).  ofa_set_params also refreshes the compute copy; in a
 * co-resident configuration the next ofa_publish_weights then publishes them. */
ofa_status ofa_get_params(ofa_handle *h, float *dev_params);
ofa_status ofa_set_params(ofa_handle *h, const float *dev_params);

/* Copies the gradient of the most recent step (device fp32 [ofa_param_count]). */
ofa_status ofa_get_grads(ofa_handle *h, float *dev_grads);

/* Statistics of the last completed call, filled on the host after a stream
 * synchronisation (this call synchronises the stream).  [3090] "Channel
 * health": the host status block; [A100] "Measured results": device time. */
typedef struct {
  int32_t status;           /* device status block: 0 or an ofa_status */
  int32_t err_phase;        /* phase index that raised it, -1 if none */
  int64_t err_step;         /* step that raised it */
  int64_t err_info;         /* extra detail (offending value) */
  uint64_t tickets_claimed; /* tickets handed out in the last persistent launch */
  uint64_t steps_done;      /* training steps completed since create (or as loaded) */
  uint64_t version;         /* latest published weight version */
  double last_call_ms;      /* device time of the last train/decode/evaluate call (hip events) */
  int32_t n_phases;         /* phases of one training step */
  int32_t n_tiles_step;     /* tiles of one training step */
  int32_t grid;             /* workgroups of the last persistent launch */
  int32_t n_tickets_step;   /* tickets of one training step (persistent executor) */
  int32_t reserved[4];
} ofa_stats;

ofa_status ofa_status_sync(ofa_handle *h, ofa_stats *out);

/* Per-phase device timestamps of the last training step run in launch-per-phase
 * or persistent mode ([3090] "Where a step's time goes": time per kernel
 * family): for phase i, t[2i] = first tile start, t[2i+1] = last tile end, in
 * device clock ticks (100 MHz).  n: capacity in pairs.  Synchronises. */
ofa_status ofa_phase_times(ofa_handle *h, uint64_t *host_t, int32_t n, int32_t *n_out,
                           char *names, size_t name_stride);

/* The same for the decode program of the last decode call (summed over its
 * positions: first tile start and last tile end of each phase). */
ofa_status ofa_decode_phase_times(ofa_handle *h, uint64_t *host_t, int32_t n, int32_t *n_out,
                                  char *names, size_t name_stride);

/* Phase trace of the last persistent call (needs OFA_DEBUG_TRACE in the config;
 * the workspace then holds the trace).  For instance i < OFA_TRACE_INSTANCES and
 * phase p of that call's program, four device times (ticks of 100 MHz) at
 * t[4(i P + p) + 0..3]: the first and the last time a workgroup started the
 * phase's work (its dependencies met), the last time one finished the work,
 * and the last time one had published it (release fence and counter update);
 * P = *n_phases.  decode != 0 selects the last decode call.  n: capacity in
 * uint64 words / 2; *n_out: entries written.  Synchronises.  ([Review]: the
 * scheduler's claim, fence and release points.) */
#define OFA_TRACE_INSTANCES 1024
ofa_status ofa_trace(ofa_handle *h, int32_t decode, uint64_t *host_t, int64_t n, int64_t *n_out,
                     int32_t *n_phases);

/* 64-bit task budget = iterations x tasks_per_unit; OFA_E_OVERFLOW if the
 * product does not fit 63 bits.  Host-only helper: the budget rule of the
 * scheduler, after [A100] "A longer run exposed a scheduler overflow" (a
 * 32-bit budget of 4,194,304 x 2,225 wrapped). */
ofa_status ofa_task_budget(uint64_t iterations, uint64_t tasks_per_unit, uint64_t *out);

/* Host-only model check of the persistent scheduler's protocol ([Review]:
 * tickets claim work, a finished phase is fenced then counted, dependents
 * acquire-read the count; [A100] "A longer run exposed a scheduler
 * overflow": counter widths).  Builds the phase tables of cfg's training
 * program (program 0) or evaluation program (program 1) for a device of n_cu
 * CUs without touching a GPU, then runs n_inst instances with n_workers host
 * threads standing in for workgroups (worker b in ticket partition b % 8):
 * 64-bit ticket claims in order per partition, waits on the completion counters
 * of each phase's dependencies, and the release either once per partition and
 * phase (per_die != 0, the share accounting of the once-per-die write-back) or
 * per ticket (per_die == 2 injects a protocol error, the count before the work,
 * which the check must catch).  Every counter starts at counter_base; seed varies the random
 * delays.  OFA_OK if every tile ran exactly once and only after all tiles of
 * its dependencies had finished, every ticket was claimed once and every
 * counter ends at base + instances x tiles; else OFA_E_STATE (or OFA_E_ARG),
 * with the reason in msg (NUL-terminated, at most msg_len bytes).  For the
 * training program it first checks that the AdamW ranges cover every parameter
 * once and that each range depends, transitively, on every phase of the step
 * that writes its gradients or reads its weights (OFA_E_STATE otherwise). */
ofa_status ofa_sched_selftest(const ofa_config *cfg, int32_t program, int32_t n_workers, int32_t n_cu,
                              int64_t n_inst, uint64_t counter_base, int32_t per_die, uint64_t seed,
                              char *msg, size_t msg_len);

/* The handle's last error message (owned by the handle), and a fixed name of a
 * status code. */
const char *ofa_last_error(const ofa_handle *h);
const char *ofa_status_string(ofa_status s);

/* Waits for the handle's stream, releases the handle's host state.  The
 * caller's workspace is untouched and may be freed afterwards. */
ofa_status ofa_destroy(ofa_handle *h);

#ifdef __cplusplus
}
#endif
#endif /* OFA_H */
