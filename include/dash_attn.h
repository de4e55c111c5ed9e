/*
 * dash_attn.h - C ABI of the deterministic attention backward for MI355X
 * (CDNA4, gfx950).
 *
 * What the library computes.  For each (batch b, head h), softmax attention
 * O = softmax(s * Q K^T) V with an optional mask (causal: query i sees keys
 * j <= i; also sliding windows and block masks, see dash_attn_desc), its
 * log-sum-exp LSE, and the backward pass: given Q, K, V, O, dO and LSE it
 * returns dQ, dK, dV.  The inputs and outputs of the backward
 * are those of the problem statement of the DASH explainer (gist.science,
 * "Technisches Resuemee" 1) and of the method outline of the euno.news
 * summary ("Methodology" 1: the backward's matrix products, score
 * computation and gradient reduction).
 *
 * Determinism.  Per the same explainer section, floating-point addition is
 * not associative, so a reproducible backward must add the per-KV-tile dQ
 * partials in a fixed order.  Every schedule except DASH_SCHED_ATOMIC adds
 * them in the order of a rank table, enforced by device-scope counters, so
 * dQ, dK and dV are bit-identical from run to run.  DASH_SCHED_ATOMIC is the
 * non-deterministic reference (unordered atomic adds).
 *
 * Schedules (explainer "Technisches Resuemee" 2.2; authors' abstract):
 *   NAIVE       Q blocks ascending; dQ order = KV tiles ascending.
 *   DESCENDING  Q blocks descending (descending Q-tile iteration); same
 *               dQ order as NAIVE.
 *   SHIFT       full mask: KV tile i visits Q blocks i, i+1, ..., 0, ..., i-1
 *               (shift scheduling); causal mask: symmetric shift, pairing
 *               KV tiles w and n-1-w in one workgroup, two phases.  dQ order
 *               = the step at which each tile reaches the block.
 *   ATOMIC      NAIVE's traversal, unordered fp32 atomic adds.
 *   AUTO        the one dash_attn_bwd_tune measured fastest for the
 *               problem on this device, else the ordered schedule the DAG
 *               model predicts fastest under the launch's placement
 *               (dash_attn_bwd_predict) with the device's costs: the
 *               defaults, or those dash_attn_bwd_calibrate fitted to
 *               measured kernel times.
 * With a window or block mask the same rules run over the tile pairs that
 * hold a visible key; SHIFT becomes a timed shift (see
 * dash_attn_schedule_tables), the summary's limitations naming
 * block-sparse masks as needing schedule extensions.
 *
 * Conventions for every call below.
 *   Layout      Q, K, V, O, dO, dQ, dK, dV: contiguous [B, H, N, d], d
 *               innermost.  LSE and delta: contiguous [B, H, N] float.
 *   dtype       One dtype for all of Q, K, V, O, dO, dQ, dK, dV (fp32 or
 *               bf16); LSE, delta and all accumulation are fp32.  bf16
 *               outputs are rounded to nearest even.
 *   LSE         Natural log of sum_j exp(s * <Q_i, K_j>) over visible j.
 *   Shapes      N_q = N_k = N; d in {64, 128}; N a multiple of the tile
 *               (64 for fp32, 128 for bf16); B, H >= 1; B*H*N < 2^31 and
 *               N*d < 2^29 (32-bit device offsets).  Anything else
 *               returns DASH_ERR_UNSUPPORTED before any launch.
 *   Pointers    Device pointers unless stated otherwise; owned by the
 *               caller; never freed or retained by the library.  Inputs
 *               are read-only; outputs may not alias inputs.
 *   Streams     `stream` is a hipStream_t (0 = the null stream).  Calls are
 *               asynchronous on it unless stated otherwise.
 *   Errors      Argument errors are returned synchronously, before any
 *               launch.  HIP launch errors return DASH_ERR_HIP.  A device
 *               ordering time-out is read after the stream has been
 *               synchronized, with dash_status_query.
 *   Memory      The library allocates no device memory: every device
 *               buffer, the backward's workspace included, is the
 *               caller's.  The schedule tables of the full and causal
 *               masks are written into the workspace by the backward's
 *               first kernel (closed forms, no host-to-device copy).  For
 *               windows and block masks the host builds the tables once
 *               per mask and schedule and keeps them in pinned host memory
 *               (a least-recently-used cache of 32 entries per kind, each
 *               freed only after the last copy from it has completed); each
 *               launch copies them into the workspace with hipMemcpyAsync
 *               on the caller's stream.  The host also caches validated
 *               tables and DAG predictions (host memory).
 *   Threads     Calls may come from several host threads; the host caches
 *               are locked.  Calls that share a workspace must be ordered
 *               on one stream.
 */
#ifndef DASH_ATTN_H
#define DASH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = 1,      /* null pointer, bad enum, negative size */
  DASH_ERR_UNSUPPORTED = 2,      /* valid but unsupported shape/dtype/schedule */
  DASH_ERR_WORKSPACE = 3,        /* workspace too small or misaligned */
  DASH_ERR_HIP = 4,              /* a HIP runtime call failed */
  DASH_ERR_SCHEDULE_INVALID = 5, /* schedule tables failed validation (cycle, coverage) */
  DASH_ERR_ORDER_TIMEOUT = 6,    /* an ordered dQ add waited past its spin limit */
  DASH_ERR_HOST_MEMORY = 7       /* a host-side table or cache allocation failed */
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;

typedef enum {
  DASH_SCHED_ATOMIC = 0,
  DASH_SCHED_NAIVE = 1,
  DASH_SCHED_DESCENDING = 2,
  DASH_SCHED_SHIFT = 3,
  DASH_SCHED_AUTO = 4  /* the ordered schedule with the shortest predicted
                          critical path (dash_schedule_choose) */
} dash_schedule;

/* Problem descriptor.  softmax_scale <= 0 selects 1/sqrt(d).
 *
 * Mask: key j is visible to query i when every given constraint holds:
 *   causal      j <= i;
 *   window > 0  a sliding window: i - j < window if causal, else
 *               |i - j| < window (0 = no window);
 *   block_mask  (host pointer, may be NULL) the entry [i / block_size]
 *               [j / block_size] of a row-major (N / block_size)^2 byte
 *               array is nonzero.  block_size must be a multiple of
 *               dash_attn_tile(desc) and divide N.  Read during the call
 *               only (the library keeps its own copy).
 * Full and causal are the pages' masks; windows and block masks are the
 * special masks the summary's limitations list names as needing schedule
 * extensions.  A query row that sees no key gets O = 0, LSE = -inf and
 * zero gradients.  With a window or block mask, N / tile must be at most
 * 2048.  Zero-initialised trailing fields give the full or causal mask. */
typedef struct {
  int32_t B, H, N, d;
  int32_t dtype;   /* dash_dtype */
  int32_t causal;  /* 0 = no causal constraint, 1 = causal */
  float softmax_scale;
  int32_t window;
  int32_t block_size;
  const uint8_t* block_mask;
} dash_attn_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* dash_status_string(dash_status s);

/* KV tile (rows) of the backward for a descriptor: 64 for fp32, 128 for
 * bf16; 0 if desc is NULL. */
int32_t dash_attn_tile(const dash_attn_desc* desc);

/* Q sub-tile (rows) of the backward: each Q block of dash_attn_tile rows
 * is processed, counted and ordered in sub-tiles of this many rows (32 for
 * d = 128, 64 for d = 64); 0 if desc is NULL. */
int32_t dash_attn_bwd_subtile(const dash_attn_desc* desc);

/*
 * Forward: O = softmax(s Q K^T) V and LSE.  q, k, v: inputs; o: output
 * [B,H,N,d]; lse: output [B,H,N] float.  Needed to produce the O and LSE
 * the backward consumes (the backward's inputs, explainer section 1).
 * A block mask needs dash_attn_fwd_ws (DASH_ERR_WORKSPACE here).
 */
dash_status dash_attn_fwd(const dash_attn_desc* desc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* stream);

/*
 * Device bytes the forward needs for this descriptor: 0 for the full,
 * causal and window masks; with a block mask, room for the tile liveness
 * (n tiles per side, n * n bytes rounded up to 256).  0 on invalid input.
 */
size_t dash_attn_fwd_workspace_size(const dash_attn_desc* desc);

/*
 * dash_attn_fwd with a caller-provided workspace (device, 256-byte aligned,
 * at least dash_attn_fwd_workspace_size bytes; may be NULL when that is 0).
 * With a block mask the call copies the tile liveness into it on `stream`
 * (asynchronously, from pinned host memory); its contents on entry do not
 * matter.  DASH_ERR_WORKSPACE if it is missing, too small or misaligned.
 */
dash_status dash_attn_fwd_ws(const dash_attn_desc* desc, const void* q, const void* k,
                             const void* v, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Backward preprocess: delta_i = sum_k dO_ik * O_ik in fp32 ([B,H,N]).
 * This row term is implied by the backward (it equals sum_j P_ij dP_ij) and
 * needs only O and dO; the pages do not name it separately.
 */
dash_status dash_attn_bwd_preprocess(const dash_attn_desc* desc, const void* o,
                                     const void* dout, float* delta, void* stream);

/*
 * Workspace bytes dash_attn_bwd needs for this descriptor and schedule;
 * 0 for an invalid or unsupported descriptor or schedule.  The size is the
 * same for every schedule: the schedules only reorder work (euno.news
 * summary, "Results": memory overhead unchanged).  Layout, 256-byte
 * aligned parts: a header (status word, work counters), the per-Q-sub-tile
 * order counters, one head's schedule tables (unit offsets, items, tiles
 * no pair touches; sized for the largest table of any schedule), and the
 * fp32 dQ accumulator [B,H,N,d].
 */
size_t dash_attn_bwd_workspace_size(const dash_attn_desc* desc, dash_schedule schedule);

/*
 * Backward: dQ, dK, dV from Q, K, V, dO, LSE and delta (from
 * dash_attn_bwd_preprocess).  workspace: device buffer of at least
 * dash_attn_bwd_workspace_size bytes, 256-byte aligned; its contents on
 * entry do not matter and on return are scratch (except the status word).
 * The call zeroes the accumulator and counters, runs the persistent
 * backward kernel with the chosen schedule, then scales and converts dQ.
 */
dash_status dash_attn_bwd(const dash_attn_desc* desc, dash_schedule schedule, const void* q,
                          const void* k, const void* v, const void* dout, const float* lse,
                          const float* delta, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments and results as dash_attn_bwd (bit-identical
 * for the ordered schedules) without a workspace argument: the workspace is
 * a built-in device array of DASH_NOALLOC_SCRATCH_BYTES per GPU, part of the
 * library's code object (allocated when the code object is loaded, held
 * until the process ends).  The call allocates nothing.
 *   Limits    the workspace dash_attn_bwd_workspace_size reports must fit
 *             the array (else DASH_ERR_WORKSPACE, before any launch; the
 *             workspace holds about 4 d + 5 bytes per query row and head,
 *             so bf16 d = 128 fits B*H*N up to about 129k, d = 64 up to
 *             about 258k); full and causal masks only (a window or
 *             block mask gives DASH_ERR_UNSUPPORTED: their tables need
 *             host memory allocated on first use).
 *   Sharing   every call on a GPU uses that GPU's one array and leaves its
 *             contents there: calls that overlap on one GPU (other streams,
 *             other threads) race and must be serialized by the caller.
 *   Status    an ordering time-out is read, after the caller synchronized
 *             the stream, with dash_status_query(DASH_NOALLOC_WORKSPACE)
 *             (the current GPU's array).
 */
#define DASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
#define DASH_NOALLOC_WORKSPACE ((const void*)1)
dash_status dash_attn_bwd_noalloc(const dash_attn_desc* desc, dash_schedule schedule,
                                  const void* q, const void* k, const void* v, const void* dout,
                                  const float* lse, const float* delta, void* dq, void* dk,
                                  void* dv, void* stream);

/*
 * Device status of the last dash_attn_bwd on this workspace: reads the
 * status word with a synchronous copy; call it after the stream the
 * backward ran on has been synchronized.  DASH_OK, or
 * DASH_ERR_ORDER_TIMEOUT if some ordered add gave up waiting (that
 * launch's results are then not valid); DASH_ERR_INVALID_ARG for NULL.
 * Each dash_attn_bwd clears the word, so it reports the last launch only.
 * DASH_NOALLOC_WORKSPACE reads the word of dash_attn_bwd_noalloc's
 * built-in array on the current GPU.
 */
dash_status dash_status_query(const void* workspace);

/*
 * Convenience: synchronizes `stream`, then dash_status_query(workspace).
 */
dash_status dash_attn_bwd_status(const void* workspace, void* stream);

/*
 * Test and diagnostic controls for dash_attn_bwd_debug.  An all-zero
 * struct gives the behaviour of dash_attn_bwd.
 *   spin_limit      0 = default; else the number of polls (each ~1 us
 *                   apart) after which an ordered add gives up and sets
 *                   DASH_ERR_ORDER_TIMEOUT.
 *   jitter_seed     non-zero: each workgroup sleeps a pseudo-random few
 *                   microseconds before each ordered add (perturbs timing
 *                   only; results of ordered schedules must not change).
 *   poison_q        0 = off; k > 0: in head 0, the first contributor to Q
 *                   sub-tile k-1 (sub-tiles of dash_attn_bwd_subtile rows)
 *                   waits for a counter value that never comes, which
 *                   forces the time-out path.
 *   partials        non-NULL: device float buffer [B,H,n_kv,N,d] (n_kv =
 *                   N / dash_attn_tile); each KV tile's unscaled dQ partial
 *                   for every Q row it meets is stored there, in addition
 *                   to the normal accumulation.
 *   kernel_events   non-NULL pair of hipEvent_t: recorded on `stream`
 *                   immediately before and after the backward kernel's
 *                   launch (excluding the workspace clear and the dQ
 *                   conversion), for timing that kernel alone.
 *   placement       where units run; results are bit-identical for every
 *                   value, only speed differs.  0 = automatic (XCD groups
 *                   with the L2-coherent accumulator for the ordered
 *                   schedules, device-wide for ATOMIC); 1 = device-wide (every workgroup takes units
 *                   from one list); 2 = XCD groups: the heads are dealt to the
 *                   XCDs, each head's units run on the workgroups of one XCD
 *                   and its accumulator is kept coherent in that XCD's L2;
 *                   3 = XCD groups with device-coherent accumulator accesses.
 *                   XCD groups fall back to device-wide when a head's units
 *                   cannot all be resident on one XCD (static schedules).
 *                   Other values: DASH_ERR_INVALID_ARG.
 *   unit_order      order in which workgroups take the units of a dynamic
 *                   schedule (NAIVE, DESCENDING); results are bit-identical
 *                   for every value.  0 = automatic (unit-major when the DAG
 *                   model predicts a makespan at least 5 % shorter, else
 *                   head by head); 1 = head by head; 2 = unit-major (unit 0
 *                   of every head, then unit 1, ...).  Ignored by static
 *                   schedules.  Other values: DASH_ERR_INVALID_ARG.
 *   wait_stats      non-NULL: device uint64 buffer of at least
 *                   4 * 4096 * 4 entries; for each workgroup g and wave w,
 *                   entries [(g*waves + w)*4 + k] receive: k=0 shader-clock
 *                   cycles spent waiting for ordered adds, k=1 ordered waits,
 *                   k=2 waits that polled more than once, k=3 cycles of the
 *                   workgroup's whole run (waves = dash_attn_tile/32;
 *                   workgroups x waves, counting 8 waves per workgroup with
 *                   layouts 1 and 2, must not exceed 4096 * 4, else
 *                   DASH_ERR_UNSUPPORTED).
 *   phase_stats     non-NULL: device uint64 buffer of at least
 *                   16 * 4096 * 4 entries; for each workgroup g and wave w,
 *                   entries [(g*waves + w)*16 + k] receive the shader-clock
 *                   cycles the wave spent in phase k of its Q sub-tiles:
 *                   0 item decode and KV tile changes, 1 S and dP products,
 *                   2 counter check and accumulator reads issued, 3 softmax
 *                   and dS, 4 dV and dK products, 5 staging the next
 *                   sub-tile, 6 the previous partial's ordered add, 7 the
 *                   sub-tile barrier, 8 the dQ product, 9 the hand-off,
 *                   10 prefetch, partial staging and counter read (atomic
 *                   adds for ATOMIC); k=15 the cycles of the whole run.  The
 *                   timer reads the clock between phases, which itself waits
 *                   for outstanding LDS accesses, so the launch runs slower
 *                   than without it; shares, not times, are the result.
 *                   Same size limit as wait_stats.  With layout 1 or 2
 *                   (also when layout 0 picks the pipeline) every one
 *                   of the 8 waves of a workgroup g writes entries
 *                   [(g*8 + v)*16 + k]: k = 0..8 its phases (the kernel
 *                   source lists them per role), k = 14 its role (1 or 2),
 *                   k = 15 its whole run.
 *   layout          which backward kernel runs; results are bit-identical
 *                   for every value (the ATOMIC schedule's unordered adds
 *                   aside).  0 = automatic: the two-stage pipeline for bf16
 *                   with d = 128 or 64, the one-stage kernel otherwise;
 *                   1 = the wave-pair layout (two waves per SIMD, each KV
 *                   slice split between a wave for S, P, dV and the dQ
 *                   product and a wave for dP, dS, dK and the ordered add);
 *                   2 = the two-stage pipeline (per SIMD, one wave computes
 *                   S, dP, P, dS and dV of a Q sub-tile while another
 *                   computes dK, dQ and the ordered dQ add of the sub-tile
 *                   before it); 3 = the one-stage kernel (one wave per KV
 *                   slice does every product of a sub-tile).  1 exists for
 *                   bf16 with d = 128 only, 2 for bf16 with d = 128 or 64:
 *                   another dtype or head dim gives DASH_ERR_UNSUPPORTED;
 *                   other values: DASH_ERR_INVALID_ARG.
 */
typedef struct {
  uint32_t spin_limit;
  uint32_t jitter_seed;
  int32_t poison_q;
  float* partials;
  void* kernel_events[2];
  uint64_t* wait_stats;
  int32_t placement;
  int32_t unit_order;
  uint64_t* phase_stats;
  int32_t layout;
} dash_bwd_debug;

dash_status dash_attn_bwd_debug(const dash_attn_desc* desc, dash_schedule schedule,
                                const void* q, const void* k, const void* v, const void* dout,
                                const float* lse, const float* delta, void* dq, void* dk,
                                void* dv, void* workspace, size_t workspace_bytes,
                                const dash_bwd_debug* dbg, void* stream);

/* ------------------------------------------------------------------ host only */

/*
 * Schedule tables for one head with n tiles (host memory, no GPU needed).
 * Outputs (caller-allocated host arrays):
 *   *n_units        number of units (workgroup work lists)
 *   unit_offsets    [n + 1]: unit u's items are [unit_offsets[u], unit_offsets[u+1])
 *   item_kv, item_q [n * n]: the items (KV tile, Q block) in processing order
 *   rank            [n * n], row-major [q][kv]: position of kv in q's dQ
 *                   order, -1 where the pair is masked or for ATOMIC
 * Returns DASH_ERR_UNSUPPORTED for SHIFT with a causal mask and odd n > 1.
 */
dash_status dash_schedule_tables(int32_t n, int32_t causal, dash_schedule schedule,
                                 int32_t* n_units, int32_t* unit_offsets, int32_t* item_kv,
                                 int32_t* item_q, int32_t* rank);

/*
 * DAG critical-path prediction for the descriptor's B*H heads (its mask's
 * tiles) run on `slots` persistent workgroups, heads taken one after the
 * other (explainer 2.1's DAG: compute and reduction nodes, data and
 * accumulation-order edges, one KV tile per processor chain).
 * cost[4] = {c_full, c_diag, r, h}: compute time of an unmasked item, of a
 * partial item (causal diagonal, window or block edge), the dQ add, and
 * the hand-off latency between consecutive contributors.
 * out[4] = {makespan, total_wait, max_slot_idle, lower_bound}.  Host only.
 * The pages' SHIFT (full and causal masks) needs slots >= units per head
 * (else DASH_ERR_UNSUPPORTED), and so does a graph of 2^31 nodes or more (2
 * per item and head); a window or block mask's SHIFT is the timed shift a
 * launch on `slots` co-resident workgroups runs.
 */
dash_status dash_schedule_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                  int32_t slots, const double cost[4], double out[4]);

/*
 * DAG prediction of a launch, host only: the schedule's tables for the
 * descriptor's mask run as dash_attn_bwd places them on `slots` co-resident
 * workgroups.  The ordered schedules run in XCD groups (each of the 8 XCDs'
 * workgroups takes the units of 1/8 of the heads) unless a static table's
 * units per head exceed one group's workgroups (then device-wide); dynamic
 * tables take units head by head, or unit-major when that is predicted at
 * least 5 % shorter.  out[4] as dash_schedule_predict, for one group's share
 * (every group carries the same share); info[4] (may be NULL) = {groups
 * (8 or 1), unit-major (0/1), heads and workgroups the model ran (the share
 * is sampled to about 2e5 items with proportionally fewer workgroups)}.
 * DASH_SCHED_AUTO predicts its candidates this way.
 */
dash_status dash_attn_bwd_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                  int32_t slots, const double cost[4], double out[4],
                                  int32_t info[4]);

/*
 * Schedule choice, host only (the explainer's significance section presents
 * DASH as a palette of strategies, heuristic and optimal, from which the
 * user picks by hardware and model configuration; this makes that pick from
 * the DAG model).  Predicts the makespan of NAIVE, DESCENDING and SHIFT
 * (the full or causal mask of n tiles) for `heads` heads on `slots` workgroups and the
 * cost model `cost` (NULL: the one-stage kernel's default {1, 0.5, 0.05,
 * 0.05} in units of one unmasked item: the dQ add and the hand-off are short
 * next to an item because the kernel overlaps the add with the next item's
 * compute; dash_attn_bwd_costs gives the costs a launch uses), and returns the one
 * with the smallest makespan (ties: SHIFT, then DESCENDING, then NAIVE).
 * (DASH_SCHED_AUTO in dash_attn_bwd makes the same choice with each
 * candidate predicted under the launch's placement, dash_attn_bwd_predict.)
 * Schedules that cannot run (SHIFT with an odd causal tile count or more
 * units per head than slots) are skipped.  predicted[3] (may be NULL)
 * receives the three makespans in enum order NAIVE, DESCENDING, SHIFT, NaN
 * where skipped.  For large problems the prediction uses a subset of the
 * heads (at most about 2e5 items).
 */
dash_status dash_schedule_choose(int32_t n, int32_t causal, int32_t heads, int32_t slots,
                                 const double* cost, dash_schedule* choice, double* predicted);

/*
 * Profiling-driven schedule choice (the summary's limitations list runtime
 * profiling-based adaptive selection as future work; the DAG model's pick
 * is the default).  Runs NAIVE, DESCENDING and SHIFT (those that can run)
 * once untimed and `reps` times timed (1..1000) on the given buffers,
 * exactly as dash_attn_bwd would (dq, dk, dv and the workspace are
 * overwritten; their final contents are those of the last schedule run),
 * times each with HIP events on `stream`, and records the fastest for this
 * shape and mask on the current device: later DASH_SCHED_AUTO launches of
 * the same shape run it.  Blocking: waits for `stream`.  *choice receives
 * the pick; times_ms[3] (may be NULL) the mean time per launch of NAIVE,
 * DESCENDING, SHIFT (NaN where a schedule cannot run).  Errors as
 * dash_attn_bwd, DASH_ERR_ORDER_TIMEOUT if an ordered add timed out.
 */
dash_status dash_attn_bwd_tune(const dash_attn_desc* desc, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* delta, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, int32_t reps, dash_schedule* choice,
                              float* times_ms, void* stream);

/*
 * Calibration of the DAG model from measured kernel times (the summary's
 * limitations list runtime-profiling-based adaptive selection as future
 * work).  Times NAIVE, DESCENDING and SHIFT as dash_attn_bwd_tune does
 * (blocking, on the caller's buffers, which are overwritten), fits the
 * model's costs to those times with dash_schedule_fit_costs, and records
 * them for this device, dtype and head dimension: later DASH_SCHED_AUTO
 * launches of any shape with that dtype and head dimension predict with
 * them (a shape dash_attn_bwd_tune measured keeps its measured pick).
 * cost_out[4] (may be NULL) receives the fitted {c_full, c_diag, r, h},
 * *residual (may be NULL) the fit's relative RMS error, times_ms[3] (may be
 * NULL) the measured times as dash_attn_bwd_tune reports them.  Errors as
 * dash_attn_bwd_tune; DASH_ERR_UNSUPPORTED if fewer than two schedules can
 * run or nothing runs (every pair masked).
 */
dash_status dash_attn_bwd_calibrate(const dash_attn_desc* desc, const void* q, const void* k,
                                    const void* v, const void* dout, const float* lse,
                                    const float* delta, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes, int32_t reps,
                                    double cost_out[4], double* residual, float* times_ms,
                                    void* stream);

/*
 * The costs DASH_SCHED_AUTO uses on the current device for the
 * descriptor's dtype and head dimension until dash_attn_bwd_calibrate fits
 * others: {1, 0.5, 0.3, 0.3} for bf16 with d = 128 or 64 (the two-stage pipeline,
 * which overlaps the products so that the ordered adds weigh more), else
 * {1, 0.5, 0.05, 0.05} (the one-stage kernel).  Queries the current device
 * only.
 */
dash_status dash_attn_bwd_costs(const dash_attn_desc* desc, double cost_out[4]);

/*
 * The fit itself, host only: the DAG model's costs for which the predicted
 * makespans of NAIVE, DESCENDING and SHIFT (dash_attn_bwd_predict's, on
 * `slots` co-resident workgroups) are proportional to measured times
 * ms[3] (<= 0 or NaN: not measured; at least two).  c_full = 1; c_diag in
 * {0.5, 0.75, 1}, r and h in {0, 0.025, 0.05, 0.1, 0.2, 0.3}; per
 * candidate, the time of one cost unit that best matches all measured
 * times in relative least squares; the candidate with the smallest
 * relative RMS error wins (ties: nearest the defaults).  cost_out[4]
 * receives the costs, *residual (may be NULL) the relative RMS error,
 * *item_ms (may be NULL) the fitted time of one cost unit in the units of
 * ms.  DASH_ERR_INVALID_ARG with fewer than two measured times or a
 * negative one; DASH_ERR_UNSUPPORTED if a measured schedule cannot run.
 */
dash_status dash_schedule_fit_costs(const dash_attn_desc* desc, int32_t slots,
                                    const double ms[3], double cost_out[4], double* residual,
                                    double* item_ms);

/*
 * The schedule dash_attn_bwd runs for `schedule` on the current device:
 * DASH_SCHED_AUTO resolves to the DAG model's pick (as dash_schedule_choose,
 * each candidate predicted under the launch's placement with the costs
 * dash_attn_bwd_costs reports) for the problem's mask, B*H heads and the
 * launch's co-resident workgroups, or to dash_attn_bwd_tune's measured pick;
 * other schedules come back unchanged.  Queries the device (occupancy),
 * launches nothing.  Errors as dash_attn_bwd's argument checks.
 */
dash_status dash_attn_bwd_resolve_schedule(const dash_attn_desc* desc, dash_schedule schedule,
                                           dash_schedule* resolved);

/*
 * The backward's schedule tables for any descriptor (any mask), host only:
 * the same tables dash_attn_bwd runs on `slots` co-resident workgroups (0:
 * this device's count for the backward; queries the device).  Two calls:
 * with any array NULL, fills sizes = {n tiles per side, units, items,
 * static, slots per head} and returns (static = 1: units run in
 * head-aligned rounds, a whole head resident; 0: from a work counter in
 * unit order); then with arrays of those sizes (sizes unchanged):
 * unit_offsets[units + 1], item_kv/item_q/item_step/item_partial[items]
 * (step: lockstep or timed step for SHIFT, else -1; partial: the pair has
 * hidden elements) and rank[n * n] (rank[q * n + kv], -1 where absent).
 *
 * SHIFT on a window or block mask is a timed shift: a step-by-step
 * simulation of s workgroup slots running one head (s = slots per head,
 * sizes[4]): one unit per KV tile with live pairs, started longest first
 * (ties: lower KV tile) as slots free up; at each step every running unit,
 * in start order, takes the remaining Q block of its own that no other
 * unit took at that step and that comes first cyclically from its own
 * diagonal (smallest (q - kv) mod n), or idles for the step.  No two units
 * meet on a block at one step (the shift's defining property, explainer
 * 2.2 B), a block's dQ order is by step, items run in step order and units
 * in start order.  Run from a work counter, such tables cannot deadlock
 * when W >= (s - 1) h + 1 for W workgroups shared by h heads, in any
 * interleaving of the heads' units; s is the largest count for which that
 * holds both in the launch's 8 XCD groups (slots / 8 workgroups, ceil(B*H
 * / 8) heads each) and device-wide.  Tile pairs that hold no visible key
 * are left out; KV tiles with none get no unit.
 */
dash_status dash_attn_schedule_tables(const dash_attn_desc* desc, dash_schedule schedule,
                                      int32_t slots, int32_t sizes[5], int32_t* unit_offsets,
                                      int32_t* item_kv, int32_t* item_q, int32_t* item_step,
                                      uint8_t* item_partial, int32_t* rank);

/*
 * dash_schedule_predict with a choice of unit order: unit_major = 1: the
 * dynamic policy takes unit 0 of every head, then unit 1, ... (0: head by
 * head, as dash_schedule_predict; ignored by static schedules).  Host only.
 */
dash_status dash_attn_schedule_predict(const dash_attn_desc* desc, dash_schedule schedule,
                                       int32_t slots, int32_t unit_major, const double cost[4],
                                       double out[4]);

/*
 * Longest path (critical path) of a general DAG, host only.  Node weights
 * [n_nodes]; edges src/dst/latency [n_edges].  Writes earliest start and
 * finish per node.  DASH_ERR_SCHEDULE_INVALID if the graph has a cycle.
 */
dash_status dash_dag_longest_path(int32_t n_nodes, const double* weights, int32_t n_edges,
                                  const int32_t* src, const int32_t* dst, const double* latency,
                                  double* start, double* finish);

/*
 * Ordering litmus (diagnostic): `workgroups` one-wave workgroups (spread
 * over all XCDs by the dispatcher, all resident at once) take turns adding
 * their row of `values` [workgroups, len] into `acc` [len], workgroup w
 * going when the counter reaches turn[w] (a permutation of
 * 0..workgroups-1), through the same counter hand-off and coherent
 * read-modify-write that the ordered dQ adds use.  turn, values, acc: device arrays; counters: device uint32[2]
 * (counter, status; cleared by the call).  spin_limit 0 = default.
 * Synchronizes the stream; returns DASH_ERR_ORDER_TIMEOUT if a hand-off
 * timed out.
 */
dash_status dash_litmus_ordered_add(int32_t workgroups, int32_t len, const int32_t* turn,
                                    const float* values, float* acc, uint32_t* counters,
                                    uint32_t spin_limit, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DASH_ATTN_H */
