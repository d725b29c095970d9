/*
 * deltalog.h -- C ABI of the DeltaLog recurrent-state decode library (MI355X, gfx950).
 *
 * Sources, cited by title and passage:
 *  [DL]   "DeltaLog: Deferred Materialization of Recurrent States for Linear
 *         Attention Decoding": Eq. 3 (the common decode step, which the paper
 *         uses as the interface every operator shares), the design section (append-merge cycle,
 *         physical state, logical-state equation), the GPU-execution section
 *         (ReplayPrep / AppendDecode / Finalize, Merge), the operator
 *         instantiations (GDN, KDA, RWKV6) and the serving-integration section
 *         (allocator, append and merge queues).
 *  [FPGA] "A Persistent-State Dataflow Accelerator for Memory-Bound Linear
 *         Attention Decode on FPGA": grouped value heads (system architecture).
 *
 * The decode step, per decoded slot s and value head h (q/k head g = h / (H_v/H_k)):
 *     S_t = diag(exp(lambda_t)) S_{t-1} + a_t b_t^T,     o_t = S_t^T q_t      [DL] Eq. 3
 * with b_t = beta_t (v_t - (diag(exp lambda_t) S_{t-1})^T k_t) and a_t = k_t for
 * delta-rule operators, and a_t, b_t given for plain operators.  The state is
 * held as a dense base plus a bounded log of (a, b, log-decay snapshot)
 * entries and merged into the base every L steps ([DL] design section).
 *
 * Conventions shared by every call
 *  - Return value: DL_OK (0) or a negative DL_ERR_* code; dl_last_error()
 *    gives a message (per host thread).  Every argument is validated before
 *    anything is enqueued: a call that fails validation leaves the pool (host
 *    mirror and device buffers) unchanged.  A call split into several launches
 *    (more slots than dl_launch_slot_limit()) that fails with DL_ERR_HIP on a
 *    later launch has enqueued the earlier launches and advanced the host
 *    mirror for their slots only: the slots of the failed launch and of those
 *    after it are unchanged on host and device.  No C++ exception crosses
 *    this ABI.
 *  - Device work is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL = the default stream).  Device faults surface as DL_ERR_HIP on a
 *    later call or at the caller's synchronization.
 *  - The caller owns every device buffer (pool buffers, inputs, outputs) and
 *    must keep it alive until the stream work that uses it has completed.  The
 *    library owns only the host-side handle and its host mirror of the live-log
 *    lengths.  Host arrays (slot ids, outputs of query calls) are read or
 *    written during the call only.
 *  - A pool is not thread-safe: one host thread and one stream per pool.
 *  - All device pointers must be 16-byte aligned; all arrays are dense,
 *    row-major, last index fastest.  "bf16" arrays hold IEEE bfloat16 bit
 *    patterns (uint16).  Outputs o_t are always fp32.
 */
#ifndef DELTALOG_H
#define DELTALOG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
#define DL_OK                   0
#define DL_ERR_INVALID_ARG     -1  /* bad descriptor, NULL pointer, bad size      */
#define DL_ERR_UNSUPPORTED     -2  /* dtype / head-dim / mode combination not built */
#define DL_ERR_SLOT_RANGE      -3  /* slot id outside [0, num_slots)              */
#define DL_ERR_DUPLICATE_SLOT  -4  /* a slot id appears twice in one call          */
#define DL_ERR_BATCH_TOO_LARGE -5  /* batch > max_batch                            */
#define DL_ERR_HIP             -6  /* HIP runtime error (launch, copy, device)     */
#define DL_ERR_DRY_RUN         -7  /* device data requested from a host-only pool  */

/* Decay granularity ([DL] Eq. 3 and Table 1): none (linear attention),
 * head-wise scalar (RetNet, GDN: one log-decay per v-head), per key (GLA,
 * RWKV6, KDA: a d_k-vector per v-head). */
enum { DL_DECAY_NONE = 0, DL_DECAY_SCALAR = 1, DL_DECAY_PER_KEY = 2 };
/* Update semantics: plain (a_t, b_t given) or delta rule (a_t = k_t,
 * b_t = beta_t (v_t - P^T k_t)). */
enum { DL_UPDATE_PLAIN = 0, DL_UPDATE_DELTA = 1 };
enum { DL_F32 = 0, DL_BF16 = 1 };

/* Pool descriptor, fixed at creation ([DL] serving-integration section: each
 * slot carries a dense base plus bounded key/value logs, log-decay snapshots
 * and live-log metadata).
 *   num_slots       P, slots in the pool (requests x layers a caller maps here),
 *                   1 <= P <= 2^24, and P * num_v_heads * (d_k / value_tile)
 *                   below 2^31 (the kernels index value tiles in 32 bits)
 *   max_batch       largest B of one dl_decode_step / dl_slot_assign / dl_merge
 *   num_v_heads     H_v <= 32768;  num_k_heads H_k (H_v % H_k == 0; grouped
 *                   value heads)
 *   d_k, d_v        head dims; the library supports d_k == d_v in {16, 32, 64, 128}
 *   merge_interval  L = [DL]'s M: one merge every L decodes of a slot; the log
 *                   holds at most L-1 entries.  1 <= L <= 64.  L == 1 makes the
 *                   pool an eager read-modify-write state (no log).
 *   decay, update   DL_DECAY_*, DL_UPDATE_*
 *   state_dtype     dense base: DL_F32 or DL_BF16
 *   in_dtype        q, k / a_t and v / b_t inputs: DL_F32 or DL_BF16
 *   value_tile      B_V, columns of the d_k x B_V value tile one GPU work unit
 *                   owns ([DL] GPU-execution section, value tiling); 0 picks the
 *                   library default from u = max_batch * num_v_heads: d when
 *                   u >= 256 or d <= 32, except 64 at d = 128 for a bf16 state
 *                   with L > 1 and a scalar or no decay while u < 2048; below
 *                   u = 256, at d = 128, 16 when u < 64 and 64 when u >= 128
 *                   with an fp32 state; else 32.  A default
 *                   whose live log would exceed the LDS staging budget is
 *                   halved until it fits or reaches the narrowest built width.
 *                   Built widths: d = 128: 128, 64, 32, 16; d = 64: 64, 32;
 *                   d = 32: 32; d = 16: 16.  Narrower tiles give more work
 *                   units per slot (lower latency at small batch) at the cost
 *                   of repeating the key-side replay work per tile.
 *   replay_split    0: every value-tile work unit computes the key-side replay
 *                   coefficients of its slot-head itself (fused).  1: a
 *                   ReplayPrep pass computes them once per (slot, v-head) into
 *                   the coef buffer and the append work units read them there
 *                   ([DL] GPU-execution section, ReplayPrep -> AppendDecode);
 *                   merging slots still replay in their own work units.
 * Factor storage follows [DL]'s operator instantiations: key factors a_t are
 * stored in in_dtype (a lossless copy of the input); value factors b_t are
 * fp32 for delta operators (cancellation-sensitive) and in_dtype for plain
 * ones (a lossless copy); decay snapshots are fp32. */
typedef struct {
    int32_t num_slots;
    int32_t max_batch;
    int32_t num_v_heads;
    int32_t num_k_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t merge_interval;
    int32_t decay;
    int32_t update;
    int32_t state_dtype;
    int32_t in_dtype;
    int32_t value_tile;
    int32_t replay_split;
} dl_pool_desc;

/* Device buffers of a pool, allocated by the caller with the sizes
 * dl_pool_sizes returns (a size may be 0, then the pointer may be NULL).
 *   base    [P, H_v, d_v / B_V, d_k, B_V]  state_dtype   dense base S_bar, value-tile
 *                                                     major: each d_k x B_V tile
 *                                                     (rows = keys) is contiguous;
 *                                                     the natural [d_k, d_v] layout
 *                                                     when B_V == d_v.  Callers
 *                                                     exchange states in the natural
 *                                                     layout via dl_slot_assign and
 *                                                     dl_read_base.
 *   klog    [P, H_k, L-1, d_k]          in_dtype      key factors a_i (one per q/k head)
 *   ulog    [P, H_v, L-1, d_v]          fp32 | in     value factors b_i
 *   lamlog  [P, H_v, L-1] (scalar) or [P, H_v, L-1, d_k] (per key)  fp32
 *                                                     log-decay snapshot of entry i:
 *                                                     the cumulative log-decay right
 *                                                     after entry i's own decay
 *   nlog    [P, H_v, d_v / B_V]         int32         live-log length per value tile (all
 *                                                     tiles of a slot hold the same value)
 *   coef    [min(max_batch, launch slot limit), H_v, 2 L]  fp32   replay coefficients of
 *                                                     one launch (replay_split only; else 0 B);
 *                                                     transient, reused launch after launch;
 *                                                     may be NULL for a pool decoded only
 *                                                     through dl_decode_step_noalloc
 * The cumulative log-decay l_bar of [DL]'s physical state is not stored: it
 * equals lamlog[n-1] when n > 0 and 0 when the log is empty. */
typedef struct {
    void    *base;
    void    *klog;
    void    *ulog;
    float   *lamlog;
    int32_t *nlog;
    float   *coef;
} dl_pool_buffers;

enum { DL_BUF_BASE = 0, DL_BUF_KLOG, DL_BUF_ULOG, DL_BUF_LAMLOG, DL_BUF_NLOG, DL_BUF_COEF, DL_NUM_BUFS };

typedef struct dl_pool dl_pool;

/* Byte size of each pool buffer, indexed by DL_BUF_*: the physical state of
 * num_slots slots ([DL] physical-state list: dense base, log entries K_i, U_i,
 * Lambda_i, live length) in the layouts above, and the split-replay
 * coefficient buffer.  Host only; allocates nothing.  Returns
 * DL_ERR_INVALID_ARG / DL_ERR_UNSUPPORTED for a descriptor that dl_pool_create
 * would refuse (same checks), else DL_OK with bytes_out filled. */
int dl_pool_sizes(const dl_pool_desc *desc, size_t bytes_out[DL_NUM_BUFS]);

/* Create a pool over caller-owned buffers: the slot pool of [DL]'s
 * serving-integration section (per-slot state with its own log counter; the
 * host handle keeps the merge schedule).  Every slot starts with an empty
 * log (nlog is zeroed here, synchronously); the base is left as the caller
 * wrote it -- use dl_slot_assign to set it.  Errors: the descriptor checks of
 * dl_pool_sizes, a NULL or non-16-byte-aligned buffer whose size is not 0
 * (DL_ERR_INVALID_ARG), DL_ERR_HIP if zeroing nlog fails; *out is NULL then.  buffers == NULL creates a
 * host-only pool: every call validates and advances the host mirror exactly as
 * it would on the device but enqueues nothing (for bookkeeping checks without
 * a GPU).  *out receives the handle. */
int dl_pool_create(const dl_pool_desc *desc, const dl_pool_buffers *buffers, dl_pool **out);

/* Free the host handle (never the caller's buffers).  NULL is a no-op. */
int dl_pool_destroy(dl_pool *pool);

/* Allocator ([DL] serving-integration section): give n slots a fresh state.
 *   slot_ids   host int32 [n], distinct, in range, n <= max_batch
 *   init_base  device [n, H_v, d_k, d_v] in state_dtype (natural layout), or
 *              NULL for a zero state
 * Copies init_base[j] into base[slot_ids[j]] (re-laid out into value tiles)
 * and empties that slot's log; the slot's previous log is discarded, not
 * merged.  Other slots are untouched. */
int dl_slot_assign(dl_pool *pool, int32_t n, const int32_t *slot_ids,
                   const void *init_base, void *stream);

/* One decode step for B slots ([DL] Eq. 3 through the append-merge cycle).
 *   slot_ids  host int32 [B], distinct, in range (B == 0 is a no-op)
 *   q         device [B, H_k, d_k]   in_dtype
 *   a_or_k    device [B, H_k, d_k]   in_dtype   a_t (plain) or k_t (delta)
 *   b_or_v    device [B, H_v, d_v]   in_dtype   b_t (plain) or v_t (delta)
 *   lambda    device fp32 [B, H_v] (scalar) or [B, H_v, d_k] (per key);
 *             must be NULL for DL_DECAY_NONE
 *   beta      device fp32 [B, H_v]; must be NULL for DL_UPDATE_PLAIN
 *   out       device fp32 [B, H_v, d_v]   o_t = S_t^T q_t (post-update state)
 * A slot whose log holds L-1 entries takes the merge step: its output is
 * computed from base + log + this token, and the base is rewritten with the
 * materialized state; its log becomes empty.  Any other slot appends this
 * token's (a_t, b_t, snapshot) at log index n and leaves the base unchanged.
 *
 * Graph capture: a call made while `stream` is capturing records its launches
 * and advances the host's live lengths as if they had run.  The kernels take
 * each slot's phase (append or merge, entry index) from the device counters,
 * so a captured step stays correct when replayed at any point of the cycle;
 * dl_get_log_len then reflects the calls made, not the replays, and the pool
 * counts its host mirror as stale from then on (see dl_flush_all).  A direct
 * call also passes the host's live lengths to the kernels, which use them to
 * start loading the log early and fall back to the device counters when they
 * differ (as after a capture); captured launches pass none. */
int dl_decode_step(dl_pool *pool, int32_t B, const int32_t *slot_ids,
                   const void *q, const void *a_or_k, const void *b_or_v,
                   const float *lambda, const float *beta, float *out, void *stream);

/* dl_decode_step for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and errors as dl_decode_step.  It allocates nothing: on a
 * replay_split pool the ReplayPrep coefficients, the one scratch buffer of the
 * step, go to a static device array of the library (4 MiB per GPU, held until
 * the process ends) instead of the pool's coef buffer, which may then be NULL
 * at dl_pool_create; on other pools, whose kernels use no scratch, it is
 * dl_decode_step.  A launch carries at most 2^20 / (num_v_heads * 2 *
 * merge_interval) slots (and at most dl_launch_slot_limit()); a pool with
 * num_v_heads * 2 * merge_interval > 2^20 is refused with DL_ERR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams or host threads) race and must not be issued.  The
 * current device must be the one the pool and the stream belong to. */
int dl_decode_step_noalloc(dl_pool *pool, int32_t B, const int32_t *slot_ids,
                           const void *q, const void *a_or_k, const void *b_or_v,
                           const float *lambda, const float *beta, float *out, void *stream);

/* W consecutive decode steps of the same B slots in one launch, with the
 * state held on chip across them ([DL] Eq. 3 applied W times; [FPGA]'s
 * persistent on-chip state with streamed per-token inputs).  Each (slot,
 * v-head, value tile) block materializes its tile of the logical state once
 * ([DL] logical-state equation), keeps it in registers through the W steps and
 * writes it back once; every slot's log is empty afterwards (as after
 * dl_merge), whatever its position in the append-merge cycle was.  For use
 * where the inputs of the W steps exist before the call (a streamed token
 * sequence, a run of draft tokens).
 *   slot_ids  host int32 [B], distinct, in range (B == 0 is a no-op)
 *   W         steps, 1 <= W <= 4096
 *   q, a_or_k device [W, B, H_k, d_k]   in_dtype, step-major
 *   b_or_v    device [W, B, H_v, d_v]   in_dtype
 *   lambda    device fp32 [W, B, H_v] or [W, B, H_v, d_k]; NULL for DL_DECAY_NONE
 *   beta      device fp32 [W, B, H_v]; NULL for DL_UPDATE_PLAIN
 *   out       device fp32 [W, B, H_v, d_v]   o of every step
 * Outputs equal those of W dl_decode_step calls on the same inputs, up to
 * rounding; the dense state is rounded to state_dtype once, at the end.
 * Errors as dl_decode_step, plus DL_ERR_INVALID_ARG for W out of range. */
int dl_decode_window(dl_pool *pool, int32_t B, const int32_t *slot_ids, int32_t W,
                     const void *q, const void *a_or_k, const void *b_or_v,
                     const float *lambda, const float *beta, float *out, void *stream);

/* Eager read-modify-write baseline of the same step ([DL]'s "state-update
 * tax": read the dense state, transform it, add the outer product, write it
 * back, every token).  Same arguments as dl_decode_step; the pool must have
 * merge_interval == 1 (no log). */
int dl_eager_step(dl_pool *pool, int32_t B, const int32_t *slot_ids,
                  const void *q, const void *a_or_k, const void *b_or_v,
                  const float *lambda, const float *beta, float *out, void *stream);

/* Materialize the logical state of n slots into their bases and empty their
 * logs ([DL] logical-state equation: S = D(l_bar) S_bar + sum_i
 * D(l_bar - Lambda_i) K_i U_i^T).  Slots with an empty log are left untouched.
 * slot_ids: host int32 [n], distinct, in range, n <= max_batch.
 * Every listed slot is launched, and each of its blocks merges what its
 * device counter holds when it runs (nothing if empty), so the result does
 * not depend on the host mirror: a merge recorded into a graph merges, at
 * each replay, the listed slots' logs as they are then.  The host mirror of
 * the listed slots becomes 0. */
int dl_merge(dl_pool *pool, int32_t n, const int32_t *slot_ids, void *stream);

/* dl_merge over every slot whose log is not empty ([DL] Algorithm 1's merge
 * for the whole pool, e.g. before the bases are read back or handed to another
 * consumer); afterwards every log is empty and every base is its slot's
 * logical state.  Idempotent.  The host
 * mirror selects the slots while it follows the device; once any call on the
 * pool has been recorded into a graph (including this one), replays may have
 * moved the device counters without it, and every slot of the pool is
 * launched instead (blocks of empty slots exit at once). */
int dl_flush_all(dl_pool *pool, void *stream);

/* Copy the bases of n slots out in the natural layout.
 *   slot_ids  host int32 [n], distinct, in range, n <= max_batch
 *   out       device [n, H_v, d_k, d_v] in state_dtype, 16-byte aligned
 * Enqueued on the stream; the pool is not modified.  A base is the slot's
 * logical state only when its log is empty: call dl_merge (or dl_flush_all)
 * first to read logical states.  DL_ERR_DRY_RUN on a host-only pool. */
int dl_read_base(dl_pool *pool, int32_t n, const int32_t *slot_ids, void *out, void *stream);

/* Host mirror of the live-log length of every slot: n_out host int32 [P]. */
int dl_get_log_len(const dl_pool *pool, int32_t *n_out);

/* What the next dl_decode_step would do for these slots, without doing it:
 * merge_out[j] = 1 if slot_ids[j] would merge, else 0; index_out[j] = its live
 * length n (the log index an append writes).  Host arrays of length B. */
int dl_schedule(const dl_pool *pool, int32_t B, const int32_t *slot_ids,
                int32_t *merge_out, int32_t *index_out);

/* Device copy of nlog, read back synchronously: n_out host int32
 * [P, H_v, d_v / B_V].
 * Waits for the stream.  DL_ERR_DRY_RUN on a host-only pool. */
int dl_read_log_len_device(dl_pool *pool, int32_t *n_out, void *stream);

/* Effective value-tile width B_V of a descriptor (> 0), or a DL_ERR_* code. */
int dl_value_tile(const dl_pool_desc *desc);

/* Message of the last failed call on this host thread ("" if none). */
const char *dl_last_error(void);

/* Largest number of slots one kernel launch carries (larger calls are split). */
int32_t dl_launch_slot_limit(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_H */
