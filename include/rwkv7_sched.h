/* rwkv7_sched.h: continuous-batching scheduler over the rwkv7 C ABI (host).
 *
 * The Albatross article (RWKV-Runner backend, "continuous batching: the
 * worker main loop") describes a worker that, in every round, handles abort
 * requests, advances each occupied state slot through its prefill / decode
 * phase, retires finished tasks and frees their slots, refills the slot pool
 * from the task queue (at most max_batch tasks, of which at most
 * max_prefill_count = max(int(batch * 0.125), 1) may still be in a prefill
 * phase), orders the rows by category (decode, then one-token prefill), runs
 * one batched forward and samples the decode rows.  Prompts shorter than
 * min_forward_seq_len (10) are prefilled one token per round inside the decode
 * batch; longer ones take a sequence prefill, and decode_prefill_ratio (5)
 * paces those: one sequence prefill per about five decode rounds.  The
 * RWKV-Server article ("RWKV-Server design: single-threaded prefill +
 * lock-free decode") names the task states PREFILL -> READY -> RUNNING ->
 * FINISHED.  Both pages give the behaviour in prose only; this is one plain
 * reading of it:
 *
 *   * a task is QUEUED until it gets a slot; admission is FIFO and stops at the
 *     first queued task that needs a prefill while max_prefill_count tasks are
 *     already in PREFILL;
 *   * admission takes the lowest free slot in [0, max_batch), resets its state
 *     and occurrence row, and sends the task to PREFILL (prompt length >= 2)
 *     or READY (a one-token prompt);
 *   * the prefill covers prompt[0 .. n-2]; the last prompt token is the
 *     task's first decode input;
 *   * a prompt of length n < min_forward_seq_len is prefilled one token per
 *     round as a row of the decode batch (its logits are not sampled);
 *   * a longer one waits for a sequence prefill (rwkv7_prefill_seq): one
 *     task per round, oldest admission first, when no row is left to decode
 *     or when decode_prefill_ratio decode rounds have passed since the last
 *     one;
 *   * READY and RUNNING tasks form the decode rows (RUNNING from then on);
 *     the rows are ordered decode rows by slot, then one-token prefill rows by
 *     slot, and rows [0, n_sample) are the decode rows;
 *   * a decode row samples its next token with the task's parameters and the
 *     uniform u_j of its j-th generated token (j = 0, 1, ...):
 *       u_j = (splitmix64 output number j+1 from state `seed`) >> 40, times
 *       2^-24
 *     (SplitMix64: Steele, Lea and Flood, OOPSLA 2014; the state advances by
 *     0x9E3779B97F4A7C15 per output, mixed with the published constants);
 *   * each generated token is an event; a task finishes after emitting its
 *     stop token (if >= 0) or its max_new_tokens-th token, or when aborted;
 *     its slot is free for the next round's admission.
 *
 * Ownership: the scheduler copies prompts; the backend's ctx and buffers
 * stay the caller's.  Calls on one scheduler must not overlap; different
 * schedulers are independent.  All functions return RWKV7_OK or an RWKV7_E*
 * status (rwkv7.h), with the message in rwkv7_last_error(). */
#ifndef RWKV7_SCHED_H
#define RWKV7_SCHED_H

#include <stdint.h>

#include "rwkv7.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rwkv7_sched rwkv7_sched; /* opaque host handle */

/* Task states. */
#define RWKV7_TASK_QUEUED 0
#define RWKV7_TASK_PREFILL 1
#define RWKV7_TASK_READY 2
#define RWKV7_TASK_RUNNING 3
#define RWKV7_TASK_FINISHED 4

/* Event kinds and finish reasons. */
#define RWKV7_EV_TOKEN 1    /* value = generated token id, index = its position */
#define RWKV7_EV_FINISHED 2 /* value = reason, index = tokens generated */
#define RWKV7_FIN_LENGTH 1
#define RWKV7_FIN_STOP 2
#define RWKV7_FIN_ABORT 3

typedef struct rwkv7_sched_config {
  int32_t max_batch;            /* slots 0 .. max_batch-1 are the scheduler's (>= 1) */
  int32_t max_prefill_count;    /* <= 0: max(int(max_batch * 0.125), 1) */
  int32_t decode_prefill_ratio; /* <= 0: 5 */
  int32_t min_forward_seq_len;  /* <= 0: 10 */
  int32_t vocab;                /* token ids of prompts and stop tokens lie in [0, vocab) */
} rwkv7_sched_config;

typedef struct rwkv7_sched_params {
  float temperature;      /* not > 0: greedy pick */
  float top_p;            /* >= 1: no nucleus cut */
  int32_t top_k;          /* <= 0: no top-k cut */
  float presence, frequency, decay; /* the penalty of rwkv7_sample / rwkv7_greedy */
  int32_t max_new_tokens; /* >= 1 */
  int32_t stop_token;     /* -1: none */
  uint64_t seed;          /* the task's uniform stream */
} rwkv7_sched_params;

/* One round's forward: B rows, each consuming tokens[b] on slots[b]; rows
 * [0, n_sample) then draw their next token with the per-row sampling
 * parameters (host arrays of n_sample entries) into ids_out[0 .. n_sample). */
typedef struct rwkv7_sched_batch {
  int32_t B;
  const int32_t* slots;
  const int32_t* tokens;
  int32_t n_sample;
  const float* temperature;
  const float* top_p;
  const int32_t* top_k;
  const float* presence;
  const float* frequency;
  const float* decay;
  const float* uniform;
} rwkv7_sched_batch;

/* What the scheduler drives.  Every callback returns RWKV7_OK or a status,
 * which the scheduler passes on (the round stops there).  All pointers are
 * host memory, valid for the call only. */
typedef struct rwkv7_sched_backend {
  void* ctx;
  /* zero the recurrent state, shifts, step counter and occurrence row of one slot */
  int (*reset)(void* ctx, int32_t slot);
  /* advance `slot` by tokens[0 .. T) (T >= 1), state only */
  int (*prefill)(void* ctx, int32_t slot, const int32_t* tokens, int32_t T);
  /* one batched forward + sampling round (see rwkv7_sched_batch) */
  int (*step)(void* ctx, const rwkv7_sched_batch* batch, int32_t* ids_out);
} rwkv7_sched_backend;

typedef struct rwkv7_sched_event {
  int64_t task;
  int32_t kind;  /* RWKV7_EV_* */
  int32_t value; /* token id, or RWKV7_FIN_* */
  int32_t index; /* token position, or the count of generated tokens */
  int32_t pad;
} rwkv7_sched_event;

typedef struct rwkv7_sched_stats {
  int32_t decode_rows;      /* rows sampled this round */
  int32_t one_prefill_rows; /* one-token prefill rows this round */
  int32_t seq_prefills;     /* sequence prefills run this round (0 or 1) */
  int32_t seq_prefill_tokens;
  int32_t admitted;         /* tasks that got a slot this round */
  int32_t finished;         /* tasks that finished this round (any reason) */
  int32_t queued;           /* tasks still waiting for a slot */
  int32_t active;           /* tasks holding a slot after the round */
} rwkv7_sched_stats;

/* Create a scheduler over `backend` (copied).  EINVAL for a null pointer,
 * max_batch < 1, vocab < 1 or a backend without all three callbacks. */
int rwkv7_sched_create(const rwkv7_sched_config* cfg, const rwkv7_sched_backend* backend,
                       rwkv7_sched** out);
int rwkv7_sched_free(rwkv7_sched* s);

/* Queue a task: prompt[0 .. n) (host, copied, n >= 1, ids in [0, vocab)).
 * *task_id receives its id (1, 2, ... in submission order).  EINVAL for a
 * bad prompt, max_new_tokens < 1 or a stop token outside [-1, vocab). */
int rwkv7_sched_submit(rwkv7_sched* s, const int32_t* prompt, int32_t n,
                       const rwkv7_sched_params* params, int64_t* task_id);

/* Request an abort; it takes effect at the start of the next round (the
 * task then emits RWKV7_EV_FINISHED with RWKV7_FIN_ABORT and frees its slot).
 * EINVAL for an unknown or already finished task. */
int rwkv7_sched_abort(rwkv7_sched* s, int64_t task_id);

/* Run one round (see the top of this file).  stats may be NULL.  A round
 * with nothing to do returns RWKV7_OK with zero counts. */
int rwkv7_sched_step(rwkv7_sched* s, rwkv7_sched_stats* stats);

/* Move up to `cap` pending events, oldest first, into out[]; *n = how many. */
int rwkv7_sched_poll(rwkv7_sched* s, rwkv7_sched_event* out, int32_t cap, int32_t* n);

/* *state = RWKV7_TASK_* of a submitted task; EINVAL for an id never issued. */
int rwkv7_sched_task_state(const rwkv7_sched* s, int64_t task_id, int32_t* state);

/* A backend over a loaded model: reset = rwkv7_reset_slots plus zeroing the
 * slot's row of occ_pool; prefill = rwkv7_prefill_seq, in pieces of at most
 * max_T tokens (prefilling a then b lands where a || b does); step =
 * rwkv7_decode_step over the B rows, then rwkv7_sample over the first
 * n_sample rows' logits, on `stream`, with one host-to-device copy of the
 * round's arrays and one synchronisation for the ids.  A non-zero device
 * error word of either workspace fails the round with RWKV7_EDEVICE.
 * pool / n_slots / ws: as for rwkv7_decode_step (ws sized for max_B rows and
 * max_T prefill tokens); occ_pool: device fp32[n_slots * vocab]; forbidden:
 * device uint8[vocab] or NULL; sample_ws: rwkv7_sample_workspace_bytes(max_B,
 * vocab) bytes.
 * Ownership: the backend allocates nothing.  Its staging lives in two
 * caller-owned, 256-byte aligned buffers whose sizes
 * rwkv7_sched_gpu_backend_bytes gives: dev_buf (device memory: the round's
 * arrays, the ids, max_B logits rows, max_T prefill tokens) and host_buf
 * (pinned host memory, e.g. hipHostMalloc or torch's pin_memory; pageable
 * memory works but makes every copy synchronous).  Both must outlive the
 * backend; rwkv7_sched_gpu_backend_free releases only its host-side record.
 * EINVAL for NULL pointers, max_B outside [1, n_slots], max_T < 1 or
 * misaligned buffers; ESHAPE for buffers or a sample workspace too small.
 * A scheduler driving it needs max_batch <= max_B (a larger round fails
 * with RWKV7_EINVAL and is not advanced). */
int rwkv7_sched_gpu_backend_bytes(const rwkv7_model* model, int32_t max_B, int32_t max_T,
                                  uint64_t* device_bytes, uint64_t* host_bytes);
int rwkv7_sched_gpu_backend(rwkv7_model* model, void* pool, int64_t n_slots, float* occ_pool,
                            const uint8_t* forbidden, int32_t max_B, int32_t max_T, void* ws, uint64_t ws_bytes,
                            void* sample_ws, uint64_t sample_ws_bytes, void* dev_buf, uint64_t dev_bytes,
                            void* host_buf, uint64_t host_bytes, void* stream, rwkv7_sched_backend* out);
int rwkv7_sched_gpu_backend_free(rwkv7_sched_backend* backend);

/* Attach a prefix-state cache (include/rwkv7_prefix.h; NULL detaches) to a
 * GPU backend.  Its sequence prefills then restore the longest cached prefix
 * of prompt[0 .. n-1), prefill only the rest, and store the result under
 * prompt[0 .. n-1), so a prompt that extends an earlier one (the next turn
 * of a conversation, a shared system prompt stored by the caller) skips the
 * tokens already consumed.  *tokens_restored / *tokens_prefilled (either may
 * be NULL) of rwkv7_sched_gpu_backend_counts report the totals. */
struct rwkv7_prefix_cache;
int rwkv7_sched_gpu_backend_set_cache(rwkv7_sched_backend* backend, struct rwkv7_prefix_cache* cache);
int rwkv7_sched_gpu_backend_counts(const rwkv7_sched_backend* backend, int64_t* tokens_restored,
                                   int64_t* tokens_prefilled);

#ifdef __cplusplus
}
#endif

#endif /* RWKV7_SCHED_H */
