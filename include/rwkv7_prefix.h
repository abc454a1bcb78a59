/* rwkv7_prefix.h: slot snapshots, slot offload and a prefix-state cache.
 *
 * An RWKV-7 sequence's whole history is its fixed-size slot (the recurrent
 * state, both token shifts and the step counter), so a prompt prefix that
 * was prefilled once can be reused by restoring that slot instead of
 * recomputing it.  The RWKV-Server article ("RWKV-Server design") moves a
 * task's state to the host when it leaves the batch and back when it is
 * picked again; the Albatross article ("boundaries and follow-up route")
 * lists a prefix-state cache whose first version is an in-memory LRU, with
 * persistence left for later.  Reading, MI355X-first:
 *
 *   * a snapshot is one slot copied out: slot_floats fp32 values in the pool's
 *     slot layout, then the int64 step counter (rwkv7_snapshot_bytes);
 *   * the cache keeps snapshots keyed by the exact token sequence that
 *     produced them, in a device arena (HBM: restoring one is a device copy)
 *     and, when that is full, an optional host arena (pinned memory: slot
 *     offload); its least recently used device entry moves to the host arena,
 *     and the least recently used host entry is dropped;
 *   * a lookup restores the longest cached prefix of a token sequence into a
 *     slot and returns its length; the state after it equals that of a slot
 *     which consumed those tokens itself, bit for bit (it is a copy).
 *
 * Every copy is queued on the caller's stream; calls of one cache must be
 * ordered on one stream (they are host calls that queue device copies).
 * Errors: RWKV7_EINVAL for null pointers or out-of-range arguments,
 * RWKV7_ESHAPE for arenas too small for one snapshot, RWKV7_EHIP for a failed
 * copy; nothing is queued then. */
#ifndef RWKV7_PREFIX_H
#define RWKV7_PREFIX_H

#include <stdint.h>

#include "rwkv7.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of one slot snapshot: slot_floats * 4 (the slot's state) + 8 (its
 * step counter). */
int rwkv7_snapshot_bytes(const rwkv7_config* cfg, uint64_t* bytes);

/* Copy slot `slot` of the pool into dst (device or host memory, at least
 * rwkv7_snapshot_bytes) / from src into the slot, on `stream`.  The pool and
 * n_slots are those of rwkv7_decode_step.  Host memory should be pinned for
 * the copy to be asynchronous; the caller synchronises the stream before
 * reading an exported snapshot on the host. */
int rwkv7_slot_export(const rwkv7_model* model, const void* pool, int64_t n_slots, int32_t slot,
                      void* dst, void* stream);
int rwkv7_slot_import(const rwkv7_model* model, void* pool, int64_t n_slots, int32_t slot,
                      const void* src, void* stream);

typedef struct rwkv7_prefix_cache rwkv7_prefix_cache; /* opaque host handle */

typedef struct rwkv7_prefix_stats {
  int64_t lookups, hits, hit_tokens;  /* lookups, those that matched, tokens matched in all */
  int64_t stores, offloads, drops;    /* snapshots stored, moved to the host arena, dropped */
  int32_t device_entries, host_entries;
  int32_t device_capacity, host_capacity;
} rwkv7_prefix_stats;

/* A cache over `arena` (device memory, arena_bytes) and, optionally,
 * `host_arena` (pinned host memory, host_bytes; NULL / 0 for none).  Each
 * arena holds floor(bytes / snapshot bytes rounded up to 256) snapshots; the
 * device arena must hold at least one.  The arenas stay the caller's. */
int rwkv7_prefix_cache_create(const rwkv7_model* model, void* arena, uint64_t arena_bytes,
                              void* host_arena, uint64_t host_bytes, rwkv7_prefix_cache** out);
int rwkv7_prefix_cache_free(rwkv7_prefix_cache* cache);

/* Store the state of `slot`, which has consumed exactly tokens[0 .. n)
 * (host int32, n >= 1), under that sequence.  Storing a sequence that is
 * already cached only marks it recently used. */
int rwkv7_prefix_cache_store(rwkv7_prefix_cache* cache, const void* pool, int64_t n_slots,
                             int32_t slot, const int32_t* tokens, int32_t n, void* stream);

/* Find the longest cached sequence equal to tokens[0 .. p) with 1 <= p <= n,
 * restore it into `slot` and set *matched = p; with no match, *matched = 0
 * and the slot is untouched. */
int rwkv7_prefix_cache_lookup(rwkv7_prefix_cache* cache, void* pool, int64_t n_slots, int32_t slot,
                              const int32_t* tokens, int32_t n, int32_t* matched, void* stream);

int rwkv7_prefix_cache_stats(const rwkv7_prefix_cache* cache, rwkv7_prefix_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* RWKV7_PREFIX_H */
