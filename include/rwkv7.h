/*
 * rwkv7.h: C ABI of librwkv7.so, the RWKV-7 decode / prefill hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * What the calls compute.  The RWKV-Server article ("RWKV 批量推理中 Prefill
 * 的正确打开方式") separates two phases (section 2 table):
 *   - decode: one token per sequence per step, an O(1) update of a
 *     fixed-size recurrent state, over B independent sequences;
 *   - prefill: one sequence, T prompt tokens, an O(n) linear scan that must
 *     leave the same state as T single-token steps.
 * Section 4 of the same article argues the two must not share a batch, so
 * they are separate calls here.  Section 5 (Task.prefill) prefills
 * prompt[:-1] and feeds the last prompt token to the first decode step; the
 * per-sequence state is (shift_state, wkv_state, elapsed_t).  The RWKV-Runner
 * Albatross article describes a pool of pre-allocated state slots and
 * presence / frequency penalties with a per-step decay before selection.
 *
 * Conventions
 *  - Every pointer argument documented as "device" is HIP device memory that
 *    the caller allocated and owns (the library allocates nothing on the
 *    device).  The model handle owns host metadata only.
 *  - Every call is asynchronous on the caller's stream (`stream` is a
 *    hipStream_t; NULL = the null stream), except rwkv7_load's validation,
 *    rwkv7_poll_error (synchronises) and the size queries (host only).
 *  - Every call returns a status: RWKV7_OK or an error code.  Host-checkable
 *    misuse (null pointers, sizes, B or T out of range, bad shapes) fails
 *    synchronously and launches nothing; rwkv7_last_error() describes it.
 *    Misuse only the device can see (a token id outside [0, V), a slot index
 *    outside [0, n_slots), a slot listed twice, an all-NaN logits row) sets
 *    bits in a sticky device word read by rwkv7_poll_error; such rows are
 *    computed on a clamped token / skipped slot so nothing is accessed out
 *    of bounds.  After any error the contents of the slots named in that
 *    call are unspecified: reset and prefill them again.
 *  - One call in flight per (model, workspace) at a time.
 */
#ifndef RWKV7_H
#define RWKV7_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define RWKV7_OK 0
#define RWKV7_EINVAL 1     /* bad argument (null pointer, out-of-range count) */
#define RWKV7_ESHAPE 2     /* a tensor or buffer has the wrong shape / size */
#define RWKV7_EHIP 3       /* a HIP runtime call failed */
#define RWKV7_EDEVICE 4    /* rwkv7_poll_error: the device error word was non-zero */
#define RWKV7_ENOTSUP 5    /* configuration not supported by this build */

/* ---- device error bits (rwkv7_poll_error) ---- */
#define RWKV7_ERR_SLOT_RANGE 1u   /* a slot index outside [0, n_slots): row skipped */
#define RWKV7_ERR_SLOT_DUP 2u     /* a slot listed twice in one call: later rows skipped */
#define RWKV7_ERR_TOKEN_RANGE 4u  /* a token id outside [0, vocab): token 0 used */
#define RWKV7_ERR_ALL_NAN 8u      /* rwkv7_greedy: a logits row was all NaN; rwkv7_sample: a row
                                     had no candidate: id 0 */

/* ---- tensor dtypes ---- */
#define RWKV7_F32 0
#define RWKV7_F16 1

/* Model dimensions.  head_size must be 64; n_embd = n_head * 64. */
typedef struct rwkv7_config {
  int32_t n_layer;   /* L */
  int32_t n_embd;    /* C */
  int32_t n_head;    /* H */
  int32_t head_size; /* N = 64 */
  int32_t ffn;       /* F, channel-mix hidden size */
  int32_t d_w;       /* decay adapter rank */
  int32_t d_a;       /* in-context-rate adapter rank */
  int32_t d_v;       /* value-residual adapter rank */
  int32_t d_g;       /* gate adapter rank */
  int32_t vocab;     /* V */
} rwkv7_config;

/* One named input tensor for rwkv7_load.  `data` is a device pointer to a
 * dense row-major array of `shape` in `dtype`.  Names and shapes (matrices
 * are (out, in) like torch.nn.Linear):
 *   emb.weight [V,C]; ln0.{weight,bias} [C]; ln_out.{weight,bias} [C];
 *   head.weight [V,C]; and for each layer l, prefix "blocks.l.":
 *   ln1.{weight,bias}, ln2.{weight,bias} [C];
 *   att.x_r, att.x_w, att.x_k, att.x_v, att.x_a, att.x_g [C] (token-shift mix);
 *   att.w0 [C], att.w1 [d_w,C], att.w2 [C,d_w];
 *   att.a0 [C], att.a1 [d_a,C], att.a2 [C,d_a];
 *   att.v0 [C], att.v1 [d_v,C], att.v2 [C,d_v]  (unused in layer 0);
 *   att.g1 [d_g,C], att.g2 [C,d_g];
 *   att.k_k [C], att.k_a [C], att.r_k [H,N];
 *   att.receptance.weight, att.key.weight, att.value.weight,
 *   att.output.weight [C,C]; att.ln_x.{weight,bias} [C];
 *   ffn.x_k [C], ffn.key.weight [F,C], ffn.key.bias [F], ffn.value.weight [C,F].
 * Matrices may be F16 or F32 (F32 is rounded to fp16 when packed); vectors
 * may be F16 or F32 (kept as fp32). */
typedef struct rwkv7_tensor {
  const char* name;
  int32_t dtype;
  int32_t ndim;
  int64_t shape[4];
  const void* data;
} rwkv7_tensor;

typedef struct rwkv7_model rwkv7_model; /* opaque host handle */

/* ---- sizes (host only) ---- */

/* Bytes of the packed weight buffer rwkv7_load fills. */
int rwkv7_packed_bytes(const rwkv7_config* cfg, uint64_t* bytes);

/* fp32 elements of one slot's state: for each layer, att_shift[C] |
 * ffn_shift[C] | S[H][N][N] (S[h][i][j]: value row i, key column j). */
int rwkv7_slot_floats(const rwkv7_config* cfg, uint64_t* n_floats);

/* Bytes of a pool of n_slots slots: n_slots * slot_floats fp32 values,
 * then (at a 256-byte aligned offset, returned in *counter_offset) one
 * int64 step counter per slot (the elapsed-token count). */
int rwkv7_state_bytes(const rwkv7_config* cfg, int64_t n_slots, uint64_t* bytes,
                      uint64_t* counter_offset);

/* Bytes of the workspace for decode steps of up to max_B rows and prefill
 * calls (any T; processed in chunks of up to max_T tokens; max_T >= 1).
 * The workspace begins with the 4-byte sticky device error word; the caller
 * zero-fills the workspace once before its first use. */
int rwkv7_workspace_bytes(const rwkv7_config* cfg, int32_t max_B, int32_t max_T,
                          uint64_t* bytes);

/* ---- model ---- */

/* Validate the tensor table (every name above exactly once, shapes, dtypes),
 * pack the weights into the caller's `packed` device buffer (>=
 * rwkv7_packed_bytes), and return a host handle in *out.  Packing is queued
 * on `stream`; the input tensors may be freed once it has completed.
 * Layout of the packed buffer: fp16 matrices with the reduction dimension
 * contiguous (r|k|v|lora-in rows fused into one matrix, each block padded to
 * 64 rows), the channel-mix value matrix twice (hidden-major for the sparse
 * path, C-major for the dense path), fp32 vectors.  */
int rwkv7_load(const rwkv7_config* cfg, const rwkv7_tensor* tensors, int32_t n_tensors,
               void* packed, uint64_t packed_bytes, void* stream, rwkv7_model** out);

/* Release the host handle (the packed buffer stays the caller's). */
int rwkv7_free(rwkv7_model* model);

/* Zero the state, both shifts and the step counter of the n listed slots
 * (slot_idx: device int32[n]). */
int rwkv7_reset_slots(const rwkv7_model* model, void* pool, int64_t n_slots,
                      const int32_t* slot_idx, int32_t n, void* ws, uint64_t ws_bytes,
                      void* stream);

/* ---- the hot path ---- */

/* One decode step: row b consumes token_ids[b] on slot slot_idx[b] and
 * writes its next-token logits to logits_out[b*V .. b*V+V) (fp32).
 * slot_idx, token_ids: device int32[B]; logits_out: device fp32[B*V].
 * Slots not listed are left bit-identical; each listed slot's counter +1.
 * 1 <= B <= the workspace's max_B and B <= n_slots. */
int rwkv7_decode_step(rwkv7_model* model, void* pool, int64_t n_slots, int32_t B,
                      const int32_t* slot_idx, const int32_t* token_ids, float* logits_out,
                      void* ws, uint64_t ws_bytes, void* stream);

/* Sequence prefill: advance slot `slot` (host int, 0 <= slot < n_slots) by
 * the T tokens token_ids[0..T) (device int32), updating its state only (no
 * logits).  T = 0 is a no-op.  The result equals T decode steps up to
 * rounding.  Serving code prefills prompt[:-1] and feeds the last prompt
 * token to rwkv7_decode_step. */
int rwkv7_prefill_seq(rwkv7_model* model, void* pool, int64_t n_slots, int32_t slot,
                      const int32_t* token_ids, int32_t T, void* ws, uint64_t ws_bytes,
                      void* stream);

/* Penalised greedy selection over logits [B*V] (device fp32).  For row b
 * with occ = occ_pool[slot_idx[b]*V ..] (device fp32, per-slot token
 * occurrence weights), in separately rounded fp32 ops:
 *   l' = l - (frequency[b]*occ + presence[b]) where occ > 0, else l;
 *   ids_out[b] = lowest index of the maximum of l' (NaN never wins; an
 *                all-NaN row gives 0 and RWKV7_ERR_ALL_NAN);
 *   occ = occ*decay[b]; then occ[id] += 1.
 * presence, frequency, decay: device fp32[B]; ids_out: device int32[B] (may
 * be passed straight back as the next step's token_ids).  `ws` is the
 * decode workspace (or any buffer of rwkv7_greedy_workspace_bytes).
 * A row whose slot lies outside [0, n_slots) (RWKV7_ERR_SLOT_RANGE) or
 * repeats an earlier row's slot (RWKV7_ERR_SLOT_DUP) reads and updates no
 * occurrences: its id is the pick on its unpenalised logits. */
int rwkv7_greedy_workspace_bytes(int32_t B, int32_t V, uint64_t* bytes);
int rwkv7_greedy(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                 const int32_t* slot_idx, const float* presence, const float* frequency,
                 const float* decay, int32_t* ids_out, void* ws, uint64_t ws_bytes,
                 void* stream);

/* rwkv7_greedy for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same selection and occurrence update, bit for bit, with its partial
 * results in a static device array of the library (64 KB per GPU, held until
 * the process ends) instead of a caller workspace.  It calls no hipMalloc /
 * hipFree.  Limit: B * ceil(V / 2048) <= 8192 row-blocks (B <= 256 at
 * V = 65536); larger calls fail with RWKV7_ESHAPE before any launch.  Device
 * error bits (as for rwkv7_greedy) are ORed into *flags_out (device uint32,
 * cleared by the caller).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, two threads) race and must be
 * serialised by the caller.  The stream must belong to the current device. */
int rwkv7_greedy_noalloc(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                         const int32_t* slot_idx, const float* presence, const float* frequency,
                         const float* decay, int32_t* ids_out, uint32_t* flags_out, void* stream);

/* Penalised temperature / top-k / top-p sampling over logits [B*V] (device
 * fp32, V <= 65536).  The Albatross article (RWKV-Runner backend) names the
 * adapter's sampling defaults (temperature 1.0, top_p 0.3, top_k 0) and the
 * worker's per-step order: forbidden-token mask, presence / frequency
 * penalty, batched sampling; it gives no formulas.  Per row b, with occ as
 * in rwkv7_greedy:
 *   l' as in rwkv7_greedy; z = l' / temperature[b] (fp32);
 *   candidates: tokens with forbidden[v] == 0 (forbidden may be NULL) and z
 *     finite;
 *   order: z descending (IEEE total order, -0 after +0), then index ascending;
 *   weight: floor(exp(z - max z) * 2^31), z - max z in fp64 and exp by a
 *     fixed sequence of fp64 operations, each rounded to nearest even and none
 *     fused (Cody-Waite reduction with ln2 split at 2^-40, the degree-13
 *     Taylor polynomial by Horner's rule, scaling by 2^n; within 2 ulp of
 *     exp), so every implementation of the definition gets the same weights;
 *   top-k (0 < top_k[b] < candidates): the first top_k[b] candidates;
 *   top-p (top_p[b] < 1): the shortest non-empty prefix of those whose weight
 *     sum reaches ceil(top_p[b] * their total) (fp64 product);
 *   draw: u = uniform[b] clamped to [0, 1 - 2^-24]; the first kept token whose
 *     running weight sum exceeds floor(u * kept total) (fp64 product);
 *   temperature not > 0: z = l' and top_k = 1 (the greedy pick);
 *   occ = occ*decay[b]; then occ[id] += 1.
 * Every decision is integer arithmetic, so the result does not depend on
 * timing.  A row without candidates gives 0 and RWKV7_ERR_ALL_NAN.  Slots
 * outside the pool or repeated as in rwkv7_greedy set RWKV7_ERR_SLOT_RANGE /
 * RWKV7_ERR_SLOT_DUP, and that row reads and updates no occurrences.
 * temperature, top_p, uniform, presence, frequency, decay: device fp32[B];
 * top_k: device int32[B]; forbidden: device uint8[V] or NULL; ids_out:
 * device int32[B].  The caller draws the uniforms.  `ws`: a device buffer of
 * rwkv7_sample_workspace_bytes (its first word is the error word read by
 * rwkv7_poll_error; about 4 V + 49 KB per row).  EINVAL for null pointers
 * or sizes, ENOTSUP for V > 65536, ESHAPE for a short workspace; nothing is
 * launched then. */
int rwkv7_sample_workspace_bytes(int32_t B, int32_t V, uint64_t* bytes);
int rwkv7_sample(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                 const int32_t* slot_idx, const float* presence, const float* frequency,
                 const float* decay, const float* temperature, const float* top_p,
                 const int32_t* top_k, const uint8_t* forbidden, const float* uniform,
                 int32_t* ids_out, void* ws, uint64_t ws_bytes, void* stream);

/* ---- int8 weights (small-batch decode) ----
 * The Albatross article (RWKV-Runner backend, "boundaries and follow-up
 * route") names int8 quantised weights as a performance item it leaves out,
 * without a scheme.  A single-token step streams every weight once, so this
 * build offers symmetric per-row int8 copies of the matrices the small-batch
 * path streams: the fused r | k | v | adapter-input matrix, W_o, the channel-mix
 * key, the channel-mix value (per hidden unit, as the sparse path reads it)
 * and the head.  Per row: m = max |w| of the packed fp16 row, s = m / 127 in
 * fp32, code = rint(w / s) (ties to even) clamped to [-127, 127], 0 where
 * s = 0; the weight used is code * s.  Bytes hold code + 128.  The adapters'
 * second stage and the embedding stay fp16; larger batches and prefill keep
 * the fp16 MFMA path.
 *
 * rwkv7_int8_bytes: size of the caller's buffer for those copies.
 * rwkv7_quantize_int8: fill it from the packed weights (queued on `stream`;
 * the buffer must stay allocated while the model is used with
 * RWKV7_OPT_INT8 = 1).  ESHAPE for a short buffer. */
int rwkv7_int8_bytes(const rwkv7_config* cfg, uint64_t* bytes);
int rwkv7_quantize_int8(rwkv7_model* model, void* buf, uint64_t bytes, void* stream);

/* Device addresses of one int8 matrix for tests: which = 0 fused input
 * matrix, 1 W_o, 2 channel-mix key, 3 channel-mix value (hidden-major) of
 * `layer`, 4 the head; *rows x *K bytes (code + 128) and *rows fp32 scales.
 * ENOTSUP before rwkv7_quantize_int8. */
int rwkv7_debug_int8_matrix(const rwkv7_model* model, int32_t layer, int32_t which, const void** codes,
                            const float** scales, int64_t* rows, int32_t* K);

/* ---- errors ---- */

/* Synchronise `stream`, read and clear the sticky device error word at the
 * start of `ws`.  *flags = the RWKV7_ERR_* bits; returns RWKV7_EDEVICE if
 * any bit was set, else RWKV7_OK. */
int rwkv7_poll_error(void* ws, void* stream, uint32_t* flags);

const char* rwkv7_status_string(int status);

/* Text of the last host-side error on this thread ("" if none). */
const char* rwkv7_last_error(void);

/* ---- tuning and measurement ---- */

#define RWKV7_OPT_USE_GRAPH 1      /* 1 (default): replay a HIP graph per decode shape */
#define RWKV7_OPT_GEMV_MAX_B 2     /* largest B served by the fp32-activation GEMV path */
#define RWKV7_OPT_SPARSE_MAX_B 3   /* largest B served by the sparse channel-mix value path */
#define RWKV7_OPT_KERNEL_TIMING 4  /* 1: bracket every launch with HIP events (no graph) */
#define RWKV7_OPT_PREFILL_CHUNK 5  /* tokens per prefill chunk (default 2048; halved until the
                                      workspace holds it) */
#define RWKV7_OPT_FUSE_LN 6        /* 1 (default): LayerNorm + token shift inside the GEMV path */
#define RWKV7_OPT_FUSE_VALUE 7     /* 1 (default): on the GEMV path (B <= 2, sparse), each key
                                      workgroup also adds its active rows' value contributions
                                      into per-workgroup partial sums, folded in a fixed order */
#define RWKV7_OPT_PREFILL_SCAN 14  /* WKV recurrence of rwkv7_prefill_seq: 0 (default) chunked
                                      for chunks of >= 32 tokens, else serial; 1 serial (one
                                      token after another); 2 chunked (16-token blocks in closed
                                      form, the state carried block to block) */
/* Tile plan of one MFMA projection (B > GEMV_MAX_B and prefill); 0 (default) = the built-in
   plan for the shape.  Otherwise the decimal digits "T N KKK P S" of the value give the
   workgroup tile (32 T rows x 32 N columns, T in {1, 2, 4}, N in {2, 4}; also T = 4, N = 1
   with loop 3 and 64- or 128-deep stages, T in {2, 4}, N = 5
   with loop 3, and T in {2, 4}, N = 8 with loop 4, both with 64-deep stages, and T = N = 8
   or T = 8, N = 10 (written as the digits 9 0: 256 x 320 tiles) with loop 4 and 32-deep
   stages), the K stage depth
   KKK (32, 64 or 128), the K loop P (0 plain, 1 pipelined LDS reads, 2 two stages of global
   loads in flight, 3 stages loaded straight into a three-deep LDS ring, 4 the same with
   eight waves (T, N in {2, 4}), 5 a deeper LDS ring of as many stages as fit about 144 KB
   (up to nine; one workgroup per CU), 6 the same in about 72 KB (two per CU), for KKK in
   {64, 128}; 3 to 6 fall back to 2 (0 for 4 x 4 tiles) where K is not a
   multiple of KKK) and the K split S (0 automatic); e.g. 2206430 = 64 x 64
   tiles, 64-deep stages, loop 3, automatic split.  Unsupported combinations fail with
   EINVAL. */
#define RWKV7_OPT_GEMM_PLAN_PROJ_IN 8     /* r, k, v and the adapters' first stage */
#define RWKV7_OPT_GEMM_PLAN_ADAPTERS 9    /* the adapters' second stage (decay, alpha, gates) */
#define RWKV7_OPT_GEMM_PLAN_PROJ_OUT 10   /* W_o + residual */
#define RWKV7_OPT_GEMM_PLAN_CMIX_KEY 11   /* channel-mix key */
#define RWKV7_OPT_GEMM_PLAN_CMIX_VALUE 12 /* dense channel-mix value */
#define RWKV7_OPT_GEMM_PLAN_HEAD 13       /* output head */

#define RWKV7_OPT_INT8 15  /* 1: decode steps of B <= 2 on the GEMV path stream the int8 copies made
                              by rwkv7_quantize_int8 (ENOTSUP before it); 0 (default): fp16 */
#define RWKV7_OPT_LN_SPLIT 16  /* workgroups per row of the LayerNorm + token-shift kernel on the
                                 MFMA decode path: 0 (default) automatic (256 / B, at least
                                 2 for B <= 256, 1 above), n > 0 at most n (capped at C / 512,
                                 or C / 256 for C / 256 odd).  Each workgroup reads the whole row for the
                                 statistics and loads and writes its share of the columns;
                                 results do not depend on it */
#define RWKV7_OPT_WKV_ADAPTERS 17  /* the adapters' second stage (decay, alpha, value gate, gate) on
                                      the MFMA decode path: 0 (default) inside the WKV kernel, one
                                      workgroup per head and block of rows, with the rows per wave
                                      chosen for B and the ranks (1; 2 up to 128 rows where the
                                      ranks sum past 512); 1 a separate MFMA projection whose
                                      outputs the WKV kernel reads; 2, 3, 4 inside the WKV kernel
                                      with 1, 2, 4 rows per wave.  Shapes without an instantiated
                                      adapter step
                                      (ranks other than 32/32/32/64, 64/64/32/320, 128/128/64/480)
                                      always take 1 */
int rwkv7_set_option(rwkv7_model* model, int32_t key, int64_t value);
int rwkv7_get_option(const rwkv7_model* model, int32_t key, int64_t* value);

/* Kernel classes for rwkv7_kernel_timing. */
#define RWKV7_K_LN_MIX 0
#define RWKV7_K_PROJ_IN 1
#define RWKV7_K_WKV 2
#define RWKV7_K_PROJ_OUT 3
#define RWKV7_K_CMIX_KEY 4
#define RWKV7_K_CMIX_VALUE 5
#define RWKV7_K_HEAD 6
#define RWKV7_K_OTHER 7
#define RWKV7_K_COUNT 8

/* Per-class launch count and summed duration (ms, from HIP events recorded
 * on the caller's stream) of launches made while RWKV7_OPT_KERNEL_TIMING
 * was 1; synchronises the recorded events.  `reset` != 0 clears them. */
int rwkv7_kernel_timing(rwkv7_model* model, int32_t kernel_class, double* total_ms,
                        int64_t* launches, int32_t reset);

/* Measure one kernel class in isolation: enqueue, `iters` times back to
 * back, the launch(es) that class makes at `layer` (0..n_layer-1; n_layer =
 * the head) of a decode step of B rows with these arguments, between two
 * HIP events on `stream`; synchronise and return the average per iteration
 * in *avg_ms.  `layer` = -1 (per-layer classes only) sweeps the class over
 * layers 0..n_layer-1 `iters` times instead, so consecutive launches read
 * different weights as they do inside a step; *avg_ms is then the average
 * per launch.  Run it after a normal decode step with the same arguments so
 * the workspace holds that step's activations.  It rewrites the listed
 * slots' state and the workspace (the repeated launches are real), so reset
 * those slots before using them again. */
int rwkv7_time_kernel(rwkv7_model* model, void* pool, int64_t n_slots, int32_t B,
                      const int32_t* slot_idx, const int32_t* token_ids, float* logits_out,
                      int32_t kernel_class, int32_t layer, int32_t iters, void* ws,
                      uint64_t ws_bytes, void* stream, double* avg_ms);

/* Measured streaming-read bandwidth: `iters` back-to-back launches of a
 * plain kernel that reads every 16-byte chunk of `buf` (device memory,
 * `bytes` long) once (8 workgroups of 256 threads per CU, grid-stride,
 * non-temporal loads when `nontemporal` != 0), after one untimed launch;
 * synchronises `stream` and returns GB/s (1e9 bytes) in *gbs.  The buffer is
 * only read.  For reporting the attainable HBM rate next to the 8 TB/s peak
 * (a buffer far beyond the 256 MB MALL), or the MALL's rate on a re-read of
 * a small one. */
int rwkv7_read_bandwidth(const void* buf, uint64_t bytes, int32_t nontemporal, int32_t iters, void* stream,
                         double* gbs);

/* Name of the kernel symbol a class launches on the decode path for batch B
 * (for matching rocprofv3 output), or "" for an unknown class. */
const char* rwkv7_kernel_name(const rwkv7_model* model, int32_t kernel_class, int32_t B);

/* ---- test hook ---- */

/* Device addresses, inside `ws`, of the sparse channel-mix buffers of the
 * last layer of the most recent decode step of B rows made with this
 * workspace: pre-activations (fp32 [B][F], bias included), the union mask
 * (uint8 [F], 1 where any row's pre-activation is > 0), the ascending
 * active list (int32 [F]) and its length (int32).  Valid only when that
 * step took the sparse path (B <= RWKV7_OPT_SPARSE_MAX_B).  The pages'
 * sparse channel-mix skips value rows whose activation is zero; this hook
 * lets a test check the skipped set exactly. */
int rwkv7_debug_cmix_buffers(const rwkv7_model* model, void* ws, int32_t B, void** pre,
                             void** mask, void** active, void** active_count);

/* Device address, inside `ws`, of the time-mix output of the last layer of
 * the most recent decode step of B rows made with this workspace, before
 * the output projection: (GroupNorm(S r) + bonus * v) * g per row, [B][C].
 * *is_f16 = 1 when that step stores it in fp16 (the MFMA path, B above the
 * GEMV limit), 0 for fp32.  The RWKV-Server article's section 2 table gives
 * the per-token state update whose readout this is; the hook lets a test
 * compare the WKV stage on its own, ahead of W_o. */
int rwkv7_debug_wkv_out(const rwkv7_model* model, void* ws, int32_t B, void** out, int32_t* is_f16);

#ifdef __cplusplus
}
#endif

#endif /* RWKV7_H */
