// Host-side launchers of the librwkv7 kernels (one translation unit each).
#pragma once

#include "common.h"

// ---------------------------------------------------------------- projections
// Rows of one GEMV workgroup for batch B and reduction length K (segments
// must start and end on multiples of it).
int gemv_rows_per_wg(int B, int K);
// Rows per workgroup that launch_gemv uses for `rows` output rows in `nseg` segments;
// four_waves: the launch has the fused LayerNorm prologue or the value epilogue.
int gemv_launch_rows(int B, int K, int rows, int nseg, bool four_waves);
bool gemv_supported(int B, int K);
hipError_t launch_gemv(const ProjArgs& a, int total_rows, hipStream_t st);
// MFMA path: A (segment activations) fp16.  `part_floats` bounds the split-K
// partial buffer a.part (nullptr: no split).
// With `deferred` non-null, a launch whose only segment is a residual add
// (EPI_RESID into fp32 rows of total_rows) leaves its split-K partials in
// a.part for the caller to add (k_ln_mix does) and sets *deferred to the
// number of K ranges; otherwise (and when not split) it sets 0.
hipError_t launch_gemm(ProjArgs a, int total_rows, int64_t part_floats, hipStream_t st,
                       int* deferred = nullptr);
// Same with an explicit tile (tm, tn: 16 x 16 blocks per wave), stage depth
// ks (64 or 128) and K split; 0 selects the default / automatic value.
hipError_t launch_gemm_cfg(ProjArgs a, int total_rows, int64_t part_floats, int tm, int tn, int ks,
                           int split, hipStream_t st, int* deferred = nullptr);
// `epi`: the epilogue shared by every segment of the launch, -1 when mixed,
// -2 for the key projection with the sparse value fused into it
const char* gemv_kernel_name(int B, int K, int epi, int rows, int nseg, bool four_waves, bool q8);
const char* gemm_kernel_name(int M, int N, int K);
// Whether launch_gemm_cfg supports tile (32 tm x 32 tn), stage depth ks and K loop pipe.
bool gemm_cfg_ok(int tm, int tn, int ks, int pipe);

// ---------------------------------------------------------------- misc
struct ValidateArgs {
  const int* slot_idx;   // caller's slots [n] (decode) or nullptr (prefill)
  const int* tokens;     // caller's tokens [n]
  int n_rows;            // rows with a slot (decode) / 0 (prefill)
  int n_tok;
  int64_t n_slots;
  int vocab;
  int seq_slot;          // prefill: the (host-validated) slot
  int* slots_out;        // [n_rows]
  int* tok_out;          // [n_tok]
  uint32_t* err;
  int64_t* counters;     // pool counters; += 1 per valid row, or += n_tok for prefill
  unsigned int* zero;    // words to clear at the start of a step (arrival counters)
  int n_zero;
};
hipError_t launch_validate(const ValidateArgs& a, hipStream_t st);

// Copy new shift rows u [B][C] into each row's slot (rows with bad slots skipped).
struct CommitArgs {
  const float* u;
  float* pool;
  int64_t slot_stride;
  int64_t n_slots;
  int64_t shift_off;
  const int* slots;
  int B, C;
};
hipError_t launch_commit_shift(const CommitArgs& a, hipStream_t st);
bool gemv_fused_ok(int B, int K);

struct EmbedArgs {
  const half_t* emb;
  const float* g;
  const float* b;
  const int* tok;
  float* x;
  int R, C;
};
hipError_t launch_embed(const EmbedArgs& a, hipStream_t st);
// decode: k_validate's row checks and k_embed in one launch (n_rows == n_tok == R)
hipError_t launch_embed_rows(const ValidateArgs& v, const EmbedArgs& a, hipStream_t st);

enum { LNMIX_DECODE = 0, LNMIX_SEQ = 1, LNMIX_PLAIN = 2 };
struct LnMixArgs {
  float* x;                 // [R][C] residual (updated when partials are folded in)
  const float* parts;       // [nparts][R][C] split-K partials of the residual projection that
                            // precedes (added into x first), or nullptr
  float* x_out;             // nullptr: the folded residual replaces x; else it goes here (needed
                            // in sequence mode, where a row also reads the previous row's x)
  int nparts;
  int C, R, mode;
  const float* g;
  const float* b;
  float* pool;              // slot pool
  int64_t slot_stride;      // floats per slot
  int64_t n_slots;          // slots in the pool (rows with other slots are skipped)
  int64_t shift_off;        // float offset of the shift vector inside a slot
  const int* slots;         // decode: sanitized slot per row (-1 = skip)
  int seq_slot;             // sequence mode: the slot
  float* shift_tmp;         // sequence mode: receives the last row's LN output
  const float* mu;          // [nq][C] token-shift mix coefficients
  int nq;
  void* out;                // [nq][R][C] (q stride out_q_stride elements)
  int out_f16;
  int64_t out_q_stride;
  int ncb;                  // workgroups per row, each owning every ncb-th 512-column pair
                            // (256-column slice for C / 256 odd); 1 = the whole row.  Above
                            // 1: not in sequence mode, and partials need x_out != x
  const float* cp_src;      // side job of workgroup 0: cp_dst[0 .. cp_n) = cp_src[...]
  float* cp_dst;            // (prefill: the previous LayerNorm's last-row output into
  int cp_n;                 // its slot's shift, once nothing reads the old one)
};
hipError_t launch_ln_mix(const LnMixArgs& a, hipStream_t st);

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st);
hipError_t launch_zero_f32(float* dst, int64_t n, hipStream_t st);

struct ResetArgs {
  float* pool;
  int64_t slot_stride;
  int64_t* counters;
  const int* slot_idx;
  int n;
  int64_t n_slots;
  uint32_t* err;
};
hipError_t launch_reset(const ResetArgs& a, hipStream_t st);

// packing
hipError_t launch_pack_matrix(half_t* dst, int64_t dst_ld, const void* src, int src_f16,
                              int64_t rows, int64_t cols, hipStream_t st);
hipError_t launch_pack_transpose(half_t* dst, const void* src, int src_f16, int64_t rows,
                                 int64_t cols, hipStream_t st);
hipError_t launch_pack_vec(float* dst, const void* src, int src_f16, int64_t n, hipStream_t st);
hipError_t launch_fill_vec(float* dst, float v, int64_t n, hipStream_t st);

// sparse channel-mix value
struct CmixArgs {
  const float* pre;           // [B][F] key pre-activations (bias included)
  const unsigned char* mask;  // [F] union over rows of (pre > 0)
  const half_t* Wv;           // [F][C] hidden-major value matrix
  float* x;                   // [B][C] residual: x += value projection
  const float* u_ffn;         // [B][C] new channel-mix shift to commit, or nullptr
  float* pool;
  int64_t slot_stride;
  int64_t n_slots;
  int64_t shift_off;
  const int* slots;
  int B, C, F;
  int* dbg_idx;               // optional: the union active list (ascending)
  int* dbg_cnt;               // optional: its length
};
hipError_t launch_cmix_sparse(const CmixArgs& a, hipStream_t st);

// Fold of the per-workgroup value partial sums written by the fused key
// projection: x[b][c] += sum over workgroups w (in order) of part[w][b][c],
// then the channel-mix shift commit; optionally the union active list.
struct CmixFoldArgs {
  const float* part;          // [nwg][B][C]
  int nwg;
  const unsigned char* mask;  // [F] union over rows of (pre > 0), for the debug list
  float* x;
  const float* u_ffn;
  float* pool;
  int64_t slot_stride;
  int64_t n_slots;
  int64_t shift_off;
  const int* slots;
  int B, C, F;
  int* dbg_idx;
  int* dbg_cnt;
};
hipError_t launch_cmix_fold(const CmixFoldArgs& a, hipStream_t st);
int cmix_sparse_max_b();
const char* cmix_sparse_kernel_name(int B);

// greedy
struct GreedyArgs {
  const float* logits;
  float* occ;
  int64_t n_slots;
  const int* slot_idx;
  const float* presence;
  const float* frequency;
  const float* decay;
  int* ids;
  float* part_val;
  int* part_idx;
  uint32_t* err;
  int B, V, nblk;
};
int greedy_blocks(int V);
hipError_t launch_greedy(const GreedyArgs& a, hipStream_t st);

// penalised temperature / top-k / top-p sampling (V <= 65536): three launches,
// the first two over G workgroups per row, the third one workgroup per row
struct SampleArgs {
  const float* logits;
  float* occ;
  int64_t n_slots;
  const int* slot_idx;
  const float* presence;
  const float* frequency;
  const float* decay;
  const float* temperature;
  const float* top_p;
  const int* top_k;
  const unsigned char* forbidden;   // [V] nonzero = never sampled, or nullptr
  const float* uniform;             // [B] draws in [0, 1)
  int* ids;
  uint32_t* err;
  uint32_t* key;                    // [B][V] workspace: ordered bits of z (0 = not a candidate)
  uint32_t* hcnt;                   // [B][4096] workspace: top-level histogram, token counts
  unsigned long long* hmass;        // [B][4096] workspace: top-level histogram, weight sums
  float* pmax;                      // [B][SAMPLE_MAX_G] workspace: per-workgroup max z
  uint32_t* rown;                   // [B] workspace: candidates per row
  unsigned long long* rowtot;       // [B] workspace: weight sum per row
  int B, V, G;                      // G = sample_groups(B, V)
};
constexpr int SAMPLE_MAX_V = 65536;
constexpr int SAMPLE_MAX_G = 64;
int sample_groups(int B, int V);
hipError_t launch_sample(const SampleArgs& a, hipStream_t st);

// int8 weights: per-row symmetric codes (byte = code + 128) and fp32 scales of W [rows][K]
hipError_t launch_read_stream(const void* buf, int64_t bytes, bool nt, int grid, hipStream_t st);
hipError_t launch_quant_rows(const half_t* W, int64_t rows, int K, uint8_t* q, float* sc, hipStream_t st);

// api.hip, for the scheduler: set the thread's last-error text and return
// `code`; a loaded model's vocabulary size.
struct rwkv7_model;
int lib_fail(int code, const char* msg);
int lib_model_vocab(const rwkv7_model* m);
int64_t lib_model_slot_floats(const rwkv7_model* m);

// ---------------------------------------------------------------- WKV
struct WkvArgs {
  float* pool;
  int64_t slot_stride;
  int64_t n_slots;         // slots in the pool (rows with other slots are skipped)
  int64_t layer_off;       // float offset of this layer inside a slot
  const int* slots;        // decode: per-row slot (-1 = skip)
  int seq_slot;            // sequence kernels: the slot
  int B, C, H, layer;
  const float* rkv;        // [B][3C]: r | k | v
  const float* lin;        // [B][Lin]: tanh(w1 x) | a1 x | v1 x | sigmoid(g1 x)
  int Lin, off_a, off_v, off_g;
  int Dw, Da, Dv, Dg;
  const half_t* w2;        // [C][Dw]
  const half_t* a2;        // [C][Da]
  const half_t* v2;        // [C][Dv]
  const half_t* g2;        // [C][Dg]
  const half_t* adp;       // the four as read by the decode / prep prologue (rwkv7_load packs them)
  const float* w0;
  const float* a0;
  const float* v0;
  const float* k_k;
  const float* k_a;
  const float* r_k;
  const float* lnx_w;
  const float* lnx_b;
  float* vfirst;           // [B][C]
  const float* lo;         // [B][4C] precomputed decay | alpha | value gate | gate, or nullptr
  int ad_rpw;              // many-row decode with lo null: the WKV kernel computes the adapters'
                           // second stage from fp16 lin, this many rows per wave (1, 2, 4); 0 = not
  const float* u_att;      // decode: [B][C] new time-mix shift to commit, or nullptr
  void* yout;              // [B][C] gated, normalised readout (fp32 or fp16)
  int yout_f16;
  // sequence path buffers ([T][C] fp32 each)
  float* q_d;
  float* q_a;
  float* q_b;
  float* q_kt;
  float* q_v;
  float* q_g;
  float* q_bonus;          // [T][H]
  float* q_brk;            // [T][H][2]: b.r and kt.r of each token and head (prefill scan)
  float* q_y;              // raw readout ([wkv_chunk_rows(T)][C] for the chunked scan)
  float* q_rec;            // chunked scan: per (16-token chunk, head) records (wkv_chunk_rec_floats)
};
hipError_t launch_pack_wkv_adapters(half_t* dst, const half_t* w2, const half_t* a2, const half_t* v2,
                                    const half_t* g2, int C, int Dw, int Da, int Dv, int Dg, hipStream_t st);
int wkv_rows_waves(int items);   // waves per workgroup of the many-row WKV decode kernel
hipError_t launch_wkv_decode(const WkvArgs& a, hipStream_t st);
hipError_t launch_wkv_prep(const WkvArgs& a, hipStream_t st);   // sequence: per (t, h)
hipError_t launch_wkv_scan(const WkvArgs& a, hipStream_t st);   // sequence: serial in t
hipError_t launch_wkv_post(const WkvArgs& a, hipStream_t st);   // sequence: GroupNorm + bonus + gate
// Chunked form of launch_wkv_prep + launch_wkv_scan (same q_v, q_g, q_bonus, q_y and
// final state, up to rounding): the head vectors and per-chunk matrices for every (16-token
// chunk, head), then the state carried chunk to chunk.  The adapter outputs come from lo
// when it is set, else they are computed in the chunk kernel from fp16 lin and the
// second-stage matrices (needs wkv_chunk_adapters_ok); q_rec needs wkv_chunk_rec_floats,
// q_y wkv_chunk_rows rows.
hipError_t launch_wkv_chunk_prep(const WkvArgs& a, hipStream_t st);
hipError_t launch_wkv_chunk_scan(const WkvArgs& a, hipStream_t st);
int64_t wkv_chunk_rec_floats(int T, int H);
bool wkv_chunk_adapters_ok(const WkvArgs& a);
// Rows of q_y the chunked scan writes (T rounded up to whole unrolled chunks; rows past T
// are padding).
int wkv_chunk_rows(int T);
