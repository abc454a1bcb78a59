// Host side of librwkv7: argument validation, packed-weight and workspace
// layouts, the decode-step and prefill launch sequences, HIP-graph replay
// of decode steps, and per-kernel event timing.  See include/rwkv7.h for the
// contract of every exported call.
#include "launch.h"
#include "../../include/rwkv7.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <string>
#include <tuple>
#include <vector>

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(RWKV7_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                      \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

constexpr uint64_t ALIGN = 256;
// shortest prefill chunk that takes the chunked WKV scan under the automatic choice
constexpr int PREFILL_CHUNKED_MIN_T = 32;
// decode graphs kept instantiated (least recently used evicted): a serving
// loop's batch size wanders over 1 .. max_batch as tasks come and go
constexpr size_t GRAPH_CACHE = 128;
inline uint64_t align_up(uint64_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline int pad64(int x) { return (x + 63) / 64 * 64; }

struct Dims {
  int L, C, H, N, F, Dw, Da, Dv, Dg, V;
  int Dwp, Dap, Dvp, Dgp, Lin, Nin;
  int64_t layer_floats;  // floats per layer inside a slot
  int64_t slot_floats;
};

int check_config(const rwkv7_config* c, Dims* d) {
  if (!c) return fail(RWKV7_EINVAL, "config is NULL");
  if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->ffn < 1 || c->vocab < 1)
    return fail(RWKV7_ESHAPE, "config dimensions must be positive");
  if (c->head_size != 64) return fail(RWKV7_ENOTSUP, "head_size must be 64 (got %d)", c->head_size);
  if (c->n_embd != c->n_head * 64) return fail(RWKV7_ESHAPE, "n_embd must equal n_head*64");
  if (c->n_embd % 256 || c->n_embd > 4096)
    return fail(RWKV7_ENOTSUP, "n_embd must be a multiple of 256 and <= 4096 (got %d)", c->n_embd);
  if (c->ffn % 128) return fail(RWKV7_ENOTSUP, "ffn must be a multiple of 128 (got %d)", c->ffn);
  const int ds[4] = {c->d_w, c->d_a, c->d_v, c->d_g};
  for (int i = 0; i < 4; ++i)
    if (ds[i] < 8 || ds[i] % 8)
      return fail(RWKV7_ENOTSUP, "adapter ranks must be positive multiples of 8");
  if ((c->d_w + c->d_a + c->d_v + c->d_g) % 32)
    return fail(RWKV7_ENOTSUP, "the adapter ranks must sum to a multiple of 32");
  Dims r;
  r.L = c->n_layer; r.C = c->n_embd; r.H = c->n_head; r.N = 64; r.F = c->ffn;
  r.Dw = c->d_w; r.Da = c->d_a; r.Dv = c->d_v; r.Dg = c->d_g; r.V = c->vocab;
  r.Dwp = pad64(r.Dw); r.Dap = pad64(r.Da); r.Dvp = pad64(r.Dv); r.Dgp = pad64(r.Dg);
  r.Lin = r.Dwp + r.Dap + r.Dvp + r.Dgp;
  if (r.Lin > 1024) return fail(RWKV7_ENOTSUP, "adapter ranks too large (padded sum %d > 1024)", r.Lin);
  r.Nin = 3 * r.C + r.Lin;
  r.layer_floats = 2LL * r.C + (int64_t)r.H * 64 * 64;
  r.slot_floats = r.layer_floats * r.L;
  if (d) *d = r;
  return RWKV7_OK;
}

// ------------------------------------------------------------ packed layout
struct LayerPtrs {
  half_t *w_in, *w2, *a2, *v2, *g2, *w_o, *w_key, *w_val_hm, *w_val_km;
  half_t* wkv_ad;   // w2 | a2 | v2 | g2 per head in the order the WKV threads read them
  float *ln1_w, *ln1_b, *ln2_w, *ln2_b, *lnx_w, *lnx_b, *mu6, *w0, *a0, *v0, *k_k, *k_a, *r_k,
      *mu_k, *b_key;
};

struct Packed {
  half_t *emb, *head;
  float *ln0_w, *ln0_b, *lnout_w, *lnout_b;
  std::vector<LayerPtrs> layers;
  uint64_t bytes;
};

// int8 copies of the matrices the small-batch GEMV path streams: per-row
// symmetric codes stored as code + 128, and fp32 row scales.
struct Q8Layer {
  uint8_t *w_in, *w_o, *w_key, *w_val;
  float *s_in, *s_o, *s_key, *s_val;
};
struct Q8 {
  uint8_t* head;
  float* s_head;
  std::vector<Q8Layer> layers;
  uint64_t bytes;
};

// With base == nullptr only the size is computed.
Q8 q8_layout(const Dims& d, char* base) {
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return p;
  };
  const uint64_t C = d.C, F = d.F, V = d.V;
  Q8 q;
  q.head = (uint8_t*)take(V * C);
  q.s_head = (float*)take(V * 4);
  for (int l = 0; l < d.L; ++l) {
    Q8Layer y;
    y.w_in = (uint8_t*)take((uint64_t)d.Nin * C);
    y.s_in = (float*)take((uint64_t)d.Nin * 4);
    y.w_o = (uint8_t*)take(C * C);
    y.s_o = (float*)take(C * 4);
    y.w_key = (uint8_t*)take(F * C);
    y.s_key = (float*)take(F * 4);
    y.w_val = (uint8_t*)take(F * C);
    y.s_val = (float*)take(F * 4);
    q.layers.push_back(y);
  }
  q.bytes = off;
  return q;
}

// With base == nullptr only the size is computed.
Packed pack_layout(const Dims& d, char* base) {
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return p;
  };
  const uint64_t C = d.C, F = d.F, V = d.V;
  Packed p;
  p.emb = (half_t*)take(V * C * 2);
  p.head = (half_t*)take(V * C * 2);
  p.ln0_w = (float*)take(C * 4);
  p.ln0_b = (float*)take(C * 4);
  p.lnout_w = (float*)take(C * 4);
  p.lnout_b = (float*)take(C * 4);
  for (int l = 0; l < d.L; ++l) {
    LayerPtrs q;
    q.w_in = (half_t*)take((uint64_t)d.Nin * C * 2);
    q.w2 = (half_t*)take(C * d.Dw * 2);
    q.a2 = (half_t*)take(C * d.Da * 2);
    q.v2 = (half_t*)take(C * d.Dv * 2);
    q.g2 = (half_t*)take(C * d.Dg * 2);
    q.wkv_ad = (half_t*)take(C * (d.Dw + d.Da + d.Dv + d.Dg) * 2);
    q.w_o = (half_t*)take(C * C * 2);
    q.w_key = (half_t*)take(F * C * 2);
    q.w_val_hm = (half_t*)take(F * C * 2);
    q.w_val_km = (half_t*)take(C * F * 2);
    q.ln1_w = (float*)take(C * 4); q.ln1_b = (float*)take(C * 4);
    q.ln2_w = (float*)take(C * 4); q.ln2_b = (float*)take(C * 4);
    q.lnx_w = (float*)take(C * 4); q.lnx_b = (float*)take(C * 4);
    q.mu6 = (float*)take(6 * C * 4);
    q.w0 = (float*)take(C * 4); q.a0 = (float*)take(C * 4); q.v0 = (float*)take(C * 4);
    q.k_k = (float*)take(C * 4); q.k_a = (float*)take(C * 4); q.r_k = (float*)take(C * 4);
    q.mu_k = (float*)take(C * 4);
    q.b_key = (float*)take(F * 4);
    p.layers.push_back(q);
  }
  p.bytes = off;
  return p;
}

// ------------------------------------------------------------ workspace layout
struct Ws {
  uint32_t* err;
  int *slots, *tok;
  float *x, *x2, *xq, *rkv, *lin, *lo, *vfirst, *yg, *xk, *pre, *xo, *shift_tmp, *shift_tmp2, *u_att, *u_ffn;
  unsigned char* mask;
  int *dbg_idx, *dbg_cnt;
  float *q_d, *q_a, *q_b, *q_kt, *q_v, *q_g, *q_bonus, *q_brk, *q_y;
  float* q_rec;           // chunked prefill scan records
  float* part;            // split-K partial sums of the MFMA projections
  int64_t part_floats;
  float* vpart;           // value partials of the fused key projection
  int vpart_nwg;
  uint64_t bytes;
};

Ws ws_layout(const Dims& d, int R, char* base) {
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return p;
  };
  const uint64_t C = d.C, F = d.F, r = R;
  Ws w;
  w.err = (uint32_t*)take(4);
  w.slots = (int*)take(r * 4);
  w.tok = (int*)take(r * 4);
  w.x = (float*)take(r * C * 4);
  w.x2 = (float*)take(r * C * 4);   // prefill: the other residual buffer
  w.xq = (float*)take(6 * r * C * 4);
  w.rkv = (float*)take(3 * r * C * 4);
  w.lin = (float*)take(r * d.Lin * 4);
  w.lo = (float*)take(r * 4 * C * 4);
  w.vfirst = (float*)take(r * C * 4);
  w.yg = (float*)take(r * C * 4);
  w.xk = (float*)take(r * C * 4);
  w.pre = (float*)take(r * F * 4);
  w.mask = (unsigned char*)take(F);
  w.xo = (float*)take(r * C * 4);
  w.shift_tmp = (float*)take(C * 4);
  w.shift_tmp2 = (float*)take(C * 4);   // prefill: the channel-mix LayerNorm's last row
  w.dbg_idx = (int*)take(F * 4);
  w.dbg_cnt = (int*)take(4);
  w.u_att = (float*)take(r * C * 4);
  w.u_ffn = (float*)take(r * C * 4);
  w.q_d = (float*)take(r * C * 4);
  w.q_a = (float*)take(r * C * 4);
  w.q_b = (float*)take(r * C * 4);
  w.q_kt = (float*)take(r * C * 4);
  w.q_v = (float*)take(r * C * 4);
  w.q_g = (float*)take(r * C * 4);
  w.q_y = (float*)take((uint64_t)wkv_chunk_rows(R) * C * 4);   // padded rows for the chunked scan
  w.q_bonus = (float*)take(r * d.H * 4);
  w.q_brk = (float*)take(r * d.H * 2 * 4);
  w.q_rec = (float*)take((uint64_t)wkv_chunk_rec_floats(R, d.H) * 4);
  w.part_floats = (int64_t)(r * 16 * C);
  w.part = (float*)take(r * 16 * C * 4);
  // value partials of the fused key projection (B <= 2 rows, 16 key rows per workgroup)
  w.vpart_nwg = (int)((F + 15) / 16);
  w.vpart = (float*)take((uint64_t)w.vpart_nwg * (r < 2 ? r : 2) * C * 4);
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------ timing
struct TimedLaunch {
  int cls;
  hipEvent_t a, b;
};

}  // namespace

struct GraphKey {
  int B;
  const void *pool, *slots, *tok, *logits, *ws;
  int64_t n_slots;
  int gemv_max, sparse_max;
  bool operator<(const GraphKey& o) const {
    return std::tie(B, pool, slots, tok, logits, ws, n_slots, gemv_max, sparse_max) <
           std::tie(o.B, o.pool, o.slots, o.tok, o.logits, o.ws, o.n_slots, o.gemv_max, o.sparse_max);
  }
};

struct GraphEntry {
  hipGraph_t graph;
  hipGraphExec_t exec;
  uint64_t last_use;
};

struct rwkv7_model {
  rwkv7_config cfg;
  Dims d;
  Packed pk;
  int64_t opt_graph = 1, opt_gemv_max = 2, opt_sparse_max = 4, opt_timing = 0, opt_chunk = 2048,
          opt_fuse_ln = 1, opt_fuse_value = 1, opt_prefill_scan = 0, opt_int8 = 0, opt_ln_split = 0,
          opt_wkv_ad = 0;
  Q8 q8{};
  bool has_q8 = false;
  // tile plan per MFMA projection (RWKV7_OPT_GEMM_PLAN_* order), 0 = built-in
  int64_t opt_plan[6] = {0, 0, 0, 0, 0, 0};
  std::vector<TimedLaunch> pending;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> free_events;
  double t_ms[RWKV7_K_COUNT] = {0};
  int64_t t_n[RWKV7_K_COUNT] = {0};
  std::map<GraphKey, GraphEntry> graphs;
  uint64_t use_clock = 0;
  hipStream_t cap_stream = nullptr;
  int device = 0;
};

namespace {

// Runs one launch, bracketed by events when timing is on.
// Restricts a launch sequence to one kernel class at one layer, repeated
// (used to time a kernel in isolation).  layer == n_layer selects the head.
struct Filter {
  int cls = -1;
  int layer = -1;
  bool any_layer = false;   // match the class at every layer
  int repeat = 1;
};

struct Launcher {
  rwkv7_model* m;
  hipStream_t st;
  bool timing;
  const Filter* flt = nullptr;
  int layer = -1;
  template <class F>
  int run(int cls, const char* what, F&& f) {
    if (flt && flt->cls >= 0) {
      if (cls != flt->cls || (!flt->any_layer && layer != flt->layer)) return RWKV7_OK;
      for (int i = 0; i < flt->repeat; ++i) {
        hipError_t e = f();
        if (e != hipSuccess) return hip_fail(e, what);
      }
      return RWKV7_OK;
    }
    hipEvent_t ea = nullptr, eb = nullptr;
    if (timing) {
      if (!m->free_events.empty()) {
        ea = m->free_events.back().first;
        eb = m->free_events.back().second;
        m->free_events.pop_back();
      } else {
        HIP_TRY(hipEventCreate(&ea), "hipEventCreate");
        HIP_TRY(hipEventCreate(&eb), "hipEventCreate");
      }
      HIP_TRY(hipEventRecord(ea, st), "hipEventRecord");
    }
    hipError_t e = f();
    if (e != hipSuccess) return hip_fail(e, what);
    if (timing) {
      HIP_TRY(hipEventRecord(eb, st), "hipEventRecord");
      m->pending.push_back({cls, ea, eb});
    }
    return RWKV7_OK;
  }
};

#define RUN(cls, what, expr)                                   \
  do {                                                         \
    int rc_ = L.run(cls, what, [&]() -> hipError_t { return (expr); }); \
    if (rc_ != RWKV7_OK) return rc_;                           \
  } while (0)

Seg mkseg(int row0, int row1, int epi, const void* act, int ld_act, void* out, int ld_out,
          const float* aux = nullptr, unsigned char* mask = nullptr) {
  Seg s;
  memset(&s, 0, sizeof s);
  s.row0 = row0; s.row1 = row1; s.epi = epi;
  s.act = act; s.ld_act = ld_act; s.out = out; s.ld_out = ld_out;
  s.aux = aux; s.mask = mask;
  return s;
}

// A tile plan code (RWKV7_OPT_GEMM_PLAN_*): decimal digits tm tn kkk p s.
struct PlanCode {
  int tm, tn, ks, pipe, split;
};
// "T N KKK P S"; the pair "9 0" (= 8 * 10 + 10) stands for T = 8, N = 10
static PlanCode decode_plan(int64_t v) {
  const int tt = (int)(v / 100000 % 100);
  return {tt == 90 ? 8 : tt / 10, tt == 90 ? 10 : tt % 10, (int)(v / 100 % 1000), (int)(v / 10 % 10),
          (int)(v % 10)};
}

// `deferred` (MFMA path): see launch_gemm; the GEMV path never defers.
hipError_t proj(bool gemv, ProjArgs& a, int total_rows, const Ws& w, hipStream_t st, int64_t plan = 0,
                int* deferred = nullptr) {
  if (deferred) *deferred = 0;
  if (gemv) return launch_gemv(a, total_rows, st);
  a.part = w.part;
  if (plan == 0) return launch_gemm(a, total_rows, w.part_floats, st, deferred);
  const PlanCode c = decode_plan(plan);
  return launch_gemm_cfg(a, total_rows, w.part_floats, c.tm, c.tn, c.ks + 1000 * c.pipe, c.split, st,
                         deferred);
}

// Input-projection segments: r | k | v | w1 | a1 | v1 | g1 of the fused matrix.
void proj_in_args(const Dims& d, const LayerPtrs& q, const Ws& w, int R, bool f16, ProjArgs& a) {
  memset(&a, 0, sizeof a);
  a.W = q.w_in;
  a.K = d.C;
  a.M = R;
  const size_t es = f16 ? 2 : 4;
  auto xq = [&](int i) { return (const void*)((const char*)w.xq + (size_t)i * R * d.C * es); };
  // the first-stage adapter outputs feed the second-stage MFMA projection:
  // fp16 on that path
  auto lin = [&](int col) { return (void*)((char*)w.lin + (size_t)col * es); };
  const int C = d.C;
  int r0 = 3 * C;
  a.seg[0] = mkseg(0, C, EPI_NONE, xq(0), C, w.rkv, 3 * C);
  a.seg[1] = mkseg(C, 2 * C, EPI_NONE, xq(2), C, w.rkv + C, 3 * C);
  a.seg[2] = mkseg(2 * C, 3 * C, EPI_NONE, xq(3), C, w.rkv + 2 * C, 3 * C);
  a.seg[3] = mkseg(r0, r0 + d.Dwp, EPI_TANH, xq(1), C, lin(0), d.Lin);
  r0 += d.Dwp;
  a.seg[4] = mkseg(r0, r0 + d.Dap, EPI_NONE, xq(4), C, lin(d.Dwp), d.Lin);
  r0 += d.Dap;
  a.seg[5] = mkseg(r0, r0 + d.Dvp, EPI_NONE, xq(3), C, lin(d.Dwp + d.Dap), d.Lin);
  r0 += d.Dvp;
  a.seg[6] = mkseg(r0, r0 + d.Dgp, EPI_SIGMOID, xq(5), C, lin(d.Dwp + d.Dap + d.Dvp), d.Lin);
  for (int i = 3; i < 7; ++i) a.seg[i].out_f16 = f16 ? 1 : 0;
  a.nseg = 7;
}

// Adapter outputs for all R rows as one MFMA projection: four blocks of C
// columns, each with its own matrix and rank, writing decay | alpha |
// value gate | gate into lo [R][4C].
void lora_args(const Dims& d, const LayerPtrs& q, const Ws& w, int R, ProjArgs& a) {
  memset(&a, 0, sizeof a);
  a.W = q.w2;
  a.K = d.Dw;
  a.M = R;
  a.nseg = 4;
  const int C = d.C;
  const half_t* W[4] = {q.w2, q.a2, q.v2, q.g2};
  const int K[4] = {d.Dw, d.Da, d.Dv, d.Dg};
  const int off[4] = {0, d.Dwp, d.Dwp + d.Dap, d.Dwp + d.Dap + d.Dvp};
  const int epi[4] = {EPI_DECAY, EPI_SIGB, EPI_SIGB, EPI_NONE};
  const float* bias[4] = {q.w0, q.a0, q.v0, nullptr};
  for (int s = 0; s < 4; ++s) {
    a.seg[s] = mkseg(s * C, (s + 1) * C, epi[s], w.lin, d.Lin, w.lo + (int64_t)s * C, 4 * C, bias[s]);
    a.seg[s].W = W[s];
    a.seg[s].K = K[s];
    a.seg[s].act_off = off[s];
  }
}

WkvArgs wkv_args(const rwkv7_model* m, int l, float* pool, int64_t n_slots, const Ws& w, int R, bool f16) {
  const Dims& d = m->d;
  const LayerPtrs& q = m->pk.layers[l];
  WkvArgs a;
  memset(&a, 0, sizeof a);
  a.pool = pool;
  a.slot_stride = d.slot_floats;
  a.n_slots = n_slots;
  a.layer_off = (int64_t)l * d.layer_floats;
  a.slots = w.slots;
  a.seq_slot = -1;
  a.B = R; a.C = d.C; a.H = d.H; a.layer = l;
  a.rkv = w.rkv; a.lin = w.lin; a.Lin = d.Lin;
  a.off_a = d.Dwp; a.off_v = d.Dwp + d.Dap; a.off_g = d.Dwp + d.Dap + d.Dvp;
  a.Dw = d.Dw; a.Da = d.Da; a.Dv = d.Dv; a.Dg = d.Dg;
  a.w2 = q.w2; a.a2 = q.a2; a.v2 = q.v2; a.g2 = q.g2; a.adp = q.wkv_ad;
  a.w0 = q.w0; a.a0 = q.a0; a.v0 = q.v0; a.k_k = q.k_k; a.k_a = q.k_a; a.r_k = q.r_k;
  a.lnx_w = q.lnx_w; a.lnx_b = q.lnx_b;
  a.vfirst = w.vfirst;
  a.yout = w.yg;
  a.yout_f16 = f16 ? 1 : 0;
  a.q_d = w.q_d; a.q_a = w.q_a; a.q_b = w.q_b; a.q_kt = w.q_kt; a.q_v = w.q_v; a.q_g = w.q_g;
  a.q_bonus = w.q_bonus; a.q_brk = w.q_brk; a.q_y = w.q_y; a.q_rec = w.q_rec;
  return a;
}

struct Path {
  bool gemv, sparse, fused, fuse_value;
};

Path decode_path(const rwkv7_model* m, int B) {
  Path p;
  p.gemv = B <= m->opt_gemv_max && gemv_supported(B, m->d.C);
  p.sparse = B <= m->opt_sparse_max && B <= cmix_sparse_max_b() && m->d.F <= 16384 &&
             m->d.F % 1024 == 0 && m->d.C % 64 == 0;
  p.fused = p.gemv && m->opt_fuse_ln && gemv_fused_ok(B, m->d.C);
  p.fuse_value = p.gemv && p.sparse && B <= 2 && m->opt_fuse_value && m->d.C % 8 == 0 &&
                 m->d.C / 8 <= 512;
  return p;
}

// Workgroups per row of the batched decode LayerNorm kernel: a few rows
// leave most CUs idle and each workgroup's time goes into its loads, so the
// row's per-column vectors are spread over several workgroups, about 256
// in all and at least two per row up to B = 256 (whole-step timing at the
// 2.9B and 7.2B shapes, B 8 to 256).
int ln_blocks(const rwkv7_model* m, int B) {
  const int ne = m->d.C / 256;
  const int units = ne % 2 == 0 ? ne / 2 : ne;
  int n = (int)m->opt_ln_split;
  if (n <= 0) n = B > 256 ? 1 : std::max(2, 256 / std::max(B, 1));
  return std::max(1, std::min(n, units));
}

// Rows per wave of the many-row WKV kernel that computes the adapters' second
// stage itself (0: a separate MFMA projection computes them).  Default, from
// whole graph-replayed steps against the separate projection: where the
// adapter operands leave registers for the first row's state (ranks summing
// to <= 512, e.g. 2.9B), one row per wave up to 128 rows and two above
// (B 8 to 256: 1.8-6.1 % faster); otherwise (7.2B) four, which spreads the
// adapter step over more rows (B 64 and 256: 2.3 and 1.8 % faster).
int wkv_ad_rows_per_wave(const rwkv7_model* m, int B) {
  switch (m->opt_wkv_ad) {
    case 1: return 0;
    case 2: return 1;
    case 3: return 2;
    case 4: return 4;
    default:
      // whole-step sweeps: one row per wave, except two up to 128 rows when
      // the ranks sum past 512 (7.2B)
      if (m->d.Dw + m->d.Da + m->d.Dv + m->d.Dg > 512) return B <= 128 ? 2 : 1;
      return 1;
  }
}

// mixing vector (index into the six time-mix coefficient rows r,w,k,v,a,g)
// read by each block of the fused input projection
constexpr int kInMix[7] = {0, 2, 3, 1, 4, 3, 5};

int enqueue_decode(rwkv7_model* m, float* pool, int64_t n_slots, int B, const int* slot_idx,
                   const int* tok, float* logits, char* ws, hipStream_t st, bool timing,
                   const Filter* flt = nullptr) {
  const Dims& d = m->d;
  Launcher L{m, st, timing, flt};
  const Ws w = ws_layout(d, B, ws);
  const Path path = decode_path(m, B);
  // GEMV path: fp32 activations; MFMA path: every projection input is
  // written in fp16 by its producer (the residual stream stays fp32)
  const bool f16 = !path.gemv;
  // int8 weights on the small-batch GEMV path when enabled
  const bool q8 = m->opt_int8 && m->has_q8 && path.gemv && B <= 2;
  const int C = d.C;
  int64_t* counters = (int64_t*)((char*)pool + align_up((uint64_t)n_slots * d.slot_floats * 4));

  ValidateArgs va{slot_idx, tok, B, B, n_slots, d.V, -1, w.slots, w.tok, w.err, counters,
                  nullptr, 0};
  EmbedArgs ea{m->pk.emb, m->pk.ln0_w, m->pk.ln0_b, w.tok, w.x, B, C};
  RUN(RWKV7_K_OTHER, "validate + embed", launch_embed_rows(va, ea, st));

  // Fused path (small B): LayerNorm + token-shift mix run inside the GEMV
  // prologues; the new shifts are committed by the following kernel (WKV
  // for the time mix, the channel-mix value for the channel mix).
  // Otherwise a LayerNorm kernel writes the mixed rows and the shift.
  // MFMA path: a residual projection split over K leaves its partial sums
  // for the LayerNorm that follows it to add into x (no reduction launch)
  // A LayerNorm that folds partials in writes the new residual to the other
  // buffer (its column blocks all read the whole old row): xc is the current one.
  int pending = 0;
  int* const defer = path.fused ? nullptr : &pending;
  const int ncb = ln_blocks(m, B);
  float* xc = w.x;
  float* xn = w.x2;
  for (int l = 0; l < d.L; ++l) {
    L.layer = l;
    const LayerPtrs& q = m->pk.layers[l];
    const int64_t lo = (int64_t)l * d.layer_floats;
    LnMixArgs la;
    memset(&la, 0, sizeof la);
    la.x = xc; la.C = C; la.R = B; la.mode = LNMIX_DECODE; la.ncb = ncb;
    if (pending) {
      la.parts = w.part; la.nparts = pending; la.x_out = xn;
      std::swap(xc, xn);
      pending = 0;
    }
    la.g = q.ln1_w; la.b = q.ln1_b;
    la.pool = pool; la.slot_stride = d.slot_floats; la.n_slots = n_slots; la.shift_off = lo;
    la.slots = w.slots; la.seq_slot = -1;
    la.mu = q.mu6; la.nq = 6;
    la.out = w.xq; la.out_f16 = f16; la.out_q_stride = (int64_t)B * C;

    ProjArgs pa;
    proj_in_args(d, q, w, B, f16, pa);
    if (q8) { pa.Wq = m->q8.layers[l].w_in; pa.Wsc = m->q8.layers[l].s_in; }
    if (path.fused) {
      pa.ln = LnPro{xc, q.ln1_w, q.ln1_b, pool, d.slot_floats, n_slots, lo, w.slots, w.u_att, LNP_MIX, 0};
      for (int s = 0; s < 7; ++s) pa.seg[s].mix = q.mu6 + (int64_t)kInMix[s] * C;
    } else {
      RUN(RWKV7_K_LN_MIX, "ln_mix(tmix)", launch_ln_mix(la, st));
    }
    RUN(RWKV7_K_PROJ_IN, "proj_in", proj(path.gemv, pa, d.Nin, w, st, m->opt_plan[0]));

    WkvArgs wa = wkv_args(m, l, pool, n_slots, w, B, f16);
    wa.u_att = path.fused ? w.u_att : nullptr;
    if (!path.gemv) {
      const int rpw = wkv_ad_rows_per_wave(m, B);
      if (rpw && wkv_chunk_adapters_ok(wa)) {
        // many rows, the adapters' second stage inside the WKV kernel
        wa.ad_rpw = rpw;
      } else {
        // many rows: the adapter outputs as one MFMA projection, WKV reads them
        ProjArgs pl;
        lora_args(d, q, w, B, pl);
        RUN(RWKV7_K_PROJ_IN, "adapters", proj(false, pl, 4 * C, w, st, m->opt_plan[1]));
        wa.lo = w.lo;
      }
    }
    RUN(RWKV7_K_WKV, "wkv", launch_wkv_decode(wa, st));

    ProjArgs po;
    memset(&po, 0, sizeof po);
    po.W = q.w_o; po.K = C; po.M = B; po.nseg = 1;
    po.seg[0] = mkseg(0, C, EPI_RESID, w.yg, C, xc, C);
    if (q8) { po.Wq = m->q8.layers[l].w_o; po.Wsc = m->q8.layers[l].s_o; }
    RUN(RWKV7_K_PROJ_OUT, "proj_out", proj(path.gemv, po, C, w, st, m->opt_plan[2], defer));

    ProjArgs pk;
    memset(&pk, 0, sizeof pk);
    pk.W = q.w_key; pk.K = C; pk.M = B; pk.nseg = 1;
    if (path.sparse)
      pk.seg[0] = mkseg(0, d.F, EPI_PRE, w.xk, C, w.pre, d.F, q.b_key, w.mask);
    else
      pk.seg[0] = mkseg(0, d.F, EPI_RELU2, w.xk, C, w.pre, d.F, q.b_key);
    if (!path.sparse) pk.seg[0].out_f16 = 1;   // the dense (MFMA) value projection's input
    if (path.fuse_value) {
      pk.vW = q.w_val_hm;
      pk.vpart = w.vpart;
      pk.vC = C;
    }
    if (q8) {
      pk.Wq = m->q8.layers[l].w_key; pk.Wsc = m->q8.layers[l].s_key;
      if (path.fuse_value) { pk.vWq = m->q8.layers[l].w_val; pk.vSc = m->q8.layers[l].s_val; }
    }
    if (path.fused) {
      pk.ln = LnPro{xc, q.ln2_w, q.ln2_b, pool, d.slot_floats, n_slots, lo + C, w.slots, w.u_ffn, LNP_MIX, 0};
      pk.seg[0].mix = q.mu_k;
    } else {
      LnMixArgs lc = la;
      lc.g = q.ln2_w; lc.b = q.ln2_b;
      lc.shift_off = lo + C;
      lc.mu = q.mu_k; lc.nq = 1;
      lc.out = w.xk; lc.out_q_stride = 0;
      lc.x = xc; lc.parts = nullptr; lc.nparts = 0; lc.x_out = nullptr;
      if (pending) {
        lc.parts = w.part; lc.nparts = pending; lc.x_out = xn;
        std::swap(xc, xn);
      }
      RUN(RWKV7_K_LN_MIX, "ln_mix(cmix)", launch_ln_mix(lc, st));
    }
    pending = 0;
    RUN(RWKV7_K_CMIX_KEY, "cmix_key", proj(path.gemv, pk, d.F, w, st, m->opt_plan[3]));

    if (path.fuse_value) {
      CmixFoldArgs fa;
      memset(&fa, 0, sizeof fa);
      fa.part = w.vpart; fa.nwg = (d.F + gemv_launch_rows(B, C, d.F, 1, true) - 1) / gemv_launch_rows(B, C, d.F, 1, true);
      fa.mask = w.mask; fa.x = xc; fa.u_ffn = path.fused ? w.u_ffn : nullptr;
      fa.pool = pool; fa.slot_stride = d.slot_floats; fa.n_slots = n_slots; fa.shift_off = lo + C;
      fa.slots = w.slots; fa.B = B; fa.C = C; fa.F = d.F;
      if (l == d.L - 1) { fa.dbg_idx = w.dbg_idx; fa.dbg_cnt = w.dbg_cnt; }
      RUN(RWKV7_K_CMIX_VALUE, "cmix_fold", launch_cmix_fold(fa, st));
    } else if (path.sparse) {
      CmixArgs ca;
      memset(&ca, 0, sizeof ca);
      ca.pre = w.pre; ca.mask = w.mask; ca.Wv = q.w_val_hm;
      ca.x = xc; ca.u_ffn = path.fused ? w.u_ffn : nullptr;
      ca.pool = pool; ca.slot_stride = d.slot_floats; ca.n_slots = n_slots; ca.shift_off = lo + C;
      ca.slots = w.slots; ca.B = B; ca.C = C; ca.F = d.F;
      if (l == d.L - 1) { ca.dbg_idx = w.dbg_idx; ca.dbg_cnt = w.dbg_cnt; }
      RUN(RWKV7_K_CMIX_VALUE, "cmix_value", launch_cmix_sparse(ca, st));
    } else {
      ProjArgs pv;
      memset(&pv, 0, sizeof pv);
      pv.W = q.w_val_km; pv.K = d.F; pv.M = B; pv.nseg = 1;
      pv.seg[0] = mkseg(0, C, EPI_RESID, w.pre, d.F, xc, C);
      RUN(RWKV7_K_CMIX_VALUE, "cmix_value", proj(false, pv, C, w, st, m->opt_plan[4], defer));
      if (path.fused) {
        CommitArgs ca{w.u_ffn, pool, d.slot_floats, n_slots, lo + C, w.slots, B, C};
        RUN(RWKV7_K_OTHER, "commit shift", launch_commit_shift(ca, st));
      }
    }
  }

  L.layer = d.L;
  ProjArgs ph;
  memset(&ph, 0, sizeof ph);
  ph.W = m->pk.head; ph.K = C; ph.M = B; ph.nseg = 1;
  ph.seg[0] = mkseg(0, d.V, EPI_NONE, w.xo, C, logits, d.V);
  if (q8) { ph.Wq = m->q8.head; ph.Wsc = m->q8.s_head; }
  if (path.fused) {
    ph.ln = LnPro{xc, m->pk.lnout_w, m->pk.lnout_b, nullptr, 0, 0, 0, nullptr, nullptr, LNP_PLAIN, 0};
  } else {
    LnMixArgs lo;
    memset(&lo, 0, sizeof lo);
    lo.x = xc; lo.C = C; lo.R = B; lo.mode = LNMIX_PLAIN; lo.ncb = ncb;
    lo.g = m->pk.lnout_w; lo.b = m->pk.lnout_b;
    lo.nq = 1; lo.mu = nullptr;
    lo.out = w.xo; lo.out_f16 = f16; lo.out_q_stride = 0;
    if (pending) { lo.parts = w.part; lo.nparts = pending; lo.x_out = xn; }
    RUN(RWKV7_K_LN_MIX, "ln_out", launch_ln_mix(lo, st));
  }
  RUN(RWKV7_K_HEAD, "head", proj(path.gemv, ph, d.V, w, st, m->opt_plan[5]));
  return RWKV7_OK;
}

int enqueue_prefill_chunk(rwkv7_model* m, float* pool, int64_t n_slots, int slot, const int* tok,
                          int T, char* ws, hipStream_t st, bool timing) {
  const Dims& d = m->d;
  Launcher L{m, st, timing};
  const Ws w = ws_layout(d, T, ws);
  const int C = d.C;
  int64_t* counters = (int64_t*)((char*)pool + align_up((uint64_t)n_slots * d.slot_floats * 4));
  float* slot_base = pool + (int64_t)slot * d.slot_floats;

  ValidateArgs va{nullptr, tok, 0, T, n_slots, d.V, slot, w.slots, w.tok, w.err, counters,
                  nullptr, 0};
  RUN(RWKV7_K_OTHER, "validate", launch_validate(va, st));
  EmbedArgs ea{m->pk.emb, m->pk.ln0_w, m->pk.ln0_b, w.tok, w.x, T, C};
  RUN(RWKV7_K_OTHER, "embed", launch_embed(ea, st));

  // The residual projections split over K leave their partials to the next
  // LayerNorm, which writes the folded residual to the other buffer (a row
  // also reads the previous row's residual, so it cannot be updated in place).
  float* xc = w.x;
  float* xn = w.x2;
  int pending = 0;
  // A LayerNorm's last-row output is the slot's new shift, but its own first
  // row still reads the old one: it goes to a temporary, copied into the slot
  // by the next LayerNorm launch (the channel-mix one for the time-mix shift,
  // the next layer's time-mix one for the channel-mix shift).
  const float* cp_ffn = nullptr;   // the previous layer's channel-mix shift, not yet in the slot
  for (int l = 0; l < d.L; ++l) {
    const LayerPtrs& q = m->pk.layers[l];
    const int64_t lo = (int64_t)l * d.layer_floats;
    LnMixArgs la;
    memset(&la, 0, sizeof la);
    la.x = xc; la.C = C; la.R = T; la.mode = LNMIX_SEQ; la.ncb = 1;
    if (cp_ffn) {
      la.cp_src = cp_ffn; la.cp_dst = slot_base + lo - d.layer_floats + C; la.cp_n = C;
    }
    if (pending) {
      la.parts = w.part; la.nparts = pending; la.x_out = xn;
      std::swap(xc, xn);
      pending = 0;
    }
    la.g = q.ln1_w; la.b = q.ln1_b;
    la.pool = pool; la.slot_stride = d.slot_floats; la.n_slots = n_slots; la.shift_off = lo;
    la.seq_slot = slot; la.shift_tmp = w.shift_tmp;
    la.mu = q.mu6; la.nq = 6;
    la.out = w.xq; la.out_f16 = 1; la.out_q_stride = (int64_t)T * C;
    RUN(RWKV7_K_LN_MIX, "ln_mix(tmix)", launch_ln_mix(la, st));

    ProjArgs pa;
    proj_in_args(d, q, w, T, true, pa);
    RUN(RWKV7_K_PROJ_IN, "proj_in", proj(false, pa, d.Nin, w, st, m->opt_plan[0]));

    WkvArgs wa = wkv_args(m, l, pool, n_slots, w, T, true);
    wa.seq_slot = slot;
    const bool chunked = m->opt_prefill_scan == 2 || (m->opt_prefill_scan == 0 && T >= PREFILL_CHUNKED_MIN_T);
    // the chunked scan computes the adapters' second stage itself when the ranks allow
    if (chunked && wkv_chunk_adapters_ok(wa)) {
      wa.lo = nullptr;
    } else {
      ProjArgs pl;
      lora_args(d, q, w, T, pl);
      RUN(RWKV7_K_PROJ_IN, "adapters", proj(false, pl, 4 * C, w, st, m->opt_plan[1]));
      wa.lo = w.lo;
    }
    if (chunked) {
      RUN(RWKV7_K_WKV, "wkv_chunk_prep", launch_wkv_chunk_prep(wa, st));
      RUN(RWKV7_K_WKV, "wkv_chunk_scan", launch_wkv_chunk_scan(wa, st));
    } else {
      RUN(RWKV7_K_WKV, "wkv_prep", launch_wkv_prep(wa, st));
      RUN(RWKV7_K_WKV, "wkv_scan", launch_wkv_scan(wa, st));
    }
    RUN(RWKV7_K_WKV, "wkv_post", launch_wkv_post(wa, st));

    ProjArgs po;
    memset(&po, 0, sizeof po);
    po.W = q.w_o; po.K = C; po.M = T; po.nseg = 1;
    po.seg[0] = mkseg(0, C, EPI_RESID, w.yg, C, xc, C);
    RUN(RWKV7_K_PROJ_OUT, "proj_out", proj(false, po, C, w, st, m->opt_plan[2], &pending));

    LnMixArgs lc = la;
    lc.g = q.ln2_w; lc.b = q.ln2_b;
    lc.shift_off = lo + C;
    lc.shift_tmp = w.shift_tmp2;
    lc.cp_src = w.shift_tmp; lc.cp_dst = slot_base + lo; lc.cp_n = C;   // this layer's time-mix shift
    lc.mu = q.mu_k; lc.nq = 1;
    lc.out = w.xk; lc.out_q_stride = 0;
    lc.x = xc; lc.parts = nullptr; lc.nparts = 0; lc.x_out = nullptr;
    if (pending) {
      lc.parts = w.part; lc.nparts = pending; lc.x_out = xn;
      std::swap(xc, xn);
      pending = 0;
    }
    RUN(RWKV7_K_LN_MIX, "ln_mix(cmix)", launch_ln_mix(lc, st));
    cp_ffn = w.shift_tmp2;

    ProjArgs pk;
    memset(&pk, 0, sizeof pk);
    pk.W = q.w_key; pk.K = C; pk.M = T; pk.nseg = 1;
    pk.seg[0] = mkseg(0, d.F, EPI_RELU2, w.xk, C, w.pre, d.F, q.b_key);
    pk.seg[0].out_f16 = 1;
    RUN(RWKV7_K_CMIX_KEY, "cmix_key", proj(false, pk, d.F, w, st, m->opt_plan[3]));

    ProjArgs pv;
    memset(&pv, 0, sizeof pv);
    pv.W = q.w_val_km; pv.K = d.F; pv.M = T; pv.nseg = 1;
    pv.seg[0] = mkseg(0, C, EPI_RESID, w.pre, d.F, xc, C);
    RUN(RWKV7_K_CMIX_VALUE, "cmix_value", proj(false, pv, C, w, st, m->opt_plan[4], &pending));
  }
  // the last layer's channel-mix shift; its value partials are not needed
  // (prefill returns no logits)
  RUN(RWKV7_K_OTHER, "shift copy",
      launch_copy_f32(slot_base + (int64_t)(d.L - 1) * d.layer_floats + C, w.shift_tmp2, C, st));
  return RWKV7_OK;
}

const char* kClassName[RWKV7_K_COUNT] = {"ln_mix", "proj_in", "wkv", "proj_out",
                                         "cmix_key", "cmix_value", "head", "other"};

void drop_graphs(rwkv7_model* m) {
  for (auto& kv : m->graphs) {
    hipGraphExecDestroy(kv.second.exec);
    hipGraphDestroy(kv.second.graph);
  }
  m->graphs.clear();
}

// Expected name -> shape, for the tensor table.
struct Expect {
  std::string name;
  std::vector<int64_t> shape;
};

std::vector<Expect> expected_tensors(const Dims& d) {
  std::vector<Expect> e;
  const int64_t C = d.C, F = d.F, V = d.V;
  e.push_back({"emb.weight", {V, C}});
  e.push_back({"ln0.weight", {C}});
  e.push_back({"ln0.bias", {C}});
  e.push_back({"ln_out.weight", {C}});
  e.push_back({"ln_out.bias", {C}});
  e.push_back({"head.weight", {V, C}});
  for (int l = 0; l < d.L; ++l) {
    const std::string p = "blocks." + std::to_string(l) + ".";
    for (const char* n : {"ln1.weight", "ln1.bias", "ln2.weight", "ln2.bias", "att.x_r", "att.x_w",
                          "att.x_k", "att.x_v", "att.x_a", "att.x_g", "att.w0", "att.a0", "att.v0",
                          "att.k_k", "att.k_a", "att.ln_x.weight", "att.ln_x.bias", "ffn.x_k"})
      e.push_back({p + n, {C}});
    e.push_back({p + "att.w1", {d.Dw, C}});
    e.push_back({p + "att.w2", {C, d.Dw}});
    e.push_back({p + "att.a1", {d.Da, C}});
    e.push_back({p + "att.a2", {C, d.Da}});
    e.push_back({p + "att.v1", {d.Dv, C}});
    e.push_back({p + "att.v2", {C, d.Dv}});
    e.push_back({p + "att.g1", {d.Dg, C}});
    e.push_back({p + "att.g2", {C, d.Dg}});
    e.push_back({p + "att.r_k", {d.H, 64}});
    for (const char* n : {"att.receptance.weight", "att.key.weight", "att.value.weight",
                          "att.output.weight"})
      e.push_back({p + n, {C, C}});
    e.push_back({p + "ffn.key.weight", {F, C}});
    e.push_back({p + "ffn.key.bias", {F}});
    e.push_back({p + "ffn.value.weight", {C, F}});
  }
  return e;
}

}  // namespace

// Library-internal entry points for the scheduler (sched.hip).
int lib_fail(int code, const char* msg) { return fail(code, "%s", msg); }
int lib_model_vocab(const rwkv7_model* m) { return m ? m->cfg.vocab : 0; }
int64_t lib_model_slot_floats(const rwkv7_model* m) { return m ? m->d.slot_floats : 0; }

// ====================================================================== C ABI
extern "C" {

const char* rwkv7_last_error(void) { return g_last_error.c_str(); }

const char* rwkv7_status_string(int s) {
  switch (s) {
    case RWKV7_OK: return "ok";
    case RWKV7_EINVAL: return "invalid argument";
    case RWKV7_ESHAPE: return "wrong shape or size";
    case RWKV7_EHIP: return "HIP runtime error";
    case RWKV7_EDEVICE: return "device-detected error";
    case RWKV7_ENOTSUP: return "not supported";
    default: return "unknown status";
  }
}

int rwkv7_packed_bytes(const rwkv7_config* cfg, uint64_t* bytes) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  *bytes = pack_layout(d, nullptr).bytes;
  return RWKV7_OK;
}

int rwkv7_slot_floats(const rwkv7_config* cfg, uint64_t* n) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!n) return fail(RWKV7_EINVAL, "n_floats is NULL");
  *n = (uint64_t)d.slot_floats;
  return RWKV7_OK;
}

int rwkv7_state_bytes(const rwkv7_config* cfg, int64_t n_slots, uint64_t* bytes,
                      uint64_t* counter_offset) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  if (n_slots < 1) return fail(RWKV7_EINVAL, "n_slots must be >= 1");
  const uint64_t co = align_up((uint64_t)n_slots * d.slot_floats * 4);
  if (counter_offset) *counter_offset = co;
  *bytes = co + align_up((uint64_t)n_slots * 8);
  return RWKV7_OK;
}

int rwkv7_workspace_bytes(const rwkv7_config* cfg, int32_t max_B, int32_t max_T, uint64_t* bytes) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  if (max_B < 1 || max_T < 1) return fail(RWKV7_EINVAL, "max_B and max_T must be >= 1");
  const int R = max_B > max_T ? max_B : max_T;
  uint64_t b = ws_layout(d, R, nullptr).bytes;
  uint64_t g = 0;
  rwkv7_greedy_workspace_bytes(max_B, d.V, &g);
  *bytes = b > g ? b : g;
  return RWKV7_OK;
}

int rwkv7_load(const rwkv7_config* cfg, const rwkv7_tensor* tensors, int32_t n_tensors,
               void* packed, uint64_t packed_bytes, void* stream, rwkv7_model** out) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!out) return fail(RWKV7_EINVAL, "out is NULL");
  *out = nullptr;
  if (!tensors || n_tensors < 1) return fail(RWKV7_EINVAL, "empty tensor table");
  if (!packed) return fail(RWKV7_EINVAL, "packed buffer is NULL");
  Packed pk = pack_layout(d, (char*)packed);
  if (packed_bytes < pk.bytes)
    return fail(RWKV7_ESHAPE, "packed buffer too small: %llu < %llu bytes",
                (unsigned long long)packed_bytes, (unsigned long long)pk.bytes);

  std::map<std::string, const rwkv7_tensor*> by_name;
  for (int i = 0; i < n_tensors; ++i) {
    const rwkv7_tensor& t = tensors[i];
    if (!t.name) return fail(RWKV7_EINVAL, "tensor %d has no name", i);
    if (by_name.count(t.name)) return fail(RWKV7_EINVAL, "tensor %s given twice", t.name);
    by_name[t.name] = &t;
  }
  const std::vector<Expect> exp = expected_tensors(d);
  if ((size_t)n_tensors != exp.size())
    for (auto& kv : by_name) {
      bool known = false;
      for (auto& e : exp) known |= e.name == kv.first;
      if (!known) return fail(RWKV7_EINVAL, "unknown tensor %s", kv.first.c_str());
    }
  for (const Expect& e : exp) {
    auto it = by_name.find(e.name);
    if (it == by_name.end()) return fail(RWKV7_EINVAL, "missing tensor %s", e.name.c_str());
    const rwkv7_tensor& t = *it->second;
    if (t.dtype != RWKV7_F32 && t.dtype != RWKV7_F16)
      return fail(RWKV7_EINVAL, "tensor %s: dtype must be F32 or F16", e.name.c_str());
    if (t.ndim != (int)e.shape.size())
      return fail(RWKV7_ESHAPE, "tensor %s: expected %zu dims, got %d", e.name.c_str(), e.shape.size(), t.ndim);
    for (size_t k = 0; k < e.shape.size(); ++k)
      if (t.shape[k] != e.shape[k])
        return fail(RWKV7_ESHAPE, "tensor %s: dim %zu is %lld, expected %lld", e.name.c_str(), k,
                    (long long)t.shape[k], (long long)e.shape[k]);
    if (!t.data) return fail(RWKV7_EINVAL, "tensor %s has no data", e.name.c_str());
  }

  hipStream_t st = (hipStream_t)stream;
  auto T = [&](const std::string& n) { return by_name[n]; };
  auto mat = [&](half_t* dst, int64_t dst_ld, const std::string& n) -> hipError_t {
    const rwkv7_tensor* t = T(n);
    return launch_pack_matrix(dst, dst_ld, t->data, t->dtype == RWKV7_F16, t->shape[0], t->shape[1], st);
  };
  auto vec = [&](float* dst, const std::string& n) -> hipError_t {
    const rwkv7_tensor* t = T(n);
    int64_t cnt = 1;
    for (int k = 0; k < t->ndim; ++k) cnt *= t->shape[k];
    return launch_pack_vec(dst, t->data, t->dtype == RWKV7_F16, cnt, st);
  };
#define PK(expr, what) HIP_TRY(expr, what)
  PK(mat(pk.emb, d.C, "emb.weight"), "pack emb");
  PK(mat(pk.head, d.C, "head.weight"), "pack head");
  PK(vec(pk.ln0_w, "ln0.weight"), "pack");
  PK(vec(pk.ln0_b, "ln0.bias"), "pack");
  PK(vec(pk.lnout_w, "ln_out.weight"), "pack");
  PK(vec(pk.lnout_b, "ln_out.bias"), "pack");
  const int64_t C = d.C;
  for (int l = 0; l < d.L; ++l) {
    const std::string p = "blocks." + std::to_string(l) + ".";
    const LayerPtrs& q = pk.layers[l];
    PK(hipMemsetAsync(q.w_in, 0, (size_t)d.Nin * C * 2, st), "zero w_in");
    PK(mat(q.w_in, C, p + "att.receptance.weight"), "pack");
    PK(mat(q.w_in + C * C, C, p + "att.key.weight"), "pack");
    PK(mat(q.w_in + 2 * C * C, C, p + "att.value.weight"), "pack");
    int64_t r0 = 3 * C;
    PK(mat(q.w_in + r0 * C, C, p + "att.w1"), "pack");
    r0 += d.Dwp;
    PK(mat(q.w_in + r0 * C, C, p + "att.a1"), "pack");
    r0 += d.Dap;
    PK(mat(q.w_in + r0 * C, C, p + "att.v1"), "pack");
    r0 += d.Dvp;
    PK(mat(q.w_in + r0 * C, C, p + "att.g1"), "pack");
    PK(mat(q.w2, d.Dw, p + "att.w2"), "pack");
    PK(mat(q.a2, d.Da, p + "att.a2"), "pack");
    PK(mat(q.v2, d.Dv, p + "att.v2"), "pack");
    PK(mat(q.g2, d.Dg, p + "att.g2"), "pack");
    PK(launch_pack_wkv_adapters(q.wkv_ad, q.w2, q.a2, q.v2, q.g2, d.C, d.Dw, d.Da, d.Dv, d.Dg, st), "pack");
    PK(mat(q.w_o, C, p + "att.output.weight"), "pack");
    PK(mat(q.w_key, C, p + "ffn.key.weight"), "pack");
    PK(mat(q.w_val_km, d.F, p + "ffn.value.weight"), "pack");
    {
      const rwkv7_tensor* t = T(p + "ffn.value.weight");
      PK(launch_pack_transpose(q.w_val_hm, t->data, t->dtype == RWKV7_F16, C, d.F, st), "pack");
    }
    PK(vec(q.ln1_w, p + "ln1.weight"), "pack"); PK(vec(q.ln1_b, p + "ln1.bias"), "pack");
    PK(vec(q.ln2_w, p + "ln2.weight"), "pack"); PK(vec(q.ln2_b, p + "ln2.bias"), "pack");
    PK(vec(q.lnx_w, p + "att.ln_x.weight"), "pack"); PK(vec(q.lnx_b, p + "att.ln_x.bias"), "pack");
    const char* mix[6] = {"att.x_r", "att.x_w", "att.x_k", "att.x_v", "att.x_a", "att.x_g"};
    for (int k = 0; k < 6; ++k) PK(vec(q.mu6 + k * C, p + mix[k]), "pack");
    PK(vec(q.w0, p + "att.w0"), "pack"); PK(vec(q.a0, p + "att.a0"), "pack");
    PK(vec(q.v0, p + "att.v0"), "pack"); PK(vec(q.k_k, p + "att.k_k"), "pack");
    PK(vec(q.k_a, p + "att.k_a"), "pack"); PK(vec(q.r_k, p + "att.r_k"), "pack");
    PK(vec(q.mu_k, p + "ffn.x_k"), "pack"); PK(vec(q.b_key, p + "ffn.key.bias"), "pack");
  }
#undef PK
  rwkv7_model* m = new rwkv7_model();
  m->cfg = *cfg;
  m->d = d;
  m->pk = pk;
  hipGetDevice(&m->device);
  *out = m;
  return RWKV7_OK;
}

int rwkv7_free(rwkv7_model* m) {
  if (!m) return RWKV7_OK;
  drop_graphs(m);
  for (auto& t : m->pending) { hipEventDestroy(t.a); hipEventDestroy(t.b); }
  for (auto& e : m->free_events) { hipEventDestroy(e.first); hipEventDestroy(e.second); }
  if (m->cap_stream) hipStreamDestroy(m->cap_stream);
  delete m;
  return RWKV7_OK;
}

static int check_pool_ws(const rwkv7_model* m, const void* pool, int64_t n_slots, const void* ws,
                         uint64_t ws_bytes, uint64_t need) {
  if (!m) return fail(RWKV7_EINVAL, "model is NULL");
  if (!pool) return fail(RWKV7_EINVAL, "pool is NULL");
  if (!ws) return fail(RWKV7_EINVAL, "workspace is NULL");
  if (n_slots < 1) return fail(RWKV7_EINVAL, "n_slots must be >= 1");
  if (ws_bytes < need)
    return fail(RWKV7_ESHAPE, "workspace too small: %llu < %llu bytes", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  return RWKV7_OK;
}

int rwkv7_reset_slots(const rwkv7_model* m, void* pool, int64_t n_slots, const int32_t* slot_idx,
                      int32_t n, void* ws, uint64_t ws_bytes, void* stream) {
  int rc = check_pool_ws(m, pool, n_slots, ws, ws_bytes, 4);
  if (rc) return rc;
  if (n < 0) return fail(RWKV7_EINVAL, "n must be >= 0");
  if (n == 0) return RWKV7_OK;
  if (!slot_idx) return fail(RWKV7_EINVAL, "slot_idx is NULL");
  const Dims& d = m->d;
  ResetArgs a;
  a.pool = (float*)pool;
  a.slot_stride = d.slot_floats;
  a.counters = (int64_t*)((char*)pool + align_up((uint64_t)n_slots * d.slot_floats * 4));
  a.slot_idx = slot_idx;
  a.n = n;
  a.n_slots = n_slots;
  a.err = (uint32_t*)ws;
  HIP_TRY(launch_reset(a, (hipStream_t)stream), "reset");
  return RWKV7_OK;
}

int rwkv7_decode_step(rwkv7_model* m, void* pool, int64_t n_slots, int32_t B,
                      const int32_t* slot_idx, const int32_t* token_ids, float* logits_out,
                      void* ws, uint64_t ws_bytes, void* stream) {
  if (!m) return fail(RWKV7_EINVAL, "model is NULL");
  if (B < 1) return fail(RWKV7_EINVAL, "B must be >= 1 (got %d)", B);
  if (B > n_slots) return fail(RWKV7_EINVAL, "B=%d exceeds n_slots=%lld", B, (long long)n_slots);
  int rc = check_pool_ws(m, pool, n_slots, ws, ws_bytes, ws_layout(m->d, B, nullptr).bytes);
  if (rc) return rc;
  if (!slot_idx || !token_ids || !logits_out)
    return fail(RWKV7_EINVAL, "slot_idx, token_ids and logits_out must be non-NULL");
  hipStream_t st = (hipStream_t)stream;
  if (m->opt_timing || !m->opt_graph)
    return enqueue_decode(m, (float*)pool, n_slots, B, slot_idx, token_ids, logits_out, (char*)ws,
                          st, m->opt_timing != 0);

  GraphKey key{B, pool, slot_idx, token_ids, logits_out, ws, n_slots, (int)m->opt_gemv_max,
               (int)m->opt_sparse_max};
  auto it = m->graphs.find(key);
  if (it == m->graphs.end()) {
    if (!m->cap_stream) HIP_TRY(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking), "hipStreamCreate");
    if (m->graphs.size() >= GRAPH_CACHE) {
      auto oldest = m->graphs.begin();
      for (auto j = m->graphs.begin(); j != m->graphs.end(); ++j)
        if (j->second.last_use < oldest->second.last_use) oldest = j;
      hipGraphExecDestroy(oldest->second.exec);
      hipGraphDestroy(oldest->second.graph);
      m->graphs.erase(oldest);
    }
    HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed), "hipStreamBeginCapture");
    rc = enqueue_decode(m, (float*)pool, n_slots, B, slot_idx, token_ids, logits_out, (char*)ws,
                        m->cap_stream, false);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(m->cap_stream, &g);
    if (rc != RWKV7_OK) {
      if (g) hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      hipGraphDestroy(g);
      return hip_fail(e, "hipGraphInstantiate");
    }
    it = m->graphs.emplace(key, GraphEntry{g, ex, 0}).first;
  }
  it->second.last_use = ++m->use_clock;
  HIP_TRY(hipGraphLaunch(it->second.exec, st), "hipGraphLaunch");
  return RWKV7_OK;
}

int rwkv7_prefill_seq(rwkv7_model* m, void* pool, int64_t n_slots, int32_t slot,
                      const int32_t* token_ids, int32_t T, void* ws, uint64_t ws_bytes,
                      void* stream) {
  if (!m) return fail(RWKV7_EINVAL, "model is NULL");
  if (T < 0) return fail(RWKV7_EINVAL, "T must be >= 0 (got %d)", T);
  if (slot < 0 || slot >= n_slots)
    return fail(RWKV7_EINVAL, "slot %d outside [0, %lld)", slot, (long long)n_slots);
  if (T == 0) return RWKV7_OK;
  if (!token_ids) return fail(RWKV7_EINVAL, "token_ids is NULL");
  int chunk = (int)(m->opt_chunk < 1 ? 1 : m->opt_chunk);
  if (chunk > T) chunk = T;
  // shrink the chunk until the workspace holds it
  while (chunk > 1 && ws_layout(m->d, chunk, nullptr).bytes > ws_bytes) chunk = (chunk + 1) / 2;
  int rc = check_pool_ws(m, pool, n_slots, ws, ws_bytes, ws_layout(m->d, chunk, nullptr).bytes);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  for (int t0 = 0; t0 < T; t0 += chunk) {
    const int n = (T - t0) < chunk ? (T - t0) : chunk;
    rc = enqueue_prefill_chunk(m, (float*)pool, n_slots, slot, token_ids + t0, n, (char*)ws, st,
                               m->opt_timing != 0);
    if (rc) return rc;
  }
  return RWKV7_OK;
}

int rwkv7_greedy_workspace_bytes(int32_t B, int32_t V, uint64_t* bytes) {
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  if (B < 1 || V < 1) return fail(RWKV7_EINVAL, "B and V must be >= 1");
  const uint64_t nb = (uint64_t)greedy_blocks(V);
  *bytes = ALIGN + align_up((uint64_t)B * nb * 4) * 2;
  return RWKV7_OK;
}

int rwkv7_greedy(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                 const int32_t* slot_idx, const float* presence, const float* frequency,
                 const float* decay, int32_t* ids_out, void* ws, uint64_t ws_bytes, void* stream) {
  if (B < 1 || V < 1) return fail(RWKV7_EINVAL, "B and V must be >= 1");
  if (n_slots < 1) return fail(RWKV7_EINVAL, "n_slots must be >= 1");
  if (!logits || !occ_pool || !slot_idx || !presence || !frequency || !decay || !ids_out || !ws)
    return fail(RWKV7_EINVAL, "null pointer argument");
  uint64_t need = 0;
  rwkv7_greedy_workspace_bytes(B, V, &need);
  if (ws_bytes < need)
    return fail(RWKV7_ESHAPE, "workspace too small: %llu < %llu bytes", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  GreedyArgs a;
  a.logits = logits; a.occ = occ_pool; a.n_slots = n_slots; a.slot_idx = slot_idx;
  a.presence = presence; a.frequency = frequency; a.decay = decay; a.ids = ids_out;
  a.nblk = greedy_blocks(V);
  char* base = (char*)ws;
  a.err = (uint32_t*)base;
  // Partial results go at the tail of the workspace, away from the decode
  // step's buffers at its head (the tail of a decode workspace holds the
  // prefill-only scan buffers).
  const uint64_t part = align_up((uint64_t)B * a.nblk * 4);
  const uint64_t tail = (ws_bytes - 2 * part) / ALIGN * ALIGN;
  a.part_val = (float*)(base + tail);
  a.part_idx = (int*)(base + tail + part);
  a.B = B; a.V = V;
  HIP_TRY(launch_greedy(a, (hipStream_t)stream), "greedy");
  return RWKV7_OK;
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free greedy
// The partial (max, index) results of rwkv7_greedy_noalloc live in this
// file-scope device array, one copy per GPU, kept until the process ends:
// value partials [B * nblk] fp32 at offset 0, index partials [B * nblk] int32
// at offset GREEDY_NOALLOC_PART.  In host code `scratch` is only a stand-in
// for the symbol; its device address comes from hipGetSymbolAddress.
namespace {
constexpr uint64_t GREEDY_NOALLOC_PART = 32768;   // bytes per partial array: 8192 (row, block) pairs
static __device__ __align__(256) unsigned char scratch[2 * GREEDY_NOALLOC_PART];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RWKV7_ENOTSUP, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RWKV7_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RWKV7_OK;
}
}  // namespace

extern "C" {

int rwkv7_greedy_noalloc(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                         const int32_t* slot_idx, const float* presence, const float* frequency,
                         const float* decay, int32_t* ids_out, uint32_t* flags_out, void* stream) {
  if (B < 1 || V < 1) return fail(RWKV7_EINVAL, "B and V must be >= 1");
  if (n_slots < 1) return fail(RWKV7_EINVAL, "n_slots must be >= 1");
  if (!logits || !occ_pool || !slot_idx || !presence || !frequency || !decay || !ids_out || !flags_out)
    return fail(RWKV7_EINVAL, "null pointer argument");
  const int nblk = greedy_blocks(V);
  if ((uint64_t)B * nblk * 4 > GREEDY_NOALLOC_PART)
    return fail(RWKV7_ESHAPE, "B * ceil(V / 2048) = %lld exceeds the %llu row-blocks of the static scratch "
                "(e.g. B <= 256 at V = 65536)", (long long)B * nblk,
                (unsigned long long)(GREEDY_NOALLOC_PART / 4));
  void* base = nullptr;
  int rc = scratch_address(&base);
  if (rc) return rc;
  GreedyArgs a;
  a.logits = logits; a.occ = occ_pool; a.n_slots = n_slots; a.slot_idx = slot_idx;
  a.presence = presence; a.frequency = frequency; a.decay = decay; a.ids = ids_out;
  a.nblk = nblk;
  a.err = flags_out;
  // every (row, block) partial is written by the first pass before the second reads it,
  // so nothing in the array needs clearing between calls
  a.part_val = (float*)base;
  a.part_idx = (int*)((char*)base + GREEDY_NOALLOC_PART);
  a.B = B; a.V = V;
  HIP_TRY(launch_greedy(a, (hipStream_t)stream), "greedy");
  return RWKV7_OK;
}

int rwkv7_read_bandwidth(const void* buf, uint64_t bytes, int32_t nontemporal, int32_t iters, void* stream,
                         double* gbs) {
  if (!buf || !gbs || bytes < 16 || iters < 1) return fail(RWKV7_EINVAL, "buf, gbs, bytes >= 16, iters >= 1");
  hipStream_t st = (hipStream_t)stream;
  hipDeviceProp_t prop;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  HIP_TRY(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
  const int grid = prop.multiProcessorCount * 8;
  HIP_TRY(launch_read_stream(buf, (int64_t)bytes, nontemporal != 0, grid, st), "read stream");   // warm-up
  hipEvent_t a = nullptr, b = nullptr;
  HIP_TRY(hipEventCreate(&a), "hipEventCreate");
  HIP_TRY(hipEventCreate(&b), "hipEventCreate");
  hipError_t e = hipEventRecord(a, st);
  for (int i = 0; i < iters && e == hipSuccess; ++i) e = launch_read_stream(buf, (int64_t)bytes, nontemporal != 0, grid, st);
  if (e == hipSuccess) e = hipEventRecord(b, st);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  if (e != hipSuccess) return hip_fail(e, "read bandwidth");
  *gbs = (double)bytes * iters / (ms * 1e-3) / 1e9;
  return RWKV7_OK;
}

// Sample workspace: error word | key [B][V] u32 | histogram
// counts [B][4096] u32 | histogram weights [B][4096] u64 | per-workgroup max
// [B][SAMPLE_MAX_G] f32 | candidates [B] u32 | weight sums [B] u64.  Fills `a`'s
// pointers when it is not null; returns the size.
static uint64_t sample_layout(int64_t B, int64_t V, SampleArgs* a, char* base = nullptr) {
  uint64_t off = ALIGN;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off += align_up(bytes);
    return base + o;
  };
  char* key = take((uint64_t)B * V * 4);
  char* hc = take((uint64_t)B * 4096 * 4);
  char* hm = take((uint64_t)B * 4096 * 8);
  char* pm = take((uint64_t)B * SAMPLE_MAX_G * 4);
  char* rn = take((uint64_t)B * 4);
  char* rt = take((uint64_t)B * 8);
  if (a) {
    a->err = (uint32_t*)base;
    a->key = (uint32_t*)key;
    a->hcnt = (uint32_t*)hc;
    a->hmass = (unsigned long long*)hm;
    a->pmax = (float*)pm;
    a->rown = (uint32_t*)rn;
    a->rowtot = (unsigned long long*)rt;
  }
  return off;
}

int rwkv7_sample_workspace_bytes(int32_t B, int32_t V, uint64_t* bytes) {
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  if (B < 1 || V < 1) return fail(RWKV7_EINVAL, "B and V must be >= 1");
  *bytes = sample_layout(B, V, nullptr);
  return RWKV7_OK;
}

int rwkv7_sample(int32_t B, int32_t V, const float* logits, float* occ_pool, int64_t n_slots,
                 const int32_t* slot_idx, const float* presence, const float* frequency,
                 const float* decay, const float* temperature, const float* top_p,
                 const int32_t* top_k, const uint8_t* forbidden, const float* uniform,
                 int32_t* ids_out, void* ws, uint64_t ws_bytes, void* stream) {
  if (B < 1 || V < 1) return fail(RWKV7_EINVAL, "B and V must be >= 1");
  if (V > SAMPLE_MAX_V) return fail(RWKV7_ENOTSUP, "V must be <= %d (got %d)", SAMPLE_MAX_V, V);
  if (n_slots < 1) return fail(RWKV7_EINVAL, "n_slots must be >= 1");
  if (!logits || !occ_pool || !slot_idx || !presence || !frequency || !decay || !temperature ||
      !top_p || !top_k || !uniform || !ids_out || !ws)
    return fail(RWKV7_EINVAL, "null pointer argument");
  uint64_t need = 0;
  rwkv7_sample_workspace_bytes(B, V, &need);
  if (ws_bytes < need)
    return fail(RWKV7_ESHAPE, "workspace too small: %llu < %llu bytes", (unsigned long long)ws_bytes,
                (unsigned long long)need);
  SampleArgs a;
  a.logits = logits; a.occ = occ_pool; a.n_slots = n_slots; a.slot_idx = slot_idx;
  a.presence = presence; a.frequency = frequency; a.decay = decay;
  a.temperature = temperature; a.top_p = top_p; a.top_k = top_k; a.forbidden = forbidden;
  a.uniform = uniform; a.ids = ids_out;
  sample_layout(B, V, &a, (char*)ws);
  a.B = B; a.V = V; a.G = sample_groups(B, V);
  HIP_TRY(launch_sample(a, (hipStream_t)stream), "sample");
  return RWKV7_OK;
}

int rwkv7_int8_bytes(const rwkv7_config* cfg, uint64_t* bytes) {
  Dims d;
  int rc = check_config(cfg, &d);
  if (rc) return rc;
  if (!bytes) return fail(RWKV7_EINVAL, "bytes is NULL");
  *bytes = q8_layout(d, nullptr).bytes;
  return RWKV7_OK;
}

int rwkv7_quantize_int8(rwkv7_model* m, void* buf, uint64_t bytes, void* stream) {
  if (!m || !buf) return fail(RWKV7_EINVAL, "model and buf must be non-NULL");
  const Dims& d = m->d;
  Q8 q = q8_layout(d, (char*)buf);
  if (bytes < q.bytes)
    return fail(RWKV7_ESHAPE, "int8 buffer of %llu bytes, %llu needed", (unsigned long long)bytes,
                (unsigned long long)q.bytes);
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(launch_quant_rows(m->pk.head, d.V, d.C, q.head, q.s_head, st), "quantize head");
  for (int l = 0; l < d.L; ++l) {
    const LayerPtrs& p = m->pk.layers[l];
    const Q8Layer& y = q.layers[l];
    HIP_TRY(launch_quant_rows(p.w_in, d.Nin, d.C, y.w_in, y.s_in, st), "quantize w_in");
    HIP_TRY(launch_quant_rows(p.w_o, d.C, d.C, y.w_o, y.s_o, st), "quantize w_o");
    HIP_TRY(launch_quant_rows(p.w_key, d.F, d.C, y.w_key, y.s_key, st), "quantize w_key");
    HIP_TRY(launch_quant_rows(p.w_val_hm, d.F, d.C, y.w_val, y.s_val, st), "quantize w_val");
  }
  m->q8 = q;
  m->has_q8 = true;
  drop_graphs(m);
  return RWKV7_OK;
}

int rwkv7_debug_int8_matrix(const rwkv7_model* m, int32_t layer, int32_t which, const void** codes,
                            const float** scales, int64_t* rows, int32_t* K) {
  if (!m || !codes || !scales || !rows || !K) return fail(RWKV7_EINVAL, "null argument");
  if (!m->has_q8) return fail(RWKV7_ENOTSUP, "no int8 weights (rwkv7_quantize_int8 first)");
  const Dims& d = m->d;
  if (which == 4) {
    *codes = m->q8.head; *scales = m->q8.s_head; *rows = d.V; *K = d.C;
    return RWKV7_OK;
  }
  if (layer < 0 || layer >= d.L || which < 0 || which > 3) return fail(RWKV7_EINVAL, "bad layer or matrix");
  const Q8Layer& y = m->q8.layers[layer];
  const uint8_t* c[4] = {y.w_in, y.w_o, y.w_key, y.w_val};
  const float* s4[4] = {y.s_in, y.s_o, y.s_key, y.s_val};
  const int64_t r[4] = {d.Nin, d.C, d.F, d.F};
  *codes = c[which]; *scales = s4[which]; *rows = r[which]; *K = d.C;
  return RWKV7_OK;
}

int rwkv7_poll_error(void* ws, void* stream, uint32_t* flags) {
  if (!ws) return fail(RWKV7_EINVAL, "workspace is NULL");
  hipStream_t st = (hipStream_t)stream;
  uint32_t v = 0;
  HIP_TRY(hipStreamSynchronize(st), "hipStreamSynchronize");
  HIP_TRY(hipMemcpy(&v, ws, 4, hipMemcpyDeviceToHost), "hipMemcpy");
  HIP_TRY(hipMemset(ws, 0, 4), "hipMemset");
  if (flags) *flags = v;
  return v ? RWKV7_EDEVICE : RWKV7_OK;
}

int rwkv7_set_option(rwkv7_model* m, int32_t key, int64_t value) {
  if (!m) return fail(RWKV7_EINVAL, "model is NULL");
  switch (key) {
    case RWKV7_OPT_USE_GRAPH: m->opt_graph = value ? 1 : 0; break;
    case RWKV7_OPT_GEMV_MAX_B:
      if (value < 0 || value > 4) return fail(RWKV7_EINVAL, "GEMV_MAX_B must be in [0, 4]");
      m->opt_gemv_max = value; break;
    case RWKV7_OPT_SPARSE_MAX_B:
      if (value < 0 || value > cmix_sparse_max_b())
        return fail(RWKV7_EINVAL, "SPARSE_MAX_B must be in [0, %d]", cmix_sparse_max_b());
      m->opt_sparse_max = value; break;
    case RWKV7_OPT_KERNEL_TIMING: m->opt_timing = value ? 1 : 0; break;
    case RWKV7_OPT_PREFILL_CHUNK:
      if (value < 1) return fail(RWKV7_EINVAL, "PREFILL_CHUNK must be >= 1");
      m->opt_chunk = value; break;
    case RWKV7_OPT_FUSE_LN: m->opt_fuse_ln = value ? 1 : 0; break;
    case RWKV7_OPT_FUSE_VALUE: m->opt_fuse_value = value ? 1 : 0; break;
    case RWKV7_OPT_PREFILL_SCAN:
      if (value < 0 || value > 2) return fail(RWKV7_EINVAL, "PREFILL_SCAN must be 0, 1 or 2");
      m->opt_prefill_scan = value; break;
    case RWKV7_OPT_INT8:
      if (value && !m->has_q8) return fail(RWKV7_ENOTSUP, "INT8 needs rwkv7_quantize_int8 first");
      m->opt_int8 = value ? 1 : 0; break;
    case RWKV7_OPT_LN_SPLIT:
      if (value < 0 || value > 16) return fail(RWKV7_EINVAL, "LN_SPLIT must be in [0, 16]");
      m->opt_ln_split = value; break;
    case RWKV7_OPT_WKV_ADAPTERS:
      if (value < 0 || value > 4) return fail(RWKV7_EINVAL, "WKV_ADAPTERS must be in [0, 4]");
      m->opt_wkv_ad = value; break;
    case RWKV7_OPT_GEMM_PLAN_PROJ_IN:
    case RWKV7_OPT_GEMM_PLAN_ADAPTERS:
    case RWKV7_OPT_GEMM_PLAN_PROJ_OUT:
    case RWKV7_OPT_GEMM_PLAN_CMIX_KEY:
    case RWKV7_OPT_GEMM_PLAN_CMIX_VALUE:
    case RWKV7_OPT_GEMM_PLAN_HEAD: {
      if (value != 0) {
        const PlanCode c = decode_plan(value);
        if (value < 0 || value >= 10000000 || !gemm_cfg_ok(c.tm, c.tn, c.ks, c.pipe))
          return fail(RWKV7_EINVAL, "GEMM plan %lld is not a supported tile configuration", (long long)value);
      }
      m->opt_plan[key - RWKV7_OPT_GEMM_PLAN_PROJ_IN] = value;
      break;
    }
    default: return fail(RWKV7_EINVAL, "unknown option %d", key);
  }
  // cached graphs bake in the kernel path: drop them when it may change
  if (key == RWKV7_OPT_GEMV_MAX_B || key == RWKV7_OPT_SPARSE_MAX_B || key == RWKV7_OPT_FUSE_LN ||
      key == RWKV7_OPT_FUSE_VALUE || key == RWKV7_OPT_INT8 || key == RWKV7_OPT_LN_SPLIT || key == RWKV7_OPT_WKV_ADAPTERS || (key >= RWKV7_OPT_GEMM_PLAN_PROJ_IN && key <= RWKV7_OPT_GEMM_PLAN_HEAD))
    drop_graphs(m);
  return RWKV7_OK;
}

int rwkv7_get_option(const rwkv7_model* m, int32_t key, int64_t* value) {
  if (!m || !value) return fail(RWKV7_EINVAL, "null argument");
  switch (key) {
    case RWKV7_OPT_USE_GRAPH: *value = m->opt_graph; break;
    case RWKV7_OPT_GEMV_MAX_B: *value = m->opt_gemv_max; break;
    case RWKV7_OPT_SPARSE_MAX_B: *value = m->opt_sparse_max; break;
    case RWKV7_OPT_KERNEL_TIMING: *value = m->opt_timing; break;
    case RWKV7_OPT_PREFILL_CHUNK: *value = m->opt_chunk; break;
    case RWKV7_OPT_FUSE_LN: *value = m->opt_fuse_ln; break;
    case RWKV7_OPT_FUSE_VALUE: *value = m->opt_fuse_value; break;
    case RWKV7_OPT_PREFILL_SCAN: *value = m->opt_prefill_scan; break;
    case RWKV7_OPT_INT8: *value = m->opt_int8; break;
    case RWKV7_OPT_LN_SPLIT: *value = m->opt_ln_split; break;
    case RWKV7_OPT_WKV_ADAPTERS: *value = m->opt_wkv_ad; break;
    case RWKV7_OPT_GEMM_PLAN_PROJ_IN:
    case RWKV7_OPT_GEMM_PLAN_ADAPTERS:
    case RWKV7_OPT_GEMM_PLAN_PROJ_OUT:
    case RWKV7_OPT_GEMM_PLAN_CMIX_KEY:
    case RWKV7_OPT_GEMM_PLAN_CMIX_VALUE:
    case RWKV7_OPT_GEMM_PLAN_HEAD: *value = m->opt_plan[key - RWKV7_OPT_GEMM_PLAN_PROJ_IN]; break;
    default: return fail(RWKV7_EINVAL, "unknown option %d", key);
  }
  return RWKV7_OK;
}

int rwkv7_kernel_timing(rwkv7_model* m, int32_t cls, double* total_ms, int64_t* launches,
                        int32_t reset) {
  if (!m) return fail(RWKV7_EINVAL, "model is NULL");
  if (cls < 0 || cls >= RWKV7_K_COUNT) return fail(RWKV7_EINVAL, "unknown kernel class %d", cls);
  for (auto& t : m->pending) {
    HIP_TRY(hipEventSynchronize(t.b), "hipEventSynchronize");
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, t.a, t.b), "hipEventElapsedTime");
    m->t_ms[t.cls] += ms;
    m->t_n[t.cls] += 1;
    m->free_events.push_back({t.a, t.b});
  }
  m->pending.clear();
  if (total_ms) *total_ms = m->t_ms[cls];
  if (launches) *launches = m->t_n[cls];
  if (reset) {
    for (int i = 0; i < RWKV7_K_COUNT; ++i) { m->t_ms[i] = 0; m->t_n[i] = 0; }
  }
  return RWKV7_OK;
}

int rwkv7_time_kernel(rwkv7_model* m, void* pool, int64_t n_slots, int32_t B,
                      const int32_t* slot_idx, const int32_t* token_ids, float* logits_out,
                      int32_t kernel_class, int32_t layer, int32_t iters, void* ws,
                      uint64_t ws_bytes, void* stream, double* avg_ms) {
  if (!m || !avg_ms) return fail(RWKV7_EINVAL, "null argument");
  if (B < 1 || B > n_slots) return fail(RWKV7_EINVAL, "B out of range");
  if (kernel_class < 0 || kernel_class >= RWKV7_K_COUNT) return fail(RWKV7_EINVAL, "bad kernel class");
  if (layer < -1 || layer > m->d.L) return fail(RWKV7_EINVAL, "layer outside [-1, n_layer]");
  if (iters < 1) return fail(RWKV7_EINVAL, "iters must be >= 1");
  int rc = check_pool_ws(m, pool, n_slots, ws, ws_bytes, ws_layout(m->d, B, nullptr).bytes);
  if (rc) return rc;
  if (!slot_idx || !token_ids || !logits_out) return fail(RWKV7_EINVAL, "null pointer argument");
  hipStream_t st = (hipStream_t)stream;
  // Rebuild the step's sanitized rows and embeddings first: other calls on
  // this workspace (rwkv7_greedy, a prefill) may have reused its buffers.
  {
    Filter pre;
    pre.cls = RWKV7_K_OTHER;
    pre.layer = -1;
    rc = enqueue_decode(m, (float*)pool, n_slots, B, slot_idx, token_ids, logits_out, (char*)ws, st,
                        false, &pre);
    if (rc) return rc;
  }
  // layer -1: sweep the class over layers 0..n_layer-1, `iters` times, so
  // every launch streams other weights than the one before it (as in a step)
  const bool sweep = layer < 0;
  if (sweep && (kernel_class == RWKV7_K_HEAD || kernel_class == RWKV7_K_OTHER))
    return fail(RWKV7_EINVAL, "layer -1 needs a per-layer kernel class");
  Filter f;
  f.cls = kernel_class;
  f.layer = layer;
  f.any_layer = sweep;
  f.repeat = sweep ? 1 : iters;
  const int passes = sweep ? iters : 1;
  const int launches = sweep ? iters * m->d.L : iters;
  hipEvent_t a, b;
  HIP_TRY(hipEventCreate(&a), "hipEventCreate");
  HIP_TRY(hipEventCreate(&b), "hipEventCreate");
  HIP_TRY(hipEventRecord(a, st), "hipEventRecord");
  for (int i = 0; i < passes && rc == RWKV7_OK; ++i)
    rc = enqueue_decode(m, (float*)pool, n_slots, B, slot_idx, token_ids, logits_out, (char*)ws, st,
                        false, &f);
  HIP_TRY(hipEventRecord(b, st), "hipEventRecord");
  HIP_TRY(hipEventSynchronize(b), "hipEventSynchronize");
  float ms = 0.f;
  hipEventElapsedTime(&ms, a, b);
  hipEventDestroy(a);
  hipEventDestroy(b);
  if (rc) return rc;
  *avg_ms = (double)ms / launches;
  return RWKV7_OK;
}

const char* rwkv7_kernel_name(const rwkv7_model* m, int32_t cls, int32_t B) {
  if (!m || cls < 0 || cls >= RWKV7_K_COUNT) return "";
  const Path p = decode_path(m, B);
  const bool q = m->opt_int8 && m->has_q8 && p.gemv && B <= 2;
  switch (cls) {
    case RWKV7_K_LN_MIX: return "k_ln_mix";
    case RWKV7_K_PROJ_IN:
      return p.gemv ? gemv_kernel_name(B, m->d.C, -1, m->d.Nin, 7, p.fused, q) : gemm_kernel_name(B, m->d.Nin, m->d.C);
    case RWKV7_K_PROJ_OUT:
      return p.gemv ? gemv_kernel_name(B, m->d.C, EPI_RESID, m->d.C, 1, false, q) : gemm_kernel_name(B, m->d.C, m->d.C);
    case RWKV7_K_CMIX_KEY:
      return p.gemv ? gemv_kernel_name(B, m->d.C, p.fuse_value ? -2 : p.sparse ? EPI_PRE : -1, m->d.F, 1,
                                      p.fused || p.fuse_value, q)
                    : gemm_kernel_name(B, m->d.F, m->d.C);
    case RWKV7_K_HEAD:
      return p.gemv ? gemv_kernel_name(B, m->d.C, EPI_NONE, m->d.V, 1, p.fused, q) : gemm_kernel_name(B, m->d.V, m->d.C);
    case RWKV7_K_WKV: {
      static char name[48];
      if (!p.gemv) {
        const Dims& d = m->d;
        WkvArgs t;
        memset(&t, 0, sizeof t);
        t.Lin = d.Lin; t.off_a = d.Dwp; t.off_v = d.Dwp + d.Dap; t.off_g = d.Dwp + d.Dap + d.Dvp;
        t.Dw = d.Dw; t.Da = d.Da; t.Dv = d.Dv; t.Dg = d.Dg;
        const int rpw = wkv_ad_rows_per_wave(m, B);
        if (rpw && wkv_chunk_adapters_ok(t)) {
          snprintf(name, sizeof name, "k_wkv_decode_ad<%d, %d, %d, %d, %d>", d.Dw, d.Da, d.Dv, d.Dg, rpw);
          return name;
        }
        return wkv_rows_waves(B * d.H) == 5 ? "k_wkv_decode_rows<5>" : "k_wkv_decode_rows<4>";
      }
      snprintf(name, sizeof name, "k_wkv_decode<%d>", (m->d.Dw + m->d.Da + m->d.Dv + m->d.Dg) / 32);
      return name;
    }
    case RWKV7_K_CMIX_VALUE:
      if (p.fuse_value) return B == 1 ? "k_cmix_fold<1>" : "k_cmix_fold<2>";
      return p.sparse ? cmix_sparse_kernel_name(B) : gemm_kernel_name(B, m->d.C, m->d.F);
    default: return kClassName[cls];
  }
}

int rwkv7_debug_cmix_buffers(const rwkv7_model* m, void* ws, int32_t B, void** pre, void** mask,
                             void** active, void** active_count) {
  if (!m || !ws || !pre || !mask || !active || !active_count)
    return fail(RWKV7_EINVAL, "null argument");
  if (B < 1) return fail(RWKV7_EINVAL, "B must be >= 1");
  const Ws w = ws_layout(m->d, B, (char*)ws);
  *pre = w.pre;
  *mask = w.mask;
  *active = w.dbg_idx;
  *active_count = w.dbg_cnt;
  return RWKV7_OK;
}

int rwkv7_debug_wkv_out(const rwkv7_model* m, void* ws, int32_t B, void** out, int32_t* is_f16) {
  if (!m || !ws || !out || !is_f16) return fail(RWKV7_EINVAL, "null argument");
  if (B < 1) return fail(RWKV7_EINVAL, "B must be >= 1");
  const Ws w = ws_layout(m->d, B, (char*)ws);
  *out = w.yg;
  *is_f16 = decode_path(m, B).gemv ? 0 : 1;
  return RWKV7_OK;
}

}  // extern "C"
