// Continuous-batching scheduler over the rwkv7 C ABI (host code), and the
// backend that drives a loaded model on one HIP stream.  The round structure
// follows the Albatross article (RWKV-Runner backend, "continuous batching:
// the worker main loop") and the task states the RWKV-Server article
// ("RWKV-Server design"); include/rwkv7_sched.h states the reading in full.
//
// The scheduler itself touches no device memory: a round is a list of host
// arrays handed to the backend's three callbacks.  State never moves between
// slots (the kernels gather rows through slot_idx), so organising a batch is
// ordering row indices, not swapping state.
#include "launch.h"
#include "../../include/rwkv7_sched.h"
#include "../../include/rwkv7_prefix.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

int sfail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int sfail(int code, const char* fmt, ...) {
  char buf[384];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return lib_fail(code, buf);
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): output number n (n >= 1) of the generator whose
// state starts at `seed`.
uint64_t splitmix64_nth(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The task's uniform for its j-th generated token: the top 24 bits, exact in fp32.
float task_uniform(uint64_t seed, int64_t j) {
  return (float)(splitmix64_nth(seed, (uint64_t)j + 1) >> 40) * (1.0f / 16777216.0f);
}

struct Task {
  int64_t id = 0;
  std::vector<int32_t> prompt;
  rwkv7_sched_params p{};
  int state = RWKV7_TASK_QUEUED;
  int slot = -1;
  bool seq = false;      // PREFILL through rwkv7_prefill_seq (else one token per round)
  int pos = 0;           // prompt tokens already fed on the one-token path
  int gen = 0;           // tokens generated
  int32_t cur = 0;       // next decode input
  int64_t admitted = 0;  // admission order
};

}  // namespace

struct rwkv7_sched {
  rwkv7_sched_config cfg{};
  rwkv7_sched_backend be{};
  int64_t next_id = 1;
  int64_t admit_seq = 0;
  int countdown = 0;  // decode rounds until the next sequence prefill may run
  std::deque<int64_t> queue;
  std::unordered_map<int64_t, Task> live;  // queued and slot-holding tasks
  std::vector<int64_t> slot_task;          // per slot: task id, 0 = free
  std::vector<int64_t> aborts;
  std::deque<rwkv7_sched_event> events;
  // one round's rows
  std::vector<int32_t> r_slot, r_tok, r_topk, r_ids;
  std::vector<float> r_temp, r_topp, r_pres, r_freq, r_dec, r_uni;
  std::vector<int64_t> r_task;

  void emit(int64_t task, int kind, int value, int index) {
    rwkv7_sched_event e{};
    e.task = task;
    e.kind = kind;
    e.value = value;
    e.index = index;
    events.push_back(e);
  }
  void finish(Task& t, int reason) {
    emit(t.id, RWKV7_EV_FINISHED, reason, t.gen);
    if (t.slot >= 0) slot_task[t.slot] = 0;
    live.erase(t.id);  // t is gone after this
  }
};

extern "C" {

int rwkv7_sched_create(const rwkv7_sched_config* cfg, const rwkv7_sched_backend* backend,
                       rwkv7_sched** out) {
  if (!cfg || !backend || !out) return sfail(RWKV7_EINVAL, "cfg, backend and out must be non-NULL");
  if (cfg->max_batch < 1) return sfail(RWKV7_EINVAL, "max_batch must be >= 1 (got %d)", cfg->max_batch);
  if (cfg->vocab < 1) return sfail(RWKV7_EINVAL, "vocab must be >= 1 (got %d)", cfg->vocab);
  if (!backend->reset || !backend->prefill || !backend->step)
    return sfail(RWKV7_EINVAL, "the backend needs reset, prefill and step callbacks");
  rwkv7_sched* s = new rwkv7_sched;
  s->cfg = *cfg;
  if (s->cfg.max_prefill_count <= 0) {
    const int m = (int)(s->cfg.max_batch * 0.125);
    s->cfg.max_prefill_count = m > 1 ? m : 1;
  }
  if (s->cfg.decode_prefill_ratio <= 0) s->cfg.decode_prefill_ratio = 5;
  if (s->cfg.min_forward_seq_len <= 0) s->cfg.min_forward_seq_len = 10;
  s->be = *backend;
  s->slot_task.assign(s->cfg.max_batch, 0);
  *out = s;
  return RWKV7_OK;
}

int rwkv7_sched_free(rwkv7_sched* s) {
  delete s;
  return RWKV7_OK;
}

int rwkv7_sched_submit(rwkv7_sched* s, const int32_t* prompt, int32_t n,
                       const rwkv7_sched_params* params, int64_t* task_id) {
  if (!s || !prompt || !params || !task_id) return sfail(RWKV7_EINVAL, "NULL argument");
  if (n < 1) return sfail(RWKV7_EINVAL, "a prompt needs at least one token (got %d)", n);
  for (int i = 0; i < n; ++i)
    if (prompt[i] < 0 || prompt[i] >= s->cfg.vocab)
      return sfail(RWKV7_EINVAL, "prompt[%d] = %d is outside [0, %d)", i, prompt[i], s->cfg.vocab);
  if (params->max_new_tokens < 1)
    return sfail(RWKV7_EINVAL, "max_new_tokens must be >= 1 (got %d)", params->max_new_tokens);
  if (params->stop_token < -1 || params->stop_token >= s->cfg.vocab)
    return sfail(RWKV7_EINVAL, "stop_token %d is outside [-1, %d)", params->stop_token, s->cfg.vocab);
  Task t;
  t.id = s->next_id++;
  t.prompt.assign(prompt, prompt + n);
  t.p = *params;
  s->queue.push_back(t.id);
  *task_id = t.id;
  s->live.emplace(t.id, std::move(t));
  return RWKV7_OK;
}

int rwkv7_sched_abort(rwkv7_sched* s, int64_t task_id) {
  if (!s) return sfail(RWKV7_EINVAL, "NULL scheduler");
  if (!s->live.count(task_id))
    return sfail(RWKV7_EINVAL, "task %lld is unknown or already finished", (long long)task_id);
  s->aborts.push_back(task_id);
  return RWKV7_OK;
}

int rwkv7_sched_task_state(const rwkv7_sched* s, int64_t task_id, int32_t* state) {
  if (!s || !state) return sfail(RWKV7_EINVAL, "NULL argument");
  auto it = s->live.find(task_id);
  if (it != s->live.end()) {
    *state = it->second.state;
    return RWKV7_OK;
  }
  if (task_id >= 1 && task_id < s->next_id) {
    *state = RWKV7_TASK_FINISHED;
    return RWKV7_OK;
  }
  return sfail(RWKV7_EINVAL, "task %lld was never submitted", (long long)task_id);
}

int rwkv7_sched_poll(rwkv7_sched* s, rwkv7_sched_event* out, int32_t cap, int32_t* n) {
  if (!s || !n || (cap > 0 && !out)) return sfail(RWKV7_EINVAL, "NULL argument");
  int k = 0;
  while (k < cap && !s->events.empty()) {
    out[k++] = s->events.front();
    s->events.pop_front();
  }
  *n = k;
  return RWKV7_OK;
}

int rwkv7_sched_step(rwkv7_sched* s, rwkv7_sched_stats* stats) {
  if (!s) return sfail(RWKV7_EINVAL, "NULL scheduler");
  rwkv7_sched_stats st{};
  const int M = s->cfg.max_batch;

  // 1. abort requests
  for (int64_t id : s->aborts) {
    auto it = s->live.find(id);
    if (it == s->live.end()) continue;  // finished meanwhile, or listed twice
    if (it->second.state == RWKV7_TASK_QUEUED) {
      for (auto q = s->queue.begin(); q != s->queue.end(); ++q)
        if (*q == id) {
          s->queue.erase(q);
          break;
        }
    }
    s->finish(it->second, RWKV7_FIN_ABORT);
    ++st.finished;
  }
  s->aborts.clear();

  // 2. admission: FIFO into the lowest free slots, prefills capped
  int in_prefill = 0;
  for (int i = 0; i < M; ++i)
    if (s->slot_task[i] && s->live[s->slot_task[i]].state == RWKV7_TASK_PREFILL) ++in_prefill;
  while (!s->queue.empty()) {
    Task& t = s->live[s->queue.front()];
    const int n = (int)t.prompt.size();
    if (n >= 2 && in_prefill >= s->cfg.max_prefill_count) break;
    int slot = -1;
    for (int i = 0; i < M && slot < 0; ++i)
      if (!s->slot_task[i]) slot = i;
    if (slot < 0) break;
    int rc = s->be.reset(s->be.ctx, slot);
    if (rc) return rc;
    s->queue.pop_front();
    t.slot = slot;
    t.admitted = s->admit_seq++;
    s->slot_task[slot] = t.id;
    if (n >= 2) {
      t.state = RWKV7_TASK_PREFILL;
      t.seq = n >= s->cfg.min_forward_seq_len;
      t.pos = 0;
      ++in_prefill;
    } else {
      t.state = RWKV7_TASK_READY;
      t.cur = t.prompt[0];
    }
    ++st.admitted;
  }

  // 3. at most one sequence prefill, paced against the decode rounds
  Task* pick = nullptr;
  bool rows_waiting = false;
  for (int i = 0; i < M; ++i) {
    if (!s->slot_task[i]) continue;
    Task& t = s->live[s->slot_task[i]];
    if (t.state == RWKV7_TASK_PREFILL && t.seq) {
      if (!pick || t.admitted < pick->admitted) pick = &t;
    } else {
      rows_waiting = true;
    }
  }
  if (pick && (!rows_waiting || s->countdown <= 0)) {
    const int T = (int)pick->prompt.size() - 1;
    int rc = s->be.prefill(s->be.ctx, pick->slot, pick->prompt.data(), T);
    if (rc) return rc;
    pick->state = RWKV7_TASK_READY;
    pick->cur = pick->prompt[T];
    s->countdown = s->cfg.decode_prefill_ratio;
    st.seq_prefills = 1;
    st.seq_prefill_tokens = T;
  }

  // 4. rows: decode rows by slot, then one-token prefill rows by slot
  s->r_slot.clear(); s->r_tok.clear(); s->r_topk.clear(); s->r_task.clear();
  s->r_temp.clear(); s->r_topp.clear(); s->r_pres.clear(); s->r_freq.clear(); s->r_dec.clear();
  s->r_uni.clear();
  for (int i = 0; i < M; ++i) {
    if (!s->slot_task[i]) continue;
    Task& t = s->live[s->slot_task[i]];
    if (t.state != RWKV7_TASK_READY && t.state != RWKV7_TASK_RUNNING) continue;
    t.state = RWKV7_TASK_RUNNING;
    s->r_slot.push_back(i);
    s->r_tok.push_back(t.cur);
    s->r_task.push_back(t.id);
    s->r_temp.push_back(t.p.temperature);
    s->r_topp.push_back(t.p.top_p);
    s->r_topk.push_back(t.p.top_k);
    s->r_pres.push_back(t.p.presence);
    s->r_freq.push_back(t.p.frequency);
    s->r_dec.push_back(t.p.decay);
    s->r_uni.push_back(task_uniform(t.p.seed, t.gen));
  }
  const int n_sample = (int)s->r_slot.size();
  for (int i = 0; i < M; ++i) {
    if (!s->slot_task[i]) continue;
    Task& t = s->live[s->slot_task[i]];
    if (t.state != RWKV7_TASK_PREFILL || t.seq) continue;
    s->r_slot.push_back(i);
    s->r_tok.push_back(t.prompt[t.pos]);
    s->r_task.push_back(t.id);
  }
  const int B = (int)s->r_slot.size();

  // 5. one batched forward + sampling
  if (B > 0) {
    s->r_ids.assign(n_sample > 0 ? n_sample : 1, -1);
    rwkv7_sched_batch b{};
    b.B = B;
    b.slots = s->r_slot.data();
    b.tokens = s->r_tok.data();
    b.n_sample = n_sample;
    b.temperature = s->r_temp.data();
    b.top_p = s->r_topp.data();
    b.top_k = s->r_topk.data();
    b.presence = s->r_pres.data();
    b.frequency = s->r_freq.data();
    b.decay = s->r_dec.data();
    b.uniform = s->r_uni.data();
    int rc = s->be.step(s->be.ctx, &b, s->r_ids.data());
    if (rc) return rc;
    for (int r = 0; r < n_sample; ++r)
      if (s->r_ids[r] < 0 || s->r_ids[r] >= s->cfg.vocab)
        return sfail(RWKV7_EDEVICE, "the backend returned token %d for row %d", s->r_ids[r], r);
    if (n_sample > 0) --s->countdown;
  }

  // 6. outputs and phase changes
  for (int r = 0; r < B; ++r) {
    Task& t = s->live[s->r_task[r]];
    if (r < n_sample) {
      const int32_t id = s->r_ids[r];
      s->emit(t.id, RWKV7_EV_TOKEN, id, t.gen);
      ++t.gen;
      t.cur = id;
      if (t.p.stop_token >= 0 && id == t.p.stop_token) {
        s->finish(t, RWKV7_FIN_STOP);
        ++st.finished;
      } else if (t.gen >= t.p.max_new_tokens) {
        s->finish(t, RWKV7_FIN_LENGTH);
        ++st.finished;
      }
    } else if (++t.pos == (int)t.prompt.size() - 1) {
      t.state = RWKV7_TASK_READY;
      t.cur = t.prompt[t.pos];
    }
  }

  st.decode_rows = n_sample;
  st.one_prefill_rows = B - n_sample;
  st.queued = (int32_t)s->queue.size();
  for (int i = 0; i < M; ++i) st.active += s->slot_task[i] != 0;
  if (stats) *stats = st;
  return RWKV7_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- GPU backend
namespace {

// Device and pinned staging of one round: int32 slots | tokens | top_k, then
// fp32 temperature | top_p | presence | frequency | decay | uniform, max_B
// entries each; the ids and both workspaces' error words come back in one
// pinned block.  Both buffers are the caller's (rwkv7_sched_gpu_backend_bytes).
constexpr int STAGE_ARRAYS = 9;

uint64_t up256(uint64_t n) { return (n + 255) & ~(uint64_t)255; }

// Byte offsets of the backend's pieces inside the caller's buffers.
struct GbLayout {
  uint64_t d_stage, d_ids, d_logits, d_tok, dev_bytes;
  uint64_t h_stage, h_back, host_bytes;
};

GbLayout gb_layout(int max_B, int V, int max_T) {
  GbLayout o;
  const uint64_t stage = (uint64_t)STAGE_ARRAYS * max_B * 4;
  o.d_stage = 0;
  o.d_ids = o.d_stage + up256(stage);
  o.d_logits = o.d_ids + up256((uint64_t)max_B * 4);
  o.d_tok = o.d_logits + up256((uint64_t)max_B * V * 4);
  o.dev_bytes = o.d_tok + up256((uint64_t)max_T * 4);
  o.h_stage = 0;
  o.h_back = up256(stage);
  o.host_bytes = o.h_back + up256((uint64_t)(max_B + 2) * 4);
  return o;
}

struct GpuBackend {
  rwkv7_model* model = nullptr;
  void* pool = nullptr;
  int64_t n_slots = 0;
  float* occ = nullptr;
  const uint8_t* forbidden = nullptr;
  int max_B = 0, V = 0, max_T = 0;
  void* ws = nullptr;
  uint64_t ws_bytes = 0;
  void* sws = nullptr;
  uint64_t sws_bytes = 0;
  hipStream_t st = nullptr;
  int32_t* h_stage = nullptr;  // caller's pinned buffer: STAGE_ARRAYS * max_B words
  int32_t* d_stage = nullptr;  // caller's device buffer from here on
  int32_t* h_back = nullptr;   // pinned: ids[max_B], err[2]
  int32_t* d_ids = nullptr;
  float* d_logits = nullptr;   // [max_B * V]
  int32_t* d_tok = nullptr;    // prefill tokens, max_T per piece
  rwkv7_prefix_cache* cache = nullptr;
  int64_t restored = 0, prefilled = 0;
};

int gb_hip(hipError_t e, const char* what) {
  return e == hipSuccess ? RWKV7_OK : sfail(RWKV7_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int gb_reset(void* ctx, int32_t slot) {
  GpuBackend* g = (GpuBackend*)ctx;
  if (slot < 0 || slot >= g->n_slots) return sfail(RWKV7_EINVAL, "slot %d outside the pool", slot);
  g->h_stage[0] = slot;
  int rc = gb_hip(hipMemcpyAsync(g->d_stage, g->h_stage, 4, hipMemcpyHostToDevice, g->st), "stage slot");
  if (rc) return rc;
  rc = rwkv7_reset_slots(g->model, g->pool, g->n_slots, g->d_stage, 1, g->ws, g->ws_bytes, g->st);
  if (rc) return rc;
  rc = gb_hip(hipMemsetAsync(g->occ + (int64_t)slot * g->V, 0, (size_t)g->V * 4, g->st), "clear occ row");
  if (rc) return rc;
  // the staging word is rewritten by the next call: wait for the copy to finish
  return gb_hip(hipStreamSynchronize(g->st), "reset sync");
}

int gb_prefill(void* ctx, int32_t slot, const int32_t* all_tokens, int32_t T_all) {
  GpuBackend* g = (GpuBackend*)ctx;
  int32_t start = 0;
  if (g->cache) {
    int rc = rwkv7_prefix_cache_lookup(g->cache, g->pool, g->n_slots, slot, all_tokens, T_all, &start, g->st);
    if (rc) return rc;
  }
  g->restored += start;
  const int32_t* tokens = all_tokens + start;
  const int32_t T = T_all - start;
  if (T == 0) return gb_hip(hipStreamSynchronize(g->st), "prefill sync");
  g->prefilled += T;
  // pieces of at most max_T tokens: prefilling a then b lands where a || b does.
  // Each piece's copy is queued behind the previous piece's kernels on the same
  // stream, so the token buffer is never overwritten while still being read.
  int rc = RWKV7_OK;
  for (int32_t done = 0; done < T; done += g->max_T) {
    const int32_t n = T - done < g->max_T ? T - done : g->max_T;
    rc = gb_hip(hipMemcpyAsync(g->d_tok, tokens + done, (size_t)n * 4, hipMemcpyHostToDevice, g->st),
                "stage prefill tokens");
    if (rc) return rc;
    rc = rwkv7_prefill_seq(g->model, g->pool, g->n_slots, slot, g->d_tok, n, g->ws, g->ws_bytes, g->st);
    if (rc) return rc;
  }
  if (g->cache) {
    rc = rwkv7_prefix_cache_store(g->cache, g->pool, g->n_slots, slot, all_tokens, T_all, g->st);
    if (rc) return rc;
  }
  return gb_hip(hipStreamSynchronize(g->st), "prefill sync");
}

int gb_step(void* ctx, const rwkv7_sched_batch* b, int32_t* ids_out) {
  GpuBackend* g = (GpuBackend*)ctx;
  const int B = b->B, S = b->n_sample, M = g->max_B;
  if (B < 1 || B > M || S < 0 || S > B)
    return sfail(RWKV7_EINVAL, "round of %d rows (%d sampled) exceeds the backend's %d", B, S, M);
  int32_t* h = g->h_stage;
  std::memcpy(h, b->slots, (size_t)B * 4);
  std::memcpy(h + M, b->tokens, (size_t)B * 4);
  if (S > 0) {
    std::memcpy(h + 2 * M, b->top_k, (size_t)S * 4);
    const float* src[6] = {b->temperature, b->top_p, b->presence, b->frequency, b->decay, b->uniform};
    for (int k = 0; k < 6; ++k) std::memcpy(h + (3 + k) * M, src[k], (size_t)S * 4);
  }
  int rc = gb_hip(hipMemcpyAsync(g->d_stage, h, (size_t)STAGE_ARRAYS * M * 4, hipMemcpyHostToDevice, g->st),
                  "stage round");
  if (rc) return rc;
  int32_t* d = g->d_stage;
  rc = rwkv7_decode_step(g->model, g->pool, g->n_slots, B, d, d + M, g->d_logits, g->ws, g->ws_bytes, g->st);
  if (rc) return rc;
  if (S > 0) {
    const float* f = (const float*)d;
    rc = rwkv7_sample(S, g->V, g->d_logits, g->occ, g->n_slots, d, f + 5 * M, f + 6 * M, f + 7 * M,
                      f + 3 * M, f + 4 * M, d + 2 * M, g->forbidden, f + 8 * M, g->d_ids, g->sws,
                      g->sws_bytes, g->st);
    if (rc) return rc;
    rc = gb_hip(hipMemcpyAsync(g->h_back, g->d_ids, (size_t)S * 4, hipMemcpyDeviceToHost, g->st), "ids back");
    if (rc) return rc;
  }
  rc = gb_hip(hipMemcpyAsync(g->h_back + M, g->ws, 4, hipMemcpyDeviceToHost, g->st), "error word");
  if (rc) return rc;
  rc = gb_hip(hipMemcpyAsync(g->h_back + M + 1, g->sws, 4, hipMemcpyDeviceToHost, g->st), "error word");
  if (rc) return rc;
  rc = gb_hip(hipStreamSynchronize(g->st), "round sync");
  if (rc) return rc;
  if (g->h_back[M] || g->h_back[M + 1]) {
    uint32_t f0 = 0, f1 = 0;
    rwkv7_poll_error(g->ws, g->st, &f0);
    rwkv7_poll_error(g->sws, g->st, &f1);
    return sfail(RWKV7_EDEVICE, "device error flags: decode 0x%x, sample 0x%x", f0, f1);
  }
  std::memcpy(ids_out, g->h_back, (size_t)S * 4);
  return RWKV7_OK;
}

void gb_release(GpuBackend* g) { delete g; }  // the buffers stay the caller's

}  // namespace

extern "C" {

int rwkv7_sched_gpu_backend_bytes(const rwkv7_model* model, int32_t max_B, int32_t max_T,
                                  uint64_t* device_bytes, uint64_t* host_bytes) {
  if (!model || !device_bytes || !host_bytes)
    return sfail(RWKV7_EINVAL, "model, device_bytes and host_bytes must be non-NULL");
  if (max_B < 1 || max_T < 1) return sfail(RWKV7_EINVAL, "max_B and max_T must be >= 1 (got %d, %d)", max_B, max_T);
  const GbLayout o = gb_layout(max_B, lib_model_vocab(model), max_T);
  *device_bytes = o.dev_bytes;
  *host_bytes = o.host_bytes;
  return RWKV7_OK;
}

int rwkv7_sched_gpu_backend(rwkv7_model* model, void* pool, int64_t n_slots, float* occ_pool,
                            const uint8_t* forbidden, int32_t max_B, int32_t max_T, void* ws, uint64_t ws_bytes,
                            void* sample_ws, uint64_t sample_ws_bytes, void* dev_buf, uint64_t dev_bytes,
                            void* host_buf, uint64_t host_bytes, void* stream, rwkv7_sched_backend* out) {
  if (!model || !pool || !occ_pool || !ws || !sample_ws || !dev_buf || !host_buf || !out)
    return sfail(RWKV7_EINVAL, "model, pool, occ_pool, ws, sample_ws, dev_buf, host_buf and out must be non-NULL");
  if (max_B < 1 || max_B > n_slots)
    return sfail(RWKV7_EINVAL, "max_B must lie in [1, n_slots] (got %d, n_slots %lld)", max_B,
                 (long long)n_slots);
  if (max_T < 1) return sfail(RWKV7_EINVAL, "max_T must be >= 1 (got %d)", max_T);
  if (((uintptr_t)dev_buf & 255) || ((uintptr_t)host_buf & 255))
    return sfail(RWKV7_EINVAL, "dev_buf and host_buf must be 256-byte aligned");
  const int V = lib_model_vocab(model);
  uint64_t need = 0;
  int rc = rwkv7_sample_workspace_bytes(max_B, V, &need);
  if (rc) return rc;
  if (sample_ws_bytes < need)
    return sfail(RWKV7_ESHAPE, "sample workspace of %llu bytes, %llu needed", (unsigned long long)sample_ws_bytes,
                 (unsigned long long)need);
  const GbLayout o = gb_layout(max_B, V, max_T);
  if (dev_bytes < o.dev_bytes || host_bytes < o.host_bytes)
    return sfail(RWKV7_ESHAPE, "backend buffers of %llu (device) / %llu (host) bytes, %llu / %llu needed",
                 (unsigned long long)dev_bytes, (unsigned long long)host_bytes,
                 (unsigned long long)o.dev_bytes, (unsigned long long)o.host_bytes);
  GpuBackend* g = new GpuBackend;
  g->model = model; g->pool = pool; g->n_slots = n_slots; g->occ = occ_pool; g->forbidden = forbidden;
  g->max_B = max_B; g->V = V; g->max_T = max_T; g->ws = ws; g->ws_bytes = ws_bytes; g->sws = sample_ws;
  g->sws_bytes = sample_ws_bytes; g->st = (hipStream_t)stream;
  char* d = (char*)dev_buf;
  char* h = (char*)host_buf;
  g->d_stage = (int32_t*)(d + o.d_stage);
  g->d_ids = (int32_t*)(d + o.d_ids);
  g->d_logits = (float*)(d + o.d_logits);
  g->d_tok = (int32_t*)(d + o.d_tok);
  g->h_stage = (int32_t*)(h + o.h_stage);
  g->h_back = (int32_t*)(h + o.h_back);
  std::memset(g->h_stage, 0, (size_t)STAGE_ARRAYS * max_B * 4);
  out->ctx = g;
  out->reset = gb_reset;
  out->prefill = gb_prefill;
  out->step = gb_step;
  return RWKV7_OK;
}

int rwkv7_sched_gpu_backend_set_cache(rwkv7_sched_backend* backend, rwkv7_prefix_cache* cache) {
  if (!backend || backend->step != gb_step || !backend->ctx)
    return sfail(RWKV7_EINVAL, "not a backend made by rwkv7_sched_gpu_backend");
  ((GpuBackend*)backend->ctx)->cache = cache;
  return RWKV7_OK;
}

int rwkv7_sched_gpu_backend_counts(const rwkv7_sched_backend* backend, int64_t* tokens_restored,
                                   int64_t* tokens_prefilled) {
  if (!backend || backend->step != gb_step || !backend->ctx)
    return sfail(RWKV7_EINVAL, "not a backend made by rwkv7_sched_gpu_backend");
  const GpuBackend* g = (const GpuBackend*)backend->ctx;
  if (tokens_restored) *tokens_restored = g->restored;
  if (tokens_prefilled) *tokens_prefilled = g->prefilled;
  return RWKV7_OK;
}

int rwkv7_sched_gpu_backend_free(rwkv7_sched_backend* backend) {
  if (!backend) return sfail(RWKV7_EINVAL, "NULL backend");
  if (backend->step != gb_step) return sfail(RWKV7_EINVAL, "not a backend made by rwkv7_sched_gpu_backend");
  if (backend->ctx) gb_release((GpuBackend*)backend->ctx);
  backend->ctx = nullptr;
  return RWKV7_OK;
}

}  // extern "C"
