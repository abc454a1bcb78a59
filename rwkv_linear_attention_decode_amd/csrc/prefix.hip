// Slot snapshots, slot offload and the prefix-state cache (include/rwkv7_prefix.h).
//
// A slot is the whole history of a sequence: its fp32 state and its step
// counter.  A snapshot is those bytes copied out, so restoring one is a
// stream-ordered copy (device to device at HBM rate, or host to device from
// the offload arena), and the restored slot is bit-identical to the one that
// was stored.  The cache index is host-side: FNV-1a prefix hashes of the
// token sequences, confirmed by comparing the tokens.
#include "launch.h"
#include "../../include/rwkv7_prefix.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <map>
#include <utility>
#include <vector>

namespace {

int pfail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int pfail(int code, const char* fmt, ...) {
  char buf[384];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return lib_fail(code, buf);
}

int phip(hipError_t e, const char* what) {
  return e == hipSuccess ? RWKV7_OK : pfail(RWKV7_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Where slot `slot` lives in a pool of n_slots slots (the rwkv7_state_bytes layout).
struct SlotAddr {
  char* state;
  char* counter;
  uint64_t state_bytes;
};

SlotAddr slot_addr(const rwkv7_model* m, const void* pool, int64_t n_slots, int32_t slot) {
  const uint64_t sf = (uint64_t)lib_model_slot_floats(m);
  const uint64_t co = ((uint64_t)n_slots * sf * 4 + 255) / 256 * 256;
  SlotAddr a;
  a.state = (char*)pool + (uint64_t)slot * sf * 4;
  a.counter = (char*)pool + co + (uint64_t)slot * 8;
  a.state_bytes = sf * 4;
  return a;
}

int check_slot(const rwkv7_model* m, const void* pool, int64_t n_slots, int32_t slot) {
  if (!m || !pool) return pfail(RWKV7_EINVAL, "model and pool must be non-NULL");
  if (n_slots < 1 || slot < 0 || slot >= n_slots)
    return pfail(RWKV7_EINVAL, "slot %d outside [0, %lld)", slot, (long long)n_slots);
  return RWKV7_OK;
}

// snapshot <-> slot: the state block, then the 8-byte counter right after it
int copy_out(const SlotAddr& a, char* dst, hipStream_t st) {
  int rc = phip(hipMemcpyAsync(dst, a.state, a.state_bytes, hipMemcpyDefault, st), "snapshot state");
  if (rc) return rc;
  return phip(hipMemcpyAsync(dst + a.state_bytes, a.counter, 8, hipMemcpyDefault, st), "snapshot counter");
}

int copy_in(const SlotAddr& a, const char* src, hipStream_t st) {
  int rc = phip(hipMemcpyAsync(a.state, src, a.state_bytes, hipMemcpyDefault, st), "restore state");
  if (rc) return rc;
  return phip(hipMemcpyAsync(a.counter, src + a.state_bytes, 8, hipMemcpyDefault, st), "restore counter");
}

// FNV-1a (Fowler, Noll, Vo), 64-bit, over the little-endian bytes of each token.
uint64_t fnv_step(uint64_t h, int32_t tok) {
  const uint32_t v = (uint32_t)tok;
  for (int i = 0; i < 4; ++i) {
    h ^= (v >> (8 * i)) & 0xFFu;
    h *= 0x100000001B3ull;
  }
  return h;
}
constexpr uint64_t FNV_OFFSET = 0xCBF29CE484222325ull;

struct Entry {
  std::vector<int32_t> toks;
  uint64_t hash = 0;
  int tier = -1;  // 0 device arena, 1 host arena, -1 unused
  int block = -1;
  uint64_t last_use = 0;
};

}  // namespace

struct rwkv7_prefix_cache {
  const rwkv7_model* m = nullptr;
  uint64_t snap = 0;   // snapshot bytes
  uint64_t stride = 0; // arena block stride
  char* arena[2] = {nullptr, nullptr};
  int cap[2] = {0, 0};
  std::vector<int> free_blocks[2];
  std::vector<Entry> entries;
  std::vector<int> free_entries;
  std::map<std::pair<int, uint64_t>, std::vector<int>> index;  // (length, hash) -> entries
  uint64_t clock = 0;
  rwkv7_prefix_stats st{};

  char* block_ptr(const Entry& e) const { return arena[e.tier] + (uint64_t)e.block * stride; }

  int find(const int32_t* toks, int n, uint64_t h) const {
    auto it = index.find({n, h});
    if (it == index.end()) return -1;
    for (int id : it->second) {
      const Entry& e = entries[id];
      bool same = true;
      for (int i = 0; i < n && same; ++i) same = e.toks[i] == toks[i];
      if (same) return id;
    }
    return -1;
  }

  int lru(int tier) const {
    int best = -1;
    for (int i = 0; i < (int)entries.size(); ++i)
      if (entries[i].tier == tier && (best < 0 || entries[i].last_use < entries[best].last_use)) best = i;
    return best;
  }

  void drop(int id) {
    Entry& e = entries[id];
    auto& v = index[{(int)e.toks.size(), e.hash}];
    for (size_t i = 0; i < v.size(); ++i)
      if (v[i] == id) {
        v.erase(v.begin() + i);
        break;
      }
    if (v.empty()) index.erase({(int)e.toks.size(), e.hash});
    free_blocks[e.tier].push_back(e.block);
    e = Entry{};
    free_entries.push_back(id);
  }

  // a free device block, making room by offloading or dropping the LRU entry
  int device_block(hipStream_t s, int* block) {
    if (free_blocks[0].empty()) {
      const int v = lru(0);
      Entry& e = entries[v];
      if (cap[1] > 0) {
        if (free_blocks[1].empty()) {
          drop(lru(1));
          ++st.drops;
        }
        const int hb = free_blocks[1].back();
        int rc = phip(hipMemcpyAsync(arena[1] + (uint64_t)hb * stride, block_ptr(e), snap, hipMemcpyDefault, s),
                      "offload snapshot");
        if (rc) return rc;
        free_blocks[1].pop_back();
        free_blocks[0].push_back(e.block);
        e.tier = 1;
        e.block = hb;
        ++st.offloads;
      } else {
        drop(v);
        ++st.drops;
      }
    }
    *block = free_blocks[0].back();
    free_blocks[0].pop_back();
    return RWKV7_OK;
  }
};

extern "C" {

int rwkv7_snapshot_bytes(const rwkv7_config* cfg, uint64_t* bytes) {
  if (!bytes) return pfail(RWKV7_EINVAL, "bytes is NULL");
  uint64_t n = 0;
  int rc = rwkv7_slot_floats(cfg, &n);
  if (rc) return rc;
  *bytes = n * 4 + 8;
  return RWKV7_OK;
}

int rwkv7_slot_export(const rwkv7_model* m, const void* pool, int64_t n_slots, int32_t slot, void* dst,
                      void* stream) {
  int rc = check_slot(m, pool, n_slots, slot);
  if (rc) return rc;
  if (!dst) return pfail(RWKV7_EINVAL, "dst is NULL");
  return copy_out(slot_addr(m, pool, n_slots, slot), (char*)dst, (hipStream_t)stream);
}

int rwkv7_slot_import(const rwkv7_model* m, void* pool, int64_t n_slots, int32_t slot, const void* src,
                      void* stream) {
  int rc = check_slot(m, pool, n_slots, slot);
  if (rc) return rc;
  if (!src) return pfail(RWKV7_EINVAL, "src is NULL");
  return copy_in(slot_addr(m, pool, n_slots, slot), (const char*)src, (hipStream_t)stream);
}

int rwkv7_prefix_cache_create(const rwkv7_model* m, void* arena, uint64_t arena_bytes, void* host_arena,
                              uint64_t host_bytes, rwkv7_prefix_cache** out) {
  if (!m || !arena || !out) return pfail(RWKV7_EINVAL, "model, arena and out must be non-NULL");
  if (host_bytes && !host_arena) return pfail(RWKV7_EINVAL, "host_bytes > 0 with a NULL host arena");
  const uint64_t snap = (uint64_t)lib_model_slot_floats(m) * 4 + 8;
  const uint64_t stride = (snap + 255) / 256 * 256;
  if (arena_bytes < stride)
    return pfail(RWKV7_ESHAPE, "the device arena holds no snapshot (%llu bytes, %llu needed)",
                 (unsigned long long)arena_bytes, (unsigned long long)stride);
  rwkv7_prefix_cache* c = new rwkv7_prefix_cache;
  c->m = m;
  c->snap = snap;
  c->stride = stride;
  c->arena[0] = (char*)arena;
  c->arena[1] = (char*)host_arena;
  c->cap[0] = (int)(arena_bytes / stride);
  c->cap[1] = host_arena ? (int)(host_bytes / stride) : 0;
  for (int t = 0; t < 2; ++t)
    for (int b = c->cap[t] - 1; b >= 0; --b) c->free_blocks[t].push_back(b);
  c->st.device_capacity = c->cap[0];
  c->st.host_capacity = c->cap[1];
  *out = c;
  return RWKV7_OK;
}

int rwkv7_prefix_cache_free(rwkv7_prefix_cache* c) {
  delete c;
  return RWKV7_OK;
}

int rwkv7_prefix_cache_store(rwkv7_prefix_cache* c, const void* pool, int64_t n_slots, int32_t slot,
                             const int32_t* tokens, int32_t n, void* stream) {
  if (!c) return pfail(RWKV7_EINVAL, "NULL cache");
  int rc = check_slot(c->m, pool, n_slots, slot);
  if (rc) return rc;
  if (!tokens || n < 1) return pfail(RWKV7_EINVAL, "a stored sequence needs n >= 1 tokens");
  uint64_t h = FNV_OFFSET;
  for (int i = 0; i < n; ++i) h = fnv_step(h, tokens[i]);
  int id = c->find(tokens, n, h);
  if (id >= 0) {
    c->entries[id].last_use = ++c->clock;
    return RWKV7_OK;
  }
  hipStream_t st = (hipStream_t)stream;
  int block = -1;
  if ((rc = c->device_block(st, &block))) return rc;
  if (c->free_entries.empty()) {
    c->entries.emplace_back();
    c->free_entries.push_back((int)c->entries.size() - 1);
  }
  id = c->free_entries.back();
  Entry& e = c->entries[id];
  e.tier = 0;
  e.block = block;
  rc = copy_out(slot_addr(c->m, pool, n_slots, slot), c->block_ptr(e), st);
  if (rc) {
    c->free_blocks[0].push_back(block);
    e = Entry{};
    return rc;
  }
  c->free_entries.pop_back();
  e.toks.assign(tokens, tokens + n);
  e.hash = h;
  e.last_use = ++c->clock;
  c->index[{n, h}].push_back(id);
  ++c->st.stores;
  return RWKV7_OK;
}

int rwkv7_prefix_cache_lookup(rwkv7_prefix_cache* c, void* pool, int64_t n_slots, int32_t slot,
                              const int32_t* tokens, int32_t n, int32_t* matched, void* stream) {
  if (!c || !matched) return pfail(RWKV7_EINVAL, "NULL argument");
  int rc = check_slot(c->m, pool, n_slots, slot);
  if (rc) return rc;
  if (n < 0 || (n > 0 && !tokens)) return pfail(RWKV7_EINVAL, "bad token sequence");
  *matched = 0;
  ++c->st.lookups;
  std::vector<uint64_t> hs(n + 1);
  hs[0] = FNV_OFFSET;
  for (int i = 0; i < n; ++i) hs[i + 1] = fnv_step(hs[i], tokens[i]);
  for (int p = n; p >= 1; --p) {
    const int id = c->find(tokens, p, hs[p]);
    if (id < 0) continue;
    Entry& e = c->entries[id];
    rc = copy_in(slot_addr(c->m, pool, n_slots, slot), c->block_ptr(e), (hipStream_t)stream);
    if (rc) return rc;
    e.last_use = ++c->clock;
    *matched = p;
    ++c->st.hits;
    c->st.hit_tokens += p;
    return RWKV7_OK;
  }
  return RWKV7_OK;
}

int rwkv7_prefix_cache_stats(const rwkv7_prefix_cache* c, rwkv7_prefix_stats* out) {
  if (!c || !out) return pfail(RWKV7_EINVAL, "NULL argument");
  *out = c->st;
  out->device_entries = c->cap[0] - (int)c->free_blocks[0].size();
  out->host_entries = c->cap[1] - (int)c->free_blocks[1].size();
  return RWKV7_OK;
}

}  // extern "C"
