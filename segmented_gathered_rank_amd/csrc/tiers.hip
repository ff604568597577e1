// Two-tier adapter residency: which adapters occupy the pool's GPU slots and
// which wait in host memory (study page "Multi-LoRA Serving", section
// "Memory: slots, tiers and paging": GPU slots at a fixed count, a larger
// host-memory LRU so that a swap is a PCIe copy, and a cold store behind it).
//
// Policy, per request for adapter a:
//   GPU tier, least recently used order: a hit refreshes a; a miss gives a
//   the lowest free slot, else the slot of the least recently used adapter,
//   which leaves the GPU tier;
//   host tier, consulted only on a GPU miss, same LRU rule: a hit means a
//   host-to-GPU copy, a miss means a load from the cold store.
// Both tiers are intrusive doubly linked lists over fixed entry arrays, so a
// request costs O(1) besides one hash lookup per tier.
//
// lora_tiers_acquire drives a slot pool with it: each GPU miss evicts the
// displaced adapter's entries and uploads the new adapter's A and B rows for
// every module from page-locked host buffers (the host tier), asynchronously
// on the caller's stream.  A host-tier miss first asks the caller's fetch
// function to fill a host buffer (the cold store is the caller's).
#include <hip/hip_runtime.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "lora.h"
#include "pool.hpp"

using lora::DeviceGuard;

namespace {

// LRU list over entries 0..cap-1: head = most recent, tail = least recent.
struct LruList {
  std::vector<int32_t> prev, next, key;
  std::unordered_map<int32_t, int32_t> where;   // key -> entry
  std::vector<int32_t> free_;                   // unused entries, lowest on top
  int32_t head = -1, tail = -1;

  void init(int32_t cap) {
    prev.assign(cap, -1);
    next.assign(cap, -1);
    key.assign(cap, -1);
    where.clear();
    where.reserve(static_cast<size_t>(cap) * 2 + 1);
    free_.clear();
    for (int32_t e = cap - 1; e >= 0; --e) free_.push_back(e);
    head = tail = -1;
  }
  void unlink(int32_t e) {
    if (prev[e] >= 0) next[prev[e]] = next[e]; else head = next[e];
    if (next[e] >= 0) prev[next[e]] = prev[e]; else tail = prev[e];
    prev[e] = next[e] = -1;
  }
  void push_front(int32_t e) {
    prev[e] = -1;
    next[e] = head;
    if (head >= 0) prev[head] = e;
    head = e;
    if (tail < 0) tail = e;
  }
  // Returns the entry of k after the access; *hit, and *evicted = the key
  // that left (-1 none).  With capacity 0 nothing is kept (entry -1).
  int32_t access(int32_t k, bool* hit, int32_t* evicted) {
    *evicted = -1;
    auto it = where.find(k);
    if (it != where.end()) {
      *hit = true;
      unlink(it->second);
      push_front(it->second);
      return it->second;
    }
    *hit = false;
    if (key.empty()) {
      *evicted = k;
      return -1;
    }
    int32_t e;
    if (!free_.empty()) {
      e = free_.back();
      free_.pop_back();
    } else {
      e = tail;
      unlink(e);
      *evicted = key[e];
      where.erase(key[e]);
    }
    key[e] = k;
    where[k] = e;
    push_front(e);
    return e;
  }
};

}  // namespace

struct lora_tiers {
  LruList gpu, host;
  int64_t gpu_hits = 0, host_hits = 0, cold = 0;
  // host buffers (page-locked), one per host entry, for the pool bound by acquire
  const lora_pool* pool = nullptr;
  void* pinned = nullptr;
  size_t entry_bytes = 0;
  std::vector<int32_t> rank;    // [host entry][module]
  std::vector<float> scale;     // [host entry][module]
  std::vector<hipEvent_t> done; // [host entry]: last upload that read the entry's buffer
  std::vector<uint8_t> pending;
};

namespace {

// One request: tier, GPU slot after it, adapter displaced from the GPU tier,
// and the host entry of the adapter (-1 if the host tier keeps nothing).
void touch_one(lora_tiers* t, int32_t id, int32_t* tier, int32_t* slot, int32_t* evicted, int32_t* host_entry) {
  bool hit = false;
  int32_t out = -1;
  *slot = t->gpu.access(id, &hit, &out);
  *evicted = (hit || out == id) ? -1 : out;
  *host_entry = -1;
  if (hit) {
    ++t->gpu_hits;
    *tier = LORA_TIER_GPU;
    return;
  }
  bool h_hit = false;
  int32_t h_out = -1;
  *host_entry = t->host.access(id, &h_hit, &h_out);
  if (h_hit) {
    ++t->host_hits;
    *tier = LORA_TIER_HOST;
  } else {
    ++t->cold;
    *tier = LORA_TIER_COLD;
  }
}

}  // namespace

extern "C" {

lora_status lora_tiers_create(lora_tiers** out, int32_t gpu_slots, int32_t host_slots) {
  if (!out) return LORA_ERR_ARG;
  *out = nullptr;
  if (gpu_slots < 1 || host_slots < 0 || gpu_slots > (1 << 24) || host_slots > (1 << 24)) return LORA_ERR_ARG;
  lora_tiers* t = new (std::nothrow) lora_tiers();
  if (!t) return LORA_ERR_ARG;
  t->gpu.init(gpu_slots);
  t->host.init(host_slots);
  *out = t;
  return LORA_OK;
}

lora_status lora_tiers_destroy(lora_tiers* t) {
  if (!t) return LORA_OK;
  lora_status st = LORA_OK;
  for (size_t e = 0; e < t->done.size(); ++e)
    if (t->done[e] && hipEventDestroy(t->done[e]) != hipSuccess) st = LORA_ERR_HIP;
  if (t->pinned && hipHostFree(t->pinned) != hipSuccess) st = LORA_ERR_HIP;
  delete t;
  return st;
}

lora_status lora_tiers_touch(lora_tiers* t, const int32_t* ids, int32_t n, int32_t* tier, int32_t* slot,
                             int32_t* evicted) {
  if (!t || n < 0 || (n > 0 && !ids)) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i) {
    int32_t tr, s, ev, he;
    touch_one(t, ids[i], &tr, &s, &ev, &he);
    if (tier) tier[i] = tr;
    if (slot) slot[i] = s;
    if (evicted) evicted[i] = ev;
  }
  return LORA_OK;
}

lora_status lora_tiers_stats(const lora_tiers* t, int64_t* gpu_hits, int64_t* host_hits, int64_t* cold_loads) {
  if (!t) return LORA_ERR_ARG;
  if (gpu_hits) *gpu_hits = t->gpu_hits;
  if (host_hits) *host_hits = t->host_hits;
  if (cold_loads) *cold_loads = t->cold;
  return LORA_OK;
}

lora_status lora_tiers_slot_of(const lora_tiers* t, int32_t id, int32_t* slot) {
  if (!t || !slot) return LORA_ERR_ARG;
  auto it = t->gpu.where.find(id);
  *slot = it == t->gpu.where.end() ? -1 : it->second;
  return LORA_OK;
}

lora_status lora_tiers_acquire(lora_tiers* t, lora_pool* p, const int32_t* ids, int32_t n,
                               lora_fetch_fn fetch, void* ctx, int32_t* slots, void* stream) {
  if (!t || !p || n < 0 || (n > 0 && (!ids || !slots)) || !fetch) return LORA_ERR_ARG;
  if (static_cast<int64_t>(t->gpu.key.size()) != p->n_slots) return LORA_ERR_SLOT;
  if (t->host.key.empty()) return LORA_ERR_ARG;   // uploads come from host buffers
  if (t->pool && t->pool != p) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0) return LORA_ERR_ARG;
  {   // a batch may not need more adapters than there are slots
    std::unordered_map<int32_t, int> seen;
    for (int32_t i = 0; i < n; ++i) seen[ids[i]] = 1;
    if (static_cast<int64_t>(seen.size()) > p->n_slots) return LORA_ERR_SLOT;
  }
  const int32_t nm = p->n_modules;
  const size_t eb = p->elem_bytes();
  auto a_bytes = [&](int32_t m) { return static_cast<size_t>(p->max_rank) * p->h_in[m] * eb; };
  auto b_bytes = [&](int32_t m) { return static_cast<size_t>(p->max_rank) * p->h_out[m] * eb; };
  const size_t ids_bytes = (static_cast<size_t>(p->max_pages_per_entry) * 4 + 15) / 16 * 16;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  if (!t->pool) {   // host buffers for this pool: every module at the rank cap, plus its page list
    size_t per = 0;
    for (int32_t m = 0; m < nm; ++m) per += a_bytes(m) + b_bytes(m) + ids_bytes;
    const size_t nh = t->host.key.size();
    if (hipHostMalloc(&t->pinned, per * nh, hipHostMallocDefault) != hipSuccess) {
      t->pinned = nullptr;
      return LORA_ERR_HIP;
    }
    t->pool = p;
    t->entry_bytes = per;
    t->rank.assign(nh * nm, 0);
    t->scale.assign(nh * nm, 0.f);
    t->done.assign(nh, nullptr);
    t->pending.assign(nh, 0);
    for (size_t e = 0; e < nh; ++e)
      if (hipEventCreateWithFlags(&t->done[e], hipEventDisableTiming) != hipSuccess) return LORA_ERR_HIP;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i = 0; i < n; ++i) {
    int32_t tier, slot, ev, he;
    touch_one(t, ids[i], &tier, &slot, &ev, &he);
    slots[i] = slot;
    if (tier == LORA_TIER_GPU) continue;
    // the entry's buffers (rows, page lists) may still feed an earlier upload
    if (t->pending[he] && hipEventSynchronize(t->done[he]) != hipSuccess) return LORA_ERR_HIP;
    t->pending[he] = 0;
    char* buf = static_cast<char*>(t->pinned) + static_cast<size_t>(he) * t->entry_bytes;
    if (tier == LORA_TIER_COLD) {   // the caller's cold store fills the host buffer
      char* q = buf;
      for (int32_t m = 0; m < nm; ++m) {
        int32_t r = 0;
        float sc = 0.f;
        if (fetch(ctx, ids[i], m, &r, &sc, q, q + a_bytes(m)) != 0) return LORA_ERR_ARG;
        if (r < 0 || r > p->max_rank) return LORA_ERR_RANK;
        t->rank[static_cast<size_t>(he) * nm + m] = r;
        t->scale[static_cast<size_t>(he) * nm + m] = sc;
        q += a_bytes(m) + b_bytes(m) + ids_bytes;
      }
    }
    // the slot's previous adapter leaves (stream-ordered), the new one is copied in
    bool loaded = false;
    for (int32_t m = 0; m < nm; ++m) loaded = loaded || p->entries[static_cast<size_t>(slot) * nm + m].rank > 0;
    if (loaded) {
      const lora_status st = lora_pool_evict(p, slot, stream);
      if (st != LORA_OK) return st;
    }
    char* q = buf;
    for (int32_t m = 0; m < nm; ++m) {
      const int32_t r = t->rank[static_cast<size_t>(he) * nm + m];
      if (r > 0) {
        const lora_status st =
            pool_upload_async(p, slot, m, r, q, q + a_bytes(m), t->scale[static_cast<size_t>(he) * nm + m],
                              reinterpret_cast<int32_t*>(q + a_bytes(m) + b_bytes(m)), s);
        if (st != LORA_OK) return st;
      }
      q += a_bytes(m) + b_bytes(m) + ids_bytes;
    }
    if (hipEventRecord(t->done[he], s) != hipSuccess) return LORA_ERR_HIP;
    t->pending[he] = 1;
  }
  return LORA_OK;
}

}  // extern "C"
