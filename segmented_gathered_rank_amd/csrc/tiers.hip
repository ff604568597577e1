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
// lora_tiers_acquire drives a slot pool with it: the GPU misses of a batch
// evict the displaced adapters' entries and upload the new adapters' A and B
// rows for every module from page-locked host buffers (the host tier), all in
// one launch and asynchronously on the caller's stream: the host only does
// bookkeeping per miss.  A host-tier miss first asks the caller's fetch
// function to fill a host buffer (the cold store is the caller's).
//
// lora_tiers_prefetch is the forecast of "Thousands of adapters" (slide 9: a
// forecast from the waiting queue and an asynchronous copy): while the batch
// in flight computes, the adapters of the next batch are uploaded on a copy
// stream.  It never displaces an adapter of the batch in flight, and it
// waits for the kernels of earlier batches (lora_tiers_batch_done marks
// them) before it reuses a slot.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
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

// Page-locked descriptors of one batched upload, and the event behind it.
struct UploadRing {
  void* buf = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  uint64_t serial = 0;   // the batch that used it last
};

struct lora_tiers {
  LruList gpu, host;
  int64_t gpu_hits = 0, host_hits = 0, cold = 0;
  // host buffers (page-locked), one per host entry, for the pool bound by acquire
  const lora_pool* pool = nullptr;
  void* pinned = nullptr;
  size_t entry_bytes = 0;
  std::vector<int32_t> rank;    // [host entry][module]
  std::vector<float> scale;     // [host entry][module]
  // batched uploads: two descriptor buffers used in turn; batch `serial` is the
  // last one launched, and host entry e's buffer was last read by batch
  // he_serial[e] through ring[he_ring[e]] (0: never)
  UploadRing ring[2];
  int ring_next = 0;
  uint64_t serial = 0;
  std::vector<uint64_t> he_serial;
  std::vector<int8_t> he_ring;
  // the batch being staged: pieces, entry writes and the host entries they read
  std::vector<lora::UploadPiece> pieces;
  std::vector<lora::EntryWrite> writes;
  std::vector<int32_t> staged_he;
  // prefetch: adapters of the batch in flight (never displaced by a prefetch),
  // the end of the two latest batches' kernels, and the end of the latest prefetch
  std::vector<int32_t> inflight;
  hipEvent_t batch_ev[2] = {nullptr, nullptr};
  int batches_done = 0;
  hipEvent_t prefetch_ev = nullptr;
  bool prefetch_pending = false;
  int64_t prefetched = 0;
};

namespace {

// One request: tier, GPU slot after it, adapter displaced from the GPU tier,
// and the host entry of the adapter (-1 if the host tier keeps nothing).
// count = false: a prefetch, not a request (the hit counters stay).
void touch_one(lora_tiers* t, int32_t id, int32_t* tier, int32_t* slot, int32_t* evicted, int32_t* host_entry,
               bool count = true) {
  bool hit = false;
  int32_t out = -1;
  *slot = t->gpu.access(id, &hit, &out);
  *evicted = (hit || out == id) ? -1 : out;
  *host_entry = -1;
  if (hit) {
    if (count) ++t->gpu_hits;
    *tier = LORA_TIER_GPU;
    return;
  }
  bool h_hit = false;
  int32_t h_out = -1;
  *host_entry = t->host.access(id, &h_hit, &h_out);
  if (h_hit) {
    if (count) ++t->host_hits;
    *tier = LORA_TIER_HOST;
  } else {
    if (count) ++t->cold;
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
  for (UploadRing& r : t->ring) {   // uploads still reading page-locked memory finish first
    if (r.ev && hipEventSynchronize(r.ev) != hipSuccess) st = LORA_ERR_HIP;
    if (r.ev && hipEventDestroy(r.ev) != hipSuccess) st = LORA_ERR_HIP;
    if (r.buf && hipHostFree(r.buf) != hipSuccess) st = LORA_ERR_HIP;
  }
  for (hipEvent_t ev : {t->batch_ev[0], t->batch_ev[1], t->prefetch_ev})
    if (ev && hipEventDestroy(ev) != hipSuccess) st = LORA_ERR_HIP;
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

namespace {

size_t a_bytes_of(const lora_pool* p, int32_t m) { return static_cast<size_t>(p->max_rank) * p->h_in[m] * p->elem_bytes(); }
size_t b_bytes_of(const lora_pool* p, int32_t m) { return static_cast<size_t>(p->max_rank) * p->h_out[m] * p->elem_bytes(); }
size_t ids_bytes_of(const lora_pool* p) { return (static_cast<size_t>(p->max_pages_per_entry) * 4 + 15) / 16 * 16; }

// Binds the tiers to pool p on first use: host buffers for every module at the
// rank cap plus its page list, one per host entry, page-locked.
lora_status bind_pool(lora_tiers* t, lora_pool* p) {
  if (t->pool) return t->pool == p ? LORA_OK : LORA_ERR_ARG;
  if (static_cast<int64_t>(t->gpu.key.size()) != p->n_slots) return LORA_ERR_SLOT;
  if (t->host.key.empty()) return LORA_ERR_ARG;   // uploads come from host buffers
  size_t per = 0;
  for (int32_t m = 0; m < p->n_modules; ++m) per += a_bytes_of(p, m) + b_bytes_of(p, m) + ids_bytes_of(p);
  const size_t nh = t->host.key.size();
  if (hipHostMalloc(&t->pinned, per * nh, hipHostMallocDefault) != hipSuccess) {
    t->pinned = nullptr;
    return LORA_ERR_HIP;
  }
  t->pool = p;
  t->entry_bytes = per;
  t->rank.assign(nh * p->n_modules, 0);
  t->scale.assign(nh * p->n_modules, 0.f);
  t->he_serial.assign(nh, 0);
  t->he_ring.assign(nh, 0);
  for (hipEvent_t* ev : {&t->batch_ev[0], &t->batch_ev[1], &t->prefetch_ev, &t->ring[0].ev, &t->ring[1].ev})
    if (hipEventCreateWithFlags(ev, hipEventDisableTiming) != hipSuccess) return LORA_ERR_HIP;
  return LORA_OK;
}

// Launches the staged batch on stream s: its descriptors go to the next ring
// buffer (once the batch that used it last has passed), one upload launch,
// one event.
lora_status flush_uploads(lora_tiers* t, lora_pool* p, hipStream_t s) {
  if (t->pieces.empty() && t->writes.empty()) return LORA_OK;
  UploadRing& r = t->ring[t->ring_next];
  if (hipEventSynchronize(r.ev) != hipSuccess) return LORA_ERR_HIP;
  const size_t pb = t->pieces.size() * sizeof(lora::UploadPiece);
  const size_t wb = t->writes.size() * sizeof(lora::EntryWrite);
  const size_t need = (pb + 255) / 256 * 256 + wb;
  if (need > r.cap) {
    if (r.buf && hipHostFree(r.buf) != hipSuccess) return LORA_ERR_HIP;
    r.buf = nullptr;
    r.cap = 0;
    const size_t cap = std::max(need, 2 * r.cap + (size_t(1) << 16));
    if (hipHostMalloc(&r.buf, cap, hipHostMallocDefault) != hipSuccess) {
      r.buf = nullptr;
      return LORA_ERR_HIP;
    }
    r.cap = cap;
  }
  char* d = static_cast<char*>(r.buf);
  std::memcpy(d, t->pieces.data(), pb);
  std::memcpy(d + (pb + 255) / 256 * 256, t->writes.data(), wb);
  lora_status st = pool_upload_batch(p, reinterpret_cast<const lora::UploadPiece*>(d),
                                     static_cast<int32_t>(t->pieces.size()),
                                     reinterpret_cast<const lora::EntryWrite*>(d + (pb + 255) / 256 * 256),
                                     static_cast<int32_t>(t->writes.size()), s);
  if (st == LORA_OK && hipEventRecord(r.ev, s) != hipSuccess) st = LORA_ERR_HIP;
  r.serial = ++t->serial;
  for (int32_t he : t->staged_he) {
    t->he_serial[he] = r.serial;
    t->he_ring[he] = static_cast<int8_t>(t->ring_next);
  }
  t->ring_next ^= 1;
  t->pieces.clear();
  t->writes.clear();
  t->staged_he.clear();
  return st;
}

// Before host entry he's buffer is overwritten: the staged batch (if it reads
// it) is launched, and the last upload that read it has completed.
lora_status free_host_entry(lora_tiers* t, lora_pool* p, int32_t he, hipStream_t s) {
  for (int32_t e : t->staged_he)
    if (e == he) {
      const lora_status st = flush_uploads(t, p, s);
      if (st != LORA_OK) return st;
      break;
    }
  const UploadRing& r = t->ring[t->he_ring[he]];
  if (t->he_serial[he] != 0 && r.serial == t->he_serial[he] && hipEventSynchronize(r.ev) != hipSuccess)
    return LORA_ERR_HIP;
  return LORA_OK;
}

// A GPU miss of adapter id in slot `slot`, host entry he: fill the host
// buffer from the cold store if needed, then stage the eviction of the slot's
// previous adapter and the uploads of the new one into the batch (flushed by
// the caller: device work happens in flush_uploads).
lora_status stage_miss(lora_tiers* t, lora_pool* p, int32_t id, int32_t tier, int32_t slot, int32_t he,
                       lora_fetch_fn fetch, void* ctx, hipStream_t s) {
  const int32_t nm = p->n_modules;
  char* buf = static_cast<char*>(t->pinned) + static_cast<size_t>(he) * t->entry_bytes;
  if (tier == LORA_TIER_COLD) {   // the caller's cold store fills the host buffer
    lora_status st = free_host_entry(t, p, he, s);
    if (st != LORA_OK) return st;
    char* q = buf;
    for (int32_t m = 0; m < nm; ++m) {
      int32_t r = 0;
      float sc = 0.f;
      if (fetch(ctx, id, m, &r, &sc, q, q + a_bytes_of(p, m)) != 0) return LORA_ERR_ARG;
      if (r < 0 || r > p->max_rank) return LORA_ERR_RANK;
      t->rank[static_cast<size_t>(he) * nm + m] = r;
      t->scale[static_cast<size_t>(he) * nm + m] = sc;
      q += a_bytes_of(p, m) + b_bytes_of(p, m) + ids_bytes_of(p);
    }
  }
  // the slot's previous adapter leaves; each module's entry is then written
  // once in the batch: the new adapter's, or empty where it has none
  pool_evict_host(p, slot);
  char* q = buf;
  for (int32_t m = 0; m < nm; ++m) {
    const int32_t r = t->rank[static_cast<size_t>(he) * nm + m];
    if (r > 0) {
      const lora_status st = pool_stage_upload(p, slot, m, r, q, q + a_bytes_of(p, m),
                                               t->scale[static_cast<size_t>(he) * nm + m], t->pieces, t->writes);
      if (st != LORA_OK) return st;
    } else {
      t->writes.push_back(lora::EntryWrite{slot * nm + m, 0, lora::SlotEntry{0, 0.f, 0, 0}});
    }
    q += a_bytes_of(p, m) + b_bytes_of(p, m) + ids_bytes_of(p);
  }
  t->staged_he.push_back(he);
  return LORA_OK;
}

}  // namespace

lora_status lora_tiers_acquire(lora_tiers* t, lora_pool* p, const int32_t* ids, int32_t n,
                               lora_fetch_fn fetch, void* ctx, int32_t* slots, void* stream) {
  if (!t || !p || n < 0 || (n > 0 && (!ids || !slots)) || !fetch) return LORA_ERR_ARG;
  if (static_cast<int64_t>(t->gpu.key.size()) != p->n_slots) return LORA_ERR_SLOT;
  if (t->host.key.empty()) return LORA_ERR_ARG;
  if (t->pool && t->pool != p) return LORA_ERR_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0) return LORA_ERR_ARG;
  std::vector<int32_t> distinct;
  {   // a batch may not need more adapters than there are slots
    std::unordered_map<int32_t, int> seen;
    for (int32_t i = 0; i < n; ++i)
      if (seen.emplace(ids[i], 1).second) distinct.push_back(ids[i]);
    if (static_cast<int64_t>(distinct.size()) > p->n_slots) return LORA_ERR_SLOT;
  }
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  lora_status st = bind_pool(t, p);
  if (st != LORA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (t->prefetch_pending) {   // this batch's kernels come after the prefetched uploads
    if (hipStreamWaitEvent(s, t->prefetch_ev, 0) != hipSuccess) return LORA_ERR_HIP;
    t->prefetch_pending = false;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t tier, slot, ev, he;
    touch_one(t, ids[i], &tier, &slot, &ev, &he);
    slots[i] = slot;
    if (tier == LORA_TIER_GPU) continue;
    st = stage_miss(t, p, ids[i], tier, slot, he, fetch, ctx, s);
    if (st != LORA_OK) {
      (void)flush_uploads(t, p, s);   // what was staged before the error still goes out
      return st;
    }
  }
  st = flush_uploads(t, p, s);
  if (st != LORA_OK) return st;
  t->inflight = std::move(distinct);
  return LORA_OK;
}

lora_status lora_tiers_batch_done(lora_tiers* t, void* stream) {
  if (!t) return LORA_ERR_ARG;
  if (!t->pool) return LORA_OK;   // nothing acquired yet
  DeviceGuard g(t->pool->device);
  if (!g.ok) return LORA_ERR_HIP;
  // keep the latest two: a prefetch waits for the batch before the one in flight
  std::swap(t->batch_ev[0], t->batch_ev[1]);
  if (hipEventRecord(t->batch_ev[1], static_cast<hipStream_t>(stream)) != hipSuccess) return LORA_ERR_HIP;
  ++t->batches_done;
  return LORA_OK;
}

lora_status lora_tiers_prefetch(lora_tiers* t, lora_pool* p, const int32_t* ids, int32_t n, lora_fetch_fn fetch,
                                void* ctx, void* copy_stream, int32_t* issued) {
  if (!t || !p || n < 0 || (n > 0 && !ids) || !fetch) return LORA_ERR_ARG;
  if (issued) *issued = 0;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0) return LORA_ERR_ARG;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  lora_status st = bind_pool(t, p);
  if (st != LORA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(copy_stream);
  // slots may still be read by kernels of batches before the one in flight
  // (with fewer than two batches done there are none)
  if (t->batches_done >= 2 && hipStreamWaitEvent(s, t->batch_ev[0], 0) != hipSuccess) return LORA_ERR_HIP;
  std::unordered_map<int32_t, int> pinned;
  for (int32_t a : t->inflight) pinned[a] = 1;
  int32_t free_slots = static_cast<int32_t>(t->gpu.key.size()) - static_cast<int32_t>(pinned.size());
  int32_t count = 0;
  for (int32_t i = 0; i < n && free_slots > 0; ++i) {
    const int32_t id = ids[i];
    if (t->gpu.where.count(id)) continue;   // resident: nothing to do (its recency is left alone)
    // the least recently used adapter must not be one of the batch in flight:
    // those were touched last, so it is not while fewer than free_slots uploads happen
    const int32_t victim = t->gpu.tail >= 0 && t->gpu.free_.empty() ? t->gpu.key[t->gpu.tail] : -1;
    if (victim >= 0 && pinned.count(victim)) break;
    int32_t tier, slot, ev, he;
    touch_one(t, id, &tier, &slot, &ev, &he, false);
    st = stage_miss(t, p, id, tier, slot, he, fetch, ctx, s);
    if (st != LORA_OK) {
      (void)flush_uploads(t, p, s);
      return st;
    }
    pinned[id] = 1;
    --free_slots;
    ++count;
  }
  st = flush_uploads(t, p, s);
  if (st != LORA_OK) return st;
  if (count > 0) {
    if (hipEventRecord(t->prefetch_ev, s) != hipSuccess) return LORA_ERR_HIP;
    t->prefetch_pending = true;
    t->prefetched += count;
  }
  if (issued) *issued = count;
  return LORA_OK;
}

}  // extern "C"
