// Host-side state of a pool (internal to the library).
#pragma once

#include <vector>

#include "common.hpp"
#include "page_alloc.hpp"

struct lora_pool {
  int32_t device = 0;
  lora_dtype dtype = LORA_BF16;
  int64_t page_elems = 0;
  int64_t n_pages = 0;
  int32_t n_slots = 0;
  int32_t n_modules = 0;
  int32_t max_rank = 0;
  int32_t max_pages_per_entry = 0;
  std::vector<int64_t> h_in, h_out;

  void* d_pages = nullptr;
  lora::SlotEntry* d_entries = nullptr;
  int32_t* d_page_ids = nullptr;
  // lora_pool_load's staging ring: kLoadRing uploads may be in flight.  Slot r
  // holds one upload's A and B rows and its page list in page-locked host
  // memory (h_staging) and device memory (d_staging); ring_done[r] is recorded
  // on the upload's stream after it, so the slot is reused only once its
  // copy and kernel are done.
  static constexpr int kLoadRing = 4;
  void* h_staging[kLoadRing] = {};
  void* d_staging[kLoadRing] = {};
  hipEvent_t ring_done[kLoadRing] = {};
  int ring_next = 0;
  size_t staging_bytes = 0;

  lora::PageAllocator alloc;
  struct Entry {
    int32_t rank = 0;
    float scale = 0.f;
    std::vector<int32_t> pages;   // A's rows then B's rows, page by page
  };
  std::vector<Entry> entries;     // [n_slots * n_modules]
  int64_t loads = 0, evicts = 0;

  size_t elem_bytes() const { return dtype == LORA_BF16 ? 2 : 4; }
  lora::PoolView view() const {
    lora::PoolView v;
    v.pages = d_pages;
    v.entries = d_entries;
    v.page_ids = d_page_ids;
    v.page_elems = page_elems;
    v.n_slots = n_slots;
    v.n_modules = n_modules;
    v.max_rank = max_rank;
    v.zero_page = static_cast<int32_t>(n_pages);
    v.ppe = max_pages_per_entry;
    return v;
  }
};

namespace lora {

// Makes the pool's device current for the lifetime of the guard.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (ok && hipGetDevice(&cur) == hipSuccess && cur != prev && prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace lora

// Asynchronous upload of one (slot, module) entry on stream s: A's rank rows
// from a, B's from b (device memory or page-locked host memory), the page
// list written to plist (rank * (h_in + h_out) / page_elems ints, readable by
// the device).  The caller keeps a, b and plist unchanged until the stream
// passes the upload.  Same checks and bookkeeping as lora_pool_load.
lora_status pool_upload_async(lora_pool* p, int32_t slot, int32_t module, int32_t rank, const void* a,
                              const void* b, float scale, int32_t* plist, hipStream_t s);

// Batched uploads (several (slot, module) entries in one launch).  A piece is
// one page: its source (device memory or page-locked host memory), its page
// and its position in the page-id table.  An entry write publishes (or, with
// rank 0, clears) one (slot, module) entry after the pieces.  Descriptors may
// themselves live in page-locked host memory.
namespace lora {
struct UploadPiece {
  const void* src;
  int32_t page;
  int32_t id_at;
};
struct EntryWrite {
  int32_t index;
  int32_t pad_;
  SlotEntry value;
};
}  // namespace lora

// Host bookkeeping of evicting every module of `slot` (pages back to the free
// list, entries empty); the caller clears the device entries (an EntryWrite of
// rank 0 per module).  Returns whether anything was loaded.
bool pool_evict_host(lora_pool* p, int32_t slot);

// Host bookkeeping of one upload: checks, allocates the pages and appends the
// pieces (A's rows from a, B's from b, page by page) and the entry write; the
// entry reads as loaded on the host at once.  No device work.
lora_status pool_stage_upload(lora_pool* p, int32_t slot, int32_t module, int32_t rank, const void* a,
                              const void* b, float scale, std::vector<lora::UploadPiece>& pieces,
                              std::vector<lora::EntryWrite>& entries);

// One launch for n_pieces pieces and n_entries entry writes (descriptors in
// device or page-locked host memory, unchanged until the stream passes it).
lora_status pool_upload_batch(lora_pool* p, const lora::UploadPiece* pieces, int32_t n_pieces,
                              const lora::EntryWrite* entries, int32_t n_entries, hipStream_t s);

