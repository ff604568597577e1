// Paged adapter store: pool creation, adapter upload into pages, eviction.
//
// The study page's GPU slots (section "Memory: slots, tiers and paging") hold the
// hot adapters; S-LoRA's unified paging ("Thousands of adapters", slide 8)
// stores rank-R adapters in R pages of H elements.  Here a page holds
// page_elems elements; each rank row of A and of B is cut into whole pages and
// a (slot, module) entry lists its pages, so adapters of any rank share one
// pool without padding to the maximum rank.
#include <cstring>
#include <new>

#include "pool.hpp"

using namespace lora;

namespace {

// Copies one upload (A's rank rows from src_a, B's from src_b, page by page)
// into its pages and publishes the slot-table entry.  One workgroup per page.
// The sources may be device memory or page-locked host memory.
template <typename T>
__global__ __launch_bounds__(256) void k_upload(T* __restrict__ pages, const T* __restrict__ src_a,
                                                const T* __restrict__ src_b,
                                                const int32_t* __restrict__ plist, int32_t n_plist,
                                                int64_t page_elems, int32_t* __restrict__ page_ids,
                                                int32_t ids_off, int32_t n_a, int32_t b_gap,
                                                SlotEntry* __restrict__ entry, SlotEntry value) {
  const int32_t piece = blockIdx.x;
  if (piece >= n_plist) return;
  const int32_t page = plist[piece];
  const T* s = piece < n_a ? src_a + static_cast<int64_t>(piece) * page_elems
                           : src_b + static_cast<int64_t>(piece - n_a) * page_elems;
  T* d = pages + static_cast<int64_t>(page) * page_elems;
  constexpr int kVec = 16 / sizeof(T);
  for (int64_t e = static_cast<int64_t>(threadIdx.x) * kVec; e < page_elems; e += 256 * kVec) {
    *reinterpret_cast<u32x4*>(d + e) = *reinterpret_cast<const u32x4*>(s + e);
  }
  if (threadIdx.x == 0) {
    page_ids[ids_off + piece + (piece >= n_a ? b_gap : 0)] = page;
    if (piece == 0) *entry = value;
  }
}

// Batched uploads: workgroup b < n_pieces copies piece b's page and records its
// page id; the workgroups after them publish the entry writes, one per thread.
// A kernel boundary orders every page before any entry that lists it, as the
// entries are only read by later kernels.
template <typename T>
__global__ __launch_bounds__(256) void k_upload_batch(T* __restrict__ pages, int64_t page_elems,
                                                      const UploadPiece* __restrict__ pieces, int32_t n_pieces,
                                                      const EntryWrite* __restrict__ writes, int32_t n_writes,
                                                      int32_t* __restrict__ page_ids, SlotEntry* __restrict__ entries) {
  const int32_t b = blockIdx.x;
  if (b < n_pieces) {
    const UploadPiece pc = pieces[b];
    const T* src = static_cast<const T*>(pc.src);
    T* d = pages + static_cast<int64_t>(pc.page) * page_elems;
    constexpr int kVec = 16 / sizeof(T);
    for (int64_t e = static_cast<int64_t>(threadIdx.x) * kVec; e < page_elems; e += 256 * kVec)
      *reinterpret_cast<u32x4*>(d + e) = *reinterpret_cast<const u32x4*>(src + e);
    if (threadIdx.x == 0) page_ids[pc.id_at] = pc.page;
    return;
  }
  const int32_t w = (b - n_pieces) * 256 + static_cast<int32_t>(threadIdx.x);
  if (w < n_writes) {
    const EntryWrite ew = writes[w];
    entries[ew.index] = ew.value;
  }
}

__global__ void k_clear_entries(SlotEntry* __restrict__ e, int32_t count) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) e[i] = SlotEntry{0, 0.f, 0, 0};
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

bool fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t words = static_cast<int64_t>(bytes / 4);
  if (words == 0) return true;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError() == hipSuccess;
}

void free_device(lora_pool* p) {
  if (p->d_pages) (void)hipFree(p->d_pages);
  if (p->d_entries) (void)hipFree(p->d_entries);
  if (p->d_page_ids) (void)hipFree(p->d_page_ids);
  for (int r = 0; r < lora_pool::kLoadRing; ++r) {
    if (p->d_staging[r]) (void)hipFree(p->d_staging[r]);
    if (p->h_staging[r]) (void)hipHostFree(p->h_staging[r]);
    if (p->ring_done[r]) (void)hipEventDestroy(p->ring_done[r]);
    p->d_staging[r] = nullptr;
    p->h_staging[r] = nullptr;
    p->ring_done[r] = nullptr;
  }
  p->d_pages = nullptr;
  p->d_entries = nullptr;
  p->d_page_ids = nullptr;
}

// Whether ptr is device memory (hipPointerGetAttributes fails for pageable
// host memory the runtime has never seen: that is host memory too, and the
// error is cleared so that later checks do not report it).
bool is_device_memory(const void* ptr) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice;
}

}  // namespace

lora_status pool_upload_async(lora_pool* p, int32_t slot, int32_t module, int32_t rank, const void* a,
                              const void* b, float scale, int32_t* plist, hipStream_t s) {
  if (slot < 0 || slot >= p->n_slots || module < 0 || module >= p->n_modules) return LORA_ERR_SLOT;
  if (rank < 1 || rank > p->max_rank) return LORA_ERR_RANK;
  const size_t ei = static_cast<size_t>(slot) * p->n_modules + module;
  if (p->entries[ei].rank != 0) return LORA_ERR_SLOT;
  const int64_t h = p->page_elems;
  const int64_t ppr_a = p->h_in[module] / h, ppr_b = p->h_out[module] / h;
  const int64_t n_plist = rank * (ppr_a + ppr_b);
  std::vector<int32_t> pages;
  if (!p->alloc.allocate(n_plist, pages)) return LORA_ERR_NO_PAGES;
  std::memcpy(plist, pages.data(), pages.size() * 4);
  const int32_t ids_off = static_cast<int32_t>(ei * p->max_pages_per_entry);
  const int32_t n_a = static_cast<int32_t>(rank * ppr_a);
  const int32_t b_gap = static_cast<int32_t>((p->max_rank - rank) * ppr_a);
  SlotEntry value{rank, scale, ids_off, ids_off + n_a + b_gap};
  if (p->dtype == LORA_BF16) {
    hipLaunchKernelGGL(k_upload<__bf16>, dim3(static_cast<unsigned>(n_plist)), dim3(256), 0, s,
                       static_cast<__bf16*>(p->d_pages), static_cast<const __bf16*>(a),
                       static_cast<const __bf16*>(b), plist, static_cast<int32_t>(n_plist), h, p->d_page_ids,
                       ids_off, n_a, b_gap, p->d_entries + ei, value);
  } else {
    hipLaunchKernelGGL(k_upload<float>, dim3(static_cast<unsigned>(n_plist)), dim3(256), 0, s,
                       static_cast<float*>(p->d_pages), static_cast<const float*>(a), static_cast<const float*>(b),
                       plist, static_cast<int32_t>(n_plist), h, p->d_page_ids, ids_off, n_a, b_gap,
                       p->d_entries + ei, value);
  }
  if (hipGetLastError() != hipSuccess) {
    p->alloc.release(pages);
    return LORA_ERR_HIP;
  }
  auto& e = p->entries[ei];
  e.rank = rank;
  e.scale = scale;
  e.pages = std::move(pages);
  ++p->loads;
  return LORA_OK;
}

bool pool_evict_host(lora_pool* p, int32_t slot) {
  bool any = false;
  for (int32_t m = 0; m < p->n_modules; ++m) {
    auto& e = p->entries[static_cast<size_t>(slot) * p->n_modules + m];
    if (e.rank == 0) continue;
    any = true;
    p->alloc.release(e.pages);
    e = lora_pool::Entry();
  }
  if (any) ++p->evicts;
  return any;
}

lora_status pool_stage_upload(lora_pool* p, int32_t slot, int32_t module, int32_t rank, const void* a,
                              const void* b, float scale, std::vector<UploadPiece>& pieces,
                              std::vector<EntryWrite>& entries) {
  if (slot < 0 || slot >= p->n_slots || module < 0 || module >= p->n_modules) return LORA_ERR_SLOT;
  if (rank < 1 || rank > p->max_rank) return LORA_ERR_RANK;
  const size_t ei = static_cast<size_t>(slot) * p->n_modules + module;
  if (p->entries[ei].rank != 0) return LORA_ERR_SLOT;
  const int64_t h = p->page_elems;
  const int64_t ppr_a = p->h_in[module] / h, ppr_b = p->h_out[module] / h;
  const int64_t n_a = rank * ppr_a, n_plist = rank * (ppr_a + ppr_b);
  std::vector<int32_t> pages;
  if (!p->alloc.allocate(n_plist, pages)) return LORA_ERR_NO_PAGES;
  const int32_t ids_off = static_cast<int32_t>(ei * p->max_pages_per_entry);
  const int32_t b_gap = static_cast<int32_t>((p->max_rank - rank) * ppr_a);
  const size_t pb = static_cast<size_t>(h) * p->elem_bytes();
  for (int64_t i = 0; i < n_plist; ++i) {
    const bool is_a = i < n_a;
    const char* src = static_cast<const char*>(is_a ? a : b) + static_cast<size_t>(is_a ? i : i - n_a) * pb;
    pieces.push_back(UploadPiece{src, pages[static_cast<size_t>(i)],
                                 static_cast<int32_t>(ids_off + i + (is_a ? 0 : b_gap))});
  }
  entries.push_back(EntryWrite{static_cast<int32_t>(ei), 0,
                               SlotEntry{rank, scale, ids_off, static_cast<int32_t>(ids_off + n_a + b_gap)}});
  auto& e = p->entries[ei];
  e.rank = rank;
  e.scale = scale;
  e.pages = std::move(pages);
  ++p->loads;
  return LORA_OK;
}

lora_status pool_upload_batch(lora_pool* p, const UploadPiece* pieces, int32_t n_pieces, const EntryWrite* entries,
                              int32_t n_entries, hipStream_t s) {
  if (n_pieces < 0 || n_entries < 0) return LORA_ERR_ARG;
  const int64_t blocks = static_cast<int64_t>(n_pieces) + (n_entries + 255) / 256;
  if (blocks == 0) return LORA_OK;
  if (blocks > INT32_MAX) return LORA_ERR_SHAPE;
  if (p->dtype == LORA_BF16)
    hipLaunchKernelGGL(k_upload_batch<__bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<__bf16*>(p->d_pages), p->page_elems, pieces, n_pieces, entries, n_entries,
                       p->d_page_ids, p->d_entries);
  else
    hipLaunchKernelGGL(k_upload_batch<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<float*>(p->d_pages), p->page_elems, pieces, n_pieces, entries, n_entries,
                       p->d_page_ids, p->d_entries);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

extern "C" {

int32_t lora_abi_version(void) { return LORA_ABI_VERSION; }

const char* lora_status_str(lora_status s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_ERR_ARG: return "invalid argument";
    case LORA_ERR_SHAPE: return "shape not supported by the pool";
    case LORA_ERR_RANK: return "rank outside [1, max_rank]";
    case LORA_ERR_NO_PAGES: return "not enough free pages";
    case LORA_ERR_SLOT: return "slot/module out of range, already loaded, or empty";
    case LORA_ERR_DTYPE: return "unsupported dtype combination";
    case LORA_ERR_HIP: return "HIP runtime error";
    case LORA_ERR_DEVICE_IDS: return "batch held adapter ids outside [-1, n_slots)";
    case LORA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

lora_status lora_pool_create(lora_pool** out, int32_t device, lora_dtype wdtype, int64_t page_elems,
                             int64_t n_pages, int32_t n_slots, int32_t n_modules, const int64_t* h_in,
                             const int64_t* h_out, int32_t max_rank) {
  if (!out || !h_in || !h_out) return LORA_ERR_ARG;
  *out = nullptr;
  if (wdtype != LORA_F32 && wdtype != LORA_BF16) return LORA_ERR_ARG;
  if (device < 0 || page_elems <= 0 || n_pages <= 0 || n_pages > INT32_MAX) return LORA_ERR_ARG;
  if (n_slots < 1 || n_slots > kMaxSlots || n_modules < 1 || n_modules > 4096) return LORA_ERR_ARG;
  if (max_rank < 1 || max_rank > kMaxRank) return LORA_ERR_RANK;
  if (page_elems % 64 != 0) return LORA_ERR_SHAPE;
  int64_t max_ppe = 0, max_in = 0, max_out = 0;
  for (int32_t m = 0; m < n_modules; ++m) {
    if (h_in[m] <= 0 || h_out[m] <= 0) return LORA_ERR_ARG;
    if (h_in[m] % page_elems != 0 || h_out[m] % page_elems != 0) return LORA_ERR_SHAPE;
    if (h_in[m] > (1 << 20) || h_out[m] > (1 << 20)) return LORA_ERR_SHAPE;
    // kernels find a page by multiplying with the page size's reciprocal: exact while width * page < 2^32
    if (h_in[m] * page_elems >= (int64_t(1) << 32) || h_out[m] * page_elems >= (int64_t(1) << 32))
      return LORA_ERR_SHAPE;
    const int64_t ppe = static_cast<int64_t>(max_rank) * (h_in[m] + h_out[m]) / page_elems;
    if (ppe > kMaxEntryPages) return LORA_ERR_SHAPE;
    if (ppe > max_ppe) max_ppe = ppe;
    if (h_in[m] > max_in) max_in = h_in[m];
    if (h_out[m] > max_out) max_out = h_out[m];
  }
  const int64_t table = static_cast<int64_t>(n_slots) * n_modules * max_ppe;
  if (table > INT32_MAX) return LORA_ERR_ARG;

  lora_pool* p = new (std::nothrow) lora_pool();
  if (!p) return LORA_ERR_ARG;
  p->device = device;
  p->dtype = wdtype;
  p->page_elems = page_elems;
  p->n_pages = n_pages;
  p->n_slots = n_slots;
  p->n_modules = n_modules;
  p->max_rank = max_rank;
  p->max_pages_per_entry = static_cast<int32_t>(max_ppe);
  p->h_in.assign(h_in, h_in + n_modules);
  p->h_out.assign(h_out, h_out + n_modules);
  p->alloc.reset(n_pages);
  p->entries.resize(static_cast<size_t>(n_slots) * n_modules);

  DeviceGuard g(device);
  if (!g.ok) { delete p; return LORA_ERR_HIP; }
  const size_t eb = p->elem_bytes();
  const size_t ab = ((static_cast<size_t>(max_rank) * (max_in + max_out) * eb) + 255) / 256 * 256;
  p->staging_bytes = ab + static_cast<size_t>(max_ppe) * 4 + 256;
  const size_t n_entries = static_cast<size_t>(n_slots) * n_modules;
  // one page past the allocator's: all zeros, read by kernels in place of rows an adapter does not have
  const size_t page_bytes = static_cast<size_t>(page_elems) * eb;
  bool ok = hipMalloc(&p->d_pages, static_cast<size_t>(n_pages + 1) * page_bytes) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&p->d_entries), n_entries * sizeof(SlotEntry)) == hipSuccess &&
            hipMalloc(reinterpret_cast<void**>(&p->d_page_ids),
                      static_cast<size_t>(table > 0 ? table : 1) * 4) == hipSuccess;
  for (int r = 0; ok && r < lora_pool::kLoadRing; ++r)
    ok = hipMalloc(&p->d_staging[r], p->staging_bytes) == hipSuccess &&
         hipHostMalloc(&p->h_staging[r], p->staging_bytes, hipHostMallocDefault) == hipSuccess &&
         hipEventCreateWithFlags(&p->ring_done[r], hipEventDisableTiming) == hipSuccess;
  ok = ok && fill_zero(static_cast<char*>(p->d_pages) + static_cast<size_t>(n_pages) * page_bytes, page_bytes, nullptr) &&
       fill_zero(p->d_entries, n_entries * sizeof(SlotEntry), nullptr) &&
       fill_zero(p->d_page_ids, static_cast<size_t>(table) * 4, nullptr) &&
       hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    free_device(p);
    delete p;
    return LORA_ERR_HIP;
  }
  *out = p;
  return LORA_OK;
}

lora_status lora_pool_destroy(lora_pool* p) {
  if (!p) return LORA_OK;
  lora_status st = LORA_OK;
  {
    DeviceGuard g(p->device);
    if (!g.ok || hipDeviceSynchronize() != hipSuccess) st = LORA_ERR_HIP;
    free_device(p);
  }
  delete p;
  return st;
}

lora_status lora_pool_load(lora_pool* p, int32_t slot, int32_t module, int32_t rank, const void* A,
                           const void* B, float scale, void* stream) {
  if (!p || !A || !B) return LORA_ERR_ARG;
  if (slot < 0 || slot >= p->n_slots || module < 0 || module >= p->n_modules) return LORA_ERR_SLOT;
  if (rank < 1 || rank > p->max_rank) return LORA_ERR_RANK;
  const size_t ei = static_cast<size_t>(slot) * p->n_modules + module;
  if (p->entries[ei].rank != 0) return LORA_ERR_SLOT;
  const int64_t h = p->page_elems;
  const int64_t ppr_a = p->h_in[module] / h, ppr_b = p->h_out[module] / h;
  const int64_t n_plist = rank * (ppr_a + ppr_b);
  std::vector<int32_t> pages;
  if (!p->alloc.allocate(n_plist, pages)) return LORA_ERR_NO_PAGES;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t eb = p->elem_bytes();
  const size_t a_bytes = static_cast<size_t>(rank) * p->h_in[module] * eb;
  const size_t b_bytes = static_cast<size_t>(rank) * p->h_out[module] * eb;
  const size_t ids_at = (a_bytes + b_bytes + 255) / 256 * 256;
  const int32_t ids_off = static_cast<int32_t>(ei * p->max_pages_per_entry);
  // A's page ids from ids_off (rank row j, page p at j*ppr_a + p); B's from
  // ids_off + max_rank*ppr_a whatever the rank, so kernels can fetch both
  // lists without waiting for the entry.
  const int32_t n_a = static_cast<int32_t>(rank * ppr_a);
  const int32_t b_gap = static_cast<int32_t>((p->max_rank - rank) * ppr_a);
  SlotEntry value{rank, scale, ids_off, ids_off + n_a + b_gap};

  DeviceGuard g(p->device);
  bool ok = g.ok;
  // the next ring slot, once the upload that used it last has passed its stream
  const int r = p->ring_next;
  ok = ok && hipEventSynchronize(p->ring_done[r]) == hipSuccess;
  char* hs = static_cast<char*>(p->h_staging[r]);
  char* ds = static_cast<char*>(p->d_staging[r]);
  if (ok) {
    // host rows and the page list are copied into the slot's page-locked buffer now (the
    // caller may reuse A and B at once); rows in device memory are copied on the stream
    const bool a_dev = is_device_memory(A), b_dev = is_device_memory(B);
    if (!a_dev) std::memcpy(hs, A, a_bytes);
    if (!b_dev) std::memcpy(hs + a_bytes, B, b_bytes);
    std::memcpy(hs + ids_at, pages.data(), pages.size() * 4);
    if (!a_dev && !b_dev) {
      ok = hipMemcpyAsync(ds, hs, ids_at + pages.size() * 4, hipMemcpyHostToDevice, s) == hipSuccess;
    } else {
      ok = hipMemcpyAsync(ds, a_dev ? A : hs, a_bytes, a_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s) ==
               hipSuccess &&
           hipMemcpyAsync(ds + a_bytes, b_dev ? B : hs + a_bytes, b_bytes,
                          b_dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, s) == hipSuccess &&
           hipMemcpyAsync(ds + ids_at, hs + ids_at, pages.size() * 4, hipMemcpyHostToDevice, s) == hipSuccess;
    }
  }
  if (ok) {
    if (p->dtype == LORA_BF16) {
      hipLaunchKernelGGL(k_upload<__bf16>, dim3(static_cast<unsigned>(n_plist)), dim3(256), 0, s,
                         static_cast<__bf16*>(p->d_pages), reinterpret_cast<const __bf16*>(ds),
                         reinterpret_cast<const __bf16*>(ds + a_bytes),
                         reinterpret_cast<const int32_t*>(ds + ids_at), static_cast<int32_t>(n_plist), h,
                         p->d_page_ids, ids_off, n_a, b_gap, p->d_entries + ei, value);
    } else {
      hipLaunchKernelGGL(k_upload<float>, dim3(static_cast<unsigned>(n_plist)), dim3(256), 0, s,
                         static_cast<float*>(p->d_pages), reinterpret_cast<const float*>(ds),
                         reinterpret_cast<const float*>(ds + a_bytes),
                         reinterpret_cast<const int32_t*>(ds + ids_at), static_cast<int32_t>(n_plist), h,
                         p->d_page_ids, ids_off, n_a, b_gap, p->d_entries + ei, value);
    }
    ok = hipGetLastError() == hipSuccess && hipEventRecord(p->ring_done[r], s) == hipSuccess;
  }
  if (!ok) {
    p->alloc.release(pages);
    return LORA_ERR_HIP;
  }
  p->ring_next = (r + 1) % lora_pool::kLoadRing;
  auto& e = p->entries[ei];
  e.rank = rank;
  e.scale = scale;
  e.pages = std::move(pages);
  ++p->loads;
  return LORA_OK;
}

lora_status lora_pool_evict(lora_pool* p, int32_t slot, void* stream) {
  if (!p) return LORA_ERR_ARG;
  if (slot < 0 || slot >= p->n_slots) return LORA_ERR_SLOT;
  const size_t e0 = static_cast<size_t>(slot) * p->n_modules;
  bool any = false;
  for (int32_t m = 0; m < p->n_modules; ++m) any |= p->entries[e0 + m].rank != 0;
  if (!any) return LORA_ERR_SLOT;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  hipLaunchKernelGGL(k_clear_entries, dim3((p->n_modules + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p->d_entries + e0, p->n_modules);
  if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
  for (int32_t m = 0; m < p->n_modules; ++m) {
    auto& e = p->entries[e0 + m];
    if (e.rank == 0) continue;
    p->alloc.release(e.pages);
    e = lora_pool::Entry();
  }
  ++p->evicts;
  return LORA_OK;
}

lora_status lora_pool_stats(const lora_pool* p, lora_pool_stats_t* out) {
  if (!p || !out) return LORA_ERR_ARG;
  std::memset(out, 0, sizeof(*out));
  out->n_pages = p->n_pages;
  out->free_pages = p->alloc.free_count();
  for (int32_t s = 0; s < p->n_slots; ++s) {
    bool any = false;
    for (int32_t m = 0; m < p->n_modules; ++m) {
      if (p->entries[static_cast<size_t>(s) * p->n_modules + m].rank != 0) {
        ++out->loaded_entries;
        any = true;
      }
    }
    out->loaded_slots += any ? 1 : 0;
  }
  out->loads = p->loads;
  out->evicts = p->evicts;
  return LORA_OK;
}

lora_status lora_pool_read(const lora_pool* p, int32_t slot, int32_t module, int32_t* rank, float* scale,
                           void* A, void* B, int32_t* pages, int32_t max_pages) {
  if (!p) return LORA_ERR_ARG;
  if (slot < 0 || slot >= p->n_slots || module < 0 || module >= p->n_modules) return LORA_ERR_SLOT;
  const auto& e = p->entries[static_cast<size_t>(slot) * p->n_modules + module];
  if (e.rank == 0) return LORA_ERR_SLOT;
  if (rank) *rank = e.rank;
  if (scale) *scale = e.scale;
  if (pages) {
    for (int32_t i = 0; i < max_pages && i < static_cast<int32_t>(e.pages.size()); ++i) pages[i] = e.pages[i];
  }
  DeviceGuard g(p->device);
  if (!g.ok || hipDeviceSynchronize() != hipSuccess) return LORA_ERR_HIP;
  const int64_t h = p->page_elems;
  const size_t eb = p->elem_bytes();
  const int64_t ppr_a = p->h_in[module] / h, ppr_b = p->h_out[module] / h;
  const char* base = static_cast<const char*>(p->d_pages);
  for (int64_t i = 0; i < static_cast<int64_t>(e.pages.size()); ++i) {
    const bool is_a = i < e.rank * ppr_a;
    void* dst = is_a ? A : B;
    if (!dst) continue;
    const int64_t local = is_a ? i : i - e.rank * ppr_a;
    char* d = static_cast<char*>(dst) + static_cast<size_t>(local) * h * eb;
    const char* src = base + static_cast<size_t>(e.pages[static_cast<size_t>(i)]) * h * eb;
    if (hipMemcpy(d, src, static_cast<size_t>(h) * eb, hipMemcpyDeviceToHost) != hipSuccess) return LORA_ERR_HIP;
  }
  (void)ppr_b;
  return LORA_OK;
}

}  // extern "C"
