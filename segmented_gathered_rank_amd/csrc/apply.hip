// C ABI of the apply path: argument checks, path selection and launches.
//
// Dispatch.  Segments shorter than kLongMin tokens (decode tokens, short
// requests) run on the GEMV path; longer ones run on matrix-core tiles when
// the pool is bf16 and its page and output widths tile evenly.  Both work
// lists come from the segment builder and stay on the device; grids are sized
// by their upper bounds and idle workgroups exit at once.
#include <algorithm>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "fused_gemm.hpp"
#include "gemv_kernels.hpp"
#include "launch_limits.hpp"
#include "mfma_kernels.hpp"
#include "pool.hpp"

using namespace lora;

namespace {

constexpr int kMaxGrid = 4096;   // persistent grids loop over work beyond this
#ifndef LORA_SHRINK_WG_TARGET
#define LORA_SHRINK_WG_TARGET 512
#endif
constexpr int kShrinkWgTarget = LORA_SHRINK_WG_TARGET;   // matrix-core shrink: split K below this many workgroups
#ifndef LORA_PAIR_WG_TARGET
#define LORA_PAIR_WG_TARGET (LORA_SHRINK_WG_TARGET / 2)
#endif
constexpr int kPairWgTarget = LORA_PAIR_WG_TARGET;   // the same per run when two runs share one launch
// LDS for the matrix-core shrink's staged A rows and page ids: three
// workgroups fit in a CU's 160 KiB
constexpr size_t kStreamLdsBudget = 52 * 1024;

SegView seg_view(const lora_segments* s) {
  SegView v;
  v.perm = s->perm;
  v.seg_start = s->seg_start;
  v.seg_slot = s->seg_slot;
  v.meta = s->meta;
  v.units = s->units;
  v.tiles = s->tiles;
  v.max_units = s->max_units;
  v.max_tiles = s->max_tiles;
  return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the apply calls.  `need_out` also checks equal h_out.
// same_out: the call also needs equal h_out (expand and BGMV; the shrink only reads h_in).
// Modules module0 .. module0 + n_modules - 1 exist and share h_in (and h_out when same_out).
lora_status check_modules(const lora_pool* p, int32_t module0, int32_t n_modules, bool same_out) {
  if (!p || n_modules < 1 || module0 < 0 || module0 + n_modules > p->n_modules) return LORA_ERR_ARG;
  for (int32_t m = module0 + 1; m < module0 + n_modules; ++m) {
    if (p->h_in[m] != p->h_in[module0] || (same_out && p->h_out[m] != p->h_out[module0])) return LORA_ERR_SHAPE;
  }
  return LORA_OK;
}

lora_status check_call(const lora_pool* p, int32_t module0, int32_t n_modules, const lora_segments* seg,
                       bool same_out) {
  if (!p || !seg) return LORA_ERR_ARG;
  if (n_modules < 1 || module0 < 0 || module0 + n_modules > p->n_modules) return LORA_ERR_ARG;
  if (seg->n_tokens < 0 || seg->n_slots < 1 || seg->n_slots > p->n_slots) return LORA_ERR_ARG;
  if (seg->n_tokens > 0 && (!seg->perm || !seg->seg_start || !seg->seg_slot || !seg->meta || !seg->units ||
                            !seg->tiles))
    return LORA_ERR_ARG;
  if (seg->max_units != max_units_of(seg->n_tokens, seg->n_slots) || seg->max_tiles != max_tiles_of(seg->n_tokens))
    return LORA_ERR_ARG;
  return check_modules(p, module0, n_modules, same_out);
}

// Element rows of a [n_tokens][ld] operand repeated per module.
lora_status check_operand(const void* ptr, int64_t ld, int64_t mstride, int64_t width, size_t eb,
                          int32_t n_tokens, int32_t n_modules, bool written, bool vec16) {
  if (!ptr) return LORA_ERR_ARG;
  if (ld < width || mstride < 0) return LORA_ERR_ARG;
  if (vec16 && (!aligned16(ptr) || (ld * static_cast<int64_t>(eb)) % 16 != 0 ||
                (mstride * static_cast<int64_t>(eb)) % 16 != 0))
    return LORA_ERR_ARG;
  if (written && n_modules > 1 && mstride < static_cast<int64_t>(n_tokens) * ld) return LORA_ERR_ARG;
  return LORA_OK;
}

bool mfma_ok(const lora_pool* p, int32_t module) {
  return p->dtype == LORA_BF16 && p->page_elems % kExpandCols == 0 && p->h_out[module] % kExpandCols == 0;
}

// Grid for a persistent loop over `bound` work items: a multiple of 8 (one
// share per XCD), at most kMaxGrid.
unsigned grid_of(int32_t bound) {
  if (bound < 1) bound = 1;
  if (bound > kMaxGrid) bound = kMaxGrid;
  return static_cast<unsigned>((bound + 7) / 8 * 8);
}

// Grid of the matrix-core kernels over at most `max_tiles` tiles: a multiple of
// 8*kTileRun, the period of their tile-to-workgroup map, at most kMaxGrid.
unsigned tile_grid_of(int32_t max_tiles) {
  constexpr int period = 8 * kTileRun;
  static_assert(kMaxGrid % period == 0, "the grid cap must be a whole number of periods");
  if (max_tiles < 1) max_tiles = 1;
  if (max_tiles > kMaxGrid) max_tiles = kMaxGrid;
  return static_cast<unsigned>((max_tiles + period - 1) / period * period);
}

// Grid of the GEMV kernels over at most `units` units: a multiple of
// 8*kUnitRun, the period of their unit-to-workgroup map, and at most
// kGemvMaxGrid (4 workgroups per CU fill the chip; more units loop).  A
// launch that finds no units costs about one dispatch of its grid.
constexpr int kGemvMaxGrid = 1024;
// Modules per dispatch group of a fused BGMV over several modules (a multiple
// of 8), and the module count from which the grouped grid is used: against a
// grid of units x modules, which runs the modules one after another, it
// measured 4% faster at 128 modules, 15% at 32, 10% at 24, 6% at 16, even at 8.
constexpr int kBgmvModuleGroup = 32;
constexpr int kBgmvGroupedFrom = 8;

// The GEMV part of a mixed shrink or expand launch (gx workgroups per module,
// after the tiles) takes its modules in the same groups from that count on.
void set_module_groups(GemvArgs& g, unsigned gx, int32_t n_modules) {
  g.module_group = n_modules >= kBgmvGroupedFrom ? std::min(kBgmvModuleGroup, n_modules) : 0;
  g.group_nx = static_cast<int32_t>(gx);
}
unsigned gemv_grid_of(int32_t units) {
  constexpr int period = 8 * kUnitRun;
  static_assert(kGemvMaxGrid % period == 0, "the grid cap must be a whole number of periods");
  if (units < 1) units = 1;
  if (units > kGemvMaxGrid) units = kGemvMaxGrid;
  return static_cast<unsigned>((units + period - 1) / period * period);
}

// Upper bound of the units of segments shorter than kLongMin tokens: one
// such segment per slot at most, each of at most ceil((kLongMin-1)/kUnitTokens) units.
int32_t max_short_units_of(const lora_segments* seg) {
  const int64_t by_slots = static_cast<int64_t>(seg->n_slots) * ((kLongMin - 1 + kUnitTokens - 1) / kUnitTokens);
  return static_cast<int32_t>(by_slots < seg->max_units ? by_slots : seg->max_units);
}

GemvArgs gemv_args(const lora_pool* p, int32_t module0, const SegView& sv, int32_t units_word) {
  GemvArgs g{};
  g.pv = p->view();
  g.sv = sv;
  g.module0 = module0;
  g.units_word = units_word;
  g.parts = 1;
  g.h_in = static_cast<int32_t>(p->h_in[module0]);
  g.h_out = static_cast<int32_t>(p->h_out[module0]);
  g.magic = static_cast<uint32_t>(((uint64_t(1) << 32) + p->page_elems - 1) / p->page_elems);
  return g;
}

int32_t ldr_of(const lora_pool* p) { return (p->max_rank + 15) / 16 * 16; }

// Workspace of the split-K shrink for `ks` splits: one partial tile per split.
size_t split_ws_bytes(const lora_pool* p, int32_t n_tokens, int32_t n_modules, int32_t ks) {
  if (ks <= 1) return 0;
  const size_t tiles = static_cast<size_t>(max_tiles_of(n_tokens));
  return tiles * n_modules * ks * kTileTokens * ldr_of(p) * sizeof(float);
}

// The K split of the matrix-core shrink: ks splits of kps elements (a multiple of 32).
struct ShrinkSplit {
  int32_t ks, kps;
};

// Whether a shrink call runs matrix-core tiles (and so may split K).
bool shrink_has_tiles(const lora_pool* p, int32_t module0, const lora_segments* seg) {
  return p->dtype == LORA_BF16 && mfma_ok(p, module0) && seg->max_tiles > 0;
}

// Split of a shrink call with a workspace of ws_bytes: enough workgroups for 256 CUs when
// the tiles alone are too few, at most kMaxSplits, at least 256 elements of K per split,
// and no more partial tiles than the workspace holds.
ShrinkSplit shrink_split(const lora_pool* p, int32_t module0, int32_t n_modules, int64_t msx,
                         const lora_segments* seg, size_t ws_bytes, int32_t wg_target = kShrinkWgTarget) {
  const int32_t h_in = static_cast<int32_t>(p->h_in[module0]);
  if (!shrink_has_tiles(p, module0, seg)) return ShrinkSplit{1, (h_in + 31) / 32 * 32};
  const bool shared = (msx == 0 && n_modules > 1 && n_modules <= kShrinkMaxModules);
  const int32_t groups = shared ? 1 : n_modules;
  const int32_t est_tiles = (seg->n_tokens + kTileTokens - 1) / kTileTokens;
  int32_t ks = wg_target / (est_tiles * groups > 0 ? est_tiles * groups : 1);
  if (ks > kMaxSplits) ks = kMaxSplits;
  if (ks > h_in / 256) ks = h_in / 256;
  if (ks < 1) ks = 1;
  while (ks > 1 && split_ws_bytes(p, seg->n_tokens, n_modules, ks) > ws_bytes) --ks;
  int32_t kps = (h_in + ks - 1) / ks;
  kps = (kps + 31) / 32 * 32;
  return ShrinkSplit{(h_in + kps - 1) / kps, kps};
}

bool allow_dynamic_lds(const void* fn, int device, size_t lds);

// The shrink launch of one run of modules (modules that share x, or one module
// after another with x stride msx): its GEMV arguments and grid, and, for bf16
// pools with matrix-core tiles, its tile arguments, grid and LDS.
struct ShrinkPlan {
  GemvArgs g;
  unsigned gx;          // GEMV workgroups per module
  bool tiles;           // matrix-core tiles (else the GEMV kernel alone)
  ShrinkArgs a;
  int32_t per_wg;       // modules one tile workgroup computes from one x slice
  int32_t groups;       // module groups (grid z of the tile part)
  int ntiles;           // 16-column tiles per module (rank cap / 16, rounded to 1, 2 or 4)
  int tnx;              // tile workgroups per split and group
  size_t lds;
  int64_t tile_blocks() const { return static_cast<int64_t>(tnx) * a.ks_count * groups; }
  int64_t gemv_blocks(int32_t n_modules) const { return static_cast<int64_t>(gx) * n_modules; }
};

// sp: the K split (shrink_split); ws holds its partial tiles when sp.ks > 1.  fold: the
// partial tiles are left in ws for the expand to add (no k_shrink_reduce launch), so
// the t rows of tokens in matrix-core tiles are not written; they sit at modules
// part_m0 .. part_m0 + n_modules - 1 of a layout of part_nm modules (one call's
// modules may come from several shrink launches).
template <typename TI>
ShrinkPlan plan_shrink(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                       int64_t msx, const lora_segments* seg, float* t, int64_t ld_t, int64_t mst, ShrinkSplit sp,
                       void* ws, bool fold, int32_t part_m0, int32_t part_nm) {
  ShrinkPlan pl{};
  const PoolView pv = p->view();
  const SegView sv = seg_view(seg);
  const int32_t h_in = static_cast<int32_t>(p->h_in[module0]);
  const bool use_mfma = mfma_ok(p, module0);
  const int32_t units_word = use_mfma ? LORA_META_N_UNITS_SHORT : LORA_META_N_UNITS_ALL;
  GemvArgs& g = pl.g;
  g = gemv_args(p, module0, sv, units_word);
  g.x = x;
  g.ld_x = ld_x;
  g.msx = msx;
  g.t = t;
  g.ld_t = ld_t;
  g.mst = mst;
  const int32_t gemv_units = use_mfma ? max_short_units_of(seg) : seg->max_units;   // what units_word can count
  g.parts = (p->max_rank + kPartRows - 1) / kPartRows;   // a work item per kPartRows rank rows of a unit
  pl.gx = gemv_grid_of(gemv_units * g.parts);
  // long segments on matrix-core tiles and short units on the GEMV path, in one launch
  pl.tiles = sizeof(TI) == 2 && use_mfma && seg->max_tiles > 0;
  if (!pl.tiles) return pl;
  const bool shared = (msx == 0 && n_modules > 1 && n_modules <= kShrinkMaxModules);
  pl.groups = shared ? 1 : n_modules;
  pl.per_wg = shared ? n_modules : 1;
  const int32_t ks = sp.ks, kps = sp.kps;
  ShrinkArgs& a = pl.a;
  a.pv = pv;
  a.sv = sv;
  a.x = static_cast<const __bf16*>(x);
  a.ld_x = ld_x;
  a.msx = shared ? 0 : msx;
  a.t = t;
  a.ld_t = ld_t;
  a.mst = mst;
  a.module0 = module0;
  a.mods_per_wg = pl.per_wg;
  a.h_in = h_in;
  a.ks_count = ks;
  a.k_per_split = kps;
  a.ldr = ldr_of(p);
  a.magic = static_cast<uint32_t>(((uint64_t(1) << 32) + p->page_elems - 1) / p->page_elems);
  a.max_pids = p->max_pages_per_entry;
  pl.ntiles = a.ldr <= 16 ? 1 : a.ldr <= 32 ? 2 : 4;
  // A rows staged in LDS at once: the whole split when they fit the LDS budget,
  // else equal sub-ranges (multiples of 32) that do
  const size_t ids_bytes = static_cast<size_t>(pl.per_wg) * a.max_pids * 4;
  const size_t row_bytes = static_cast<size_t>(pl.per_wg) * 16 * pl.ntiles * 2;   // per k of A rows
  int32_t kc_max = static_cast<int32_t>((kStreamLdsBudget - ids_bytes) / row_bytes) - 16;
  kc_max = std::max(32, kc_max / 32 * 32);
  const int32_t n_sub = (kps + kc_max - 1) / kc_max;
  a.kc = ((kps + n_sub - 1) / n_sub + 31) / 32 * 32;
  pl.lds = std::max(stream_lds_bytes(pl.per_wg, pl.ntiles, a.kc, a.max_pids), gemv_lds_bytes<1, __bf16>());
  a.part = ks > 1 ? static_cast<float*>(ws) : nullptr;
  a.part_m0 = fold ? part_m0 : 0;
  a.part_nm = fold && part_nm > 0 ? part_nm : n_modules;   // k_shrink_reduce reads this launch's layout
  pl.tnx = static_cast<int>(tile_grid_of(seg->max_tiles));
  set_module_groups(g, pl.gx, n_modules);
  return pl;
}

template <typename TI>
lora_status launch_shrink(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                          int64_t msx, const lora_segments* seg, float* t, int64_t ld_t, int64_t mst,
                          ShrinkSplit sp, void* ws, hipStream_t s, bool fold = false, int32_t part_m0 = 0,
                          int32_t part_nm = 0) {
  ShrinkPlan pl =
      plan_shrink<TI>(p, module0, n_modules, x, ld_x, msx, seg, t, ld_t, mst, sp, ws, fold, part_m0, part_nm);
  if (pl.tiles) {
    const int32_t ks = pl.a.ks_count;
    const int64_t n_blocks = pl.tile_blocks() + pl.gemv_blocks(n_modules);
    if (!grid_fits(n_blocks, kMfmaThreads)) return LORA_ERR_SHAPE;   // beyond one launch (nothing launched yet)
    const dim3 grid(static_cast<unsigned>(n_blocks)), block(kMfmaThreads);
#define LORA_SHRINK_LAUNCH(M, NT)                                                                              \
  hipLaunchKernelGGL((k_shrink_mixed<M, NT, kStreamDepth>), grid, block, pl.lds, s, pl.a, pl.g, pl.tnx, ks, \
                     pl.groups, static_cast<int>(pl.gx), n_modules)
#define LORA_SHRINK_NT(M)                                 \
  do {                                                    \
    if (pl.ntiles == 1) LORA_SHRINK_LAUNCH(M, 1);         \
    else if (pl.ntiles == 2) LORA_SHRINK_LAUNCH(M, 2);    \
    else LORA_SHRINK_LAUNCH(M, 4);                        \
  } while (0)
    switch (pl.per_wg) {
      case 1: LORA_SHRINK_NT(1); break;
      case 2: LORA_SHRINK_NT(2); break;
      case 3: LORA_SHRINK_NT(3); break;
      default: LORA_SHRINK_NT(4); break;
    }
#undef LORA_SHRINK_NT
#undef LORA_SHRINK_LAUNCH
    if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
    if (ks > 1 && !fold) {
      hipLaunchKernelGGL(k_shrink_reduce, dim3(tile_grid_of(seg->max_tiles), n_modules), block, 0, s, pl.a);
      if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
    }
    return LORA_OK;
  }
  hipLaunchKernelGGL((k_gemv<1, TI, TI>), dim3(pl.gx, n_modules), dim3(kGemvThreads), 0, s, pl.g);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// The two shrink launches of an attention layer's runs, q,k,v sharing x (3 modules
// per tile workgroup) and o with its own x, as one launch: its grid holds both
// runs' tiles, then both runs' GEMV items, so the two x streams overlap instead of
// each ramping up and draining alone.  Both plans have matrix-core tiles, one
// module group each, the same K split and tile width; returns false when the runs
// are not of that shape (nothing launched).
bool launch_shrink_pair(const ShrinkPlan& p1, int32_t n1, const ShrinkPlan& p2, int32_t n2, hipStream_t s,
                        int device, lora_status* st) {
  if (!p1.tiles || !p2.tiles || p1.per_wg != 3 || n1 != 3 || p2.per_wg != 1 || n2 != 1 || p1.groups != 1 ||
      p2.groups != 1 || p1.ntiles != p2.ntiles || p1.a.ks_count != p2.a.ks_count || p1.tnx != p2.tnx ||
      p1.gx != p2.gx)
    return false;
  const int64_t n_blocks = p1.tile_blocks() + p2.tile_blocks() + p1.gemv_blocks(n1) + p2.gemv_blocks(n2);
  if (!grid_fits(n_blocks, kMfmaThreads)) return false;
  const size_t lds = std::max(p1.lds, p2.lds);
  const dim3 grid(static_cast<unsigned>(n_blocks)), block(kMfmaThreads);
  const int ks = p1.a.ks_count, gx = static_cast<int>(p1.gx);
#define LORA_PAIR_LAUNCH(NT)                                                                                     \
  do {                                                                                                           \
    if (!allow_dynamic_lds(reinterpret_cast<const void*>(&k_shrink_pair<3, 1, NT, kStreamDepth>), device, lds)) { \
      *st = LORA_ERR_HIP;                                                                                        \
      return true;                                                                                               \
    }                                                                                                            \
    hipLaunchKernelGGL((k_shrink_pair<3, 1, NT, kStreamDepth>), grid, block, lds, s, p1.a, p1.g, p2.a, p2.g,     \
                       p1.tnx, ks, gx, n1, n2);                                                                  \
  } while (0)
  if (p1.ntiles == 1) LORA_PAIR_LAUNCH(1);
  else if (p1.ntiles == 2) LORA_PAIR_LAUNCH(2);
  else LORA_PAIR_LAUNCH(4);
#undef LORA_PAIR_LAUNCH
  *st = hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  return true;
}

// Work items per unit of a fused BGMV launch: with few modules the units leave
// most of the GPU idle and each unit's chain of round trips sets the latency,
// so a unit is split into column ranges, each item running the whole shrink
// (from the same XCD's L2 after the first) and its range of the expand: as many
// ranges as the resident workgroups (four per CU) hold beside the launch's
// units, at most one 4-column chunk per thread.  A single module of 64 decode
// tokens over 32 slots (48 units at most) takes 4 ranges of 4096 columns:
// 28.2 -> 20.4 us per call; the 128-module launch keeps 1.
int32_t bgmv_parts(int device, int32_t n_modules, int32_t max_units, int32_t h_out) {
  static std::mutex mu;
  static std::map<int, int> cus_of;
  int cus = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus_of.find(device);
    if (it == cus_of.end()) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
        (void)hipGetLastError();
        cus = 0;
      }
      cus_of.emplace(device, cus);
    } else {
      cus = it->second;
    }
  }
  const int64_t resident = 4 * static_cast<int64_t>(cus);
  const int64_t items = static_cast<int64_t>(n_modules) * std::max(max_units, 1);
  const int32_t by_cols = std::max(1, h_out / (4 * kGemvThreads));
  const int64_t by_room = resident / items;
  return static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(by_cols, by_room)));
}

static_assert(LORA_IDS_MAX_TOKENS == kWaveSegTokens, "the ids path builds the unit list on one wave");

// The fused BGMV from the ids (k_bgmv_ids): grid as launch_bgmv's, one workgroup
// per unit 64 tokens can hold over the pool's slots.
template <typename TI, typename TO>
lora_status launch_bgmv_ids(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                            int64_t msx, const int32_t* ids, int32_t n, void* y, int64_t ld_y, int64_t msy,
                            hipStream_t s) {
  GemvArgs g = gemv_args(p, module0, SegView{}, LORA_META_N_UNITS_ALL);   // the kernel fills g.sv in LDS
  g.x = x;
  g.ld_x = ld_x;
  g.msx = msx;
  g.y = y;
  g.ld_y = ld_y;
  g.msy = msy;
  g.pack = 1;
  int32_t nbits = 0;
  while ((1 << nbits) < p->n_slots) ++nbits;
  const int32_t units = max_units_of(n, p->n_slots);
  g.parts = bgmv_parts(p->device, n_modules, units, static_cast<int32_t>(p->h_out[module0]));
  g.x_stream = (msx == 0 && n_modules > 1) || g.parts > 1 ? 0 : 1;   // x rows read by one work item only are streamed
  if (n_modules >= kBgmvGroupedFrom) {
    const unsigned gxg = static_cast<unsigned>(units * g.parts);
    if (static_cast<int64_t>(n_modules) * gxg * kGemvThreads > static_cast<int64_t>(UINT32_MAX)) return LORA_ERR_SHAPE;
    g.module_group = std::min(kBgmvModuleGroup, n_modules);
    g.group_nx = static_cast<int32_t>(gxg);
    hipLaunchKernelGGL((k_bgmv_ids<TI, TO>), dim3(gxg * static_cast<unsigned>(n_modules)), dim3(kGemvThreads), 0, s,
                       g, ids, n, nbits);
  } else {
    hipLaunchKernelGGL((k_bgmv_ids<TI, TO>), dim3(gemv_grid_of(units * g.parts), n_modules), dim3(kGemvThreads), 0, s,
                       g, ids, n, nbits);
  }
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Raises kernel `fn`'s dynamic LDS limit on `device` to at least `lds` bytes
// (the default is 64 KiB).  Safe to call from several host threads.
bool allow_dynamic_lds(const void* fn, int device, size_t lds) {
  if (lds <= 64 * 1024) return true;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> allowed;
  std::lock_guard<std::mutex> lock(mu);
  size_t& cur = allowed[std::make_pair(fn, device)];
  if (lds <= cur) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  cur = lds;
  return true;
}

// Column blocks per workgroup of the matrix-core expand.  A launch runs in
// about ceil(workgroups / resident workgroups) rounds, and a round lasts
// about (blocks per workgroup + 2) block times: a workgroup's tile prologue
// and t staging cost about two blocks.  The group size (kept even across a
// tile's groups) that minimizes that product is taken, the larger on a tie.  Measured on the
// encoder layer and prefill projections it picks the fastest of 4, 6 and 8
// blocks for every shape (768 columns: 6 blocks, 25.6 us against 27.8 us
// with 4 and 2; 3072 columns: 8 blocks, 71.5 us against 74.8 us).
int expand_group_blocks(int n_blocks, int tiles, int n_modules, int resident) {
  int best_g = 1;
  int64_t best = INT64_MAX;
  for (int g = 1; g <= kExpandBlocks; ++g) {
    const int groups = (n_blocks + g - 1) / g;
    const int gb = (n_blocks + groups - 1) / groups;
    const int64_t wgs = static_cast<int64_t>(tiles) * groups * n_modules;
    const int64_t cost = ((wgs + resident - 1) / resident) * (gb + 2);
    if (cost <= best) {   // ties go to the larger group: fewer prologues
      best = cost;
      best_g = gb;
    }
  }
  return best_g;
}

// Workgroups of k_expand_mixed<TO, PQ> resident on the whole device at `lds` bytes
// of dynamic LDS (occupancy per CU times CUs), cached per device and LDS size;
// 0 on a HIP error.
template <typename TO, int PQ>
int expand_resident_groups(int device, size_t lds) {
  static std::mutex mu;
  static std::map<std::pair<int, size_t>, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(device, lds);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_expand_mixed<TO, PQ>),
                                                   kMfmaThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int resident = std::max(1, per_cu) * std::max(1, cus);
  cache.emplace(key, resident);
  return resident;
}

// Dynamic LDS of k_expand_mixed<TO, *> at rank cap ldr: up to 78 KiB at rank 64
// with fp32 y (gfx950: 160 KiB per workgroup).
template <typename TO>
size_t expand_mixed_lds(int ldr) {
  return std::max(expand_lds_bytes(ldr, static_cast<int>(sizeof(TO))), gemv_lds_bytes<2, __bf16>());
}

// expand_resident_groups<TO, PQ> once the kernel may take `lds` bytes of
// dynamic LDS (the occupancy query needs that limit in place); 0 on a HIP error.
template <typename TO, int PQ>
int expand_resident_ready(int device, size_t lds) {
  if (!allow_dynamic_lds(reinterpret_cast<const void*>(&k_expand_mixed<TO, PQ>), device, lds)) return 0;
  return expand_resident_groups<TO, PQ>(device, lds);
}

// The matrix-core expand launch: tiles of long segments, then the GEMV items of
// short units (gx workgroups per module); PQ as for expand_mfma_body.
template <typename TO, int PQ>
lora_status expand_mixed_call(const lora_pool* p, ExpandArgs& ea, GemvArgs& g, const lora_segments* seg, unsigned gx,
                              int32_t n_modules, hipStream_t s) {
  const size_t lds = expand_mixed_lds<TO>(ea.ldr);
  const int resident = expand_resident_ready<TO, PQ>(p->device, lds);
  if (resident <= 0) return LORA_ERR_HIP;
  const int n_blocks = ea.h_out / kExpandCols;
  ea.blocks = expand_group_blocks(n_blocks, (seg->n_tokens + kTileTokens - 1) / kTileTokens, n_modules, resident);
  const int tnx = static_cast<int>(tile_grid_of(seg->max_tiles));
  const int col_groups = (n_blocks + ea.blocks - 1) / ea.blocks;
  const int64_t n_wgs = static_cast<int64_t>(tnx) * col_groups * n_modules + static_cast<int64_t>(gx) * n_modules;
  if (!grid_fits(n_wgs, kMfmaThreads)) return LORA_ERR_SHAPE;   // beyond one launch (nothing launched yet)
  set_module_groups(g, gx, n_modules);
  hipLaunchKernelGGL((k_expand_mixed<TO, PQ>), dim3(static_cast<unsigned>(n_wgs)), dim3(kMfmaThreads), lds, s, ea, g,
                     tnx, col_groups, n_modules, static_cast<int>(gx), n_modules);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// part: the shrink's K-split partial tiles of these modules (ks splits), summed
// into the T tiles in place of t's rows; nullptr: t.
template <typename TI, typename TO>
lora_status launch_expand(const lora_pool* p, int32_t module0, int32_t n_modules, const float* t, int64_t ld_t,
                          int64_t mst, const lora_segments* seg, void* y, int64_t ld_y, int64_t msy,
                          hipStream_t s, const float* part = nullptr, int32_t ks = 1) {
  const PoolView pv = p->view();
  const SegView sv = seg_view(seg);
  const int32_t h_out = static_cast<int32_t>(p->h_out[module0]);
  const bool use_mfma = mfma_ok(p, module0);
  const int32_t units_word = use_mfma ? LORA_META_N_UNITS_SHORT : LORA_META_N_UNITS_ALL;
  GemvArgs g = gemv_args(p, module0, sv, units_word);
  g.t = const_cast<float*>(t);
  g.ld_t = ld_t;
  g.mst = mst;
  g.y = y;
  g.ld_y = ld_y;
  g.msy = msy;
  const int32_t gemv_units = use_mfma ? max_short_units_of(seg) : seg->max_units;   // what units_word can count
  // a work item per column range of at least 64 quads, as many ranges as 16-row blocks of rank
  const int32_t col_ranges = static_cast<int32_t>(p->h_out[module0] / 4 / 64);
  g.parts = std::max(1, std::min((p->max_rank + 15) / 16, col_ranges));
  const unsigned gx = gemv_grid_of(gemv_units * g.parts);
  if constexpr (sizeof(TI) == 2) {
    // long segments on matrix-core tiles and short units on the GEMV path, in one launch
    if (use_mfma && seg->max_tiles > 0) {
      ExpandArgs ea;
      ea.pv = pv;
      ea.sv = sv;
      ea.t = t;
      ea.ld_t = ld_t;
      ea.mst = mst;
      ea.y = y;
      ea.ld_y = ld_y;
      ea.msy = msy;
      ea.module0 = module0;
      ea.h_out = h_out;
      ea.ldr = ldr_of(p);
      ea.b_ids_at = static_cast<int32_t>(p->max_rank * (p->h_in[module0] / p->page_elems));
      ea.part = part;
      ea.ks = part ? ks : 1;
      switch (part ? ea.ldr / 16 : 0) {   // 16-byte column groups of a partial tile row per thread
        case 0: return expand_mixed_call<TO, 0>(p, ea, g, seg, gx, n_modules, s);
        case 1: return expand_mixed_call<TO, 1>(p, ea, g, seg, gx, n_modules, s);
        case 2: return expand_mixed_call<TO, 2>(p, ea, g, seg, gx, n_modules, s);
        case 3: return expand_mixed_call<TO, 3>(p, ea, g, seg, gx, n_modules, s);
        default: return expand_mixed_call<TO, 4>(p, ea, g, seg, gx, n_modules, s);
      }
    }
  }
  hipLaunchKernelGGL((k_gemv<2, TI, TO>), dim3(gx, n_modules), dim3(kGemvThreads), 0, s, g);
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Whether n_modules modules from module0 fit one packed work item: at most
// kBgmvMaxPack modules, their stacked rank rows within a unit's t, and all their
// page ids within its LDS table.
bool packable(const lora_pool* p, int32_t module0, int32_t n_modules) {
  const int64_t ids_per = static_cast<int64_t>(p->max_rank) * ((p->h_in[module0] + p->h_out[module0]) / p->page_elems);
  return n_modules >= 2 && n_modules <= kBgmvMaxPack && n_modules * p->max_rank <= kMaxRank &&
         n_modules * ids_per <= kMaxEntryPages;
}

// packed: the modules share x and one work item takes all of them (k_bgmv_packed).
template <typename TI, typename TO>
lora_status launch_bgmv(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                        int64_t msx, const lora_segments* seg, void* y, int64_t ld_y, int64_t msy, hipStream_t s,
                        bool packed = false) {
  GemvArgs g = gemv_args(p, module0, seg_view(seg), LORA_META_N_UNITS_ALL);
  g.x = x;
  g.ld_x = ld_x;
  g.msx = msx;
  g.y = y;
  g.ld_y = ld_y;
  g.msy = msy;
  const bool shared_x = msx == 0 && n_modules > 1;
  g.pack = packed ? n_modules : 1;
  g.parts = packed ? 1 : bgmv_parts(p->device, n_modules, seg->max_units, static_cast<int32_t>(p->h_out[module0]));
  const unsigned gx = gemv_grid_of(seg->max_units * g.parts);
  // x rows read by one work item only are streamed
  g.x_stream = ((!shared_x || packed) && g.parts == 1) ? 1 : 0;
  if (packed) {
    hipLaunchKernelGGL((k_bgmv_packed<TI, TO>), dim3(gx, 1), dim3(kGemvThreads), 0, s, g);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  // several modules: one 1-D grid taken in groups of up to kBgmvModuleGroup modules.  There a
  // workgroup's unit is its place inside the group, so the grid needs no period: one
  // workgroup per unit the segments can hold (fewer empty workgroups between the groups)
  const unsigned gxg =
      static_cast<unsigned>(std::min<int32_t>(std::max<int32_t>(seg->max_units * g.parts, 1), kGemvMaxGrid));
  if (n_modules >= kBgmvGroupedFrom &&
      static_cast<int64_t>(n_modules) * gxg * kGemvThreads <= static_cast<int64_t>(UINT32_MAX)) {
    g.module_group = std::min(kBgmvModuleGroup, n_modules);
    g.group_nx = static_cast<int32_t>(gxg);
    hipLaunchKernelGGL((k_gemv<0, TI, TO>), dim3(gxg * static_cast<unsigned>(n_modules)), dim3(kGemvThreads), 0, s,
                       g);
  } else {
    hipLaunchKernelGGL((k_gemv<0, TI, TO>), dim3(gx, n_modules), dim3(kGemvThreads), 0, s, g);
  }
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Argument checks of the shrink calls.
lora_status shrink_checks(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                          int64_t msx, const lora_segments* seg, const float* t, int64_t ld_t, int64_t mst) {
  lora_status st = check_call(p, module0, n_modules, seg, false);
  if (st != LORA_OK) return st;
  const int32_t n = seg->n_tokens;
  st = check_operand(x, ld_x, msx, p->h_in[module0], p->elem_bytes(), n, n_modules, false, true);
  if (st != LORA_OK) return st;
  // t takes 16-byte stores (the K-split sum writes four rank columns at once)
  return check_operand(t, ld_t, mst, p->max_rank, 4, n, n_modules, true, true);
}

// A checked shrink call on the current device (fold, part_m0, part_nm as for launch_shrink).
lora_status shrink_call(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                        int64_t msx, const lora_segments* seg, float* t, int64_t ld_t, int64_t mst, ShrinkSplit sp,
                        void* ws, hipStream_t s, bool fold = false, int32_t part_m0 = 0, int32_t part_nm = 0) {
  if (p->dtype == LORA_BF16)
    return launch_shrink<__bf16>(p, module0, n_modules, x, ld_x, msx, seg, t, ld_t, mst, sp, ws, s, fold, part_m0,
                                 part_nm);
  return launch_shrink<float>(p, module0, n_modules, x, ld_x, msx, seg, t, ld_t, mst, sp, ws, s, fold, part_m0,
                              part_nm);
}

// Argument checks of the expand calls (modules of one shape).
lora_status expand_checks(const lora_pool* p, int32_t module0, int32_t n_modules, const float* t, int64_t ld_t,
                          int64_t mst, const lora_segments* seg, const void* y, int64_t ld_y, int64_t msy,
                          lora_dtype ydtype) {
  lora_status st = check_call(p, module0, n_modules, seg, true);
  if (st != LORA_OK) return st;
  if (ydtype != LORA_F32 && ydtype != LORA_BF16) return LORA_ERR_DTYPE;
  const int32_t n = seg->n_tokens;
  st = check_operand(t, ld_t, mst, p->max_rank, 4, n, n_modules, false, false);
  if (st != LORA_OK) return st;
  return check_operand(y, ld_y, msy, p->h_out[module0], ydtype == LORA_BF16 ? 2 : 4, n, n_modules, true, true);
}

// A checked expand call on the current device; part / ks as for launch_expand.
lora_status expand_call(const lora_pool* p, int32_t module0, int32_t n_modules, const float* t, int64_t ld_t,
                        int64_t mst, const lora_segments* seg, void* y, int64_t ld_y, int64_t msy, lora_dtype ydtype,
                        hipStream_t s, const float* part = nullptr, int32_t ks = 1) {
  if (p->dtype == LORA_BF16) {
    if (ydtype == LORA_BF16)
      return launch_expand<__bf16, __bf16>(p, module0, n_modules, t, ld_t, mst, seg, y, ld_y, msy, s, part, ks);
    return launch_expand<__bf16, float>(p, module0, n_modules, t, ld_t, mst, seg, y, ld_y, msy, s, part, ks);
  }
  if (ydtype == LORA_BF16)
    return launch_expand<float, __bf16>(p, module0, n_modules, t, ld_t, mst, seg, y, ld_y, msy, s);
  return launch_expand<float, float>(p, module0, n_modules, t, ld_t, mst, seg, y, ld_y, msy, s);
}

// The fused base + adapter pass: checks shared by both weight formats, then the
// launch.  Exactly one of w (bf16 W^T) and w8 (e4m3 W^T with column scales) is
// given; their own alignment is checked by the caller.
lora_status fused_call(const lora_pool* p, int32_t module, const void* x, int64_t ld_x, const void* w,
                       const uint8_t* w8, int64_t ld_w, const float* w_scale, const int32_t* ids, int32_t n_tokens,
                       void* y, int64_t ld_y, void* stream) {
  if (!p || module < 0 || module >= p->n_modules || n_tokens < 0) return LORA_ERR_ARG;
  if (p->dtype != LORA_BF16) return LORA_ERR_DTYPE;
  const int64_t h_in = p->h_in[module], h_out = p->h_out[module];
  if (h_in / p->page_elems > kFgMaxPpr || p->n_slots > kFgMaxSlots) return LORA_ERR_SHAPE;
  if (!x || !y) return LORA_ERR_ARG;
  if (ld_x < h_in || ld_w < h_in || ld_y < h_out) return LORA_ERR_ARG;
  // a tile's 256 rows of x or W^T are addressed with 32-bit byte offsets
  if (ld_x > (int64_t(1) << 22) || ld_w > (int64_t(1) << 22)) return LORA_ERR_SHAPE;
  if (!aligned16(x) || (ld_x * 2) % 16 != 0) return LORA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(y) & 7u) != 0 || (ld_y * 2) % 8 != 0) return LORA_ERR_ARG;
  if (n_tokens == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  FusedArgs fa{};
  fa.pv = p->view();
  fa.x = static_cast<const __bf16*>(x);
  fa.w = static_cast<const __bf16*>(w);
  fa.w8 = w8;
  fa.w_scale = w_scale;
  fa.ids = ids;
  fa.y = static_cast<__bf16*>(y);
  fa.ld_x = ld_x;
  fa.ld_w = ld_w;
  fa.ld_y = ld_y;
  fa.n = n_tokens;
  fa.h_in = static_cast<int32_t>(h_in);
  fa.h_out = static_cast<int32_t>(h_out);
  fa.module = module;
  const int64_t n_rt = (static_cast<int64_t>(n_tokens) + kFgBM - 1) / kFgBM;
  fa.n_ct = static_cast<int32_t>((h_out + kFgBN - 1) / kFgBN);
  const int64_t tiles = n_rt * fa.n_ct;
  if (tiles > (int64_t(1) << 30)) return LORA_ERR_SHAPE;
  fa.n_tiles = static_cast<int32_t>(tiles);
  const unsigned grid = static_cast<unsigned>((tiles + 7) / 8 * 8);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w8) {
    if (ids)
      hipLaunchKernelGGL((k_fused_gemm<true, true>), dim3(grid), dim3(kFgThreads), 0, s, fa);
    else
      hipLaunchKernelGGL((k_fused_gemm<false, true>), dim3(grid), dim3(kFgThreads), 0, s, fa);
  } else {
    if (ids)
      hipLaunchKernelGGL((k_fused_gemm<true, false>), dim3(grid), dim3(kFgThreads), 0, s, fa);
    else
      hipLaunchKernelGGL((k_fused_gemm<false, false>), dim3(grid), dim3(kFgThreads), 0, s, fa);
  }
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

// Device memory of lora_shrink_noalloc's K-split partial tiles, in place of a
// caller workspace: one copy per GPU, held until the process ends, shared by
// every lora_shrink_noalloc call on that GPU.
static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on `device`, which must be current: taken with
// hipGetSymbolAddress on the first call for that device and kept; nullptr if
// HIP cannot give it.  Host code uses only this address, never the array's
// name (a host-side stand-in).
void* scratch_on_device(int device) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = ptrs.find(device);
  if (it != ptrs.end()) return it->second;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  ptrs.emplace(device, ptr);
  return ptr;
}

}  // namespace

extern "C" {

size_t lora_shrink_workspace_bytes(const lora_pool* p, int32_t n_tokens, int32_t n_modules) {
  if (!p || n_tokens < 0 || n_modules < 1) return 0;
  return split_ws_bytes(p, n_tokens, n_modules, kMaxSplits);
}

lora_status lora_shrink(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                        int64_t module_stride_x, const lora_segments* seg, float* t, int64_t ld_t,
                        int64_t module_stride_t, void* ws, size_t ws_bytes, void* stream) {
  const lora_status st = shrink_checks(p, module0, n_modules, x, ld_x, module_stride_x, seg, t, ld_t, module_stride_t);
  if (st != LORA_OK) return st;
  const int32_t n = seg->n_tokens;
  if (ws_bytes > 0 && (!ws || !aligned16(ws))) return LORA_ERR_ARG;
  if (n == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  const ShrinkSplit sp = shrink_split(p, module0, n_modules, module_stride_x, seg, ws_bytes);
  return shrink_call(p, module0, n_modules, x, ld_x, module_stride_x, seg, t, ld_t, module_stride_t, sp, ws,
                     static_cast<hipStream_t>(stream));
}

lora_status lora_shrink_noalloc(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                                int64_t module_stride_x, const lora_segments* seg, float* t, int64_t ld_t,
                                int64_t module_stride_t, void* stream) {
  lora_status st = shrink_checks(p, module0, n_modules, x, ld_x, module_stride_x, seg, t, ld_t, module_stride_t);
  if (st != LORA_OK) return st;
  if (seg->n_tokens == 0) return LORA_OK;
  // the split lora_shrink makes with a workspace of lora_shrink_workspace_bytes, if it fits the scratch
  const ShrinkSplit sp = shrink_split(p, module0, n_modules, module_stride_x, seg, SIZE_MAX);
  const size_t need = split_ws_bytes(p, seg->n_tokens, n_modules, sp.ks);
  if (need > static_cast<size_t>(LORA_NOALLOC_SCRATCH_BYTES)) return LORA_ERR_WORKSPACE;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_device(p->device);
    if (!ws) return LORA_ERR_HIP;
  }
  return shrink_call(p, module0, n_modules, x, ld_x, module_stride_x, seg, t, ld_t, module_stride_t, sp, ws,
                     static_cast<hipStream_t>(stream));
}

lora_status lora_expand(const lora_pool* p, int32_t module0, int32_t n_modules, const float* t, int64_t ld_t,
                        int64_t module_stride_t, const lora_segments* seg, void* y, int64_t ld_y,
                        int64_t module_stride_y, lora_dtype ydtype, void* stream) {
  const lora_status st =
      expand_checks(p, module0, n_modules, t, ld_t, module_stride_t, seg, y, ld_y, module_stride_y, ydtype);
  if (st != LORA_OK) return st;
  if (seg->n_tokens == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  return expand_call(p, module0, n_modules, t, ld_t, module_stride_t, seg, y, ld_y, module_stride_y, ydtype,
                     static_cast<hipStream_t>(stream));
}

lora_status lora_apply_sgmv(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                            int64_t module_stride_x, const lora_segments* seg, float* t, int64_t ld_t,
                            int64_t module_stride_t, void* y, int64_t ld_y, int64_t module_stride_y,
                            lora_dtype ydtype, void* ws, size_t ws_bytes, void* stream) {
  const lora_x_run run{x, ld_x, module_stride_x, n_modules};
  return lora_apply_sgmv_multi(p, module0, n_modules, &run, 1, seg, t, ld_t, module_stride_t, y, ld_y,
                               module_stride_y, ydtype, ws, ws_bytes, stream);
}

lora_status lora_apply_sgmv_multi(const lora_pool* p, int32_t module0, int32_t n_modules, const lora_x_run* runs,
                                  int32_t n_runs, const lora_segments* seg, float* t, int64_t ld_t,
                                  int64_t module_stride_t, void* y, int64_t ld_y, int64_t module_stride_y,
                                  lora_dtype ydtype, void* ws, size_t ws_bytes, void* stream) {
  if (!runs || n_runs < 1 || n_runs > n_modules) return LORA_ERR_ARG;
  lora_status st = expand_checks(p, module0, n_modules, t, ld_t, module_stride_t, seg, y, ld_y, module_stride_y,
                                 ydtype);
  if (st != LORA_OK) return st;
  int32_t m = module0;
  for (int32_t r = 0; r < n_runs; ++r) {   // consecutive runs covering the modules, each with its x
    if (runs[r].n_modules < 1 || m + runs[r].n_modules > module0 + n_modules) return LORA_ERR_ARG;
    st = shrink_checks(p, m, runs[r].n_modules, runs[r].x, runs[r].ld_x, runs[r].module_stride_x, seg,
                       t + static_cast<int64_t>(m - module0) * module_stride_t, ld_t, module_stride_t);
    if (st != LORA_OK) return st;
    m += runs[r].n_modules;
  }
  if (m != module0 + n_modules) return LORA_ERR_ARG;
  if (ws_bytes > 0 && (!ws || !aligned16(ws))) return LORA_ERR_ARG;
  if (seg->n_tokens == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one K split for every run (the expand adds one set of splits per module): the
  // smallest the runs choose, then as small as the workspace needs for all modules.  Two
  // bf16 runs share one shrink launch, so each aims at half the workgroups.
  const bool paired = n_runs == 2 && p->dtype == LORA_BF16;
  int32_t ks = kMaxSplits;
  m = module0;
  for (int32_t r = 0; r < n_runs; ++r) {
    ks = std::min(ks, shrink_split(p, m, runs[r].n_modules, runs[r].module_stride_x, seg, SIZE_MAX,
                                   paired ? kPairWgTarget : kShrinkWgTarget).ks);
    m += runs[r].n_modules;
  }
  while (ks > 1 && split_ws_bytes(p, seg->n_tokens, n_modules, ks) > ws_bytes) --ks;
  const int32_t h_in = static_cast<int32_t>(p->h_in[module0]);
  const int32_t kps = ((h_in + ks - 1) / ks + 31) / 32 * 32;
  const ShrinkSplit sp{(h_in + kps - 1) / kps, kps};
  // partial tiles exist only where the shrink splits K, on its matrix-core tiles
  const bool fold = sp.ks > 1 && shrink_has_tiles(p, module0, seg);
  if (paired) {   // q,k,v beside o: one launch for both runs when it fits
    const int32_t n0 = runs[0].n_modules;
    const ShrinkPlan p0 = plan_shrink<__bf16>(p, module0, n0, runs[0].x, runs[0].ld_x, runs[0].module_stride_x, seg,
                                              t, ld_t, module_stride_t, sp, ws, fold, 0, n_modules);
    const ShrinkPlan p1 = plan_shrink<__bf16>(p, module0 + n0, runs[1].n_modules, runs[1].x, runs[1].ld_x,
                                              runs[1].module_stride_x, seg, t + static_cast<int64_t>(n0) * module_stride_t,
                                              ld_t, module_stride_t, sp, ws, fold, n0, n_modules);
    if (launch_shrink_pair(p0, n0, p1, runs[1].n_modules, s, p->device, &st)) {
      if (st != LORA_OK) return st;
      return expand_call(p, module0, n_modules, t, ld_t, module_stride_t, seg, y, ld_y, module_stride_y, ydtype, s,
                         fold ? static_cast<const float*>(ws) : nullptr, sp.ks);
    }
  }
  m = module0;
  for (int32_t r = 0; r < n_runs; ++r) {
    st = shrink_call(p, m, runs[r].n_modules, runs[r].x, runs[r].ld_x, runs[r].module_stride_x, seg,
                     t + static_cast<int64_t>(m - module0) * module_stride_t, ld_t, module_stride_t, sp, ws, s, fold,
                     m - module0, n_modules);
    if (st != LORA_OK) return st;
    m += runs[r].n_modules;
  }
  return expand_call(p, module0, n_modules, t, ld_t, module_stride_t, seg, y, ld_y, module_stride_y, ydtype, s,
                     fold ? static_cast<const float*>(ws) : nullptr, sp.ks);
}

lora_status lora_apply_bgmv(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                            int64_t module_stride_x, const lora_segments* seg, void* y, int64_t ld_y,
                            int64_t module_stride_y, lora_dtype ydtype, void* stream) {
  lora_status st = check_call(p, module0, n_modules, seg, true);
  if (st != LORA_OK) return st;
  if (ydtype != LORA_F32 && ydtype != LORA_BF16) return LORA_ERR_DTYPE;
  const int32_t n = seg->n_tokens;
  st = check_operand(x, ld_x, module_stride_x, p->h_in[module0], p->elem_bytes(), n, n_modules, false, true);
  if (st != LORA_OK) return st;
  st = check_operand(y, ld_y, module_stride_y, p->h_out[module0], ydtype == LORA_BF16 ? 2 : 4, n, n_modules, true,
                     true);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == LORA_BF16) {
    if (ydtype == LORA_BF16)
      return launch_bgmv<__bf16, __bf16>(p, module0, n_modules, x, ld_x, module_stride_x, seg, y, ld_y,
                                         module_stride_y, s);
    return launch_bgmv<__bf16, float>(p, module0, n_modules, x, ld_x, module_stride_x, seg, y, ld_y,
                                      module_stride_y, s);
  }
  if (ydtype == LORA_BF16)
    return launch_bgmv<float, __bf16>(p, module0, n_modules, x, ld_x, module_stride_x, seg, y, ld_y,
                                      module_stride_y, s);
  return launch_bgmv<float, float>(p, module0, n_modules, x, ld_x, module_stride_x, seg, y, ld_y, module_stride_y,
                                   s);
}

lora_status lora_apply_bgmv_ids(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x, int64_t ld_x,
                                int64_t module_stride_x, const int32_t* ids, int32_t n_tokens, void* y, int64_t ld_y,
                                int64_t module_stride_y, lora_dtype ydtype, void* stream) {
  lora_status st = check_modules(p, module0, n_modules, true);
  if (st != LORA_OK) return st;
  if (n_tokens < 0) return LORA_ERR_ARG;
  if (n_tokens > LORA_IDS_MAX_TOKENS) return LORA_ERR_SHAPE;
  if (ydtype != LORA_F32 && ydtype != LORA_BF16) return LORA_ERR_DTYPE;
  st = check_operand(x, ld_x, module_stride_x, p->h_in[module0], p->elem_bytes(), n_tokens, n_modules, false, true);
  if (st != LORA_OK) return st;
  st = check_operand(y, ld_y, module_stride_y, p->h_out[module0], ydtype == LORA_BF16 ? 2 : 4, n_tokens, n_modules,
                     true, true);
  if (st != LORA_OK) return st;
  if (n_tokens == 0) return LORA_OK;
  if (!ids) return LORA_ERR_ARG;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == LORA_BF16) {
    if (ydtype == LORA_BF16)
      return launch_bgmv_ids<__bf16, __bf16>(p, module0, n_modules, x, ld_x, module_stride_x, ids, n_tokens, y, ld_y,
                                             module_stride_y, s);
    return launch_bgmv_ids<__bf16, float>(p, module0, n_modules, x, ld_x, module_stride_x, ids, n_tokens, y, ld_y,
                                          module_stride_y, s);
  }
  if (ydtype == LORA_BF16)
    return launch_bgmv_ids<float, __bf16>(p, module0, n_modules, x, ld_x, module_stride_x, ids, n_tokens, y, ld_y,
                                          module_stride_y, s);
  return launch_bgmv_ids<float, float>(p, module0, n_modules, x, ld_x, module_stride_x, ids, n_tokens, y, ld_y,
                                       module_stride_y, s);
}

lora_status lora_apply_bgmv_packed(const lora_pool* p, int32_t module0, int32_t n_modules, const void* x,
                                   int64_t ld_x, const lora_segments* seg, void* y, int64_t ld_y,
                                   int64_t module_stride_y, lora_dtype ydtype, void* stream) {
  lora_status st = check_call(p, module0, n_modules, seg, true);
  if (st != LORA_OK) return st;
  if (ydtype != LORA_F32 && ydtype != LORA_BF16) return LORA_ERR_DTYPE;
  if (!packable(p, module0, n_modules)) return LORA_ERR_SHAPE;
  const int32_t n = seg->n_tokens;
  st = check_operand(x, ld_x, 0, p->h_in[module0], p->elem_bytes(), n, n_modules, false, true);
  if (st != LORA_OK) return st;
  st = check_operand(y, ld_y, module_stride_y, p->h_out[module0], ydtype == LORA_BF16 ? 2 : 4, n, n_modules, true,
                     true);
  if (st != LORA_OK) return st;
  if (n == 0) return LORA_OK;
  DeviceGuard g(p->device);
  if (!g.ok) return LORA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == LORA_BF16) {
    if (ydtype == LORA_BF16)
      return launch_bgmv<__bf16, __bf16>(p, module0, n_modules, x, ld_x, 0, seg, y, ld_y, module_stride_y, s, true);
    return launch_bgmv<__bf16, float>(p, module0, n_modules, x, ld_x, 0, seg, y, ld_y, module_stride_y, s, true);
  }
  if (ydtype == LORA_BF16)
    return launch_bgmv<float, __bf16>(p, module0, n_modules, x, ld_x, 0, seg, y, ld_y, module_stride_y, s, true);
  return launch_bgmv<float, float>(p, module0, n_modules, x, ld_x, 0, seg, y, ld_y, module_stride_y, s, true);
}

lora_status lora_fused_gemm(const lora_pool* p, int32_t module, const void* x, int64_t ld_x, const void* w,
                            int64_t ld_w, const int32_t* ids, int32_t n_tokens, void* y, int64_t ld_y,
                            void* stream) {
  if (!w) return LORA_ERR_ARG;
  if (!aligned16(w) || (ld_w * 2) % 16 != 0) return LORA_ERR_ARG;
  return fused_call(p, module, x, ld_x, w, nullptr, ld_w, nullptr, ids, n_tokens, y, ld_y, stream);
}

lora_status lora_fused_gemm_fp8w(const lora_pool* p, int32_t module, const void* x, int64_t ld_x, const void* w8,
                                 int64_t ld_w, const float* w_scale, const int32_t* ids, int32_t n_tokens, void* y,
                                 int64_t ld_y, void* stream) {
  if (!w8 || !w_scale) return LORA_ERR_ARG;
  if (!aligned16(w8) || ld_w % 16 != 0 || !aligned16(w_scale)) return LORA_ERR_ARG;
  return fused_call(p, module, x, ld_x, nullptr, static_cast<const uint8_t*>(w8), ld_w, w_scale, ids, n_tokens, y,
                    ld_y, stream);
}

}  // extern "C"
