// Segment builder: groups a batch's tokens by adapter slot on the GPU.
//
// The Fastino article's batching kernel and the SGMV of the "Multi-LoRA
// Serving - S-LoRA/Punica Batching" study page (section "The kernel trick:
// gather, do not merge") both work on runs of tokens that use one adapter.
// This file builds those runs: a stable counting sort of token indices by
// slot, plus the offsets and work lists the apply kernels read.
//
// Building blocks (per wave of 64 lanes, one 64-token batch at a time):
//   match   lanes holding the same id find each other: one ballot when the
//           batch holds a single id (prefill, encoder), else one ballot per
//           id bit.  A token's rank among equal ids of its batch is the
//           count of matching lanes below it.
//   count   LDS atomics into a histogram row (one add for a single-id batch).
//   rows    each scanning wave owns a contiguous range of tokens and counts
//           into its own LDS histogram row; rows in wave order, ranges in
//           token order and ranks in lane order make the sort stable.
//   layout  per slot: total, then one block-wide scan of five counters
//           (tokens, segments, GEMV units of short and of long segments,
//           matrix-core tiles) in slot order gives every offset.
//
// Two schedules, chosen by the host from the tokens per histogram row:
//   one workgroup   count rows -> layout -> scatter, one launch; the ids of a
//                   wave's range stay in registers between count and scatter.
//   chunked         k_seg_count (grid: per-chunk slot counts) -> k_seg_scan
//                   (one workgroup: per-slot prefix over chunks into chunk
//                   offsets, layout) ->
//                   k_seg_scatter (grid: rows and scatter inside each chunk,
//                   from the chunk's offsets).  Spreads the matching of large
//                   batches over the whole chip.
// All counts stay on the device: no host synchronization.
#include "common.hpp"
#include "segments_wave.hpp"

using namespace lora;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsWords = 16384;      // 64 KiB: histogram rows (+ one row of totals)
constexpr int kIdBatch = 4;           // 64-token batches a wave loads at once (a small unroll keeps the
                                      // kernel short: it runs cold in one CU's instruction cache)
constexpr int kRound = 64 * kIdBatch; // tokens a wave loads at once
constexpr int kChunkTokens = 1024;    // chunked schedule: tokens per workgroup (minimum)
constexpr int kChunkWords = 1 << 19;  // chunked schedule: bound on chunks * n_slots
constexpr int kMaxChunks = 256;       // chunked schedule: bound on chunks (the scan walks them per slot)
#ifndef LORA_SEG_ONE_PER_ROW
#define LORA_SEG_ONE_PER_ROW 512
#endif
// Batches of up to this many tokens per histogram row use one workgroup.
constexpr int kOneGroupPerRow = LORA_SEG_ONE_PER_ROW;

int rows_of(int n_slots) {
  const int v = kLdsWords / n_slots - 1;
  return v > kWaves ? kWaves : v;
}

#ifndef LORA_SEG_WAVE_TOKENS
#define LORA_SEG_WAVE_TOKENS 512
#endif
#ifndef LORA_SEG_QUAD_TOKENS
#define LORA_SEG_QUAD_TOKENS 2048
#endif
// Threads of the one-workgroup schedule: one wave, four, or sixteen, as the
// batch grows (slots per thread stay at most 4 in the smaller two).
int one_group_threads(int n, int n_slots) {
  if (n <= LORA_SEG_WAVE_TOKENS && n_slots <= 4 * 64) return 64;
  if (n <= LORA_SEG_QUAD_TOKENS && n_slots <= 4 * 256) return 256;
  return kThreads;
}

// Chunked schedule: tokens per chunk (a multiple of 64) and number of chunks;
// 0 chunks means the one-workgroup schedule.
int chunk_tokens_of(int n, int n_slots) {
  if (static_cast<int64_t>(n) <= static_cast<int64_t>(kOneGroupPerRow) * rows_of(n_slots)) return 0;
  int gmax = kChunkWords / n_slots;
  if (gmax > kMaxChunks) gmax = kMaxChunks;
  if (gmax < 1) gmax = 1;
  int c = (n + gmax - 1) / gmax;
  if (c < kChunkTokens) c = kChunkTokens;
  return (c + 63) / 64 * 64;
}
int chunks_of(int n, int n_slots) {
  const int c = chunk_tokens_of(n, n_slots);
  return c ? (n + c - 1) / c : 0;
}
size_t work_words_of(int n, int n_slots) {
  const size_t g = static_cast<size_t>(chunks_of(n, n_slots));
  return g ? 2 * g * n_slots + n_slots + g : 0;   // chunk counts, chunk offsets, slot bases, bad ids
}

// Ids of tokens [base, base + kRound) clamped to end - 1 (base < end): every
// load is unconditional so all are in flight at once; callers mask t >= end.
__device__ __forceinline__ void load_ids(const int32_t* __restrict__ ids, int base, int end, int lane,
                                         int (&idv)[kIdBatch]) {
#pragma unroll
  for (int i = 0; i < kIdBatch; ++i) idv[i] = ids[min(base + i * 64 + lane, end - 1)];
}

// Counts one round of tokens into the LDS histogram `row`: one add when the
// batch holds a single id, else one LDS atomic per token (counting needs no
// ranks).  Returns this lane's count of ids outside [-1, n_slots).
__device__ __forceinline__ int count_round(const int (&idv)[kIdBatch], int base, int end, int lane,
                                           int n_slots, int32_t* row) {
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kIdBatch; ++i) {
    const int t = base + i * 64 + lane;
    const int id = idv[i];
    const bool in = t < end;
    const bool valid = in && id >= 0 && id < n_slots;
    bad += (in && (id < -1 || id >= n_slots)) ? 1 : 0;
    const uint64_t vm = __ballot(valid);
    const int first = __builtin_amdgcn_readfirstlane(id);
    if (__ballot(valid && id == first) == vm) {
      if (valid && lowest_lane(vm) == lane) atomicAdd(&row[id], __popcll(vm));
    } else if (valid) {
      atomicAdd(&row[id], 1);
    }
  }
  return bad;
}

// Scatters one round: a token goes to its row's cursor for its slot plus its
// rank among the equal ids below it in the batch.
__device__ __forceinline__ void scatter_round(const int (&idv)[kIdBatch], int base, int end, int lane,
                                              int n_slots, int nbits, int32_t* row, int32_t* __restrict__ perm) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int i = 0; i < kIdBatch; ++i) {
    const int t = base + i * 64 + lane;
    const int id = idv[i];
    const bool valid = t < end && id >= 0 && id < n_slots;
    const uint64_t peers = peers_of(id, valid, nbits);
    if (valid) perm[row[id] + __popcll(peers & below)] = t;
    if (valid && lowest_lane(peers) == lane) row[id] += __popcll(peers);
  }
}

// Block sum of a per-thread count; `cell` is an LDS word zeroed before a
// barrier that precedes this call.  Result valid after the next barrier.
__device__ __forceinline__ void block_add(int v, int lane, int* cell) {
  const int w = lane63(wave_scan<false>(v));
  if (lane == 0 && w) atomicAdd(cell, w);
}

// Batches of up to 64 tokens: one wave, one token per lane (segments_of_wave).
__global__ __launch_bounds__(64) void k_segments_tiny(const int32_t* __restrict__ ids, int32_t n_tokens,
                                                      int32_t n_slots, int32_t nbits, SegOut o) {
  __shared__ uint32_t table[64];
  segments_of_wave(ids, n_tokens, n_slots, nbits, o, table);
}

// Long segments whose unit and tile records the whole workgroup writes
// together; a batch with more falls back to each owning wave writing its own.
constexpr int kLongDesc = 512;

template <int W>
struct LayoutLds {
  int wsum[W][7];   // per wave: inclusive counter totals, max segment length
  int woff[W][6];   // per wave: exclusive offsets
  int tot[6];
  // long segment d: slot, length, first position, first unit (after the short
  // units) and first tile; ld_u0 / ld_t0 end with the totals
  int ld_slot[kLongDesc], ld_run[kLongDesc], ld_first[kLongDesc];
  int ld_u0[kLongDesc + 1], ld_t0[kLongDesc + 1];
};

// Largest d < n with a[d] <= v, for a strictly increasing a with a[0] <= v.
__device__ __forceinline__ int last_at_most(const int* a, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Block-wide layout (a workgroup of TH threads) from the per-slot totals
// `total` (LDS).  Thread tid owns slots [s0, s1) (consecutive, in slot order,
// the same partition the caller used to fill `total`).  Writes meta,
// seg_start/seg_slot and both work lists and calls base_of(s, first position
// in perm) for each slot that has tokens.
template <int TH, class BaseFn>
__device__ void layout_segments(const int32_t* total, int n_tokens, int n_slots, int s0, int s1, int bpt,
                                int bad_total, const SegOut& o, LayoutLds<TH / 64>& L, BaseFn base_of) {
  constexpr int W = TH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int own[6] = {0, 0, 0, 0, 0, 0};   // tokens, segments, short units, long units, tiles, long segments
  int mx = 0;
  for (int s = s0; s < s1; ++s) {
    const int run = total[s];
    if (run > 0) {
      const int nu = (run + kUnitTokens - 1) / kUnitTokens;
      own[0] += run;
      own[1] += 1;
      if (run >= kLongMin) {
        own[3] += nu;
        own[4] += (run + kTileTokens - 1) / kTileTokens;
        own[5] += 1;
      } else {
        own[2] += nu;
      }
      mx = max(mx, run);
    }
  }
  int incl[6];
#pragma unroll
  for (int q = 0; q < 6; ++q) incl[q] = wave_scan<false>(own[q]);
  const int wmx = lane63(wave_scan<true>(mx));
  if (W > 1 && lane == 63) {
#pragma unroll
    for (int q = 0; q < 6; ++q) L.wsum[wave][q] = incl[q];
    L.wsum[wave][6] = wmx;
  }
  if constexpr (W > 1) __syncthreads();
  if (wave == 0) {
    int tq[6], m;
    if constexpr (W == 1) {   // one wave: its totals are the workgroup's, its offsets 0
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        tq[q] = lane63(incl[q]);
        if (lane == 0) L.woff[0][q] = 0;
      }
      m = wmx;
    } else {
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        const int v = lane < W ? L.wsum[lane][q] : 0;
        const int c = wave_scan<false>(v);
        if (lane < W) L.woff[lane][q] = c - v;
        tq[q] = lane63(c);
      }
      m = lane63(wave_scan<true>(lane < W ? L.wsum[lane][6] : 0));
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < 6; ++q) L.tot[q] = tq[q];
      L.ld_u0[min(tq[5], kLongDesc)] = tq[3];
      L.ld_t0[min(tq[5], kLongDesc)] = tq[4];
      int32_t* meta = o.meta;
      meta[LORA_META_N_SEG] = tq[1];
      meta[LORA_META_N_ACTIVE] = tq[0];
      meta[LORA_META_MAX_SEG_LEN] = m;
      meta[LORA_META_N_BAD] = bad_total;
      meta[LORA_META_N_UNITS_SHORT] = tq[2];
      meta[LORA_META_N_UNITS_ALL] = tq[2] + tq[3];
      meta[LORA_META_N_TILES] = tq[4];
      meta[LORA_META_UNIT_TOKENS] = kUnitTokens;
      meta[LORA_META_TILE_TOKENS] = kTileTokens;
      meta[LORA_META_LONG_MIN] = kLongMin;
      meta[LORA_META_N_TOKENS] = n_tokens;
      meta[LORA_META_N_SLOTS] = n_slots;
      o.seg_start[tq[1]] = tq[0];
    }
    for (int q = 12 + lane; q < LORA_META_WORDS; q += 64) o.meta[q] = 0;   // reserved words
  }
  __syncthreads();

  int off[6];
#pragma unroll
  for (int q = 0; q < 6; ++q) off[q] = L.woff[wave][q] + incl[q] - own[q];
  const int long_at = L.tot[2];   // long-segment units follow all short ones
  const int n_long = L.tot[5];
  const bool spread = n_long <= kLongDesc;   // uniform
  int2* units = reinterpret_cast<int2*>(o.units);
  int2* tiles = reinterpret_cast<int2*>(o.tiles);
  for (int b = 0; b < bpt; ++b) {
    const int s = s0 + b;
    const int run = (s < s1) ? total[s] : 0;
    const int nu = (run + kUnitTokens - 1) / kUnitTokens;
    if (run > 0) {
      o.seg_slot[off[1]] = s;
      o.seg_start[off[1]] = off[0];
      base_of(s, off[0]);
      if (run < kLongMin) {   // at most kLongMin / kUnitTokens entries: written by this lane
        for (int u = 0; u < nu; ++u) units[off[2] + u] = unit_record(s, run, u, off[0]);
      } else if (spread) {    // described here, written below by the whole workgroup
        L.ld_slot[off[5]] = s;
        L.ld_run[off[5]] = run;
        L.ld_first[off[5]] = off[0];
        L.ld_u0[off[5]] = off[3];
        L.ld_t0[off[5]] = off[4];
      }
    }
    // long segments, when too many to describe: the whole wave writes each one's entries
    uint64_t lm = spread ? 0ull : __ballot(run >= kLongMin);
    while (lm) {
      const int src = lowest_lane(lm);
      lm &= lm - 1;
      const int r = __builtin_amdgcn_readlane(run, src);
      const int slot = __builtin_amdgcn_readlane(s, src);
      const int sb = __builtin_amdgcn_readlane(off[0], src);
      const int u0 = long_at + __builtin_amdgcn_readlane(off[3], src);
      const int t0 = __builtin_amdgcn_readlane(off[4], src);
      const int lnu = (r + kUnitTokens - 1) / kUnitTokens;
      for (int u = lane; u < lnu; u += 64) units[u0 + u] = unit_record(slot, r, u, sb);
      const int ntl = (r + kTileTokens - 1) / kTileTokens;
      for (int u = lane; u < ntl; u += 64)
        tiles[t0 + u] = make_int2(slot + (min(kTileTokens, r - u * kTileTokens) << 16), sb + u * kTileTokens);
    }
    if (run > 0) {
      if (run >= kLongMin) {
        off[3] += nu;
        off[4] += (run + kTileTokens - 1) / kTileTokens;
        off[5] += 1;
      } else {
        off[2] += nu;
      }
      off[0] += run;
      off[1] += 1;
    }
  }
  // the long segments' unit and tile records, spread over the workgroup: record i
  // belongs to the last segment whose first record is at most i
  if (spread && n_long > 0) {   // uniform
    __syncthreads();
    const int n_lu = L.tot[3], n_t = L.tot[4];
    for (int i = threadIdx.x; i < n_lu; i += TH) {
      const int d = last_at_most(L.ld_u0, n_long, i);
      units[long_at + i] = unit_record(L.ld_slot[d], L.ld_run[d], i - L.ld_u0[d], L.ld_first[d]);
    }
    for (int i = threadIdx.x; i < n_t; i += TH) {
      const int d = last_at_most(L.ld_t0, n_long, i);
      const int u = i - L.ld_t0[d], r = L.ld_run[d];
      tiles[i] = make_int2(L.ld_slot[d] + (min(kTileTokens, r - u * kTileTokens) << 16),
                           L.ld_first[d] + u * kTileTokens);
    }
  }
}

// Per-slot exclusive prefix over V <= W rows plus `base`, written back into the rows.
template <int W>
__device__ __forceinline__ void rows_to_cursors(int32_t* hist, int n_slots, int V, int s, int base) {
  int c[W];
#pragma unroll
  for (int w = 0; w < W; ++w) c[w] = hist[min(w, V - 1) * n_slots + s];
  int run = base;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    if (w < V) {
      hist[w * n_slots + s] = run;
      run += c[w];
    }
  }
}
template <int W>
__device__ __forceinline__ int rows_total(const int32_t* hist, int n_slots, int V, int s) {
  int c[W];
#pragma unroll
  for (int w = 0; w < W; ++w) c[w] = hist[min(w, V - 1) * n_slots + s];
  int run = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) run += (w < V) ? c[w] : 0;
  return run;
}

// ------------------------------------------------------------ one workgroup
// TH threads (V <= TH / 64 histogram rows).  Every thread runs the layout's
// code, so a small batch takes a small workgroup: with 1024 threads the
// layout alone took about 3 us for 32 slots, all of it instruction issue.
template <int TH>
__global__ __launch_bounds__(TH) void k_segments_one(const int32_t* __restrict__ ids, int32_t n_tokens,
                                                     int32_t n_slots, int32_t V, int32_t nbits, SegOut o) {
  constexpr int W = TH / 64;
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                  // [V][n_slots]: counts, then cursors
  int32_t* total = lds + V * n_slots;   // [n_slots]
  __shared__ LayoutLds<W> L;
  __shared__ int bad_cell;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < V * n_slots; i += TH) hist[i] = 0;
  if (tid == 0) bad_cell = 0;
  __syncthreads();

  // count: wave w < V owns tokens [w*span, (w+1)*span); waves >= V own none
  const int span = ((n_tokens + V - 1) / V + 63) / 64 * 64;
  const int beg = min(n_tokens, wave * span);
  const int end = min(n_tokens, beg + span);
  int32_t* row = hist + min(wave, V - 1) * n_slots;
  int idv[kIdBatch];
  int bad = 0;
  for (int base = beg; base < end; base += kRound) {
    load_ids(ids, base, end, lane, idv);
    bad += count_round(idv, base, end, lane, n_slots, row);
  }
  block_add(bad, lane, &bad_cell);
  const int bpt = (n_slots + TH - 1) / TH;
  const int s0 = min(n_slots, tid * bpt);
  const int s1 = min(n_slots, s0 + bpt);
  __syncthreads();

  for (int s = s0; s < s1; ++s) total[s] = rows_total<W>(hist, n_slots, V, s);
  layout_segments<TH>(total, n_tokens, n_slots, s0, s1, bpt, bad_cell, o, L,
                      [&](int s, int base) { rows_to_cursors<W>(hist, n_slots, V, s, base); });
  __syncthreads();

  // scatter: same ranges, same order as the count
  const bool one_round = end - beg <= kRound;
  for (int base = beg; base < end; base += kRound) {
    if (!one_round) load_ids(ids, base, end, lane, idv);
    scatter_round(idv, base, end, lane, n_slots, nbits, row, o.perm);
  }
}

// ------------------------------------------------------------ chunked
// Per-chunk slot counts: cnt[g][s] (global), bad ids per chunk: bad[g].
__global__ __launch_bounds__(kThreads) void k_seg_count(const int32_t* __restrict__ ids, int32_t n_tokens,
                                                        int32_t n_slots, int32_t chunk, int32_t* __restrict__ cnt,
                                                        int32_t* __restrict__ bad_of) {
  extern __shared__ int32_t lds[];   // [n_slots]
  __shared__ int bad_cell;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;
  const int cb = g * chunk, ce = min(n_tokens, cb + chunk);
  for (int i = tid; i < n_slots; i += kThreads) lds[i] = 0;
  if (tid == 0) bad_cell = 0;
  __syncthreads();
  int bad = 0;
  int idv[kIdBatch];
  for (int base = cb + wave * kRound; base < ce; base += kWaves * kRound) {
    load_ids(ids, base, ce, lane, idv);
    bad += count_round(idv, base, ce, lane, n_slots, lds);
  }
  block_add(bad, lane, &bad_cell);
  __syncthreads();
  int32_t* dst = cnt + static_cast<size_t>(g) * n_slots;
  for (int s = tid; s < n_slots; s += kThreads) dst[s] = lds[s];
  if (tid == 0) bad_of[g] = bad_cell;
}

// One workgroup: per slot, the sum of the chunk counts (OFFSETS: also their
// exclusive prefix, coff[g][s] = chunk g's first position within slot s);
// then the layout (OFFSETS: with slot_base[s] = first position of slot s in
// perm).  Thread tid takes slots tid + k * kThreads (k < kBpt) and keeps 32
// counter loads in flight: the counters come from other XCDs' L2 slices, so
// each round trip is long.
template <int kBpt, bool OFFSETS>
__device__ __forceinline__ void totals_and_layout(int32_t n_tokens, int32_t n_slots, int32_t n_chunks,
                                                  const int32_t* __restrict__ cnt, int32_t* __restrict__ coff,
                                                  const int32_t* __restrict__ bad_of,
                                                  int32_t* __restrict__ slot_base, SegOut o, int32_t* total,
                                                  LayoutLds<kWaves>& L, int& bad_cell) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) bad_cell = 0;
  __syncthreads();
  int bad = 0;
  for (int g = tid; g < n_chunks; g += kThreads) bad += bad_of[g];
  block_add(bad, lane, &bad_cell);
  constexpr int kG = 32 / kBpt;
  int sl[kBpt], run[kBpt];
#pragma unroll
  for (int k = 0; k < kBpt; ++k) {
    sl[k] = min(tid + k * kThreads, n_slots - 1);
    run[k] = 0;
  }
  for (int g0 = 0; g0 < n_chunks; g0 += kG) {
    int c[kG][kBpt];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int32_t* row = cnt + static_cast<size_t>(min(g0 + j, n_chunks - 1)) * n_slots;
#pragma unroll
      for (int k = 0; k < kBpt; ++k) c[j][k] = row[sl[k]];
    }
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      if (g0 + j < n_chunks) {
        int32_t* row = OFFSETS ? coff + static_cast<size_t>(g0 + j) * n_slots : nullptr;
#pragma unroll
        for (int k = 0; k < kBpt; ++k) {
          if (OFFSETS && tid + k * kThreads < n_slots) row[tid + k * kThreads] = run[k];
          run[k] += c[j][k];
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kBpt; ++k)
    if (tid + k * kThreads < n_slots) total[tid + k * kThreads] = run[k];
  __syncthreads();
  const int bpt = (n_slots + kThreads - 1) / kThreads;
  const int s0 = min(n_slots, tid * bpt);
  const int s1 = min(n_slots, s0 + bpt);
  layout_segments<kThreads>(total, n_tokens, n_slots, s0, s1, bpt, bad_cell, o, L, [&](int s, int base) {
    if constexpr (OFFSETS) slot_base[s] = base;
  });
}

template <int kBpt>
__global__ __launch_bounds__(kThreads) void k_seg_scan(int32_t n_tokens, int32_t n_slots, int32_t n_chunks,
                                                       const int32_t* __restrict__ cnt, int32_t* __restrict__ coff,
                                                       const int32_t* __restrict__ bad_of,
                                                       int32_t* __restrict__ slot_base, SegOut o) {
  extern __shared__ int32_t total[];   // [n_slots]
  __shared__ LayoutLds<kWaves> L;
  __shared__ int bad_cell;
  totals_and_layout<kBpt, true>(n_tokens, n_slots, n_chunks, cnt, coff, bad_of, slot_base, o, total, L, bad_cell);
}

// Rows, cursors and scatter inside chunk g, starting from the chunk's offsets.
template <int kBpt>
__global__ __launch_bounds__(kThreads) void k_seg_scatter(const int32_t* __restrict__ ids, int32_t n_tokens,
                                                          int32_t n_slots, int32_t V, int32_t nbits, int32_t chunk,
                                                          const int32_t* __restrict__ cnt,
                                                          const int32_t* __restrict__ coff,
                                                          const int32_t* __restrict__ slot_base,
                                                          int32_t* __restrict__ perm) {
  extern __shared__ int32_t hist[];   // [V][n_slots]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;
  const int cb = g * chunk, ce = min(n_tokens, cb + chunk);
  for (int i = tid; i < V * n_slots; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int span = ((ce - cb + V - 1) / V + 63) / 64 * 64;
  const int beg = min(ce, cb + wave * span);
  const int end = min(ce, beg + span);
  int32_t* row = hist + min(wave, V - 1) * n_slots;
  int idv[kIdBatch];
  for (int base = beg; base < end; base += kRound) {
    load_ids(ids, base, end, lane, idv);
    count_round(idv, base, end, lane, n_slots, row);
  }
  // this chunk's count, offset and slot base of each slot, all loads at once
  const size_t gr = static_cast<size_t>(g) * n_slots;
  int cg[kBpt], base_of[kBpt];
#pragma unroll
  for (int k = 0; k < kBpt; ++k) {
    const int s = min(tid + k * kThreads, n_slots - 1);
    cg[k] = cnt[gr + s];
    base_of[k] = slot_base[s] + coff[gr + s];   // slot_base is only written for slots with tokens
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kBpt; ++k) {
    const int s = tid + k * kThreads;
    if (s < n_slots && cg[k] > 0) rows_to_cursors<kWaves>(hist, n_slots, V, s, base_of[k]);
  }
  __syncthreads();
  const bool one_round = end - beg <= kRound;
  for (int base = beg; base < end; base += kRound) {
    if (!one_round) load_ids(ids, base, end, lane, idv);
    scatter_round(idv, base, end, lane, n_slots, nbits, row, perm);
  }
}

// The chunked schedule in two launches, for at most kPlaceWords chunk
// counters: after k_seg_count, workgroup 0 sums each slot's counts and lays out
// the segments, units and tiles (as k_seg_scan, without the offsets), while
// workgroup 1 + g counts chunk g's rows, derives from the counters each slot's
// first position in perm (the exclusive prefix of the slot totals) and the
// chunk's offset within it (the counts of chunks before g), and scatters the
// chunk.  The layout is then off the scatter's critical path, and no launch
// waits for it.
constexpr int kPlaceWords = 1 << 16;
template <int kBpt>
__global__ __launch_bounds__(kThreads) void k_seg_place(const int32_t* __restrict__ ids, int32_t n_tokens,
                                                        int32_t n_slots, int32_t V, int32_t nbits, int32_t chunk,
                                                        int32_t n_chunks, const int32_t* __restrict__ cnt,
                                                        const int32_t* __restrict__ bad_of, SegOut o) {
  extern __shared__ int32_t lds[];   // chunk: rows [V][n_slots], slot bases [n_slots]; layout: totals
  __shared__ LayoutLds<kWaves> L;
  __shared__ int bad_cell;
  if (blockIdx.x == 0) {   // uniform
    totals_and_layout<kBpt, false>(n_tokens, n_slots, n_chunks, cnt, nullptr, bad_of, nullptr, o, lds, L, bad_cell);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = static_cast<int>(blockIdx.x) - 1;
  int32_t* hist = lds;
  int32_t* sbase = lds + V * n_slots;
  const int cb = g * chunk, ce = min(n_tokens, cb + chunk);
  for (int i = tid; i < V * n_slots; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int span = ((ce - cb + V - 1) / V + 63) / 64 * 64;
  const int beg = min(ce, cb + wave * span);
  const int end = min(ce, beg + span);
  int32_t* row = hist + min(wave, V - 1) * n_slots;
  int idv[kIdBatch];
  for (int base = beg; base < end; base += kRound) {
    load_ids(ids, base, end, lane, idv);
    count_round(idv, base, end, lane, n_slots, row);
  }
  // per slot: the total over all chunks, the counts of the chunks before g, and
  // chunk g's own count (32 counter loads in flight per thread)
  constexpr int kG = 32 / kBpt;
  int sl[kBpt], tot[kBpt], pre[kBpt], cg[kBpt];
#pragma unroll
  for (int k = 0; k < kBpt; ++k) {
    sl[k] = min(tid + k * kThreads, n_slots - 1);
    tot[k] = pre[k] = cg[k] = 0;
  }
  for (int g0 = 0; g0 < n_chunks; g0 += kG) {
    int c[kG][kBpt];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int32_t* crow = cnt + static_cast<size_t>(min(g0 + j, n_chunks - 1)) * n_slots;
#pragma unroll
      for (int k = 0; k < kBpt; ++k) c[j][k] = crow[sl[k]];
    }
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int gj = g0 + j;
#pragma unroll
      for (int k = 0; k < kBpt; ++k) {
        const int v = gj < n_chunks ? c[j][k] : 0;
        tot[k] += v;
        pre[k] += gj < g ? v : 0;
        cg[k] = gj == g ? v : cg[k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kBpt; ++k)
    if (tid + k * kThreads < n_slots) sbase[tid + k * kThreads] = tot[k];
  __syncthreads();
  // exclusive prefix of the slot totals, in place: thread tid takes slots s0 .. s1 - 1
  {
    const int bpt = (n_slots + kThreads - 1) / kThreads;
    const int s0 = min(n_slots, tid * bpt), s1 = min(n_slots, s0 + bpt);
    int sum = 0;
    for (int s = s0; s < s1; ++s) sum += sbase[s];
    const int incl = wave_scan<false>(sum);
    if (lane == 63) L.wsum[wave][0] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += L.wsum[w][0];
    for (int s = s0; s < s1; ++s) {
      const int v = sbase[s];
      sbase[s] = run;
      run += v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kBpt; ++k) {
    const int s = tid + k * kThreads;
    if (s < n_slots && cg[k] > 0) rows_to_cursors<kWaves>(hist, n_slots, V, s, sbase[s] + pre[k]);
  }
  __syncthreads();
  const bool one_round = end - beg <= kRound;
  for (int base = beg; base < end; base += kRound) {
    if (!one_round) load_ids(ids, base, end, lane, idv);
    scatter_round(idv, base, end, lane, n_slots, nbits, row, o.perm);
  }
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

template <class K>
bool lds_limit(K* k) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             kLdsWords * 4) == hipSuccess;
}
bool set_lds_limit() {   // gfx950 allows 160 KiB of LDS per workgroup; these use up to 64 KiB + static
  static const bool ok = lds_limit(&k_segments_one<64>) && lds_limit(&k_segments_one<256>) &&
                         lds_limit(&k_segments_one<1024>) && lds_limit(&k_seg_scatter<1>) &&
                         lds_limit(&k_seg_scatter<2>) && lds_limit(&k_seg_scatter<4>) &&
                         lds_limit(&k_seg_scatter<8>) && lds_limit(&k_seg_place<1>) &&
                         lds_limit(&k_seg_place<2>) && lds_limit(&k_seg_place<4>) && lds_limit(&k_seg_place<8>);
  return ok;
}

// Slots per thread of the chunked kernels, rounded up to 1, 2, 4 or 8.
int bpt_class(int n_slots) {
  const int bpt = (n_slots + kThreads - 1) / kThreads;
  return bpt <= 1 ? 1 : bpt <= 2 ? 2 : bpt <= 4 ? 4 : 8;
}

}  // namespace

extern "C" {

size_t lora_segments_bytes(int32_t n_tokens, int32_t n_slots) {
  if (n_tokens < 0 || n_slots < 1 || n_slots > kMaxSlots || n_tokens > (1 << 24)) return 0;
  const int32_t S = max_segs_of(n_tokens, n_slots);
  size_t b = 0;
  b += align256(static_cast<size_t>(n_tokens) * 4);                    // perm
  b += align256(static_cast<size_t>(S + 1) * 4);                       // seg_start
  b += align256(static_cast<size_t>(S > 0 ? S : 1) * 4);               // seg_slot
  b += align256(LORA_META_WORDS * 4);                                  // meta
  b += align256(static_cast<size_t>(max_units_of(n_tokens, n_slots)) * 8);  // units
  b += align256(static_cast<size_t>(max_tiles_of(n_tokens)) * 8 + 8);  // tiles
  b += align256(work_words_of(n_tokens, n_slots) * 4);                 // chunked schedule's counts
  return b;
}

lora_status lora_segments_bind(void* buf, size_t bytes, int32_t n_tokens, int32_t n_slots,
                               lora_segments* out) {
  if (!out || !buf || n_tokens < 0 || n_slots < 1 || n_slots > kMaxSlots) return LORA_ERR_ARG;
  if (n_tokens > (1 << 24)) return LORA_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(buf) % 256 != 0) return LORA_ERR_ARG;
  if (bytes < lora_segments_bytes(n_tokens, n_slots)) return LORA_ERR_WORKSPACE;
  const int32_t S = max_segs_of(n_tokens, n_slots);
  char* p = static_cast<char*>(buf);
  out->perm = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(n_tokens) * 4);
  out->seg_start = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(S + 1) * 4);
  out->seg_slot = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(S > 0 ? S : 1) * 4);
  out->meta = reinterpret_cast<int32_t*>(p);
  p += align256(LORA_META_WORDS * 4);
  out->units = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(max_units_of(n_tokens, n_slots)) * 8);
  out->tiles = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<size_t>(max_tiles_of(n_tokens)) * 8 + 8);
  out->work = work_words_of(n_tokens, n_slots) ? reinterpret_cast<int32_t*>(p) : nullptr;
  out->n_tokens = n_tokens;
  out->n_slots = n_slots;
  out->max_segs = S;
  out->max_units = max_units_of(n_tokens, n_slots);
  out->max_tiles = max_tiles_of(n_tokens);
  out->n_chunks = chunks_of(n_tokens, n_slots);
  return LORA_OK;
}

lora_status lora_build_segments(const int32_t* ids, const lora_segments* seg, void* stream) {
  if (!seg) return LORA_ERR_ARG;
  if (seg->n_tokens < 0 || seg->n_tokens > (1 << 24) || seg->n_slots < 1 || seg->n_slots > kMaxSlots)
    return LORA_ERR_ARG;
  if (seg->n_tokens == 0) return LORA_OK;
  if (!ids || !seg->perm || !seg->seg_start || !seg->seg_slot || !seg->meta || !seg->units || !seg->tiles)
    return LORA_ERR_ARG;
  const int32_t n = seg->n_tokens, n_slots = seg->n_slots;
  const int32_t G = chunks_of(n, n_slots);
  if (seg->n_chunks != G || (G > 0 && !seg->work)) return LORA_ERR_ARG;   // not laid out by lora_segments_bind
  const int32_t V = rows_of(n_slots);
  if (V < 1) return LORA_ERR_ARG;
  int32_t nbits = 0;
  while ((1 << nbits) < n_slots) ++nbits;
  if (!set_lds_limit()) return LORA_ERR_HIP;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const SegOut o{seg->perm, seg->seg_start, seg->seg_slot, seg->meta, seg->units, seg->tiles};
  if (G == 0 && n <= kWaveSegTokens) {
    hipLaunchKernelGGL(k_segments_tiny, dim3(1), dim3(64), 0, st, ids, n, n_slots, nbits, o);
  } else if (G == 0) {
    const int th = one_group_threads(n, n_slots);
    const int32_t v = std::min<int32_t>(V, th / 64);
    const size_t lds = static_cast<size_t>(v + 1) * n_slots * 4;
    if (th == 64)
      hipLaunchKernelGGL(k_segments_one<64>, dim3(1), dim3(64), lds, st, ids, n, n_slots, v, nbits, o);
    else if (th == 256)
      hipLaunchKernelGGL(k_segments_one<256>, dim3(1), dim3(256), lds, st, ids, n, n_slots, v, nbits, o);
    else
      hipLaunchKernelGGL(k_segments_one<1024>, dim3(1), dim3(1024), lds, st, ids, n, n_slots, v, nbits, o);
  } else {
    const int32_t chunk = chunk_tokens_of(n, n_slots);
    int32_t* cnt = seg->work;
    int32_t* coff = cnt + static_cast<size_t>(G) * n_slots;
    int32_t* slot_base = coff + static_cast<size_t>(G) * n_slots;
    int32_t* bad_of = slot_base + n_slots;
    const size_t row_bytes = static_cast<size_t>(n_slots) * 4;
    const size_t rows_bytes = static_cast<size_t>(V) * row_bytes;
    hipLaunchKernelGGL(k_seg_count, dim3(G), dim3(kThreads), row_bytes, st, ids, n, n_slots, chunk, cnt, bad_of);
    const bool place = static_cast<int64_t>(G) * n_slots <= kPlaceWords;
#define LORA_SEG_CHUNKED(KB)                                                                                    \
  do {                                                                                                          \
    if (place) {                                                                                                \
      hipLaunchKernelGGL(k_seg_place<KB>, dim3(G + 1), dim3(kThreads), rows_bytes + row_bytes, st, ids, n,      \
                         n_slots, V, nbits, chunk, G, cnt, bad_of, o);                                          \
    } else {                                                                                                    \
      hipLaunchKernelGGL(k_seg_scan<KB>, dim3(1), dim3(kThreads), row_bytes, st, n, n_slots, G, cnt, coff,      \
                         bad_of, slot_base, o);                                                                 \
      hipLaunchKernelGGL(k_seg_scatter<KB>, dim3(G), dim3(kThreads), rows_bytes, st, ids, n, n_slots, V, nbits, \
                         chunk, cnt, coff, slot_base, seg->perm);                                               \
    }                                                                                                           \
  } while (0)
    switch (bpt_class(n_slots)) {
      case 1: LORA_SEG_CHUNKED(1); break;
      case 2: LORA_SEG_CHUNKED(2); break;
      case 4: LORA_SEG_CHUNKED(4); break;
      default: LORA_SEG_CHUNKED(8); break;
    }
#undef LORA_SEG_CHUNKED
  }
  return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_segments_check(const lora_segments* seg, void* stream, int32_t* meta_out) {
  if (!seg || !seg->meta) return LORA_ERR_ARG;
  int32_t meta[LORA_META_WORDS] = {0};
  if (seg->n_tokens > 0) {
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return LORA_ERR_HIP;
    if (hipMemcpy(meta, seg->meta, sizeof(meta), hipMemcpyDeviceToHost) != hipSuccess) return LORA_ERR_HIP;
  } else {
    meta[LORA_META_UNIT_TOKENS] = kUnitTokens;
    meta[LORA_META_TILE_TOKENS] = kTileTokens;
    meta[LORA_META_LONG_MIN] = kLongMin;
    meta[LORA_META_N_SLOTS] = seg->n_slots;
  }
  if (meta_out)
    for (int i = 0; i < LORA_META_WORDS; ++i) meta_out[i] = meta[i];
  return meta[LORA_META_N_BAD] > 0 ? LORA_ERR_DEVICE_IDS : LORA_OK;
}

}  // extern "C"
