// GEMV (vector ALU) path: short segments and decode tokens.
//
// A work unit is up to kUnitTokens tokens of one segment, i.e. tokens that
// share one adapter (the study page's BGMV, where each decode token brings
// its own adapter, and its SGMV segments; section "The kernel trick: gather,
// do not merge").  One workgroup of kGemvThreads threads takes a unit and
// reads each gathered page of its adapter once for all its tokens.  Every
// lane issues all of its loads for a phase back to back, and a unit has few
// dependent round trips, which is what bounds a decode step made of many
// small units:
//   (1) its work-list record (slot, first token, token count) together with
//       the unit count;
//   (2) the slot table entry, every page id the entry can use (the page
//       table has a fixed layout per (slot, module), so no id waits for the
//       entry) and the token indices;
//   (3) the x rows, staged in LDS;
//   then the A batches and the B batches, each a full load of the workgroup.
//
// shrink: t[tb][j] = sum_k x[tok_tb][k] * A[j][k].  The unit's x rows are
//         staged in LDS (16-byte coalesced loads).  Wave w owns rank rows
//         w, w+W, ... (W waves); a lane takes eight 16-byte chunks of the row
//         (a wave reads 1 KiB of the row per instruction) and keeps NT
//         partial sums, folded across the wave by DPP row operations (lane
//         distance < 16) and ds_bpermute (16, 32): no LDS reduction, no float
//         atomics, a fixed summation order.
// expand: y[tok_tb][c] = round(y + scale * sum_j t[tb][j] * B[j][c]).  A
//         thread owns 4 consecutive columns (8-byte loads of bf16, 16-byte of
//         fp32), loads up to 16 rank rows of B and its y rows at once, and
//         updates y in place with one rounding per element.
#pragma once

#include "common.hpp"
#include "segments_wave.hpp"

namespace lora {

#ifndef LORA_GEMV_THREADS
#define LORA_GEMV_THREADS 256
#endif
#ifndef LORA_SHRINK_BATCH
#define LORA_SHRINK_BATCH 8
#endif
#ifndef LORA_EXPAND_BATCH
#define LORA_EXPAND_BATCH 16
#endif
#ifndef LORA_SHRINK_ROWS
#define LORA_SHRINK_ROWS 2
#endif
#ifndef LORA_UNIT_RUN
#define LORA_UNIT_RUN 8
#endif
constexpr int kGemvThreads = LORA_GEMV_THREADS;
constexpr int kBgmvMaxPack = 4;                     // modules sharing x that one fused BGMV work item takes
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kXSliceBytes = 32768;                 // LDS for the staged x rows of a unit
constexpr int kShrinkBatch = LORA_SHRINK_BATCH;     // 16-byte chunks of a row in flight per lane
constexpr int kShrinkRows = LORA_SHRINK_ROWS;       // rank rows a wave streams at once
constexpr int kUnitRun = LORA_UNIT_RUN;             // consecutive units one XCD takes (a power of 2)
constexpr int kPartRows = 8;                        // rank rows per work item of the shrink-only kernel:
                                                    // one pass of the 4 waves (2 rows each)
template <typename TI>
constexpr int kExpandBatch = sizeof(TI) == 2 ? LORA_EXPAND_BATCH : 8;   // rank rows of B in flight per thread
// The fused BGMV reads x and updates y with streaming accesses: each x row and
// each y element is touched by one work item only.
#ifndef LORA_BGMV_NT_XY
#define LORA_BGMV_NT_XY 1
#endif

template <typename TI>
struct XSlice {
  static constexpr int kElems = kXSliceBytes / (kUnitTokens * static_cast<int>(sizeof(TI)));
};

// Page of element k of a row: k / h, with h's reciprocal (exact for k*h < 2^32).
__device__ __forceinline__ int page_of(int k, uint32_t magic, int ppr) {
  return ppr == 1 ? 0 : static_cast<int>(__umulhi(static_cast<uint32_t>(k), magic));
}

// Four consecutive elements as floats / stored with one rounding.
template <typename T> struct Quad;
template <> struct Quad<__bf16> {
  uint32_t lo, hi;
  __device__ __forceinline__ void load(const __bf16* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    lo = v.x;
    hi = v.y;
  }
  __device__ __forceinline__ void load_nt(const __bf16* p) {
    const u32x2 v = ld16<LORA_NT_PAGES != 0>(reinterpret_cast<const u32x2*>(p));
    lo = v.x;
    hi = v.y;
  }
  __device__ __forceinline__ void zero() { lo = hi = 0u; }
  __device__ __forceinline__ void unpack(float (&f)[4]) const {
    f[0] = bf16lo(lo); f[1] = bf16hi(lo); f[2] = bf16lo(hi); f[3] = bf16hi(hi);
  }
  static __device__ __forceinline__ void store(__bf16* p, const float (&f)[4]) {
    __bf16 h[4] = {static_cast<__bf16>(f[0]), static_cast<__bf16>(f[1]), static_cast<__bf16>(f[2]),
                   static_cast<__bf16>(f[3])};
    *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, h);
  }
  // streaming (non-temporal) load and store, for y elements touched once
  __device__ __forceinline__ void load_stream(const __bf16* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    lo = v.x;
    hi = v.y;
  }
  static __device__ __forceinline__ void store_stream(__bf16* p, const float (&f)[4]) {
    __bf16 h[4] = {static_cast<__bf16>(f[0]), static_cast<__bf16>(f[1]), static_cast<__bf16>(f[2]),
                   static_cast<__bf16>(f[3])};
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, h), reinterpret_cast<u32x2*>(p));
  }
};
template <> struct Quad<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) { v = ld16<LORA_NT_PAGES != 0>(reinterpret_cast<const f32x4*>(p)); }
  __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void unpack(float (&f)[4]) const { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  static __device__ __forceinline__ void store(float* p, const float (&f)[4]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  }
  __device__ __forceinline__ void load_stream(const float* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  static __device__ __forceinline__ void store_stream(float* p, const float (&f)[4]) {
    __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(p));
  }
};

struct UnitLds {
  float t[kUnitTokens * kMaxRank];
  int32_t pid[kMaxEntryPages];
  int32_t toks[kUnitTokens];
};

// Copies x[tok][k0 .. k0+len) of the unit's tokens into xs[tb][0 .. len);
// stream: streaming loads (no other work item of the launch reads these rows).
// The x rows of a unit go straight from memory into LDS (global_load_lds: no
// registers, no wait between loads), so the slice lands in one round trip.
// Wave w takes the 64-chunk groups w, w + W, ... of the rows; one instruction
// moves a group (lane i lands at byte 16 i of the group's LDS base; lanes past
// the row stay idle).  The barrier after it waits for these loads.
constexpr int kCpolNt = 2;   // cache-policy bit of a non-temporal load
template <typename TI>
__device__ __forceinline__ void stage_x(const TI* __restrict__ x, int64_t ld_x, const int32_t* toks, int nt,
                                        int k0, int len, TI* xs, bool stream) {
  constexpr int V = 16 / sizeof(TI);
  constexpr int S = XSlice<TI>::kElems;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per_tok = len / V;                 // 16-byte chunks per row
  const int groups = (per_tok + 63) >> 6;      // 64-chunk groups per row
  for (int gi = wave; gi < nt * groups; gi += kGemvWaves) {   // wave-uniform
    const int tb = gi / groups, g = gi - tb * groups;
    const int c = 64 * g + lane;
    if (c < per_tok) {
      const void* src = x + static_cast<int64_t>(toks[tb]) * ld_x + k0 + c * V;
      const lds_addr_t dst = to_lds(xs + tb * S + 64 * g * V);
      if (stream) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kCpolNt);
      else __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  }
}

// KEEP: the unit's segment spans several units, whose workgroups read the
// same pages, so they are loaded through the caches; a page read by one
// unit only is streamed with non-temporal loads.
// Where the stacked rank rows of up to kBgmvMaxPack modules that share x
// start (rstart[0] = 0; a module past the pack starts past every row), and
// the page ids per module (module mi's at L.pid[mi * ids_per]).
struct Stack {
  int rstart[kBgmvMaxPack];
  int ids_per;
};

// STACK: rank rows [j_begin, j_end) are the stacked rows of the modules of st.
template <typename TI, int NT, bool KEEP, bool STACK = false>
__device__ __forceinline__ void shrink_unit(const TI* __restrict__ x, int64_t ld_x, UnitLds& L, int nt,
                                            const TI* __restrict__ pages, int pid0, int32_t h, uint32_t magic,
                                            int32_t h_in, int32_t j_begin, int32_t j_end, TI* xs, bool x_stream,
                                            const Stack& st = Stack{}) {
  constexpr int S = XSlice<TI>::kElems;
  constexpr int CE = 16 / sizeof(TI);  // elements per 16-byte chunk
  constexpr int SR = kShrinkRows;      // rank rows a wave streams at once
  constexpr int V = SR * NT;           // partial sums per lane
  constexpr int G = 64 / V;            // lanes holding the same reduced value
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ppr = h_in / h;
  (void)magic;
  const int n_slices = (h_in + S - 1) / S;

  // base address of rank rows jw + kGemvWaves*q (q < SR) in page p, one per wave
  auto row_bases = [&](int jw, int p, const TI* (&base)[SR]) {
#pragma unroll
    for (int q = 0; q < SR; ++q) {
      const int j = min(jw + kGemvWaves * q, j_end - 1);  // rows past the range repeat its last
      int slot_ix = pid0 + j * ppr + p;
      if constexpr (STACK) {   // the module whose rows hold j, and j's row in it
        int jm = j, base_ix = 0;
#pragma unroll
        for (int k = 1; k < kBgmvMaxPack; ++k)
          if (j >= st.rstart[k]) {
            jm = j - st.rstart[k];
            base_ix = k * st.ids_per;
          }
        slot_ix = base_ix + jm * ppr + p;
      }
      const int pid = __builtin_amdgcn_readfirstlane(L.pid[slot_ix]);
      base[q] = pages + (static_cast<int64_t>(pid) - p) * h;
    }
  };
  Chunk<TI> raw[SR][kShrinkBatch];
  auto load_batch = [&](const TI* (&base)[SR], int kb, int kp1) {
#pragma unroll
    for (int q = 0; q < SR; ++q)
#pragma unroll
      for (int i = 0; i < kShrinkBatch; ++i) {
        const int k = kb + (lane + 64 * i) * CE;
        if constexpr (KEEP) raw[q][i].load(base[q] + static_cast<uint32_t>(min(k, kp1 - CE)));
        else raw[q][i].load_nt(base[q] + static_cast<uint32_t>(min(k, kp1 - CE)));
      }
  };

  // acc[q*NT + tb]: this lane's partial sums of rank row jw + kGemvWaves*q, token tb
  float acc[64];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  auto compute_batch = [&](int kb, int kp1, int k0) {
#pragma unroll
    for (int i = 0; i < kShrinkBatch; ++i) {
      const int k = kb + (lane + 64 * i) * CE;
      if (k < kp1) {
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
          if (tb < nt) {
            float xv[CE];
            Chunk<TI> xc;
            xc.load(xs + tb * S + (k - k0));
            xc.unpack(xv);
#pragma unroll
            for (int q = 0; q < SR; ++q) {
              float av[CE];
              raw[q][i].unpack(av);
#pragma unroll
              for (int e = 0; e < CE; ++e) acc[q * NT + tb] = fmaf(av[e], xv[e], acc[q * NT + tb]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the x reads of later chunks from piling up
    }
  };

  if (n_slices == 1) {
    stage_x<TI>(x, ld_x, L.toks, nt, 0, h_in, xs, x_stream);
    __syncthreads();
  }
  // wave w streams rows j0 + w + kGemvWaves*q for q < SR, rank rows [j_begin, j_end)
  for (int j0 = j_begin; j0 < j_end; j0 += kGemvWaves * SR) {
    const int jw = j0 + wave;
    for (int sl = 0; sl < n_slices; ++sl) {
      const int k0 = sl * S;
      const int len = min(S, h_in - k0);
      if (n_slices > 1) {
        __syncthreads();
        stage_x<TI>(x, ld_x, L.toks, nt, k0, len, xs, x_stream);
        __syncthreads();
      }
      if (jw >= j_end) continue;         // wave-uniform
      // pages of the rows that overlap [k0, k0+len): one base address per row for the whole wave
      for (int p = k0 / h; p * h < k0 + len; ++p) {
        const int kp0 = max(k0, p * h), kp1 = min(k0 + len, (p + 1) * h);
        const TI* base[SR];
        row_bases(jw, p, base);
        for (int kb = kp0; kb < kp1; kb += 64 * CE * kShrinkBatch) {
          load_batch(base, kb, kp1);
          compute_batch(kb, kp1, k0);
        }
      }
    }
    if (jw < j_end) {
      const float r = wave_transpose_reduce<V>(acc, lane);
      const int idx = lane / G;
      const int q = idx / NT, tb = idx - q * NT;
      const int j = jw + kGemvWaves * q;
      if ((lane % G) == 0 && j < j_end && tb < nt) L.t[tb * kMaxRank + j] = r;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
  }
  __syncthreads();
}

// NTY: y is read and written with streaming accesses (each element is touched
// by this work item only).
// STACKED: the unit's t columns of this adapter start at toff and the next
// columns belong to another module, so rows past the rank are masked.
template <typename TI, typename TO, int NT, bool KEEP, bool NTY, bool STACKED = false>
__device__ __forceinline__ void expand_unit(TO* __restrict__ y, int64_t ld_y, const UnitLds& L, int nt,
                                            const TI* __restrict__ pages, int pid0, int32_t h, uint32_t magic,
                                            int32_t h_out, int32_t rank, float scale, int q_begin, int q_end,
                                            int toff = 0) {
  constexpr int EB = kExpandBatch<TI>; // rank rows of B in flight
  const int n_quads = h_out >> 2;
  const int ppr = h_out / h;
  int64_t yoff[NT];
#pragma unroll
  for (int tb = 0; tb < NT; ++tb) yoff[tb] = static_cast<int64_t>(L.toks[tb < nt ? tb : 0]) * ld_y;

  // A wave covers 256 consecutive columns; when the page size is a multiple
  // of 256 they lie in one page, so each rank row has one base address for
  // the wave and every load needs one 32-bit lane offset.
  const bool wave_page = (h % 256) == 0;
  (void)n_quads;
  for (int c0 = q_begin + threadIdx.x; c0 < q_end; c0 += kGemvThreads) {
    const int kq = c0 << 2;
    int p = page_of(kq, magic, ppr);
    if (wave_page) p = __builtin_amdgcn_readfirstlane(p);
    const int off = kq - p * h;
    Quad<TO> yq[NT];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      if constexpr (NTY) yq[tb].load_stream(y + yoff[tb] + kq);
      else yq[tb].load(y + yoff[tb] + kq);
    }
    float acc[NT][4];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tb][e] = 0.f;
    for (int j0 = 0; j0 < rank; j0 += EB) {
      Quad<TI> raw[EB];
#pragma unroll
      for (int jj = 0; jj < EB; ++jj) {
        const int j = min(j0 + jj, rank - 1);    // rows past the rank repeat the last (their t is 0)
        int pid = L.pid[pid0 + j * ppr + p];
        if (wave_page) pid = __builtin_amdgcn_readfirstlane(pid);
        if constexpr (KEEP) raw[jj].load(pages + static_cast<int64_t>(pid) * h + static_cast<uint32_t>(off));
        else raw[jj].load_nt(pages + static_cast<int64_t>(pid) * h + static_cast<uint32_t>(off));
      }
#pragma unroll
      for (int jj = 0; jj < EB; ++jj) {
        float bv[4];
        raw[jj].unpack(bv);
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
          // t is the same for the whole workgroup: keep it in a scalar register (rows past
          // the rank read zeros, except in a stacked block, where they are masked)
          float tv = __builtin_bit_cast(
              float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, L.t[tb * kMaxRank + toff + j0 + jj])));
          if constexpr (STACKED) tv = j0 + jj < rank ? tv : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tb][e] = fmaf(tv, bv[e], acc[tb][e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      if (tb < nt) {
        float yv[4];
        yq[tb].unpack(yv);
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[e] = fmaf(scale, acc[tb][e], yv[e]);
        if constexpr (NTY) Quad<TO>::store_stream(y + yoff[tb] + kq, yv);
        else Quad<TO>::store(y + yoff[tb] + kq, yv);
      }
    }
  }
}

// Loads a unit's tokens and every page id its entry can hold into LDS and
// clears its t rows.  The page table has a fixed layout per (slot, module):
// A's ids from `ids` (rank row j, page p at j*ppr_a + p), B's from
// ids + max_rank*ppr_a; none of these loads waits for the entry.  Begins and
// ends with a barrier.
__device__ __forceinline__ void unit_prologue(const SegView& sv, const int32_t* __restrict__ ids, int pos, int nt,
                                              int n_ids, UnitLds& L) {
  __syncthreads();   // the previous unit is done with LDS
  const int tid = threadIdx.x;
  if (tid < kUnitTokens) L.toks[tid] = tid < nt ? sv.perm[pos + tid] : 0;
  for (int i = tid; i < n_ids; i += kGemvThreads) L.pid[i] = ids[i];
  for (int i = tid; i < kUnitTokens * kMaxRank; i += kGemvThreads) L.t[i] = 0.f;
  __syncthreads();
}

// Unit of workgroup bx of module m (see item_of_block): runs of kUnitRun units per XCD.
__device__ __forceinline__ int unit_of_block(int bx, int m) { return item_of_block<kUnitRun>(bx, m); }

struct GemvArgs {
  PoolView pv;
  SegView sv;
  int32_t module0;
  int32_t units_word;   // meta word holding the unit count to process
  int32_t parts;        // work items per unit: rank-row blocks (MODE 1) or column ranges (MODE 0, 2; in
                        // MODE 0 each range's item runs the whole shrink)
  int32_t h_in, h_out;
  uint32_t magic;       // reciprocal of the page size
  const void* x;
  int64_t ld_x, msx;
  float* t;
  int64_t ld_t, mst;
  void* y;
  int64_t ld_y, msy;
  int32_t module_group;   // modules per dispatch group of the GEMV grid (0: one module after another)
  int32_t group_nx;       // ... and each module's unit workgroups
  int32_t pack;           // fused BGMV: modules sharing x that one work item takes (1: none); the
                          // grid's module coordinate then counts packs
  int32_t x_stream;       // fused BGMV: no two work items read the same x rows (stream them)
};

// LDS of the GEMV body: the unit's tables, then (shrink modes) its staged x rows.
template <int MODE, typename TI>
constexpr size_t gemv_xs_offset() { return (sizeof(UnitLds) + 15) / 16 * 16; }
template <int MODE, typename TI>
constexpr size_t gemv_lds_bytes() {
  return gemv_xs_offset<MODE, TI>() + ((MODE == 2) ? 16 : kUnitTokens * XSlice<TI>::kElems * sizeof(TI));
}

// One work item of the GEMV path: unit `rec` (see the segment builder's unit
// records) of module m, part `part` of it.  MODE 0: fused BGMV (t kept in
// LDS); 1: shrink only (t to memory, part = block of kPartRows rank rows); 2:
// expand only (t from memory, part = column range of `parts`).  Begins with a
// barrier (the previous item is done with LDS).
template <int MODE, typename TI, typename TO>
__device__ __forceinline__ void gemv_item(const GemvArgs& a, int m, int2 rec, int part, UnitLds& L, TI* xs) {
  const TI* xm = static_cast<const TI*>(a.x) + m * a.msx;
  float* tm = a.t + m * a.mst;
  TO* ym = static_cast<TO*>(a.y) + m * a.msy;
  const TI* pages = static_cast<const TI*>(a.pv.pages);
  const int32_t h = static_cast<int32_t>(a.pv.page_elems);
  const int ppr_a = a.h_in / h, ppr_b = a.h_out / h;
  const int ids_a = (MODE == 2) ? 0 : a.pv.max_rank * ppr_a;   // page ids loaded for A
  const int ids_b = (MODE == 1) ? 0 : a.pv.max_rank * ppr_b;   // ... and for B, after A's
  const int slot = rec.x & 0xffff, nt = (rec.x >> 16) & 0xff, pos = rec.y;
  // pages several work items read (a segment of several units, or a unit split into
  // column ranges) go through the caches; the others are streamed
  const bool keep = ((rec.x >> 24) & 1) || (MODE == 0 && a.parts > 1);
  const int ei = slot * a.pv.n_modules + a.module0 + m;
  const SlotEntry e = a.pv.entries[ei];
  const int32_t* ids = a.pv.page_ids + static_cast<int64_t>(ei) * a.pv.ppe;
  unit_prologue(a.sv, (MODE == 2) ? ids + a.pv.max_rank * ppr_a : ids, pos, nt, ids_a + ids_b, L);
  if (e.rank <= 0) return;
  // rank rows of this part (shrink-only kernel) or all of them
  const int j_begin = (MODE == 1) ? part * kPartRows : 0;
  const int j_end = (MODE == 1) ? min(e.rank, j_begin + kPartRows) : e.rank;
  if (j_begin >= j_end) return;         // uniform: this part has no rows of this rank
  if constexpr (MODE != 2) {
    const bool x_stream = MODE == 0 && LORA_BGMV_NT_XY != 0 && a.x_stream != 0;
#define LORA_SHRINK_CALL(N, K) \
  shrink_unit<TI, N, K>(xm, a.ld_x, L, nt, pages, 0, h, a.magic, a.h_in, j_begin, j_end, xs, x_stream)
    if (keep) {
      if (nt == 1) LORA_SHRINK_CALL(1, true);
      else if (nt == 2) LORA_SHRINK_CALL(2, true);
      else LORA_SHRINK_CALL(4, true);
    } else {
      if (nt == 1) LORA_SHRINK_CALL(1, false);
      else if (nt == 2) LORA_SHRINK_CALL(2, false);
      else LORA_SHRINK_CALL(4, false);
    }
#undef LORA_SHRINK_CALL
  }
  if constexpr (MODE == 1) {
    const int nr = j_end - j_begin;
    for (int i = threadIdx.x; i < nt * nr; i += kGemvThreads) {
      const int tb = i / nr, j = j_begin + (i - tb * nr);
      tm[static_cast<int64_t>(L.toks[tb]) * a.ld_t + j] = L.t[tb * kMaxRank + j];
    }
  }
  if constexpr (MODE == 2) {
    for (int i = threadIdx.x; i < nt * e.rank; i += kGemvThreads) {
      const int tb = i / e.rank, j = i - tb * e.rank;
      L.t[tb * kMaxRank + j] = tm[static_cast<int64_t>(L.toks[tb]) * a.ld_t + j];
    }
    __syncthreads();
  }
  if constexpr (MODE != 1) {
    // column quads of this part: ranges of whole waves (64 quads), the last one ragged
    const int n_quads = a.h_out >> 2;
    const int per = ((n_quads + a.parts - 1) / a.parts + 63) / 64 * 64;
    const int q_begin = part * per;
    const int q_end = min(n_quads, q_begin + per);
    if (q_begin >= q_end) return;       // uniform
    constexpr bool nty = MODE == 0 && LORA_BGMV_NT_XY != 0;
#define LORA_EXPAND_CALL(N, K)                                                                               \
  expand_unit<TI, TO, N, K, nty>(ym, a.ld_y, L, nt, pages, ids_a, h, a.magic, a.h_out, e.rank, e.scale, q_begin, \
                                 q_end)
    if (keep) {
      if (nt == 1) LORA_EXPAND_CALL(1, true);
      else if (nt == 2) LORA_EXPAND_CALL(2, true);
      else LORA_EXPAND_CALL(4, true);
    } else {
      if (nt == 1) LORA_EXPAND_CALL(1, false);
      else if (nt == 2) LORA_EXPAND_CALL(2, false);
      else LORA_EXPAND_CALL(4, false);
    }
#undef LORA_EXPAND_CALL
  }
}

// Fused BGMV work item for a pack of np = a.pack modules that share x (q, k, v
// of one layer: the slide deck "Thousands of adapters", slide 5, adapts the
// attention projections): unit `rec` of modules g*np .. g*np + np - 1.  The
// x rows are staged once; the modules' rank rows are shrunk as one stacked
// block of sum(rank) rows; then each module's y is expanded from its own t
// columns.  Per module, the rank rows keep the wave and batch they have in a
// one-module item when every rank is a multiple of 8.
template <typename TI, typename TO>
__device__ __forceinline__ void gemv_item_packed(const GemvArgs& a, int g, int2 rec, UnitLds& L, TI* xs) {
  const int np = a.pack;
  const int m0 = g * np;
  const TI* xm = static_cast<const TI*>(a.x) + m0 * a.msx;
  const TI* pages = static_cast<const TI*>(a.pv.pages);
  const int32_t h = static_cast<int32_t>(a.pv.page_elems);
  const int ppr_a = a.h_in / h, ppr_b = a.h_out / h;
  const int ids_a = a.pv.max_rank * ppr_a;
  const int ids_per = ids_a + a.pv.max_rank * ppr_b;   // page ids of one module's entry
  const int slot = rec.x & 0xffff, nt = (rec.x >> 16) & 0xff, pos = rec.y;
  const bool keep = (rec.x >> 24) & 1;
  const int e0 = slot * a.pv.n_modules + a.module0 + m0;
  int rk[kBgmvMaxPack];   // ranks of the pack's entries (0 past np or for an empty entry)
#pragma unroll
  for (int mi = 0; mi < kBgmvMaxPack; ++mi) rk[mi] = mi < np ? max(a.pv.entries[e0 + mi].rank, 0) : 0;
  int rows = 0;
#pragma unroll
  for (int mi = 0; mi < kBgmvMaxPack; ++mi) rows += rk[mi];
  // prologue: tokens, every module's page ids, stacked row starts; t cleared
  __syncthreads();   // the previous item is done with LDS
  const int tid = threadIdx.x;
  if (tid < kUnitTokens) L.toks[tid] = tid < nt ? a.sv.perm[pos + tid] : 0;
  for (int i = tid; i < np * ids_per; i += kGemvThreads) {
    const int mi = i / ids_per;
    L.pid[i] = a.pv.page_ids[static_cast<int64_t>(e0 + mi) * a.pv.ppe + (i - mi * ids_per)];
  }
  for (int i = tid; i < kUnitTokens * kMaxRank; i += kGemvThreads) L.t[i] = 0.f;
  __syncthreads();
  if (rows <= 0) return;
  Stack st;
  st.ids_per = ids_per;
  st.rstart[0] = 0;
#pragma unroll
  for (int mi = 1; mi < kBgmvMaxPack; ++mi) st.rstart[mi] = mi < np ? st.rstart[mi - 1] + rk[mi - 1] : rows;
  const bool x_stream = LORA_BGMV_NT_XY != 0 && a.x_stream != 0;
#define LORA_SHRINK_CALL(N, K) \
  shrink_unit<TI, N, K, true>(xm, a.ld_x, L, nt, pages, 0, h, a.magic, a.h_in, 0, rows, xs, x_stream, st)
  if (keep) {
    if (nt == 1) LORA_SHRINK_CALL(1, true);
    else if (nt == 2) LORA_SHRINK_CALL(2, true);
    else LORA_SHRINK_CALL(4, true);
  } else {
    if (nt == 1) LORA_SHRINK_CALL(1, false);
    else if (nt == 2) LORA_SHRINK_CALL(2, false);
    else LORA_SHRINK_CALL(4, false);
  }
#undef LORA_SHRINK_CALL
  constexpr bool nty = LORA_BGMV_NT_XY != 0;
  int toff = 0;   // t columns of module mi start after those of the modules before it
  for (int mi = 0; mi < np; ++mi) {
    const SlotEntry em = a.pv.entries[e0 + mi];
    if (em.rank <= 0) continue;   // uniform
    TO* ym = static_cast<TO*>(a.y) + (m0 + mi) * a.msy;
#define LORA_EXPAND_CALL(N, K)                                                                                  \
  expand_unit<TI, TO, N, K, nty, true>(ym, a.ld_y, L, nt, pages, mi * ids_per + ids_a, h, a.magic, a.h_out,    \
                                       em.rank, em.scale, 0, a.h_out >> 2, toff)
    if (keep) {
      if (nt == 1) LORA_EXPAND_CALL(1, true);
      else if (nt == 2) LORA_EXPAND_CALL(2, true);
      else LORA_EXPAND_CALL(4, true);
    } else {
      if (nt == 1) LORA_EXPAND_CALL(1, false);
      else if (nt == 2) LORA_EXPAND_CALL(2, false);
      else LORA_EXPAND_CALL(4, false);
    }
#undef LORA_EXPAND_CALL
    toff += em.rank;
  }
}

// The work items of module b.y for one workgroup of a grid of b.nx workgroups per
// module.  b.nx is a multiple of 8*kUnitRun (see unit_of_block).  it0 >= 0 names
// the workgroup's first work item in place of unit_of_block.
template <int MODE, typename TI, typename TO>
__device__ __forceinline__ void gemv_body(const GemvArgs& a, const Blk b, UnitLds& L, TI* xs, int it0 = -1) {
  const int m = b.y;
  const int2* units = reinterpret_cast<const int2*>(a.sv.units);
  // the unit count and this workgroup's first record travel together
  const int n_units = a.sv.meta[a.units_word];
  // work item it = unit * parts + part; high-rank units of the two-kernel path split into parts
  // so that a unit's serial batches spread over several workgroups
  const int parts = a.parts;
  const int n_items = n_units * parts;
  int it = it0 >= 0 ? it0 : unit_of_block(b.x, m);
  int2 rec = units[min(it / parts, a.sv.max_units - 1)];
  for (; it < n_items; it += b.nx) {
    const int u = it / parts, part = it - u * parts;
    if (it >= b.nx) rec = units[u];
    gemv_item<MODE, TI, TO>(a, m, rec, part, L, xs);
  }
}

// Workgroup lin of a 1-D GEMV grid of nm modules x nx workgroups taken in
// groups of gm modules (the last may be shorter), the modules varying fastest
// inside a group: the workgroups in flight at any time cover a few modules at
// once and, for a group of a multiple of 8 modules laid out from a multiple of
// 8 workgroups, every workgroup of module m runs on XCD m % 8.  Returns its
// coordinates and sets it0 to its first work item.
__device__ __forceinline__ Blk blk_of_module_groups(int lin, int nx, int nm, int gm, int& it0) {
  const int g = lin / (gm * nx), local = lin - g * gm * nx;
  const int size = min(gm, nm - g * gm);
  it0 = local / size;
  return Blk{0, g * gm + local % size, 0, nx, nm, 1};
}

// With a.module_group > 0 (MODE 0) the grid is 1-D, modules x group_nx
// workgroups in groups of module_group modules (blk_of_module_groups).
template <int MODE, typename TI, typename TO>
__global__ __launch_bounds__(kGemvThreads, 4) void k_gemv(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[gemv_lds_bytes<MODE, TI>()];
  Blk b = blk_of_launch();
  int it0 = -1;
  if (MODE == 0 && a.module_group > 0)
    b = blk_of_module_groups(static_cast<int>(blockIdx.x), a.group_nx,
                             static_cast<int>(gridDim.x) / a.group_nx, a.module_group, it0);
  gemv_body<MODE, TI, TO>(a, b, *reinterpret_cast<UnitLds*>(lds),
                          reinterpret_cast<TI*>(lds + gemv_xs_offset<MODE, TI>()), it0);
}

// Fused BGMV straight from the batch's adapter ids, for batches of at most
// kWaveSegTokens tokens: each decode token brings its own adapter index, as in
// the study page's BGMV.  Wave 0 of every workgroup builds the batch's unit
// list in LDS (segments_of_wave: the lists the segment builder writes), and the
// workgroup then runs its unit as k_gemv<0> does.  The 64 ids take the place
// of the work-list record in the first round trip, and the step needs no
// separate segment build launch.  Grid as k_gemv<0>.
constexpr int kIdsMaxUnits = kWaveSegTokens / kUnitTokens + kWaveSegTokens;   // units of 64 tokens, any slots
template <typename TI, typename TO>
__global__ __launch_bounds__(kGemvThreads, 4) void k_bgmv_ids(GemvArgs a, const int32_t* __restrict__ ids,
                                                              int32_t n_tokens, int32_t nbits) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[gemv_lds_bytes<0, TI>()];
  __shared__ int32_t perm_s[kWaveSegTokens], seg_start_s[kWaveSegTokens + 1], seg_slot_s[kWaveSegTokens];
  __shared__ int32_t meta_s[LORA_META_WORDS];
  __shared__ int2 units_s[kIdsMaxUnits], tiles_s[2];
  if (threadIdx.x < 64)   // wave 0; its slot table lives where the x rows go later
    segments_of_wave(ids, n_tokens, a.pv.n_slots, nbits,
                     SegOut{perm_s, seg_start_s, seg_slot_s, meta_s, reinterpret_cast<int32_t*>(units_s),
                            reinterpret_cast<int32_t*>(tiles_s)},
                     reinterpret_cast<uint32_t*>(lds + gemv_xs_offset<0, TI>()));
  __syncthreads();
  a.sv.perm = perm_s;
  a.sv.seg_start = seg_start_s;
  a.sv.seg_slot = seg_slot_s;
  a.sv.meta = meta_s;
  a.sv.units = reinterpret_cast<const int32_t*>(units_s);
  a.sv.tiles = reinterpret_cast<const int32_t*>(tiles_s);
  a.sv.max_units = kIdsMaxUnits;
  a.sv.max_tiles = 1;
  Blk b = blk_of_launch();
  int it0 = -1;
  if (a.module_group > 0)
    b = blk_of_module_groups(static_cast<int>(blockIdx.x), a.group_nx, static_cast<int>(gridDim.x) / a.group_nx,
                             a.module_group, it0);
  gemv_body<0, TI, TO>(a, b, *reinterpret_cast<UnitLds*>(lds), reinterpret_cast<TI*>(lds + gemv_xs_offset<0, TI>()),
                       it0);
}

// Fused BGMV over packs of a.pack modules that share x (gemv_item_packed): a
// grid of units x 1; each workgroup loops over units like k_gemv's.  Three
// waves per SIMD: the stacked row lookup and the per-module expands do not
// fit k_gemv's register budget without spilling.
template <typename TI, typename TO>
__global__ __launch_bounds__(kGemvThreads, 3) void k_bgmv_packed(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[gemv_lds_bytes<0, TI>()];
  UnitLds& L = *reinterpret_cast<UnitLds*>(lds);
  TI* xs = reinterpret_cast<TI*>(lds + gemv_xs_offset<0, TI>());
  const int2* units = reinterpret_cast<const int2*>(a.sv.units);
  const int n_units = a.sv.meta[LORA_META_N_UNITS_ALL];
  int it = unit_of_block(static_cast<int>(blockIdx.x), 0);
  int2 rec = units[min(it, a.sv.max_units - 1)];
  for (; it < n_units; it += static_cast<int>(gridDim.x)) {
    if (it >= static_cast<int>(gridDim.x)) rec = units[it];
    gemv_item_packed<TI, TO>(a, static_cast<int>(blockIdx.y), rec, L, xs);
  }
}

}  // namespace lora
