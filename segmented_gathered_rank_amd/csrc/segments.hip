// Segment builder: groups a batch's tokens by adapter slot on the GPU.
//
// The Fastino article describes the kernel as grouping "a batch's tokens by
// adapter"; the study page's SGMV works on "contiguous segments of tokens
// sharing an adapter".  This is a stable counting sort of token indices by
// slot, done by one workgroup of 16 wave64s:
//
//   count   each scanning wave owns a contiguous range of tokens and counts
//           its ids into its own LDS histogram row.  Lanes holding the same
//           id find each other with one ballot per id bit (a multi-split
//           match), so one leader lane updates the row per distinct id.
//   scan    per slot, an exclusive prefix over the waves' rows (in wave
//           order) and the slot total; then a block scan over slots of five
//           counters at once: tokens, segments, GEMV units of short and of
//           long segments, and matrix-core tiles.  Non-empty slots write
//           seg_slot/seg_start and their work-list entries.
//   scatter each wave walks its range again in token order; a token's
//           position is its wave's cursor for the slot plus its rank among
//           earlier lanes with the same id.  Ranges are in token order and
//           cursors in wave order, so the sort is stable.
//
// All counts stay on the device: no host synchronization.
#include "common.hpp"

using namespace lora;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsWords = 16384;   // 64 KiB: V histogram rows + one row of totals
constexpr int kIdBatch = 16;       // ids each lane loads at once

// Mask of the lanes whose (valid) id equals this lane's id.
__device__ __forceinline__ uint64_t match_peers(int id, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((id >> b) & 1);
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__global__ __launch_bounds__(kThreads) void k_build_segments(
    const int32_t* __restrict__ ids, int32_t n_tokens, int32_t n_slots, int32_t V, int32_t nbits,
    int32_t* __restrict__ perm, int32_t* __restrict__ seg_start, int32_t* __restrict__ seg_slot,
    int32_t* __restrict__ meta, int32_t* __restrict__ units, int32_t* __restrict__ tiles) {
  extern __shared__ int32_t lds[];
  int32_t* hist = lds;                      // [V][n_slots]: counts, then cursors
  int32_t* total = lds + V * n_slots;       // [n_slots]
  __shared__ int scan_w[kWaves][5];
  __shared__ int scan_tot[5];
  __shared__ int max_w[kWaves];
  __shared__ int bad_w[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < V * n_slots; i += kThreads) hist[i] = 0;
  __syncthreads();

  // ---- count: wave w < V owns tokens [w*span, (w+1)*span); each lane loads
  //      kIdBatch ids at once, then the wave matches them 64 at a time in order
  const int span = ((n_tokens + V - 1) / V + 63) / 64 * 64;
  const int beg = wave * span;
  const int end = min(n_tokens, beg + span);
  int bad = 0;
  if (wave < V) {
    int32_t* row = hist + wave * n_slots;
    for (int base = beg; base < end; base += 64 * kIdBatch) {
      int idv[kIdBatch];
#pragma unroll
      for (int i = 0; i < kIdBatch; ++i) {
        const int t = base + i * 64 + lane;
        idv[i] = t < end ? ids[t] : -1;
      }
#pragma unroll
      for (int i = 0; i < kIdBatch; ++i) {
        const int t = base + i * 64 + lane;
        const int id = idv[i];
        const bool valid = id >= 0 && id < n_slots;
        if (t < end && (id < -1 || id >= n_slots)) ++bad;
        const uint64_t peers = match_peers(id, valid, nbits);
        if (valid && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane) row[id] += __popcll(peers);
      }
    }
  }
  for (int m = 32; m >= 1; m >>= 1) bad += __shfl_xor(bad, m, 64);
  if (lane == 0) bad_w[wave] = bad;
  __syncthreads();

  // ---- scan: thread tid owns slots [s0, s1), consecutive, in slot order
  const int bpt = (n_slots + kThreads - 1) / kThreads;
  const int s0 = min(n_slots, tid * bpt);
  const int s1 = min(n_slots, s0 + bpt);
  int own[5] = {0, 0, 0, 0, 0};   // tokens, segments, short units, long units, tiles
  int mx = 0;
  for (int s = s0; s < s1; ++s) {
    int run = 0;
    for (int w = 0; w < V; ++w) {
      const int c = hist[w * n_slots + s];
      hist[w * n_slots + s] = run;
      run += c;
    }
    total[s] = run;
    if (run > 0) {
      own[0] += run;
      own[1] += 1;
      if (run >= kLongMin) {
        own[3] += (run + kUnitTokens - 1) / kUnitTokens;
        own[4] += (run + kTileTokens - 1) / kTileTokens;
      } else {
        own[2] += (run + kUnitTokens - 1) / kUnitTokens;
      }
      mx = max(mx, run);
    }
  }
  int v[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    v[q] = own[q];
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(v[q], d, 64);
      if (lane >= d) v[q] += o;
    }
  }
  for (int m = 32; m >= 1; m >>= 1) mx = max(mx, __shfl_xor(mx, m, 64));
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 5; ++q) scan_w[wave][q] = v[q];
    max_w[wave] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    int acc[5] = {0, 0, 0, 0, 0};
    int m = 0, b = 0;
    for (int w = 0; w < kWaves; ++w) {
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        const int t = scan_w[w][q];
        scan_w[w][q] = acc[q];
        acc[q] += t;
      }
      m = max(m, max_w[w]);
      b += bad_w[w];
    }
#pragma unroll
    for (int q = 0; q < 5; ++q) scan_tot[q] = acc[q];
    meta[LORA_META_N_SEG] = acc[1];
    meta[LORA_META_N_ACTIVE] = acc[0];
    meta[LORA_META_MAX_SEG_LEN] = m;
    meta[LORA_META_N_BAD] = b;
    meta[LORA_META_N_UNITS_SHORT] = acc[2];
    meta[LORA_META_N_UNITS_ALL] = acc[2] + acc[3];
    meta[LORA_META_N_TILES] = acc[4];
    meta[LORA_META_UNIT_TOKENS] = kUnitTokens;
    meta[LORA_META_TILE_TOKENS] = kTileTokens;
    meta[LORA_META_LONG_MIN] = kLongMin;
    meta[LORA_META_N_TOKENS] = n_tokens;
    meta[LORA_META_N_SLOTS] = n_slots;
    for (int q = 12; q < LORA_META_WORDS; ++q) meta[q] = 0;
    seg_start[acc[1]] = acc[0];
  }
  __syncthreads();

  // ---- segments, work lists and cursors.  Slots are visited in order b of
  //      each thread's block; a slot's work-list entries are written by all 64
  //      lanes of its wave (its counters are broadcast from the owning lane).
  int off[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) off[q] = scan_w[wave][q] + v[q] - own[q];
  const int long_units_at = scan_tot[2];   // long-segment units follow all short ones
  for (int b = 0; b < bpt; ++b) {
    const int s = s0 + b;
    const int run = (s < s1) ? total[s] : 0;
    for (int src = 0; src < 64; ++src) {
      const int r = __shfl(run, src, 64);
      if (r == 0) continue;                 // wave-uniform
      const int sbase = __shfl(off[0], src, 64);
      const int ssi = __shfl(off[1], src, 64);
      const int nu = (r + kUnitTokens - 1) / kUnitTokens;
      if (r >= kLongMin) {
        const int u0 = long_units_at + __shfl(off[3], src, 64);
        const int t0 = __shfl(off[4], src, 64);
        for (int u = lane; u < nu; u += 64) {
          units[2 * (u0 + u)] = ssi;
          units[2 * (u0 + u) + 1] = sbase + u * kUnitTokens;
        }
        const int ntl = (r + kTileTokens - 1) / kTileTokens;
        for (int u = lane; u < ntl; u += 64) {
          tiles[2 * (t0 + u)] = ssi;
          tiles[2 * (t0 + u) + 1] = sbase + u * kTileTokens;
        }
      } else {
        const int u0 = __shfl(off[2], src, 64);
        for (int u = lane; u < nu; u += 64) {
          units[2 * (u0 + u)] = ssi;
          units[2 * (u0 + u) + 1] = sbase + u * kUnitTokens;
        }
      }
    }
    if (run > 0) {
      seg_slot[off[1]] = s;
      seg_start[off[1]] = off[0];
      for (int w = 0; w < V; ++w) hist[w * n_slots + s] += off[0];
      const int nu = (run + kUnitTokens - 1) / kUnitTokens;
      if (run >= kLongMin) {
        off[3] += nu;
        off[4] += (run + kTileTokens - 1) / kTileTokens;
      } else {
        off[2] += nu;
      }
      off[0] += run;
      off[1] += 1;
    }
  }
  __syncthreads();

  // ---- scatter, stable: same ranges, same order as the count
  if (wave < V) {
    int32_t* row = hist + wave * n_slots;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = beg; base < end; base += 64 * kIdBatch) {
      int idv[kIdBatch];
#pragma unroll
      for (int i = 0; i < kIdBatch; ++i) {
        const int t = base + i * 64 + lane;
        idv[i] = t < end ? ids[t] : -1;
      }
#pragma unroll
      for (int i = 0; i < kIdBatch; ++i) {
        const int t = base + i * 64 + lane;
        const int id = idv[i];
        const bool valid = id >= 0 && id < n_slots;
        const uint64_t peers = match_peers(id, valid, nbits);
        if (valid) perm[row[id] + __popcll(peers & lt)] = t;
        if (valid && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane) row[id] += __popcll(peers);
      }
    }
  }
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

extern "C" {

size_t lora_segments_bytes(int32_t n_tokens, int32_t n_slots) {
  if (n_tokens < 0 || n_slots < 1) return 0;
  const int32_t S = max_segs_of(n_tokens, n_slots);
  size_t b = 0;
  b += align256(static_cast<size_t>(n_tokens) * 4);                    // perm
  b += align256(static_cast<size_t>(S + 1) * 4);                       // seg_start
  b += align256(static_cast<size_t>(S > 0 ? S : 1) * 4);               // seg_slot
  b += align256(LORA_META_WORDS * 4);                                  // meta
  b += align256(static_cast<size_t>(max_units_of(n_tokens, n_slots)) * 8);  // units
  b += align256(static_cast<size_t>(max_tiles_of(n_tokens)) * 8 + 8);  // tiles
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
  out->n_tokens = n_tokens;
  out->n_slots = n_slots;
  out->max_segs = S;
  out->max_units = max_units_of(n_tokens, n_slots);
  out->max_tiles = max_tiles_of(n_tokens);
  return LORA_OK;
}

lora_status lora_build_segments(const int32_t* ids, const lora_segments* seg, void* stream) {
  if (!seg) return LORA_ERR_ARG;
  if (seg->n_tokens < 0 || seg->n_slots < 1 || seg->n_slots > kMaxSlots) return LORA_ERR_ARG;
  if (seg->n_tokens == 0) return LORA_OK;
  if (!ids || !seg->perm || !seg->seg_start || !seg->seg_slot || !seg->meta || !seg->units || !seg->tiles)
    return LORA_ERR_ARG;
  const int32_t n_slots = seg->n_slots;
  int32_t V = kLdsWords / n_slots - 1;
  if (V > kWaves) V = kWaves;
  if (V < 1) return LORA_ERR_ARG;
  int32_t nbits = 0;
  while ((1 << nbits) < n_slots) ++nbits;
  const size_t lds = static_cast<size_t>(V + 1) * n_slots * 4;
  static bool lds_set = false;   // gfx950 allows 160 KiB of LDS per workgroup
  if (!lds_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_build_segments),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsWords * 4) != hipSuccess)
      return LORA_ERR_HIP;
    lds_set = true;
  }
  hipLaunchKernelGGL(k_build_segments, dim3(1), dim3(kThreads), lds, static_cast<hipStream_t>(stream), ids,
                     seg->n_tokens, n_slots, V, nbits, seg->perm, seg->seg_start, seg->seg_slot, seg->meta,
                     seg->units, seg->tiles);
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
