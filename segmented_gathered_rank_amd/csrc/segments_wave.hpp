// Wave-level building blocks of the segment build ("Multi-LoRA Serving -
// S-LoRA/Punica Batching", section "The kernel trick: gather, do not merge":
// tokens are grouped by adapter before the gathered products), and the build
// of a batch of at most 64 tokens on one wave, shared by the segment builder
// and the decode kernel that starts from the ids.
#pragma once

#include "common.hpp"

namespace lora {

template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}
// Inclusive scan over the 64 lanes with DPP: row shifts by 1, 2, 4, 8 inside
// each row of 16 lanes, then the row broadcasts of lane 15 and lane 31.
// Lanes outside a shift's row read 0, the identity of both operations
// (values are non-negative).
template <bool kMax>
__device__ __forceinline__ int wave_scan(int v) {
  auto op = [](int a, int b) { return kMax ? (a > b ? a : b) : a + b; };
  v = op(v, dpp0<0x111, 0xf>(v));
  v = op(v, dpp0<0x112, 0xf>(v));
  v = op(v, dpp0<0x114, 0xf>(v));
  v = op(v, dpp0<0x118, 0xf>(v));
  v = op(v, dpp0<0x142, 0xa>(v));
  v = op(v, dpp0<0x143, 0xc>(v));
  return v;
}
__device__ __forceinline__ int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

__device__ __forceinline__ int lowest_lane(uint64_t m) {
  return __ffsll(static_cast<unsigned long long>(m)) - 1;
}

// Mask of the lanes whose (valid) id equals this lane's id; 0 for an invalid lane.
__device__ __forceinline__ uint64_t peers_of(int id, bool valid, int nbits) {
  const uint64_t vm = __ballot(valid);
  const int first = __builtin_amdgcn_readfirstlane(id);
  if (__ballot(valid && id == first) == vm) return valid ? vm : 0ull;   // one id in the batch
  uint64_t peers = vm;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((id >> b) & 1);
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return valid ? peers : 0ull;
}

// Where a segment build writes its lists (device or LDS memory).
struct SegOut {
  int32_t *perm, *seg_start, *seg_slot, *meta, *units, *tiles;
};

// GEMV work unit u of a segment of `run` tokens of `slot` that starts at
// position `first` of perm: (slot + 65536 * tokens in the unit + 2^24 if the
// segment has more than one unit, position).
__device__ __forceinline__ int2 unit_record(int slot, int run, int u, int first) {
  return make_int2(slot + (min(kUnitTokens, run - u * kUnitTokens) << 16) + ((run > kUnitTokens) ? (1 << 24) : 0),
                   first + u * kUnitTokens);
}

// A decode batch on one wave: lane i holds token i.  A token's place in perm
// is the number of valid tokens of smaller slots plus its rank among its
// slot's tokens (ballot match per id bit); a segment's first token (its
// slot's lowest lane) writes the segment's entries, which need the count of
// smaller slots' segments, tokens, units and tiles: summed over the segments'
// first lanes only, one packed word each.  The same lists as the workgroup
// builders, without their histogram, barriers and layout phases.  Called by
// all 64 lanes of one wave; n_tokens <= kWaveSegTokens.
constexpr int kWaveSegTokens = 64;
// table: 64 words of LDS the wave may use (or null): with at most 64 slots the
// sums over smaller slots come from one scan over a slot table instead of a
// loop over the segments.
__device__ __forceinline__ void segments_of_wave(const int32_t* __restrict__ ids, int32_t n_tokens, int32_t n_slots,
                                                 int32_t nbits, SegOut o, uint32_t* table = nullptr) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const bool in = lane < n_tokens;
  const int id = in ? ids[lane] : -1;
  const bool valid = in && id >= 0 && id < n_slots;
  const int n_bad = __popcll(__ballot(in && (id < -1 || id >= n_slots)));
  const uint64_t peers = peers_of(id, valid, nbits);   // lanes of the same slot (0 if invalid)
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int len = __popcll(peers);
  const bool first = valid && (peers & below) == 0ull;
  const bool is_long = len >= kLongMin;
  const int nu = (len + kUnitTokens - 1) / kUnitTokens;
  const int nt = is_long ? (len + kTileTokens - 1) / kTileTokens : 0;
  // a first lane's contribution, 7 bits a field (every sum stays below 128 at 64 tokens; the
  // tile count keeps the top 4 bits: only a segment of all 64 tokens has a tile):
  // 1 segment | its tokens | its short-segment units | its long-segment units | its tiles
  const uint32_t mine = first ? 1u | (static_cast<uint32_t>(len) << 7) | (static_cast<uint32_t>(is_long ? 0 : nu) << 14) |
                                    (static_cast<uint32_t>(is_long ? nu : 0) << 21) |
                                    (static_cast<uint32_t>(nt) << 28)
                              : 0u;
  uint32_t before = 0;   // the same sums over the segments of smaller slots
  if (table != nullptr && n_slots <= 64) {   // uniform
    // slot s's record at table[s], then its exclusive prefix over the slots (each field's sum
    // stays inside its bits, so the packed words add field by field)
    table[lane] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (first) table[id] = mine;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint32_t v = table[lane];
    const uint32_t incl = static_cast<uint32_t>(wave_scan<false>(static_cast<int>(v)));
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    table[lane] = incl - v;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (valid) before = table[id];
  } else {
    for (uint64_t fm = __ballot(first); fm; fm &= fm - 1) {
      const int j = lowest_lane(fm);
      const int idj = __builtin_amdgcn_readlane(id, j);
      const uint32_t pj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine), j));
      if (valid && idj < id) before += pj;
    }
  }
  const int seg = before & 127, start = (before >> 7) & 127, su = (before >> 14) & 127;
  const int lu = (before >> 21) & 127, tl = static_cast<int>(before >> 28);
  if (valid) o.perm[start + __popcll(peers & below)] = lane;
  const int n_seg = __popcll(__ballot(first));
  const int n_active = __popcll(__ballot(valid));
  const int n_short = lane63(wave_scan<false>(first && !is_long ? nu : 0));
  const int n_long_units = lane63(wave_scan<false>(first && is_long ? nu : 0));
  const int n_tiles = lane63(wave_scan<false>(first ? nt : 0));
  const int max_len = lane63(wave_scan<true>(len));
  if (first) {
    o.seg_slot[seg] = id;
    o.seg_start[seg] = start;
    int2* units = reinterpret_cast<int2*>(o.units);
    if (!is_long) {
      for (int u = 0; u < nu; ++u) units[su + u] = unit_record(id, len, u, start);
    } else {
      for (int u = 0; u < nu; ++u) units[n_short + lu + u] = unit_record(id, len, u, start);
      int2* tiles = reinterpret_cast<int2*>(o.tiles);
      for (int u = 0; u < nt; ++u)
        tiles[tl + u] = make_int2(id + (min(kTileTokens, len - u * kTileTokens) << 16), start + u * kTileTokens);
    }
  }
  if (lane == 0) o.seg_start[n_seg] = n_active;
  if (lane < LORA_META_WORDS) {   // one store for the whole meta block
    int v = 0;
    switch (lane) {
      case LORA_META_N_SEG: v = n_seg; break;
      case LORA_META_N_ACTIVE: v = n_active; break;
      case LORA_META_MAX_SEG_LEN: v = max_len; break;
      case LORA_META_N_BAD: v = n_bad; break;
      case LORA_META_N_UNITS_SHORT: v = n_short; break;
      case LORA_META_N_UNITS_ALL: v = n_short + n_long_units; break;
      case LORA_META_N_TILES: v = n_tiles; break;
      case LORA_META_UNIT_TOKENS: v = kUnitTokens; break;
      case LORA_META_TILE_TOKENS: v = kTileTokens; break;
      case LORA_META_LONG_MIN: v = kLongMin; break;
      case LORA_META_N_TOKENS: v = n_tokens; break;
      case LORA_META_N_SLOTS: v = n_slots; break;
      default: v = 0; break;
    }
    o.meta[lane] = v;
  }
}

}  // namespace lora
