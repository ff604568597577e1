// Shared definitions of the HIP side: device structs, vector loads/stores,
// wave64 reductions.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

// Work decomposition fixed by the library (recorded in the segment meta).
#ifndef LORA_UNIT_TOKENS
#define LORA_UNIT_TOKENS 4
#endif
constexpr int kUnitTokens = LORA_UNIT_TOKENS;     // tokens per GEMV work unit
constexpr int kTileTokens = 64;    // tokens per matrix-core tile
constexpr int kLongMin = 64;       // segments this long or longer use matrix-core tiles
constexpr int kMaxRank = LORA_MAX_RANK;
constexpr int kMaxSlots = 8192;   // the segment builder's LDS histogram bound
constexpr int kMaxEntryPages = 1024;  // pages of one (slot, module) entry (an LDS table in the GEMV kernels)

// One (slot, module) entry of the device slot table.
struct SlotEntry {
  int32_t rank;    // 0 = empty
  float scale;
  int32_t a_off;   // offset of A's page list in the page-id table
  int32_t b_off;   // offset of B's page list in the page-id table
};

// Read-only view of a pool, passed to kernels by value.
struct PoolView {
  const void* pages;          // n_pages * page_elems elements
  const SlotEntry* entries;   // [n_slots * n_modules]
  const int32_t* page_ids;    // page lists
  int64_t page_elems;
  int32_t n_slots;
  int32_t n_modules;
  int32_t max_rank;           // rank cap of the pool
  int32_t ppe;                // page-table words per (slot, module): A's ids, then B's from max_rank*ppr_a
  int32_t zero_page;          // a page of zeros (index n_pages)
};

struct SegView {
  const int32_t* perm;
  const int32_t* seg_start;
  const int32_t* seg_slot;
  const int32_t* meta;
  const int32_t* units;
  const int32_t* tiles;
  int32_t max_units;
  int32_t max_tiles;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte loads for data read once per launch; on
// gfx950 they sustain a higher share of HBM bandwidth than plain loads.
#ifndef LORA_NT_PAGES
#define LORA_NT_PAGES 1
#endif
#ifndef LORA_NT_ROWS
#define LORA_NT_ROWS 0
#endif
template <bool NT, typename V>
__device__ __forceinline__ V ld16(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// LDS address of a pointer into shared memory, for the direct global-to-LDS loads
// (global_load_lds: each lane's 16 bytes land at the wave's LDS base + 16 * lane).
typedef __attribute__((address_space(3))) void* lds_addr_t;
__device__ __forceinline__ lds_addr_t to_lds(void* p) {
  return reinterpret_cast<lds_addr_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Raw 16-byte chunk of 8 bf16 or 4 f32 values.
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> {
  static constexpr int kElems = 8;
  u32x4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void load_nt(const __bf16* p) {
    v = ld16<LORA_NT_PAGES != 0>(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void unpack(float (&f)[8]) const {
    f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    f[4] = bf16lo(v.z); f[5] = bf16hi(v.z); f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
  }
};
template <> struct Chunk<float> {
  static constexpr int kElems = 4;
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) {
    v = ld16<LORA_NT_PAGES != 0>(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void unpack(float (&f)[4]) const { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
};

// Eight consecutive elements (one or two 16-byte chunks) as floats.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8]) {
  if constexpr (sizeof(T) == 2) {
    Chunk<__bf16> c; c.load(p); c.unpack(f);
  } else {
    f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// Stores eight floats, rounding to nearest even for bf16 (one rounding).
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&f)[8]) {
  if constexpr (sizeof(T) == 2) {
    __bf16 h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<__bf16>(f[e]);
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, h);
  } else {
    reinterpret_cast<f32x4*>(p)[0] = f32x4{f[0], f[1], f[2], f[3]};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{f[4], f[5], f[6], f[7]};
  }
}

// v from lane (lane ^ M) of the wave.  Masks below 16 use DPP row operations;
// 16 and 32 go through the LDS crossbar (ds_bpermute).
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  int x = __builtin_bit_cast(int, v);
  if constexpr (M == 1) {
    x = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror: i -> 7-i
    x = __builtin_amdgcn_update_dpp(0, x, 0x1B, 0xF, 0xF, false);   // quad_perm [3,2,1,0]: ^3
  } else if constexpr (M == 8) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else {
    return __shfl_xor(v, M, 64);
  }
  return __builtin_bit_cast(float, x);
}

// Transpose-reduction of V values held by every lane of a wave64.
// On return v[0] of lane l holds the sum over all 64 lanes of value
// index l / (64 / V).  log2(V) halving exchanges, then a butterfly.
template <int M, int C>
__device__ __forceinline__ void tr_step(float (&v)[64], int lane) {
  const bool upper = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < C / 2; ++i) {
    float a = v[i], b = v[i + C / 2];
    float keep = upper ? b : a;
    float send = upper ? a : b;
    v[i] = keep + xor_lane<M>(send);
  }
}

template <int V>
__device__ __forceinline__ float wave_transpose_reduce(float (&v)[64], int lane) {
  static_assert(V == 1 || V == 2 || V == 4 || V == 8 || V == 16 || V == 32 || V == 64, "V");
  if constexpr (V >= 2) tr_step<32, V>(v, lane);
  if constexpr (V >= 4) tr_step<16, V / 2>(v, lane);
  if constexpr (V >= 8) tr_step<8, V / 4>(v, lane);
  if constexpr (V >= 16) tr_step<4, V / 8>(v, lane);
  if constexpr (V >= 32) tr_step<2, V / 16>(v, lane);
  if constexpr (V >= 64) tr_step<1, V / 32>(v, lane);
  float s = v[0];
  // butterfly over the lanes that still hold partial sums of the same index
  if constexpr (V <= 1) s += xor_lane<32>(s);
  if constexpr (V <= 2) s += xor_lane<16>(s);
  if constexpr (V <= 4) s += xor_lane<8>(s);
  if constexpr (V <= 8) s += xor_lane<4>(s);
  if constexpr (V <= 16) s += xor_lane<2>(s);
  if constexpr (V <= 32) s += xor_lane<1>(s);
  return s;
}

// Work item of workgroup bx of plane `plane` (a module or a split), in a grid
// of a multiple of 8*R workgroups: runs of R consecutive items (mostly pieces
// of one segment, so one adapter) stay on one XCD and its L2 (workgroup bx
// runs on XCD bx % 8), the runs go round-robin over the XCDs, and the
// round-robin starts one XCD further for each plane, so that the XCDs share
// the items evenly whatever their count.  A bijection of [0, gridDim.x) that
// does not depend on the item count, so a workgroup can read its work-list
// record together with that count.
template <int R>
__device__ __forceinline__ int item_of_block(int bx, int plane) {
  const int run = ((bx & 7) - plane) & 7, k = bx >> 3;
  return (k / R) * (8 * R) + run * R + (k % R);
}
constexpr int kTileRun = 2;   // consecutive matrix-core tiles one XCD takes

// A workgroup's coordinates in the grid of its kernel body.  A body that
// has a launch of its own takes the launch's; one that shares a launch with
// another body takes those of its part of the launch, laid out x fastest as
// the hardware dispatches (so a part that starts at a multiple of 8 keeps
// the XCD of every block: block i goes to XCD i % 8).
struct Blk {
  int x, y, z, nx, ny, nz;
};
__device__ __forceinline__ Blk blk_of_launch() {
  return Blk{static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z),
             static_cast<int>(gridDim.x),  static_cast<int>(gridDim.y),  static_cast<int>(gridDim.z)};
}
// Block `lin` of a grid nx x ny x nz.
__device__ __forceinline__ Blk blk_of_linear(int lin, int nx, int ny, int nz) {
  const int x = lin % nx, yz = lin / nx;
  return Blk{x, yz % ny, yz / ny, nx, ny, nz};
}

// Upper bounds of the segment work lists (host and device agree on them).
__host__ __device__ inline int32_t max_segs_of(int32_t n_tokens, int32_t n_slots) {
  return n_tokens < n_slots ? n_tokens : n_slots;
}
__host__ __device__ inline int32_t max_units_of(int32_t n_tokens, int32_t n_slots) {
  return (n_tokens + kUnitTokens - 1) / kUnitTokens + max_segs_of(n_tokens, n_slots);
}
__host__ __device__ inline int32_t max_tiles_of(int32_t n_tokens) {
  // a long segment has >= kLongMin tokens, so there are at most n/kLongMin of them
  return (n_tokens + kTileTokens - 1) / kTileTokens + n_tokens / kLongMin;
}

}  // namespace lora
