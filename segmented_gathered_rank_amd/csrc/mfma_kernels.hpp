// Matrix-core path for long segments (SGMV "for contiguous segments of tokens
// sharing an adapter, as in prefill": study page, "The kernel trick").  A
// segment of L >= kLongMin tokens is a dense grouped contraction, so it is cut
// into tiles of kTileTokens tokens and run on CDNA4 MFMA.
//
// shrink (bf16 in, fp32 accumulate): T[64 x r] = X[64 x K] * A^T[K x r] with
//   v_mfma_f32_16x16x32_bf16.  Wave w owns tokens 16w..16w+15 of the tile;
//   one MFMA takes a 16 x 32 slice of X (each lane 8 consecutive bf16 of one
//   token row) and a 32 x 16 slice of A^T (each lane 8 consecutive bf16 of one
//   rank row), so both operands stream straight from row-major memory.  When
//   several modules share x (q, k, v), one workgroup computes all of them from
//   one read of the x slice.  K may be split across workgroups; the partial
//   tiles then go to a workspace and the last workgroup to finish a tile adds
//   them in split order (an atomic ticket decides who is last, the sum order
//   does not depend on it: deterministic).
// expand (fp32 t, bf16 B, y bf16 or fp32): Y[64 x 128] += s * T[64 x r] B[r x 128]
//   with v_mfma_f32_32x32x2_f32, so t stays in fp32.  T, the B tile and the
//   y tile are staged in LDS with 16-byte coalesced loads; the epilogue adds
//   s*acc to y in fp32 and rounds once on the way out.
#pragma once

#include "common.hpp"

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 256;
constexpr int kShrinkMaxModules = 4;   // modules sharing one x slice in a workgroup
constexpr int kExpandCols = 128;       // output columns per expand workgroup

__device__ __forceinline__ bf16x8 ld_bf16x8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

struct ShrinkArgs {
  PoolView pv;
  SegView sv;
  const __bf16* x;
  int64_t ld_x, msx;          // msx: x offset between module groups (grid z)
  float* t;
  int64_t ld_t, mst;          // mst: t offset between modules
  int32_t module0;
  int32_t mods_per_wg;        // modules computed from one x slice
  int32_t h_in;
  int32_t ks_count;           // K splits (grid y)
  int32_t k_per_split;        // multiple of 32
  int32_t ldr;                // rank columns of a partial tile (multiple of 16)
  float* part;                // [tiles][groups][mods_per_wg][ks_count][64][ldr]
  int32_t* tickets;           // [tiles][groups], zero between calls
};

__global__ __launch_bounds__(kMfmaThreads) void k_shrink_mfma(ShrinkArgs a) {
  __shared__ int32_t toks_s[kTileTokens];
  __shared__ int last_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = blockIdx.y;
  const int grp = blockIdx.z;
  const int groups = gridDim.z;
  const int n_tiles = a.sv.meta[LORA_META_N_TILES];
  const int32_t h = static_cast<int32_t>(a.pv.page_elems);
  const __bf16* pages = static_cast<const __bf16*>(a.pv.pages);
  const int k_begin = ks * a.k_per_split;
  const int k_end = min(a.h_in, k_begin + a.k_per_split);
  const int ppr = a.h_in / h;
  const int kq = (lane >> 4) * 8;        // this lane's k offset inside a 32-wide slice
  const int mrow = wave * 16 + (lane & 15);

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int seg = a.sv.tiles[2 * tile], pos = a.sv.tiles[2 * tile + 1];
    const int len = min(kTileTokens, a.sv.seg_start[seg + 1] - pos);
    const int slot = a.sv.seg_slot[seg];
    __syncthreads();
    if (tid < kTileTokens) toks_s[tid] = tid < len ? a.sv.perm[pos + tid] : -1;
    __syncthreads();

    SlotEntry e[kShrinkMaxModules];
#pragma unroll
    for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
      e[mi] = SlotEntry{0, 0.f, 0, 0};
      if (mi < a.mods_per_wg)
        e[mi] = a.pv.entries[slot * a.pv.n_modules + a.module0 + grp * a.mods_per_wg + mi];
    }
    const int tok = toks_s[mrow];
    const __bf16* xrow = a.x + grp * a.msx + static_cast<int64_t>(tok < 0 ? 0 : tok) * a.ld_x + kq;

    f32x4 acc[kShrinkMaxModules][4];
#pragma unroll
    for (int mi = 0; mi < kShrinkMaxModules; ++mi)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mi][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int p = k_begin / h; p * h < k_end; ++p) {
      const int kb = max(k_begin, p * h), ke = min(k_end, (p + 1) * h);
      const __bf16* arow[kShrinkMaxModules][4];
#pragma unroll
      for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int j = nt * 16 + (lane & 15);
          arow[mi][nt] = nullptr;
          if (mi < a.mods_per_wg && j < e[mi].rank)
            arow[mi][nt] = pages + static_cast<int64_t>(a.pv.page_ids[e[mi].a_off + j * ppr + p]) * h -
                           static_cast<int64_t>(p) * h + kq;
        }
      }
      for (int k = kb; k < ke; k += 32) {
        const bf16x8 xf = tok >= 0 ? ld_bf16x8(xrow + k) : bf16x8{};
#pragma unroll
        for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
          if (mi >= a.mods_per_wg) break;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            if (nt * 16 >= e[mi].rank) break;
            const bf16x8 af = arow[mi][nt] ? ld_bf16x8(arow[mi][nt] + k) : bf16x8{};
            acc[mi][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, af, acc[mi][nt], 0, 0, 0);
          }
        }
      }
    }

    // D layout: lane l holds rows 4*(l>>4)+i (token rows of this wave), column l&15 (rank)
    const int rbase = wave * 16 + (lane >> 4) * 4;
    if (a.ks_count == 1) {
#pragma unroll
      for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
        if (mi >= a.mods_per_wg) break;
        float* tm = a.t + (grp * a.mods_per_wg + mi) * a.mst;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int j = nt * 16 + (lane & 15);
          if (nt * 16 >= e[mi].rank) break;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tk = toks_s[rbase + i];
            if (tk >= 0 && j < e[mi].rank) tm[static_cast<int64_t>(tk) * a.ld_t + j] = acc[mi][nt][i];
          }
        }
      }
      continue;
    }

    // split K: write this split's partial tile, take a ticket, the last one reduces
    const int64_t tile_block = static_cast<int64_t>(kTileTokens) * a.ldr;
    const int64_t base_tg = (static_cast<int64_t>(tile) * groups + grp) * a.mods_per_wg;
#pragma unroll
    for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
      if (mi >= a.mods_per_wg) break;
      float* pp = a.part + ((base_tg + mi) * a.ks_count + ks) * tile_block;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt * 16 >= e[mi].rank) break;
        const int j = nt * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[(rbase + i) * a.ldr + j] = acc[mi][nt][i];
      }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&a.tickets[static_cast<int64_t>(tile) * groups + grp], 1);
      last_s = (prev == a.ks_count - 1);
    }
    __syncthreads();
    if (!last_s) continue;
    __threadfence();
#pragma unroll
    for (int mi = 0; mi < kShrinkMaxModules; ++mi) {
      if (mi >= a.mods_per_wg) break;
      const int rank = e[mi].rank;
      float* tm = a.t + (grp * a.mods_per_wg + mi) * a.mst;
      const float* pp = a.part + (base_tg + mi) * a.ks_count * tile_block;
      for (int idx = tid; idx < kTileTokens * rank; idx += kMfmaThreads) {
        const int r = idx / rank, j = idx - r * rank;
        const int tk = toks_s[r];
        if (tk < 0) continue;
        float s = 0.f;
        for (int q = 0; q < a.ks_count; ++q)
          s += __hip_atomic_load(pp + q * tile_block + r * a.ldr + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tm[static_cast<int64_t>(tk) * a.ld_t + j] = s;
      }
    }
    if (tid == 0) a.tickets[static_cast<int64_t>(tile) * groups + grp] = 0;
  }
}

template <typename TO>
__global__ __launch_bounds__(kMfmaThreads) void k_expand_mfma(PoolView pv, int32_t module0, SegView sv,
                                                             const float* __restrict__ t, int64_t ld_t,
                                                             int64_t mst, TO* __restrict__ y, int64_t ld_y,
                                                             int64_t msy, int32_t h_out) {
  constexpr int TN = kExpandCols;
  constexpr int TLD = kMaxRank + 1;   // T_s row stride (floats)
  constexpr int BLD = TN + 16;        // B_s row stride (bf16)
  constexpr int YLD = TN + 4;         // Y_s row stride (floats)
  constexpr int CPR = TN / 8;         // 16-byte chunks per B row / per bf16 y row
  __shared__ float T_s[kTileTokens * TLD];
  __shared__ __bf16 B_s[kMaxRank * BLD];
  __shared__ float Y_s[kTileTokens * YLD];
  __shared__ int32_t toks_s[kTileTokens];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = blockIdx.z;
  const int c0 = blockIdx.y * TN;
  const int n_tiles = sv.meta[LORA_META_N_TILES];
  const int32_t h = static_cast<int32_t>(pv.page_elems);
  const __bf16* pages = static_cast<const __bf16*>(pv.pages);
  const float* tm = t + m * mst;
  TO* ym = y + m * msy;
  const int ppr = h_out / h;
  const int p = c0 / h;              // the column tile lies inside page p of each row
  const int off = c0 - p * h;

  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int seg = sv.tiles[2 * tile], pos = sv.tiles[2 * tile + 1];
    const int len = min(kTileTokens, sv.seg_start[seg + 1] - pos);
    const int slot = sv.seg_slot[seg];
    const SlotEntry e = pv.entries[slot * pv.n_modules + module0 + m];
    if (e.rank <= 0) continue;
    const int rank = e.rank;
    const int r2 = (rank + 1) & ~1;
    __syncthreads();
    if (tid < kTileTokens) toks_s[tid] = tid < len ? sv.perm[pos + tid] : -1;
    __syncthreads();
    // T tile [64][r2] (fp32), zero past rank and for rows without a token
    for (int idx = tid; idx < kTileTokens * r2; idx += kMfmaThreads) {
      const int r = idx / r2, j = idx - r * r2;
      const int tk = toks_s[r];
      T_s[r * TLD + j] = (tk >= 0 && j < rank) ? tm[static_cast<int64_t>(tk) * ld_t + j] : 0.f;
    }
    // B tile [r2][TN] (bf16), rank row j, columns c0..c0+TN of that row
    for (int idx = tid; idx < r2 * CPR; idx += kMfmaThreads) {
      const int j = idx / CPR, c = (idx - j * CPR) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (j < rank) {
        const __bf16* src = pages + static_cast<int64_t>(pv.page_ids[e.b_off + j * ppr + p]) * h + off + c;
        v = *reinterpret_cast<const u32x4*>(src);
      }
      *reinterpret_cast<u32x4*>(&B_s[j * BLD + c]) = v;
    }
    // y tile [64][TN] as fp32
    for (int idx = tid; idx < kTileTokens * CPR; idx += kMfmaThreads) {
      const int r = idx / CPR, c = (idx - r * CPR) * 8;
      const int tk = toks_s[r];
      if (tk >= 0) {
        float f[8];
        load8(ym + static_cast<int64_t>(tk) * ld_y + c0 + c, f);
        *reinterpret_cast<f32x4*>(&Y_s[r * YLD + c]) = f32x4{f[0], f[1], f[2], f[3]};
        *reinterpret_cast<f32x4*>(&Y_s[r * YLD + c + 4]) = f32x4{f[4], f[5], f[6], f[7]};
      }
    }
    __syncthreads();

    // wave w: columns 32w..32w+31, rows 0..31 (acc0) and 32..63 (acc1)
    f32x16 acc0 = {}, acc1 = {};
    const int col = wave * 32 + (lane & 31);
    const int kh = lane >> 5;
    for (int kk = 0; kk < r2; kk += 2) {
      const int kr = kk + kh;
      const float a0 = T_s[(lane & 31) * TLD + kr];
      const float a1 = T_s[(32 + (lane & 31)) * TLD + kr];
      const float b = static_cast<float>(B_s[kr * BLD + col]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc1, 0, 0, 0);
    }
    // D layout: lane l, register v -> row 8*(v/4) + 4*(l/32) + v%4, column l%32
    const float s = e.scale;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * kh + (v & 3);
      Y_s[row * YLD + col] = fmaf(s, acc0[v], Y_s[row * YLD + col]);
      Y_s[(row + 32) * YLD + col] = fmaf(s, acc1[v], Y_s[(row + 32) * YLD + col]);
    }
    __syncthreads();
    for (int idx = tid; idx < kTileTokens * CPR; idx += kMfmaThreads) {
      const int r = idx / CPR, c = (idx - r * CPR) * 8;
      const int tk = toks_s[r];
      if (tk >= 0) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&Y_s[r * YLD + c]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&Y_s[r * YLD + c + 4]);
        const float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        store8(ym + static_cast<int64_t>(tk) * ld_y + c0 + c, f);
      }
    }
  }
}

}  // namespace lora
