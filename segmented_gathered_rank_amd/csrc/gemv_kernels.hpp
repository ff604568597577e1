// GEMV (vector ALU) path: short segments and decode tokens.
//
// A work unit is up to kUnitTokens tokens of one segment, i.e. tokens that
// share one adapter ("BGMV ... one adapter per decode token" and SGMV's
// segments, study page "The kernel trick").  One 256-thread workgroup takes a
// unit and reads each gathered page of its adapter once for all its tokens.
//
// shrink: t[tb][j] = sum_k x[tok_tb][k] * A[j][k].  The 256 threads split k
//         (16-byte loads, 8 elements each, so a wave reads 1 KiB of a row
//         per instruction); each lane keeps RG x NT partial sums, which a
//         wave64 transpose-reduction (DPP row ops and ds_bpermute) folds into
//         one sum per lane, and four wave partials are added in LDS in a
//         fixed order (deterministic, no float atomics).
// expand: y[tok_tb][c] = round(y + scale * sum_j t[tb][j] * B[j][c]).  Each
//         thread owns 8 consecutive columns, streams the rank rows of B with
//         16-byte loads (16 rows in flight) and updates y in place, one
//         rounding per element.
#pragma once

#include "common.hpp"

namespace lora {

constexpr int kGemvThreads = 256;

template <typename TI, int NT>
__device__ __forceinline__ void shrink_unit(const TI* __restrict__ x, int64_t ld_x, const int32_t* toks,
                                            int nt, const TI* __restrict__ pages,
                                            const int32_t* __restrict__ pids_a, int32_t h, int32_t h_in,
                                            int32_t rank, float* t_s, float* red_s) {
  constexpr int RG = (NT >= 8) ? 8 : 16;   // rank rows per pass
  constexpr int V = RG * NT;               // partial sums per lane
  constexpr int G = 64 / V;                // lanes holding the same reduced value
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_chunks = h_in >> 3;
  const int ppr = h_in / h;
  int64_t xoff[NT];
#pragma unroll
  for (int tb = 0; tb < NT; ++tb) xoff[tb] = static_cast<int64_t>(toks[tb < nt ? tb : 0]) * ld_x;

  for (int g = 0; g < rank; g += RG) {
    float acc[64];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int c = tid; c < n_chunks; c += kGemvThreads) {
      const int k = c << 3;
      const int p = k / h;
      const int off = k - p * h;
      float xv[NT][8];
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (tb < nt) {
          load8(x + xoff[tb] + k, xv[tb]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[tb][e] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const int j = g + q;
        if (j < rank) {
          float av[8];
          load8(pages + static_cast<int64_t>(pids_a[j * ppr + p]) * h + off, av);
#pragma unroll
          for (int tb = 0; tb < NT; ++tb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q * NT + tb] = fmaf(av[e], xv[tb][e], acc[q * NT + tb]);
          }
        }
      }
    }
    const float r = wave_transpose_reduce<V>(acc, lane);
    if ((lane % G) == 0) red_s[wave * 64 + lane / G] = r;
    __syncthreads();
    if (tid < V) {
      const float s = ((red_s[tid] + red_s[64 + tid]) + red_s[128 + tid]) + red_s[192 + tid];
      const int q = tid / NT, tb = tid % NT;
      if (g + q < rank && tb < nt) t_s[tb * kMaxRank + g + q] = s;
    }
    __syncthreads();
  }
}

template <typename TI, typename TO, int NT>
__device__ __forceinline__ void expand_unit(TO* __restrict__ y, int64_t ld_y, const int32_t* toks, int nt,
                                            const TI* __restrict__ pages, const int32_t* __restrict__ pids_b,
                                            int32_t h, int32_t h_out, int32_t rank, float scale,
                                            const float* t_s) {
  constexpr int JB = (sizeof(TI) == 2) ? 16 : 8;   // rank rows of B in flight
  const int tid = threadIdx.x;
  const int n_chunks = h_out >> 3;
  const int ppr = h_out / h;
  int64_t yoff[NT];
#pragma unroll
  for (int tb = 0; tb < NT; ++tb) yoff[tb] = static_cast<int64_t>(toks[tb < nt ? tb : 0]) * ld_y;

  for (int c = tid; c < n_chunks; c += kGemvThreads) {
    const int k = c << 3;
    const int p = k / h;
    const int off = k - p * h;
    float acc[NT][8];
#pragma unroll
    for (int tb = 0; tb < NT; ++tb)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[tb][e] = 0.f;
    for (int j0 = 0; j0 < rank; j0 += JB) {
      float bv[JB][8];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (j0 + jj < rank) {
          load8(pages + static_cast<int64_t>(pids_b[(j0 + jj) * ppr + p]) * h + off, bv[jj]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[jj][e] = 0.f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
#pragma unroll
        for (int tb = 0; tb < NT; ++tb) {
          const float tv = t_s[tb * kMaxRank + j0 + jj];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[tb][e] = fmaf(tv, bv[jj][e], acc[tb][e]);
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < NT; ++tb) {
      if (tb < nt) {
        TO* yp = y + yoff[tb] + k;
        float yv[8];
        load8(yp, yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) yv[e] = fmaf(scale, acc[tb][e], yv[e]);
        store8(yp, yv);
      }
    }
  }
}

// Loads a unit's tokens into LDS and clears its t rows.  Ends with a barrier.
__device__ __forceinline__ void unit_prologue(const SegView& sv, int pos, int nt, int32_t* toks_s, float* t_s) {
  __syncthreads();   // the previous unit is done with the LDS buffers
  if (threadIdx.x < kUnitTokens) toks_s[threadIdx.x] = threadIdx.x < nt ? sv.perm[pos + threadIdx.x] : 0;
  for (int i = threadIdx.x; i < kUnitTokens * kMaxRank; i += kGemvThreads) t_s[i] = 0.f;
  __syncthreads();
}

// Fused BGMV: shrink and expand of each unit, t kept in LDS.
template <typename TI, typename TO>
__global__ __launch_bounds__(kGemvThreads) void k_bgmv(PoolView pv, int32_t module0, SegView sv,
                                                      const TI* __restrict__ x, int64_t ld_x, int64_t msx,
                                                      TO* __restrict__ y, int64_t ld_y, int64_t msy,
                                                      int32_t h_in, int32_t h_out) {
  __shared__ float t_s[kUnitTokens * kMaxRank];
  __shared__ float red_s[4 * 64];
  __shared__ int32_t toks_s[kUnitTokens];
  const int m = blockIdx.y;
  const int n_units = sv.meta[LORA_META_N_UNITS_ALL];
  const TI* xm = x + m * msx;
  TO* ym = y + m * msy;
  const TI* pages = static_cast<const TI*>(pv.pages);
  const int32_t h = static_cast<int32_t>(pv.page_elems);
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int seg = sv.units[2 * u], pos = sv.units[2 * u + 1];
    const int nt = min(kUnitTokens, sv.seg_start[seg + 1] - pos);
    const int slot = sv.seg_slot[seg];
    const SlotEntry e = pv.entries[slot * pv.n_modules + module0 + m];
    if (e.rank <= 0) continue;
    unit_prologue(sv, pos, nt, toks_s, t_s);
    const int32_t* pa = pv.page_ids + e.a_off;
    const int32_t* pb = pv.page_ids + e.b_off;
    if (nt == 1) {
      shrink_unit<TI, 1>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
      expand_unit<TI, TO, 1>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    } else if (nt == 2) {
      shrink_unit<TI, 2>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
      expand_unit<TI, TO, 2>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    } else if (nt <= 4) {
      shrink_unit<TI, 4>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
      expand_unit<TI, TO, 4>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    } else {
      shrink_unit<TI, 8>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
      expand_unit<TI, TO, 8>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    }
  }
}

// Shrink only: t rows written to global memory (t[tok][j], j < rank).
// units_word selects the unit list: short segments only, or all segments.
template <typename TI>
__global__ __launch_bounds__(kGemvThreads) void k_shrink_gemv(PoolView pv, int32_t module0, SegView sv,
                                                             int32_t units_word, const TI* __restrict__ x,
                                                             int64_t ld_x, int64_t msx, float* __restrict__ t,
                                                             int64_t ld_t, int64_t mst, int32_t h_in) {
  __shared__ float t_s[kUnitTokens * kMaxRank];
  __shared__ float red_s[4 * 64];
  __shared__ int32_t toks_s[kUnitTokens];
  const int m = blockIdx.y;
  const int n_units = sv.meta[units_word];
  const TI* xm = x + m * msx;
  float* tm = t + m * mst;
  const TI* pages = static_cast<const TI*>(pv.pages);
  const int32_t h = static_cast<int32_t>(pv.page_elems);
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int seg = sv.units[2 * u], pos = sv.units[2 * u + 1];
    const int nt = min(kUnitTokens, sv.seg_start[seg + 1] - pos);
    const int slot = sv.seg_slot[seg];
    const SlotEntry e = pv.entries[slot * pv.n_modules + module0 + m];
    if (e.rank <= 0) continue;
    unit_prologue(sv, pos, nt, toks_s, t_s);
    const int32_t* pa = pv.page_ids + e.a_off;
    if (nt == 1) shrink_unit<TI, 1>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
    else if (nt == 2) shrink_unit<TI, 2>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
    else if (nt <= 4) shrink_unit<TI, 4>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
    else shrink_unit<TI, 8>(xm, ld_x, toks_s, nt, pages, pa, h, h_in, e.rank, t_s, red_s);
    for (int i = threadIdx.x; i < nt * e.rank; i += kGemvThreads) {
      const int tb = i / e.rank, j = i - tb * e.rank;
      tm[static_cast<int64_t>(toks_s[tb]) * ld_t + j] = t_s[tb * kMaxRank + j];
    }
  }
}

// Expand only: t rows read from global memory.
template <typename TI, typename TO>
__global__ __launch_bounds__(kGemvThreads) void k_expand_gemv(PoolView pv, int32_t module0, SegView sv,
                                                             int32_t units_word, const float* __restrict__ t,
                                                             int64_t ld_t, int64_t mst, TO* __restrict__ y,
                                                             int64_t ld_y, int64_t msy, int32_t h_out) {
  __shared__ float t_s[kUnitTokens * kMaxRank];
  __shared__ int32_t toks_s[kUnitTokens];
  const int m = blockIdx.y;
  const int n_units = sv.meta[units_word];
  const float* tm = t + m * mst;
  TO* ym = y + m * msy;
  const TI* pages = static_cast<const TI*>(pv.pages);
  const int32_t h = static_cast<int32_t>(pv.page_elems);
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int seg = sv.units[2 * u], pos = sv.units[2 * u + 1];
    const int nt = min(kUnitTokens, sv.seg_start[seg + 1] - pos);
    const int slot = sv.seg_slot[seg];
    const SlotEntry e = pv.entries[slot * pv.n_modules + module0 + m];
    if (e.rank <= 0) continue;
    unit_prologue(sv, pos, nt, toks_s, t_s);
    for (int i = threadIdx.x; i < nt * e.rank; i += kGemvThreads) {
      const int tb = i / e.rank, j = i - tb * e.rank;
      t_s[tb * kMaxRank + j] = tm[static_cast<int64_t>(toks_s[tb]) * ld_t + j];
    }
    __syncthreads();
    const int32_t* pb = pv.page_ids + e.b_off;
    if (nt == 1) expand_unit<TI, TO, 1>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    else if (nt == 2) expand_unit<TI, TO, 2>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    else if (nt <= 4) expand_unit<TI, TO, 4>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
    else expand_unit<TI, TO, 8>(ym, ld_y, toks_s, nt, pages, pb, h, h_out, e.rank, e.scale, t_s);
  }
}

}  // namespace lora
