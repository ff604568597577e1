// Matrix-core path for long segments (the study page's SGMV, meant for runs
// of tokens with one adapter such as a prefill; section "The kernel trick:
// gather, do not merge").  A
// segment of L >= kLongMin tokens is a dense grouped contraction, so it is cut
// into tiles of kTileTokens tokens and run on CDNA4 MFMA.
//
// shrink (bf16 in, fp32 accumulate): T[64 x r] = X[64 x K] * A^T[K x r] with
//   v_mfma_f32_16x16x32_bf16.  Wave w owns tokens 16w..16w+15 of the tile;
//   one MFMA takes a 16 x 32 slice of X (each lane 8 consecutive bf16 of one
//   token row, loaded straight from row-major memory: a wave's load covers 64
//   bytes of 16 rows, and the next step's load the rest of their 128-byte
//   lines) and a 32 x 16 slice of A^T (each lane 8 consecutive bf16 of one
//   rank row, from the A rows staged in LDS).  When
//   several modules share x (q, k, v), one workgroup computes all of them from
//   one read of the x slice.  K may be split across workgroups to fill the
//   chip; the partial tiles then go to a workspace and a second launch adds
//   them in split order (deterministic; the launch boundary orders the writes
//   and reads, so no device-wide fence is needed inside a kernel).
// expand (fp32 t, bf16 B, y bf16 or fp32): Y[64 x 128] += s * T[64 x r] B[r x 128]
//   with v_mfma_f32_32x32x16_bf16.  t is split into three bf16 parts whose sum
//   is t exactly, so the matrix cores multiply by t itself (three MFMAs per K
//   step of 16 instead of eight fp32 32x32x2 steps); formed transposed so that
//   the accumulators map onto y rows (see expand_mfma_body).
#pragma once

#include "common.hpp"
#include "gemv_kernels.hpp"   // Quad<T>: four-element loads and stores

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 256;
constexpr int kShrinkMaxModules = 4;   // modules sharing one x slice in a workgroup
constexpr int kExpandCols = 128;       // output columns per expand block
#ifndef LORA_EXPAND_BLOCKS
#define LORA_EXPAND_BLOCKS 8
#endif
constexpr int kExpandBlocks = LORA_EXPAND_BLOCKS;   // column blocks per expand workgroup, at most

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
  uint32_t magic;             // reciprocal of the page size
  int32_t ks_count;           // K splits (grid y)
  int32_t k_per_split;        // multiple of 32
  int32_t kc;                 // K of A rows staged in LDS at a time (multiple of 32)
  int32_t ldr;                // rank rows per module in LDS and columns of a partial tile (multiple of 16)
  int32_t max_pids;           // page ids per entry in LDS
  float* part;                // partial tiles [tile][part_nm][ks_count][64][ldr]; this launch's
  int32_t part_m0, part_nm;   // module m at part_m0 + m of part_nm (a call's modules may span launches)
};

#ifndef LORA_STAGE_BATCH
#define LORA_STAGE_BATCH 8
#endif
constexpr int kMaxSplits = 8;                     // K splits of the shrink at most
constexpr int kStageBatch = LORA_STAGE_BATCH;     // 16-byte chunks of A each thread loads at once when staging

// Streaming shrink tile: 64 tokens x one K split, for MODS modules that share
// the x slice.  The A rows of the split (every module, rank rows padded to
// the tile width) are staged in LDS once, while the first x loads are
// already in flight.  After that one barrier the four waves are independent:
// wave w owns tokens 16w..16w+15 and streams its x fragments straight from
// memory, D steps of 32 k ahead of the matrix cores, to the end of the split
// with no further barrier; A comes from LDS.  A split whose A rows do not fit
// in LDS is run as consecutive sub-ranges of a.kc elements, each staged the
// same way.
// Grid (b): x over tiles, y over K splits, z over module groups.
template <int MODS, int NTILES, int D>
__device__ __forceinline__ void shrink_stream_body(const ShrinkArgs& a, const Blk b, unsigned char* smem) {
  static_assert(MODS >= 1 && MODS <= kShrinkMaxModules && NTILES >= 1 && NTILES <= 4 && D >= 1, "tile shape");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = b.y;
  const int grp = b.z;
  const int groups = b.nz;
  const int n_tiles = a.sv.meta[LORA_META_N_TILES];
  const int32_t h = static_cast<int32_t>(a.pv.page_elems);
  const __bf16* pages = static_cast<const __bf16*>(a.pv.pages);
  const int k_split = ks * a.k_per_split;
  const int k_split_end = min(a.h_in, k_split + a.k_per_split);
  // A_s row stride (bf16): kc / 2 + 8 words, 8 mod 16.  A 16-byte fragment read serves
  // its lanes in four rounds of 16, each round two runs of 8 lanes (0-7 with 24-31,
  // 8-15 with 16-23, and the same in the upper half); lane l reads row l % 16 at
  // column group l / 16, so a round's 16 reads cover 16 distinct 4-bank groups with
  // this stride.  With kc + 8 (4 mod 16 words) lanes 0 and 31 met in one group.
  const int ALD = a.kc + 16;
  __bf16* A_s = reinterpret_cast<__bf16*>(smem);              // [MODS][16*NTILES][ALD]
  int32_t* pid_s = reinterpret_cast<int32_t*>(smem + static_cast<size_t>(MODS) * 16 * NTILES * ALD * 2);
  __shared__ int32_t toks_s[kTileTokens];
  const int ppr = a.h_in / h;
  const int kq = (lane >> 4) * 8;        // this lane's k offset inside a 32-wide step
  const int mrow = wave * 16 + (lane & 15);

  const int2* tiles = reinterpret_cast<const int2*>(a.sv.tiles);
  int tile = item_of_block<kTileRun>(b.x, b.y + b.ny * b.z);
  int2 rec = tiles[min(tile, a.sv.max_tiles - 1)];
  const int n_ids = min(a.ldr, a.pv.max_rank) * ppr;
  for (; tile < n_tiles; tile += b.nx) {
    if (tile >= b.nx) rec = tiles[tile];
    const int slot = rec.x & 0xffff, len = rec.x >> 16, pos = rec.y;
    int rank[MODS];
#pragma unroll
    for (int mi = 0; mi < MODS; ++mi) rank[mi] = a.pv.entries[slot * a.pv.n_modules + a.module0 + grp * MODS + mi].rank;
    __syncthreads();                     // the previous tile is done with toks_s and pid_s
    if (tid < kTileTokens) toks_s[tid] = tid < len ? a.sv.perm[pos + tid] : -1;
#pragma unroll
    for (int mi = 0; mi < MODS; ++mi) {
      const int32_t* ids =
          a.pv.page_ids + static_cast<int64_t>(slot * a.pv.n_modules + a.module0 + grp * MODS + mi) * a.pv.ppe;
      for (int i = tid; i < n_ids; i += kMfmaThreads) pid_s[mi * a.max_pids + i] = ids[i];
    }
    __syncthreads();
    // rows without a token read row 0 of x: an output row depends only on its own x row,
    // and those rows are never stored
    const int tok = toks_s[mrow];
    f32x4 acc[MODS][NTILES];
#pragma unroll
    for (int mi = 0; mi < MODS; ++mi)
#pragma unroll
      for (int nt = 0; nt < NTILES; ++nt) acc[mi][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k_begin = k_split; k_begin < k_split_end; k_begin += a.kc) {
    const int klen = min(a.kc, k_split_end - k_begin);
    const int n = klen >> 5;               // 32-wide steps of the sub-range
    const __bf16* xrow = a.x + grp * a.msx + static_cast<int64_t>(tok < 0 ? 0 : tok) * a.ld_x + k_begin + kq;
    if (k_begin != k_split) __syncthreads();   // every wave is done with the previous sub-range's A

    // x prologue: steps 0..D-1 (a split shorter than D steps repeats its last step)
    bf16x8 xb[D];
#pragma unroll
    for (int i = 0; i < D; ++i) xb[i] = ld_bf16x8(xrow + 32 * min(i, n - 1));
    // A rows of the split into LDS.  Rows past a module's rank read its last row: they only
    // feed output columns past the rank, which are never stored.
    const int cpr = klen >> 3;                                  // 16-byte chunks per row
    // through registers, kStageBatch chunks per thread at a time, every lane busy
    auto stage_regs = [&]() {
      const int n_chunks = MODS * 16 * NTILES * cpr;
      for (int c0 = 0; c0 < n_chunks; c0 += kMfmaThreads * kStageBatch) {
        u32x4 av[kStageBatch];
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int idx = min(c0 + tid + kMfmaThreads * q, n_chunks - 1);
          const int row = idx / cpr, c = idx - row * cpr;
          const int mi = row / (16 * NTILES), j = row - mi * (16 * NTILES);
          int rank_mi = 0;
#pragma unroll
          for (int m2 = 0; m2 < MODS; ++m2)
            if (m2 == mi) rank_mi = rank[m2];
          const int jj = max(0, min(j, rank_mi - 1));
          const int k = k_begin + c * 8;
          const int pg = ppr == 1 ? 0 : static_cast<int>(__umulhi(static_cast<uint32_t>(k), a.magic));
          const int pid = rank_mi > 0 ? pid_s[mi * a.max_pids + jj * ppr + pg] : 0;
          av[q] = *reinterpret_cast<const u32x4*>(pages + static_cast<int64_t>(pid) * h + (k - pg * h));
        }
#pragma unroll
        for (int q = 0; q < kStageBatch; ++q) {
          const int idx = c0 + tid + kMfmaThreads * q;
          if (idx < n_chunks) {
            const int row = idx / cpr, c = idx - row * cpr;
            *reinterpret_cast<u32x4*>(A_s + static_cast<size_t>(row) * ALD + c * 8) = av[q];
          }
        }
      }
    };
    // straight from memory into LDS (global_load_lds, no registers), all rows in one round
    // trip, for rows of 1 KiB or more.  Wave w takes rows w, w + 4, ...; one instruction
    // moves up to 64 chunks of a row (lane i lands at byte 16 i of the instruction's LDS
    // base; lanes past the row stay idle).  Only shapes whose A slice fits such rows in the
    // LDS budget (modules x 16-column tiles <= 3) compile it: the others would lose a wave.
    auto stage_dma = [&]() {
      for (int row = wave; row < MODS * 16 * NTILES; row += kMfmaThreads / 64) {
        const int mi = row / (16 * NTILES), j = row - mi * (16 * NTILES);
        int rank_mi = 0;
#pragma unroll
        for (int m2 = 0; m2 < MODS; ++m2)
          if (m2 == mi) rank_mi = rank[m2];
        const int jj = max(0, min(j, rank_mi - 1));
        for (int c0 = 0; c0 < cpr; c0 += 64) {
          const int c = c0 + lane;
          if (c < cpr) {
            const int k = k_begin + c * 8;
            const int pg = ppr == 1 ? 0 : static_cast<int>(__umulhi(static_cast<uint32_t>(k), a.magic));
            const int pid = rank_mi > 0 ? pid_s[mi * a.max_pids + jj * ppr + pg] : 0;
            __builtin_amdgcn_global_load_lds(pages + static_cast<int64_t>(pid) * h + (k - pg * h),
                                             to_lds(A_s + static_cast<size_t>(row) * ALD + c0 * 8), 16, 0, 0);
          }
        }
      }
    };
    if constexpr (MODS * NTILES <= 3) {
      if (cpr >= 64) stage_dma();   // uniform
      else stage_regs();
    } else {
      stage_regs();
    }
    __syncthreads();   // A has landed (the barrier waits for the loads into LDS)

    // this lane's A row of each (module, 16-column tile) in LDS
    const __bf16* arow = A_s + static_cast<size_t>(lane & 15) * ALD + kq;
    auto consume = [&](int i, int s) {
#pragma unroll
      for (int mi = 0; mi < MODS; ++mi)
#pragma unroll
        for (int nt = 0; nt < NTILES; ++nt)
          if (nt * 16 < rank[mi]) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(arow + static_cast<size_t>(mi * 16 * NTILES + nt * 16) * ALD + 32 * s);
            acc[mi][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[i], af, acc[mi][nt], 0, 0, 0);
          }
    };
    int s0 = 0;
    for (; s0 + 2 * D <= n; s0 += D) {   // every refill is in range
#pragma unroll
      for (int i = 0; i < D; ++i) {
        consume(i, s0 + i);
        xb[i] = ld_bf16x8(xrow + 32 * (s0 + D + i));
      }
    }
    // the last 1..2D-1 steps: buffer i holds step s0+i, then step s0+D+i
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s0 + i < n) consume(i, s0 + i);
      if (s0 + D + i < n) xb[i] = ld_bf16x8(xrow + 32 * (s0 + D + i));
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (s0 + D + i < n) consume(i, s0 + D + i);
    }

    // D layout: lane l holds rows 4*(l>>4)+i (token rows of this wave), column l&15 (rank)
    const int rbase = wave * 16 + (lane >> 4) * 4;
    if (a.ks_count == 1) {
#pragma unroll
      for (int mi = 0; mi < MODS; ++mi) {
        float* tm = a.t + (grp * MODS + mi) * a.mst;
#pragma unroll
        for (int nt = 0; nt < NTILES; ++nt) {
          const int j = nt * 16 + (lane & 15);
          if (nt * 16 >= rank[mi]) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tk = toks_s[rbase + i];
            if (tk >= 0 && j < rank[mi]) tm[static_cast<int64_t>(tk) * a.ld_t + j] = acc[mi][nt][i];
          }
        }
      }
      continue;
    }
    // split K: this split's partial tile goes to the workspace; k_shrink_reduce
    // (the next launch on the stream) adds the splits in order
    const int64_t tile_block = static_cast<int64_t>(kTileTokens) * a.ldr;
    const int64_t base_tg = static_cast<int64_t>(tile) * a.part_nm + a.part_m0 + grp * MODS;
#pragma unroll
    for (int mi = 0; mi < MODS; ++mi) {
      float* pp = a.part + ((base_tg + mi) * a.ks_count + ks) * tile_block;
#pragma unroll
      for (int nt = 0; nt < NTILES; ++nt) {
        if (nt * 16 >= rank[mi]) continue;
        const int j = nt * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) pp[(rbase + i) * a.ldr + j] = acc[mi][nt][i];
      }
    }
  }
}

// LDS of shrink_stream_body: a sub-range's A rows [mods][16*ntiles][kc + 16] bf16 and
// the tile's A page ids [mods][max_pids].
__host__ __device__ inline size_t stream_lds_bytes(int mods, int ntiles, int kc, int max_pids) {
  return static_cast<size_t>(mods) * 16 * ntiles * (kc + 16) * 2 + static_cast<size_t>(mods) * max_pids * 4;
}

// Prefetch depth of shrink_stream_body: 32-wide steps of x in flight per wave
// (16 bytes per lane each).
#ifndef LORA_STREAM_DEPTH
#define LORA_STREAM_DEPTH 8
#endif
constexpr int kStreamDepth = LORA_STREAM_DEPTH;

// Sum of the K splits of each tile, in split order: t[tok][j] = sum_q part[q].
// One workgroup per (tile, module); grid (tiles, groups * mods_per_wg).
__global__ __launch_bounds__(kMfmaThreads) void k_shrink_reduce(ShrinkArgs a) {
  const int n_tiles = a.sv.meta[LORA_META_N_TILES];
  const int gm = blockIdx.y;                        // group * mods_per_wg + module in group
  const int64_t tile_block = static_cast<int64_t>(kTileTokens) * a.ldr;
  const int2* tiles = reinterpret_cast<const int2*>(a.sv.tiles);
  int tile = item_of_block<kTileRun>(blockIdx.x, static_cast<int>(blockIdx.y + gridDim.y * blockIdx.z));
  int2 rec = tiles[min(tile, a.sv.max_tiles - 1)];
  for (; tile < n_tiles; tile += gridDim.x) {
    if (tile >= static_cast<int>(gridDim.x)) rec = tiles[tile];
    const int slot = rec.x & 0xffff, len = rec.x >> 16, pos = rec.y;
    const int rank = a.pv.entries[slot * a.pv.n_modules + a.module0 + gm].rank;
    const float* pp = a.part + (static_cast<int64_t>(tile) * gridDim.y + gm) * a.ks_count * tile_block;
    float* tm = a.t + gm * a.mst;
    // items: (token row r, 4 rank columns from 4q); two items per thread at a time, with
    // every split's 16-byte load of both in flight together
    const int nq = (rank + 3) >> 2;
    const int n_items = len * nq;
    constexpr int U = 2;
    for (int i0 = threadIdx.x; i0 < n_items; i0 += U * kMfmaThreads) {
      f32x4 part[U][kMaxSplits];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = min(i0 + u * kMfmaThreads, n_items - 1);
        const int r = idx / nq, j = (idx - r * nq) * 4;
#pragma unroll
        for (int q = 0; q < kMaxSplits; ++q)
          part[u][q] = *reinterpret_cast<const f32x4*>(pp + min(q, a.ks_count - 1) * tile_block + r * a.ldr + j);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = i0 + u * kMfmaThreads;
        if (idx >= n_items) continue;
        const int r = idx / nq, j = (idx - r * nq) * 4;
        f32x4 sum = part[u][0];
#pragma unroll
        for (int q = 1; q < kMaxSplits; ++q)
          if (q < a.ks_count) sum += part[u][q];   // splits added in order
        float* dst = tm + static_cast<int64_t>(a.sv.perm[pos + r]) * a.ld_t + j;
        if (j + 4 <= rank) {
          *reinterpret_cast<f32x4*>(dst) = sum;
        } else {                                    // columns past the rank are not written
          for (int e = 0; e < rank - j; ++e) dst[e] = sum[e];
        }
      }
    }
  }
}

// Expand tile: 64 tokens x up to kExpandBlocks blocks of kExpandCols columns of one
// module.  The product is formed transposed, Y^T[cols x tokens] += B^T[cols x r]
// T^T[r x tokens] (v_mfma_f32_32x32x2_f32: lane l holds token l%32 and, for
// i = 0..3, columns 8i + 4(l/32) .. +3 of its wave's 32).  y moves between HBM
// and an LDS tile with coalesced 16-byte row accesses (a wave covers whole
// rows), and between LDS and the MFMA layout with 8- or 16-byte accesses.
// T (fp32) is staged once per tile, the B block (bf16) once per column block.
// LDS of expand_mfma_body for pool rank cap ldr and y element size ysz: the
// three bf16 parts of the T tile [3][64][r16+8], the B block [r16][kExpandBRow]
// (bf16, rank rows as stored) and the y block [64][128 + 16/ysz].
constexpr int kExpandBRow = kExpandCols + 32;   // B block row stride (bf16): 80 words, 16 mod 64 banks
__host__ __device__ inline int expand_r16(int ldr) { return (ldr + 15) & ~15; }
__host__ __device__ inline size_t expand_lds_bytes(int ldr, int ysz) {
  const size_t ld = static_cast<size_t>(expand_r16(ldr) + 8);
  return 3 * kTileTokens * ld * 2 + static_cast<size_t>(expand_r16(ldr)) * kExpandBRow * 2 +
         static_cast<size_t>(kTileTokens) * (kExpandCols + 16 / ysz) * ysz;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
// LDS transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane 4r + q gives the
// address of 4 consecutive bf16 values; lane i receives, in slot r, value i % 4 of lane
// 4r + i / 4's four.  So with lane 4r + q pointing at column c + 4q of row j + r, lane i
// gets rows j .. j + 3 of column c + i.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<lds_bf16x4_t*>(reinterpret_cast<uintptr_t>(p)));
}

struct ExpandArgs {
  PoolView pv;
  SegView sv;
  const float* t;
  int64_t ld_t, mst;          // mst: t offset between modules
  void* y;
  int64_t ld_y, msy;          // msy: y offset between modules
  int32_t module0;
  int32_t h_out;
  int32_t ldr;                // rank cap of the pool rounded up to 16
  int32_t b_ids_at;           // offset of B's page ids in a (slot, module) page table
  int32_t blocks;             // column blocks per workgroup (<= kExpandBlocks)
  const float* part;          // the shrink's K-split partial tiles [tile][module][split][64][ldr] (PQ > 0)
  int32_t ks;                 // their split count
};

// Grid (b): x over tiles, y over groups of ea.blocks column blocks, z over modules.
// PQ = 0: the T tile comes from t (rows by token id).  PQ = ldr / 16 > 0: it is
// the sum, in split order, of the shrink's K-split partial tiles (rows by tile
// row), which the shrink leaves in the workspace in place of t: each thread
// loads PQ 16-byte column groups of its row per split, the first batch of
// splits together with the tile's entry, token ids and page ids.
template <typename TO, int PQ>
__device__ __forceinline__ void expand_mfma_body(const ExpandArgs& ea, const Blk b, unsigned char* smem) {
  const PoolView& pv = ea.pv;
  const SegView& sv = ea.sv;
  const int32_t module0 = ea.module0, h_out = ea.h_out, ldr = ea.ldr, b_ids_at = ea.b_ids_at;
  const int64_t ld_t = ea.ld_t, mst = ea.mst, ld_y = ea.ld_y, msy = ea.msy;
  const float* __restrict__ t = ea.t;
  TO* __restrict__ y = static_cast<TO*>(ea.y);
  constexpr int TN = kExpandCols;
  constexpr int YLD = TN + 16 / sizeof(TO);           // Y_s row stride (elements)
  constexpr int YCPR = TN * sizeof(TO) / 16;          // 16-byte chunks per y row of the block
  constexpr int YCH = kTileTokens * YCPR / kMfmaThreads;   // y chunks per thread
  constexpr int YV = 16 / sizeof(TO);                 // elements per 16-byte chunk
  const int r16 = expand_r16(ldr);
  const int LD = r16 + 8;                             // row stride of T3_s (bf16)
  __bf16* T3_s = reinterpret_cast<__bf16*>(smem);                                  // [3][64][LD]
  __bf16* B_s = T3_s + 3 * kTileTokens * LD;                                       // [r16][kExpandBRow]
  TO* Y_s = reinterpret_cast<TO*>(B_s + r16 * kExpandBRow);                         // [64][YLD]
  __shared__ int32_t toks_s[kTileTokens];
  __shared__ int32_t bids_s[kMaxEntryPages];   // B page ids of the tile's (slot, module): row j, page p at j*ppr + p

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = b.z;
  const int n_tiles = sv.meta[LORA_META_N_TILES];
  const int32_t h = static_cast<int32_t>(pv.page_elems);
  const __bf16* pages = static_cast<const __bf16*>(pv.pages);
  const float* tm = t + m * mst;
  TO* ym = y + m * msy;
  const int ppr = h_out / h;
  const int l32 = lane & 31, kh = lane >> 5;

  // the tile count and this workgroup's first tile record travel together; the
  // entry, the B page ids (fixed table layout, from b_ids_at) and the token ids
  // then load in one round trip, and t, y and the B rows in the next
  const int2* tiles = reinterpret_cast<const int2*>(sv.tiles);
  int tile = item_of_block<kTileRun>(b.x, b.y + b.ny * b.z);
  int2 rec = tiles[min(tile, sv.max_tiles - 1)];
  const int n_bids = pv.max_rank * ppr;
  // partial tiles: splits [s0, s0 + PG) of tile tl into pt (PG * PQ * 4 registers per batch)
  constexpr int PG = PQ <= 2 ? kMaxSplits : kMaxSplits / 2;
  constexpr int PQN = PQ > 0 ? PQ : 1;
  const int64_t tile_block = static_cast<int64_t>(kTileTokens) * ldr;
  f32x4 pt[PG][PQN];
  auto load_parts = [&](int tl, int s0) {
    int lt = tid;
    __asm__ volatile("" : "+v"(lt));   // per-call thread offsets: nothing hoisted out of the tile loop
    const float* pp = ea.part + ((static_cast<int64_t>(tl) * b.nz + m) * ea.ks + s0) * tile_block +
                      (lt >> 2) * ldr + 4 * (lt & 3);
#pragma unroll
    for (int u = 0; u < PG; ++u)
#pragma unroll
      for (int q = 0; q < PQN; ++q)
        if (s0 + u < ea.ks) pt[u][q] = *reinterpret_cast<const f32x4*>(pp + u * tile_block + 16 * q);
  };
  for (; tile < n_tiles; tile += b.nx) {
    if (tile >= b.nx) rec = tiles[tile];
    if constexpr (PQ > 0) load_parts(tile, 0);   // with the entry, token and page id loads
    const int slot = rec.x & 0xffff, len = rec.x >> 16, pos = rec.y;
    const int ei = slot * pv.n_modules + module0 + m;
    const SlotEntry e = pv.entries[ei];
    const int32_t* bids = pv.page_ids + static_cast<int64_t>(ei) * pv.ppe + b_ids_at;
    __syncthreads();   // the previous tile is done with LDS
    if (tid < kTileTokens) toks_s[tid] = tid < len ? sv.perm[pos + tid] : -1;
    for (int i = tid; i < n_bids; i += kMfmaThreads) bids_s[i] = bids[i];
    __syncthreads();
    if (e.rank <= 0) continue;                 // uniform
    const int rank = e.rank;
    const int rk = (rank + 15) & ~15;          // contraction length: rank rounded up to the MFMA's K
    const int first = toks_s[0];
    // y block cb [64][TN]: coalesced 16-byte chunks, rows without a token read the first token's;
    // B block [rk <= 32 rows][TN] (bf16): rank row j, columns c0..c0+TN of that row
    u32x4 yv[YCH], bv[2];
    // B chunk idx of a block (16-byte chunks, TN / 8 = 16 per rank row, chunk column fastest):
    // a row's 16 chunks are loaded and stored by 16 consecutive lanes
    static_assert(TN / 8 == 16, "16 chunks per rank row of a block");
    auto b_row = [](int idx) { return idx >> 4; };
    auto b_col = [](int idx) { return (idx & 15) * 8; };
    auto issue = [&](int cb, u32x4 (&yq)[YCH], u32x4 (&bq)[2]) {
      const int c0 = (b.y * ea.blocks + cb) * TN;
      const int p = c0 / h;                    // the column block lies inside page p of each row
      const int off = c0 - p * h;
#pragma unroll
      for (int q = 0; q < YCH; ++q) {
        const int idx = tid + kMfmaThreads * q;
        const int r = idx / YCPR, c = (idx % YCPR) * YV;
        const int tk = toks_s[r];
        yq[q] = ld16<LORA_NT_ROWS != 0>(
            reinterpret_cast<const u32x4*>(ym + static_cast<int64_t>(tk >= 0 ? tk : first) * ld_y + c0 + c));
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = min(tid + kMfmaThreads * q, rk * (TN / 8) - 1);
        const int j = b_row(idx), c = b_col(idx);
        bq[q] = *reinterpret_cast<const u32x4*>(pages + static_cast<int64_t>(bids_s[min(j, rank - 1) * ppr + p]) * h +
                                                off + c);
      }
    };
    // B chunk (row j, columns c..c+7) into the block as stored, zero for rows past the rank;
    // the matrix-core loop reads it transposed (lds_read_tr16)
    auto put_b = [&](int j, int c, u32x4 v) {
      if (j >= rank) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&B_s[j * kExpandBRow + c]) = v;
    };
    const int n_cb = min(ea.blocks, (h_out - b.y * ea.blocks * TN + TN - 1) / TN);
    // T tile: t = hi + mid + lo, three bf16 values whose sum is t exactly (3 x 8 significand
    // bits cover fp32's 24), so the bf16 matrix cores multiply by t itself.  From t: thread ->
    // row tid/4, columns (tid%4) + 4q, its loads going out with block 0's.  Each later block's
    // loads are issued as soon as the block before it is staged in LDS.
    // put_t: the three parts of t at T3_s row r, column j (zero past the rank and for rows
    // without a token)
    auto put_t = [&](int r, int j, float t_rj, bool live) {
      const float v = live ? t_rj : 0.f;
      const __bf16 hi = static_cast<__bf16>(v);
      const float r1 = v - static_cast<float>(hi);
      const __bf16 mid = static_cast<__bf16>(r1);
      const __bf16 lo = static_cast<__bf16>(r1 - static_cast<float>(mid));
      T3_s[r * LD + j] = hi;
      T3_s[(kTileTokens + r) * LD + j] = mid;
      T3_s[(2 * kTileTokens + r) * LD + j] = lo;
    };
    if constexpr (PQ > 0) {
      // thread -> tile row tid/4, columns 16q + 4(tid%4) .. +3; splits added in order.  The
      // empty asm keeps the LDS addresses from being hoisted out of the tile loop (they would
      // stay live across the matrix-core blocks and spill)
      int r = tid >> 2, c = 4 * (tid & 3);
      __asm__ volatile("" : "+v"(r), "+v"(c));
      const bool row_live = toks_s[r] >= 0;
      f32x4 sum[PQN];
#pragma unroll
      for (int q = 0; q < PQN; ++q) sum[q] = pt[0][q];
#pragma unroll
      for (int u = 1; u < PG; ++u)
#pragma unroll
        for (int q = 0; q < PQN; ++q)
          if (u < ea.ks) sum[q] += pt[u][q];
      for (int s0 = PG; s0 < ea.ks; s0 += PG) {   // rank caps above 32: the remaining splits
        load_parts(tile, s0);
#pragma unroll
        for (int u = 0; u < PG; ++u)
#pragma unroll
          for (int q = 0; q < PQN; ++q)
            if (s0 + u < ea.ks) sum[q] += pt[u][q];
      }
      if (n_cb > 0) issue(0, yv, bv);   // after the partials are summed: their registers are free
#pragma unroll
      for (int q = 0; q < PQN; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * q + c + e;
          if (j < rk) put_t(r, j, sum[q][e], row_live && j < rank);
        }
    } else {
      const int r = tid >> 2, jq = tid & 3;
      const int tk = toks_s[r];
      const float* trow = tm + static_cast<int64_t>(tk >= 0 ? tk : first) * ld_t;
      float tv[kMaxRank / 4];
#pragma unroll
      for (int q = 0; q < kMaxRank / 4; ++q) tv[q] = trow[min(jq + 4 * q, rank - 1)];
      if (n_cb > 0) issue(0, yv, bv);
#pragma unroll
      for (int q = 0; q < kMaxRank / 4; ++q) {
        const int j = jq + 4 * q;
        if (j < rk) put_t(r, j, tv[q], tk >= 0 && j < rank);
      }
    }
#pragma unroll 1
    for (int cb = 0; cb < kExpandBlocks; ++cb) {   // not unrolled: a full unroll spills
      if (cb >= n_cb) break;                   // uniform
      const int c0 = (b.y * ea.blocks + cb) * TN;
      const int p = c0 / h;
      const int off = c0 - p * h;
      __syncthreads();                         // the previous block's B_s / Y_s reads are done
#pragma unroll
      for (int q = 0; q < YCH; ++q) {
        const int idx = tid + kMfmaThreads * q;
        const int r = idx / YCPR, c = (idx % YCPR) * YV;
        *reinterpret_cast<u32x4*>(Y_s + r * YLD + c) = yv[q];
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + kMfmaThreads * q;
        if (idx < rk * (TN / 8)) put_b(b_row(idx), b_col(idx), bv[q]);
      }
      for (int base = 2 * kMfmaThreads; base < rk * (TN / 8); base += kMfmaThreads) {   // ranks above 32
        const int idx = base + tid;
        if (idx < rk * (TN / 8)) {
          const int j = b_row(idx), c = b_col(idx);
          put_b(j, c, *reinterpret_cast<const u32x4*>(
                          pages + static_cast<int64_t>(bids_s[min(j, rank - 1) * ppr + p]) * h + off + c));
        }
      }
      // the next block's y and B loads fly during this block's matrix-core work, epilogue and
      // store (same registers, now free: no occupancy cost)
      if (cb + 1 < n_cb) issue(cb + 1, yv, bv);
      __syncthreads();

      // Y^T[col][token] += B^T[col][j] T^T[j][token] on v_mfma_f32_32x32x16_bf16: A = B^T
      // (lane -> column l%32 of the wave's 32, j = 8(l/32)..+8), B = one part of T^T (lane ->
      // token l%32 or 32 + l%32, same j), K = 16 per step
      // A from the stored B block by two transpose reads of 4 rank rows: in lane group
      // g = l / 16, lane 4r + q points at row 8(g / 2) + r (+ 4) and column
      // 32 w + 16(g % 2) + 4q, so lane l gets rows j0 .. j0 + 7 of column 32 w + l % 32
      const int tg = lane >> 4, tl = lane & 15;
      const __bf16* bt = B_s + (8 * (tg >> 1) + (tl >> 2)) * kExpandBRow + wave * 32 + 16 * (tg & 1) + 4 * (tl & 3);
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll 1
      for (int kk = 0; kk < rk; kk += 16) {
        const int j0 = kk + 8 * kh;
        const bf16x4 a_lo = lds_read_tr16(bt + kk * kExpandBRow);
        const bf16x4 a_hi = lds_read_tr16(bt + (kk + 4) * kExpandBRow);
        const bf16x8 a = __builtin_shufflevector(a_lo, a_hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int part = 0; part < 3; ++part) {
          const __bf16* tp = T3_s + part * kTileTokens * LD;
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&tp[l32 * LD + j0]);
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&tp[(32 + l32) * LD + j0]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc1, 0, 0, 0);
        }
      }
      // epilogue in LDS: lane l, register 4i+j: column 32w + 8i + 4(l/32) + j, token l%32 (+32)
      const float s = e.scale;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = wave * 32 + 8 * i + 4 * kh;
        float v[4];
        Quad<TO> q0;
        q0.load(Y_s + l32 * YLD + col);
        q0.unpack(v);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = fmaf(s, acc0[4 * i + j], v[j]);
        Quad<TO>::store(Y_s + l32 * YLD + col, v);
        Quad<TO> q1;
        q1.load(Y_s + (32 + l32) * YLD + col);
        q1.unpack(v);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = fmaf(s, acc1[4 * i + j], v[j]);
        Quad<TO>::store(Y_s + (32 + l32) * YLD + col, v);
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < YCH; ++q) {
        const int idx = tid + kMfmaThreads * q;
        const int r = idx / YCPR, c = (idx % YCPR) * YV;
        const int tk = toks_s[r];
        if (tk >= 0)
          *reinterpret_cast<u32x4*>(ym + static_cast<int64_t>(tk) * ld_y + c0 + c) =
              *reinterpret_cast<const u32x4*>(Y_s + r * YLD + c);
      }
    }
  }
}

// A mixed batch in one launch (decode tokens and short segments next to long
// segments, the study page's "one kernel for a mixed batch"): the first
// tnx*tny*tnz workgroups run matrix-core tiles, the rest run GEMV work items
// (a grid of gnx x gny, gny = modules).  Both parts start at multiples of 8 workgroups,
// so each keeps its XCD-aware map, and both take their LDS from the launch's
// dynamic LDS, sized for the larger of the two.
template <int MODS, int NTILES, int D>
__global__ __launch_bounds__(kMfmaThreads) void k_shrink_mixed(ShrinkArgs a, GemvArgs g, int tnx, int tny, int tnz,
                                                               int gnx, int gny) {
  static_assert(kMfmaThreads == kGemvThreads, "both parts run on one workgroup size");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lin = static_cast<int>(blockIdx.x), tile_blocks = tnx * tny * tnz;
  if (lin < tile_blocks) {
    shrink_stream_body<MODS, NTILES, D>(a, blk_of_linear(lin, tnx, tny, tnz), smem);
  } else {
    int it0 = -1;
    const Blk b = g.module_group > 0 ? blk_of_module_groups(lin - tile_blocks, gnx, gny, g.module_group, it0)
                                     : blk_of_linear(lin - tile_blocks, gnx, gny, 1);
    gemv_body<1, __bf16, __bf16>(g, b, *reinterpret_cast<UnitLds*>(smem),
                                 reinterpret_cast<__bf16*>(smem + gemv_xs_offset<1, __bf16>()), it0);
  }
}

// Two shrink launches in one (see launch_shrink_pair): the tiles of run 1 (M1
// modules sharing x), the tiles of run 2 (M2), then the GEMV items of run 1 (n1
// modules) and of run 2 (n2).  Each part starts at a multiple of 8 workgroups.
template <int M1, int M2, int NTILES, int D>
__global__ __launch_bounds__(kMfmaThreads) void k_shrink_pair(ShrinkArgs a1, GemvArgs g1, ShrinkArgs a2, GemvArgs g2,
                                                              int tnx, int tny, int gnx, int n1, int n2) {
  static_assert(kMfmaThreads == kGemvThreads, "both parts run on one workgroup size");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int lin = static_cast<int>(blockIdx.x);
  const int tile_blocks = tnx * tny;
  if (lin < tile_blocks) {
    shrink_stream_body<M1, NTILES, D>(a1, blk_of_linear(lin, tnx, tny, 1), smem);
    return;
  }
  lin -= tile_blocks;
  if (lin < tile_blocks) {
    shrink_stream_body<M2, NTILES, D>(a2, blk_of_linear(lin, tnx, tny, 1), smem);
    return;
  }
  lin -= tile_blocks;
  UnitLds& L = *reinterpret_cast<UnitLds*>(smem);
  __bf16* xs = reinterpret_cast<__bf16*>(smem + gemv_xs_offset<1, __bf16>());
  if (lin < gnx * n1) {
    gemv_body<1, __bf16, __bf16>(g1, blk_of_linear(lin, gnx, n1, 1), L, xs);
    return;
  }
  lin -= gnx * n1;
  gemv_body<1, __bf16, __bf16>(g2, blk_of_linear(lin, gnx, n2, 1), L, xs);
}

// Partial tiles of rank caps of 32 or more (PQ >= 2) need the registers of a
// third resident workgroup; at those caps the LDS tile leaves room for at most
// three (32), or two (48, 64), anyway.
template <typename TO, int PQ>
__global__ __launch_bounds__(kMfmaThreads, (sizeof(TO) == 2 && PQ <= 1) ? 3 : 2) void k_expand_mixed(ExpandArgs ea, GemvArgs g,
                                                                                      int tnx, int tny, int tnz,
                                                                                      int gnx, int gny) {
  static_assert(kMfmaThreads == kGemvThreads, "both parts run on one workgroup size");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lin = static_cast<int>(blockIdx.x), tile_blocks = tnx * tny * tnz;
  if (lin < tile_blocks) {
    expand_mfma_body<TO, PQ>(ea, blk_of_linear(lin, tnx, tny, tnz), smem);
  } else {
    int it0 = -1;
    const Blk b = g.module_group > 0 ? blk_of_module_groups(lin - tile_blocks, gnx, gny, g.module_group, it0)
                                     : blk_of_linear(lin - tile_blocks, gnx, gny, 1);
    gemv_body<2, __bf16, TO>(g, b, *reinterpret_cast<UnitLds*>(smem),
                             reinterpret_cast<__bf16*>(smem + gemv_xs_offset<2, __bf16>()), it0);
  }
}

}  // namespace lora
