// Base product and adapter term in one matrix-core kernel:
//   y_i = x_i W + s_a (x_i A_a^T) B_a
// for a batch whose tokens come in runs of one adapter, such as prefills.
// The study page's section "The kernel trick: gather, do not merge" runs the
// shared base matmul once and then applies each adapter's low-rank update; its
// FLOP count puts the update at about 2r/d of the base.  Computing both in one
// pass over x gets close to that: the shrink reads the x tiles the base
// product has already staged, and the expand adds into the base accumulators
// before y is written once.
//
// Tile: 256 tokens x 256 output columns, 8 waves, each 128 tokens x 64
// columns, on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The product
// is formed transposed (Y^T = W^T X^T: the A operand is a row of W^T, the B
// operand a token row of x), so each lane's four accumulators are four
// consecutive output columns of one token, stored as one 8-byte write.  K
// advances 64 per step through two LDS buffers; global_load_lds moves the x,
// W^T and adapter-A tiles straight from memory into LDS (no register
// staging), 16-byte chunks XOR-swizzled by row so fragment reads are
// conflict-free.  The next step's loads are in flight while the current
// step's MFMAs run.
//
// Adapter units.  At tile start the workgroup collects the distinct adapters
// of its 256 tokens (ascending slot order) and cuts each into units of 16
// rank rows.  The first one or two units ride along with the base product:
// their A rows are staged with each step, and wave (wm, wn) computes
// t^T = A_u X^T for tokens 128 wm + 32 wn .. +32 from x fragments it already
// holds.  A tile with more units (several adapters, or ranks above 32) runs
// a further pass over K per unit that computes t alone.  During
// the last step of a pass the units' B rows for the tile's columns are
// fetched into the idle LDS buffer.  After the pass t is masked to the tokens
// of each unit's adapter, scaled, split into two bf16 parts (hi + lo carry 16
// significand bits) and multiplied by B on the same MFMA shape into the base
// accumulators.  Rows an adapter does not have read the pool's zero page.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "mfma_kernels.hpp"   // bf16x8

namespace lora {

constexpr int kFgThreads = 512;
constexpr int kFgWaves = kFgThreads / 64;
constexpr int kFgBM = 256;        // tokens per tile
constexpr int kFgBN = 256;        // output columns per tile
constexpr int kFgBK = 64;         // k per pipeline step
constexpr int kFgTileBytes = kFgBM * kFgBK * 2;   // one [256][64] bf16 tile
constexpr int kFgPassUnits = 2;   // 16-rank units per pass over K, at most
constexpr int kFgMaxPpr = 32;     // A pages per rank row (h_in / page_elems) at most
constexpr int kFgMaxBpages = 8;   // B pages a tile's 256 columns touch, at most (page >= 64)
constexpr int kFgMaxSlots = 8192; // slot ids a tile's bitmap covers
constexpr int kFgMaxUnits = kFgBM * 4;   // 256 distinct adapters x 4 units (rank 64)
constexpr int kFgTRow = 144;      // bytes per token row of the t exchange (128 + 16: no bank conflicts)
constexpr int kFgBOff = 16384;    // B rows in the idle stage buffer's second half, after T

#ifndef LORA_FG_SWIZZLE
#define LORA_FG_SWIZZLE 1
#endif

struct FusedArgs {
  PoolView pv;
  const __bf16* x;        // [n][ld_x]
  const __bf16* w;        // W^T: [h_out][ld_w], row c = weights of output column c
  const uint8_t* w8;      // W8 kernel: W^T as OCP e4m3 codes, [h_out][ld_w] bytes
  const float* w_scale;   // W8 kernel: [h_out] scale of each output column
  const int32_t* ids;     // [n]; unused by the base-only kernel
  __bf16* y;              // [n][ld_y], written
  int64_t ld_x, ld_w, ld_y;
  int32_t n, h_in, h_out, module;
  int32_t n_ct;           // column tiles
  int32_t n_tiles;        // row tiles x column tiles
};

// XOR key of row r's 16-byte chunks in a [rows][64] bf16 LDS tile, and the
// byte offset of logical chunk c (0..7) of row r.  A fragment read has 16
// lanes on 16 consecutive rows at the same logical chunk; with this key any 8
// consecutive rows from an even row, and any 16 from a multiple of 16, hit
// distinct 16-byte bank groups, so the read is conflict-free whether the LDS
// serves 128 or 256 bytes per clock.
__device__ __forceinline__ int fg_swz_key(int r) {
#if LORA_FG_SWIZZLE == 1
  return ((r >> 1) & 7) ^ ((r & 1) << 2);
#else
  return r & 7;
#endif
}
__device__ __forceinline__ int fg_swz(int r, int c) { return r * 128 + ((c ^ fg_swz_key(r)) << 4); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t fg_lds_ptr(void* p) {
  return reinterpret_cast<lds_ptr_t>(reinterpret_cast<uintptr_t>(p));
}

struct FgShared {
  // two pipeline stages of [256][64] bf16 x and W^T tiles; after a pass the
  // idle one holds t (first half) and the units' B rows (second half)
  alignas(16) unsigned char stage[2][2][kFgTileBytes];
  alignas(16) unsigned char astage[2][kFgPassUnits * 16 * kFgBK * 2];   // adapter A rows per stage
  int32_t ids[kFgBM];
  uint32_t bitmap[kFgMaxSlots / 32];
  int32_t dslot[kFgBM];            // distinct adapters of the tile, ascending
  int32_t drank[kFgBM];
  float dscale[kFgBM];
  int32_t da_off[kFgBM], db_off[kFgBM];
  int32_t unit[kFgMaxUnits];       // (distinct index << 2) | unit of 16 ranks
  int32_t pid[kFgPassUnits][16][kFgMaxPpr];        // A pages of the pass's units
  int32_t bpid[kFgPassUnits][16][kFgMaxBpages];    // B pages of the pass's units over the tile's columns
  int32_t wsum[kFgWaves];
};

// Exclusive prefix sum over the workgroup's threads; returns the total in *total.
__device__ __forceinline__ int fg_block_scan(int v, int32_t* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kFgWaves; ++w) {
    const int s = wsum[w];
    if (w < wave) base += s;
    tot += s;
  }
  *total = tot;
  __syncthreads();   // wsum is reused by the next scan
  return base + incl - v;
}

__device__ __forceinline__ bf16x8 fg_lds8(const unsigned char* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

template <int V>
using fg_int = std::integral_constant<int, V>;

// Two OCP e4m3 codes (the low or high half of w) widened to two bf16 values.
// Every e4m3 value has at most 4 significant bits and an exponent inside
// bf16's range, so the widening is exact (scale 1).
__device__ __forceinline__ uint32_t fg_e4m3x2_to_bf16x2(uint32_t w, bool high) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

// LORA false: base product only.  W8: W^T given as e4m3 codes with a scale per
// output column (W8A16: the codes are widened to bf16 on their way into LDS,
// exactly, and the column scale multiplies the base product before the
// adapter term is added).
template <bool LORA, bool W8>
__global__ __launch_bounds__(kFgThreads, 1) void k_fused_gemm(FusedArgs a) {
  __shared__ FgShared sh;
  constexpr int CB = 4;   // 16-column blocks per wave
  constexpr int SB = 2;   // 16-token shrink blocks per wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in scalar registers
  const int wm = wave >> 2, wn = wave & 3;   // tokens 128 wm .. +128, columns 64 wn .. +64
  const int l16 = lane & 15, lq = lane >> 4;

  // tile of this workgroup: the tiles one XCD takes are consecutive, so the
  // column tiles of a token tile share its x rows in that XCD's L2
  const int per_xcd = gridDim.x >> 3;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= a.n_tiles) return;
  const int rt = tile / a.n_ct, ct = tile - rt * a.n_ct;
  const int row0 = rt * kFgBM, col0 = ct * kFgBN;
  const int nk = a.h_in / kFgBK;

  // ---- staging: per K step each wave moves 4 blocks of 8 rows x 128 B of
  // the x tile and 4 of the W^T tile straight into LDS (lane i lands at byte
  // 16 i of its block).  Lane i fetches the logical chunk that the swizzle
  // puts at its LDS position: row 8 b + i / 8, physical chunk i % 8.  Rows
  // past the end repeat the last row (their results are never stored).
  const int lr = lane >> 3;
  const char* xbase = reinterpret_cast<const char*>(a.x + static_cast<int64_t>(row0) * a.ld_x);
  const char* wbase = reinterpret_cast<const char*>(a.w + static_cast<int64_t>(col0) * a.ld_w);
  uint32_t xoff[4], woff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * (wave + 8 * q) + lr;
    const int lc = (lane & 7) ^ fg_swz_key(r);
    xoff[q] = static_cast<uint32_t>((min(r, a.n - 1 - row0) * a.ld_x + 8 * lc) * 2);
    woff[q] = static_cast<uint32_t>((min(r, a.h_out - 1 - col0) * a.ld_w + 8 * lc) * 2);
  }
  auto load_x = [&](int kt, int buf) {
    const char* xb = xbase + kt * (kFgBK * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(xb + xoff[q], fg_lds_ptr(sh.stage[buf][0] + 1024 * (wave + 8 * q)), 16, 0, 0);
  };
  auto load_w = [&](int kt, int buf) {
    const char* wb = wbase + kt * (kFgBK * 2);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(wb + woff[q], fg_lds_ptr(sh.stage[buf][1] + 1024 * (wave + 8 * q)), 16, 0, 0);
  };
  // W8: each thread moves two 16-byte pieces of e4m3 codes per K step (rows
  // i / 4 of the tile, k 16 (i % 4) .. +16, for i = tid, tid + 512) through
  // registers, widened to four bf16 chunks in the same swizzled layout
  const uint8_t* w8base = W8 ? a.w8 + static_cast<int64_t>(col0) * a.ld_w : nullptr;
  uint32_t w8off[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + kFgThreads * q;
    const int r = i >> 2;
    w8off[q] = static_cast<uint32_t>(min(r, a.h_out - 1 - col0) * a.ld_w + 16 * (i & 3));
  }
  u32x4 w8reg[2];
  auto issue_w8 = [&](int kt) {
#pragma unroll
    for (int q = 0; q < 2; ++q) w8reg[q] = *reinterpret_cast<const u32x4*>(w8base + kt * kFgBK + w8off[q]);
  };
  auto store_w8 = [&](int buf) {
    unsigned char* Ws = sh.stage[buf][1];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = tid + kFgThreads * q;
      const int r = i >> 2, c = 2 * (i & 3);
      const u32x4 v = w8reg[q];
      const u32x4 lo{fg_e4m3x2_to_bf16x2(v.x, false), fg_e4m3x2_to_bf16x2(v.x, true),
                     fg_e4m3x2_to_bf16x2(v.y, false), fg_e4m3x2_to_bf16x2(v.y, true)};
      const u32x4 hi{fg_e4m3x2_to_bf16x2(v.z, false), fg_e4m3x2_to_bf16x2(v.z, true),
                     fg_e4m3x2_to_bf16x2(v.w, false), fg_e4m3x2_to_bf16x2(v.w, true)};
      *reinterpret_cast<u32x4*>(Ws + fg_swz(r, c)) = lo;
      *reinterpret_cast<u32x4*>(Ws + fg_swz(r, c + 1)) = hi;
    }
  };
  load_x(0, 0);
  if constexpr (W8) {
    issue_w8(0);
    store_w8(0);
  } else {
    load_w(0, 0);
  }

  // ---- the tile's adapters and units
  int n_units = 0;
  if constexpr (LORA) {
    int id = -1;
    if (tid < kFgBM && row0 + tid < a.n) {
      id = a.ids[row0 + tid];
      if (id < 0 || id >= a.pv.n_slots) id = -1;
    }
    const int n_words = (a.pv.n_slots + 31) >> 5;
    for (int i = tid; i < n_words; i += kFgThreads) sh.bitmap[i] = 0u;
    __syncthreads();
    if (id >= 0) atomicOr(&sh.bitmap[id >> 5], 1u << (id & 31));
    __syncthreads();
    // distinct ids in ascending order: thread i takes bitmap word i (n_slots <= 8192)
    const uint32_t word = tid < n_words ? sh.bitmap[tid] : 0u;
    int n_dist = 0;
    int off = fg_block_scan(__popc(word), sh.wsum, &n_dist);
    for (uint32_t w = word; w; w &= w - 1) sh.dslot[off++] = tid * 32 + __ffs(w) - 1;
    if (tid < kFgBM) sh.ids[tid] = id;
    __syncthreads();
    int nu = 0;
    if (tid < n_dist) {
      const SlotEntry e = a.pv.entries[static_cast<int64_t>(sh.dslot[tid]) * a.pv.n_modules + a.module];
      sh.drank[tid] = e.rank;
      sh.dscale[tid] = e.scale;
      sh.da_off[tid] = e.a_off;
      sh.db_off[tid] = e.b_off;
      nu = (max(e.rank, 0) + 15) >> 4;
    }
    int uoff = fg_block_scan(nu, sh.wsum, &n_units);
    for (int j = 0; j < nu; ++j) sh.unit[uoff + j] = (tid << 2) | j;
    __syncthreads();
  }

  const int h = static_cast<int>(a.pv.page_elems);
  const int ppr_a = a.h_in / h, ppr_b = a.h_out / h;
  const int cp0 = col0 / h;   // first B page column index of this tile
  const __bf16* pages = static_cast<const __bf16*>(a.pv.pages);

  // page ids of units u0 .. u0 + np - 1: A rows pid[u][rank row][k page], and
  // B rows bpid[u][rank row][page - cp0] over the tile's columns; the zero
  // page stands in for rows past the rank
  auto load_pids = [&](int u0, int np) {
    const int na = np * 16 * ppr_a;
    for (int i = tid; i < na; i += kFgThreads) {
      const int u = i / (16 * ppr_a), rest = i - u * 16 * ppr_a;
      const int jr = rest / ppr_a, kp = rest - jr * ppr_a;
      const int un = sh.unit[u0 + u], d = un >> 2;
      const int jj = ((un & 3) << 4) + jr;
      sh.pid[u][jr][kp] = jj < sh.drank[d] ? a.pv.page_ids[sh.da_off[d] + jj * ppr_a + kp] : a.pv.zero_page;
    }
    const int ncp = (min(col0 + kFgBN, a.h_out) - 1) / h - cp0 + 1;
    const int nb = np * 16 * ncp;
    for (int i = tid; i < nb; i += kFgThreads) {
      const int u = i / (16 * ncp), rest = i - u * 16 * ncp;
      const int jr = rest / ncp, ci = rest - jr * ncp;
      const int un = sh.unit[u0 + u], d = un >> 2;
      const int jj = ((un & 3) << 4) + jr;
      sh.bpid[u][jr][ci] =
          jj < sh.drank[d] ? a.pv.page_ids[sh.db_off[d] + jj * ppr_b + cp0 + ci] : a.pv.zero_page;
    }
  };
  // A rows of the pass's P units into astage: waves 0 .. 2P - 1 move one
  // block of 8 rank rows each (row 16 u + jr of the staged tile)
  const int arow = 8 * wave + lr;
  const int alc = (lane & 7) ^ fg_swz_key(arow);
  auto load_a = [&](auto P_, int kt, int buf) {
    constexpr int P = decltype(P_)::value;
    if (wave < 2 * P) {
      const int k0 = kt * kFgBK;
      const int kp = ppr_a == 1 ? 0 : k0 / h;
      const int pid = sh.pid[arow >> 4][arow & 15][kp];
      const __bf16* src = pages + static_cast<int64_t>(pid) * h + (k0 - kp * h) + 8 * alc;
      __builtin_amdgcn_global_load_lds(src, fg_lds_ptr(sh.astage[buf] + 1024 * wave), 16, 0, 0);
    }
  };
  // B rows of the pass's P units for the tile's columns into dst:
  // [u][rank row][256 columns] bf16, 1 KB blocks of two rank rows; columns
  // past h_out read the zero page
  auto load_b = [&](auto P_, unsigned char* dst) {
    constexpr int P = decltype(P_)::value;
    const int col = col0 + 8 * (lane & 31);
    const bool in = col < a.h_out;
    const int cp = in ? col / h : cp0;
    const int cin = in ? col - cp * h : 0;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int b = wave + kFgWaves * q;   // block: unit b / 8, rank rows 2 (b % 8) .. +2
      const int jr = 2 * (b & 7) + (lane >> 5);
      const int pid = in ? sh.bpid[b >> 3][jr][cp - cp0] : a.pv.zero_page;
      __builtin_amdgcn_global_load_lds(pages + static_cast<int64_t>(pid) * h + cin,
                                       fg_lds_ptr(dst + 1024 * b), 16, 0, 0);
    }
  };

  f32x4 acc[CB][8];
#pragma unroll
  for (int i = 0; i < CB; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 tacc[SB][kFgPassUnits];

  // LDS rows of this lane's fragments
  const int wrow = 64 * wn + l16;    // W^T rows (output columns) of col block cb: + 16 cb
  const int xrow = 128 * wm + l16;   // x rows (tokens) of token block tb: + 16 tb
  const int srow = 128 * wm + 32 * wn + l16;   // x rows of this wave's shrink tokens: + 16 i
  unsigned char* const idle = sh.stage[nk & 1][0];   // the buffer no step of a pass's last one reads

  // One pass over K.  BASE: the base product with the shrink of P units
  // riding along; otherwise the shrink alone.  During the last step the P
  // units' B rows go to the idle buffer.
  auto kloop = [&](auto P_, auto BASE_) {
    constexpr int P = decltype(P_)::value;
    constexpr bool BASE = decltype(BASE_)::value != 0;
#pragma unroll
    for (int i = 0; i < SB; ++i)
#pragma unroll
      for (int u = 0; u < kFgPassUnits; ++u) tacc[i][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int buf) {
      const unsigned char* Xs = sh.stage[buf][0];
      const unsigned char* Ws = sh.stage[buf][1];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = 4 * ks + lq;
        bf16x8 xs[SB];   // x fragments of this wave's shrink tokens
        if constexpr (BASE) {
          bf16x8 wf[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) wf[cb] = fg_lds8(Ws, fg_swz(wrow + 16 * cb, c));
#pragma unroll
          for (int tb = 0; tb < 8; ++tb) {
            const bf16x8 xf = fg_lds8(Xs, fg_swz(xrow + 16 * tb, c));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              acc[cb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[cb], xf, acc[cb][tb], 0, 0, 0);
            if constexpr (P > 0) {   // token blocks SB wn .. SB wn + SB - 1, picked without a branch
              if (tb < SB) xs[tb] = xf;
              else xs[tb % SB] = tb / SB == wn ? xf : xs[tb % SB];
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < SB; ++i) xs[i] = fg_lds8(Xs, fg_swz(srow + 16 * i, c));
        }
        if constexpr (P > 0) {
#pragma unroll
          for (int u = 0; u < P; ++u) {
            const bf16x8 af = fg_lds8(sh.astage[buf], fg_swz(16 * u + l16, c));
#pragma unroll
            for (int i = 0; i < SB; ++i)
              tacc[i][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, xs[i], tacc[i][u], 0, 0, 0);
          }
        }
      }
    };
    // The last step is peeled so that the loop body has no branch (a branch
    // there makes the compiler shuttle the accumulators between register files).
    for (int kt = 0; kt < nk - 1; ++kt) {
      const int buf = kt & 1;
      load_x(kt + 1, buf ^ 1);   // that buffer's readers passed the last barrier
      if constexpr (BASE && !W8) load_w(kt + 1, buf ^ 1);
      if constexpr (BASE && W8) issue_w8(kt + 1);
      if constexpr (P > 0) load_a(P_, kt + 1, buf ^ 1);
      step(buf);
      if constexpr (BASE && W8) store_w8(buf ^ 1);   // widened after this step's reads of buf
      __syncthreads();
    }
    if constexpr (P > 0) load_b(P_, idle + kFgTileBytes + kFgBOff);
    step((nk - 1) & 1);
    __syncthreads();   // also: the B rows have landed
  };

  // t of units u0 .. u0 + P - 1 -> LDS, masked to each unit's adapter and
  // rank rows and scaled; then acc^T += B^T_u [cols x 32] . T_u [32 x tokens]
  // where k 0..15 pair hi with ranks 0..15 and k 16..31 pair lo with them
  auto expand = [&](auto P_, int u0) {
    constexpr int P = decltype(P_)::value;
    unsigned char* T_s = idle;                                 // [256 tokens][kFgTRow]
    const unsigned char* B_s = idle + kFgTileBytes + kFgBOff;  // [u][16 ranks][256 cols] bf16
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const int tok = srow + 16 * i;
      const int id = sh.ids[tok];
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int un = sh.unit[u0 + u], d = un >> 2;
        float s = 0.f;
        int rows = 0;
        if (sh.dslot[d] == id) {
          s = sh.dscale[d];
          rows = sh.drank[d] - ((un & 3) << 4);
        }
        __bf16 hi[4], lo[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float t = 4 * lq + v < rows ? tacc[i][u][v] * s : 0.f;
          hi[v] = static_cast<__bf16>(t);
          lo[v] = static_cast<__bf16>(t - static_cast<float>(hi[v]));
        }
        unsigned char* trow = T_s + tok * kFgTRow + u * 64;
        *reinterpret_cast<u32x2*>(trow + 8 * lq) = __builtin_bit_cast(u32x2, hi);
        *reinterpret_cast<u32x2*>(trow + 32 + 8 * lq) = __builtin_bit_cast(u32x2, lo);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < P; ++u) {
      bf16x8 bfr[CB];   // lane: output column wrow + 16 cb, ranks 8 (lq & 1) .. +8
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const unsigned short* bp = reinterpret_cast<const unsigned short*>(
            B_s + u * 8192 + (8 * (lq & 1)) * 512 + 2 * (wrow + 16 * cb));
        unsigned short e[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) e[r] = bp[256 * r];
        bfr[cb] = __builtin_bit_cast(bf16x8, e);
      }
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) {
        const bf16x8 tf = fg_lds8(T_s, (xrow + 16 * tb) * kFgTRow + u * 64 + 16 * lq);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[cb], tf, acc[cb][tb], 0, 0, 0);
      }
    }
  };

  // W8: the base accumulators times each output column's scale (before any
  // adapter term is added).  Lane: columns col0 + 64 wn + 16 cb + 4 lq .. +4.
  auto scale_base = [&]() {
    if constexpr (W8) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int col = col0 + 64 * wn + 16 * cb + 4 * lq;
        const f32x4 sc = col < a.h_out ? *reinterpret_cast<const f32x4*>(a.w_scale + col) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < 8; ++tb) acc[cb][tb] *= sc;
      }
    }
  };

  // ---- pass 0: the base product with up to two units
  if constexpr (LORA) {
    const int np0 = min(n_units, kFgPassUnits);
    if (np0 > 0) {
      load_pids(0, np0);
      __syncthreads();
    }
    if (np0 == 2) {
      load_a(fg_int<2>{}, 0, 0);
      __syncthreads();
      kloop(fg_int<2>{}, fg_int<1>{});
      scale_base();
      expand(fg_int<2>{}, 0);
    } else if (np0 == 1) {
      load_a(fg_int<1>{}, 0, 0);
      __syncthreads();
      kloop(fg_int<1>{}, fg_int<1>{});
      scale_base();
      expand(fg_int<1>{}, 0);
    } else {
      __syncthreads();
      kloop(fg_int<0>{}, fg_int<1>{});
      scale_base();
    }
    // ---- further passes, one unit at a time, shrink only
    for (int u0 = np0; u0 < n_units; ++u0) {
      __syncthreads();   // the previous pass's LDS reads are done
      load_pids(u0, 1);
      __syncthreads();
      load_x(0, 0);
      load_a(fg_int<1>{}, 0, 0);
      __syncthreads();
      kloop(fg_int<1>{}, fg_int<0>{});
      expand(fg_int<1>{}, u0);
    }
  } else {
    __syncthreads();   // stage 0 has landed (the barrier waits for the loads)
    kloop(fg_int<0>{}, fg_int<1>{});
    scale_base();
  }

  // ---- y: lane holds output columns 4 lq .. +4 of col block cb for token
  // 16 tb + l16; one rounding to bf16 per element
#pragma unroll
  for (int tb = 0; tb < 8; ++tb) {
    const int tok = row0 + xrow + 16 * tb;
    if (tok >= a.n) continue;
    __bf16* yr = a.y + static_cast<int64_t>(tok) * a.ld_y;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = col0 + 64 * wn + 16 * cb + 4 * lq;
      if (col >= a.h_out) continue;
      __bf16 o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = static_cast<__bf16>(acc[cb][tb][v]);
      *reinterpret_cast<u32x2*>(yr + col) = __builtin_bit_cast(u32x2, o);
    }
  }
}

}  // namespace lora
