// tile_schedule.h -- the grouped GEMM's tile schedule, shared by the GEMM
// (which derives its own tile without a table) and the routing kernels
// (which write the FC1 and FC2 tables of the expert layer while they hold
// the expert offsets).
//
// Tiles are numbered m-tile major with the n-tiles inner, m-tiles group by
// group (ceil(rows_g / BM) per group).  Workgroups are dealt to the 8 XCDs
// round robin (workgroup b runs on XCD b % 8), and the tiles are cut into 8
// contiguous ranges of about equal estimated cost, one per XCD, at m-tile
// boundaries: consecutive tiles share A rows and, inside a group, B rows,
// which then stay in that XCD's L2, and no XCD runs dry long before the
// others.  Workgroup b takes tile b / 8 of its XCD's range.  A tile with v
// valid 32-row blocks and S K-stages costs kCostFixed + S (kCostStage + v)
// units: its prologue and epilogue, and the B decode and loads of every
// stage, do not shrink with its rows.
#pragma once

#include <algorithm>
#include <cstdint>

#include "nvfp4_device.h"

namespace nvfp4 {

constexpr int kKS = 128;                    // K per stage
constexpr uint32_t kCostFixed = 24, kCostStage = 2;
constexpr uint32_t kCostMaxStages = 16;     // keeps the total cost inside 32 bits

__device__ __forceinline__ uint32_t tile_cost(uint32_t v, uint32_t stages) {
  return kCostFixed + stages * (kCostStage + v);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v = wave_incl_scan_dpp(v, [](uint32_t x, uint32_t y) { return x + y; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_incl_sum_u32(uint32_t v) {
  return wave_incl_scan_dpp(v, [](uint32_t x, uint32_t y) { return x + y; });
}

// One GEMM launch's tile table: one {group, row0, row1, n-tile} entry per
// workgroup position (group < 0: no tile), for bm-row tiles, ntn n-tiles per
// m-tile, K (the cost model's stages) and the launch's `blocks` positions.
// `fixed` is the cost model's per-tile term for the kernel the table serves.
// `split_tail` (tables of one n-tile, for kernels that take any row range up
// to bm rows): the compute units of one XCD.  An XCD whose range leaves r
// m-tiles for a last, partial round of that many workgroups, with 2 r at most
// that many, gets those r m-tiles as 2 r half-height tiles, so its last round
// ends sooner; the grid needs split_tail / 2 more positions per XCD.
struct TileTableSpec {
  int4* table;
  int32_t bm;
  int64_t k, ntn, blocks;
  uint32_t fixed = kCostFixed;
  uint32_t split_tail = 0;
};

constexpr int kMaxTableGroups = 1024;

// LDS of the table builder (the calling kernel declares one): the offsets
// and the inclusive prefix sums of the groups' m-tile counts and costs (a
// group's own count and cost are recomputed from its offsets).
struct TileTableLds {
  int32_t off[kMaxTableGroups + 1];
  uint32_t ic[kMaxTableGroups], ik[kMaxTableGroups];   // inclusive prefix sums
  uint32_t wc[4], wk[4], f0[8], f1[8];
};

// m-tiles of a group of n rows (cnt), whole ones (full) and their cost
// (per-tile term `fixed`).
template <int BM>
__device__ __forceinline__ void group_tiles(int64_t n, uint32_t stages, uint32_t fixed,
                                            uint32_t full_cost, uint32_t* cnt, uint32_t* full,
                                            uint32_t* cost) {
  *cnt = 0; *full = 0; *cost = 0;
  if (n > 0) {
    const uint32_t f = (uint32_t)(n / BM), rem = (uint32_t)(n % BM);
    *full = f;
    *cnt = f + (rem ? 1u : 0u);
    *cost = f * full_cost + (rem ? fixed + stages * (kCostStage + (rem + 31) / 32) : 0u);
  }
}

// Writes entries first, first + stride, ... of the table from the offsets
// off[0..G] (global or LDS), exactly as the GEMM's own lookup derives each
// workgroup's tile (which uses the fixed term kCostFixed; a table may carry
// another): per-group m-tile counts and costs with their inclusive
// prefix sums over the groups, the 8 XCD cut points (the first m-tiles whose
// preceding cost reaches x/8 of the total), then for every position b its
// XCD range position, m-tile, n-tile, group and rows.  A 256-thread
// workgroup calls it (it synchronises the workgroup), G <= kMaxTableGroups.
// The offsets are read once into LDS; the entries need no memory reads.
template <int BM>
__device__ void build_tile_table(const int32_t* off, int G, const TileTableSpec& t, int64_t first,
                                 int64_t stride, TileTableLds& s) {
  constexpr int PER = kMaxTableGroups / 256;    // groups per thread, contiguous
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const uint32_t stages = (uint32_t)std::min<int64_t>(t.k / kKS, kCostMaxStages);
  const uint32_t full_cost = t.fixed + stages * (kCostStage + BM / 32);
  int32_t o[PER + 1];
#pragma unroll
  for (int i = 0; i <= PER; ++i) {
    const int gi = PER * tid + i;
    o[i] = gi <= G ? off[gi] : 0;
  }
  uint32_t lc = 0, lk = 0;
  uint32_t pc[PER], pk[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int gi = PER * tid + i;
    uint32_t cnt = 0, cost = 0, full = 0;
    if (gi < G) {
      group_tiles<BM>((int64_t)o[i + 1] - (int64_t)o[i], stages, t.fixed, full_cost, &cnt, &full,
                      &cost);
      s.off[gi] = o[i];
      if (gi == G - 1) s.off[G] = o[i + 1];
    }
    lc += cnt; lk += cost;
    pc[i] = lc; pk[i] = lk;                        // inclusive within the thread
  }
  const uint32_t ic = wave_incl_sum_u32(lc), ik = wave_incl_sum_u32(lk);
  if (lane == kWave - 1) { s.wc[w] = ic; s.wk[w] = ik; }
  __syncthreads();
  uint32_t bc = ic - lc, bk = ik - lk;             // exclusive over the workgroup
  for (int j = 0; j < w; ++j) { bc += s.wc[j]; bk += s.wk[j]; }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int gi = PER * tid + i;
    if (gi < G) { s.ic[gi] = bc + pc[i]; s.ik[gi] = bk + pk[i]; }
  }
  __syncthreads();
  const uint32_t tiles = s.ic[G - 1], total = s.ik[G - 1];
  // XCD x's m-tile range [f0, f1): the first m-tile of the first group whose
  // inclusive cost reaches the cut, as in the GEMM's lookup
  auto find = [&](uint32_t c) -> uint32_t {
    int lo = 0, hi = G;                            // first group with ik >= c
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s.ik[mid] >= c) hi = mid; else lo = mid + 1;
    }
    if (lo >= G) return tiles;
    uint32_t cnt, full, cost;
    group_tiles<BM>((int64_t)s.off[lo + 1] - (int64_t)s.off[lo], stages, t.fixed, full_cost, &cnt,
                    &full, &cost);
    const uint32_t ec = s.ic[lo] - cnt, ek = s.ik[lo] - cost;
    uint32_t j = c > ek ? (c - ek + full_cost - 1) / full_cost : 0u;
    if (j > full) j = cnt;                         // inside the partial tile: take the next one
    return ec + j;
  };
  if (tid < 8) {
    const int x = tid;
    s.f0[x] = find((uint32_t)((uint64_t)total * x / 8));
    s.f1[x] = x == 7 ? tiles : find((uint32_t)((uint64_t)total * (x + 1) / 8));
  }
  __syncthreads();
  const uint32_t un = (uint32_t)t.ntn;
  const bool split = t.split_tail != 0 && un == 1;
  for (int64_t b = first; b < t.blocks; b += stride) {
    const int x = (int)(b % 8);
    const uint32_t pos = (uint32_t)(b / 8);
    // m-tile of this position, and which half of it (-1: the whole tile)
    uint32_t mt = 0;
    int half = -1;
    bool live;
    if (split) {
      const uint32_t cnt = s.f1[x] - s.f0[x];
      const uint32_t r = cnt % t.split_tail;
      const uint32_t ns = 2 * r <= t.split_tail ? r : 0u;   // m-tiles cut in two
      const uint32_t nf = cnt - ns;
      live = pos < nf + 2 * ns;
      if (pos < nf) {
        mt = s.f0[x] + pos;
      } else {
        mt = s.f0[x] + nf + (pos - nf) / 2;
        half = (int)((pos - nf) & 1u);
      }
    } else {
      live = s.f0[x] * un + pos < s.f1[x] * un;
      mt = (s.f0[x] * un + pos) / un;
    }
    int4 e = make_int4(-1, 0, 0, 0);
    if (live) {
      int lo = 0, hi = G - 1;                      // first group with ic > mt
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s.ic[mid] > mt) hi = mid; else lo = mid + 1;
      }
      const int64_t n = (int64_t)s.off[lo + 1] - (int64_t)s.off[lo];
      const uint32_t cnt = (uint32_t)((n + BM - 1) / BM);
      int32_t r0 = s.off[lo] + (int32_t)(mt - (s.ic[lo] - cnt)) * BM;
      int32_t r1 = std::min<int32_t>(r0 + BM, s.off[lo + 1]);
      if (half >= 0) {                             // rows [r0 + BM/2 h, + BM/2) of the tile
        r0 += half * (BM / 2);
        r1 = std::min<int32_t>(r1, r0 + BM / 2);
      }
      const int ntile = split ? 0 : (int)(s.f0[x] * un + pos - mt * un);
      if (r0 < r1) e = make_int4(lo, r0, r1, ntile);
    }
    t.table[b] = e;
  }
  __syncthreads();                                 // the LDS arrays may be reused next
}

// The first n (0-2) of the tables t0, t1: this thread's entries first,
// first + stride, ... of each (256-thread workgroups).
__device__ __forceinline__ void build_tile_tables(const int32_t* off, int G, const TileTableSpec& t0,
                                                  const TileTableSpec& t1, int n, int64_t first,
                                                  int64_t stride, TileTableLds& s) {
  auto one = [&](const TileTableSpec& t) {
    if (t.bm == 32) build_tile_table<32>(off, G, t, first, stride, s);
    else build_tile_table<128>(off, G, t, first, stride, s);
  };
  if (n > 0) one(t0);
  if (n > 1) one(t1);
}

}  // namespace nvfp4
