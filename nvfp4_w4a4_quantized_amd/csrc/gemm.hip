// gemm.hip -- W4A4 NVFP4 grouped GEMM on gfx950 matrix cores.
//
// Decode strategy.  CDNA4's block-scaled MFMA takes one power-of-two (E8M0)
// scale per 32 K elements; NVFP4 carries an E4M3 scale per 16 (miniTE
// Technical Report §2.2, §5.1), so the scaled FP4 MFMA cannot reproduce the
// format.  Instead each operand element is decoded exactly to fp16: the FP4
// code through the gfx950 FP4->f16 conversion (scale 1.0), then one packed
// f16 multiply by the block scale.  q * s_b has at most 6 significant bits
// and lies in [2^-10, 2688], so the product is exact in fp16; the f16 x f16
// products are exact in the fp32 accumulator of v_mfma_f32_32x32x16_f16.  The
// per-row and per-expert FP32 outer scales are applied once per output in
// the epilogue (miniTE Technical Report §5.4: the accumulator is multiplied
// by the per-row factor and, optionally, a per-column one; miniTE summary
// §4.2: FP32 rescaling after the block-scaled product).
//
// Structure: see the kernel comment below.  Group boundaries come from the
// device offsets, so the host never reads them: every workgroup derives its
// (group, m-tile) from a wave-wide scan of the per-group tile counts, or
// reads it from a tile table that a kernel holding the offsets wrote
// beforehand (tile_schedule.h); surplus workgroups exit.
#include <type_traits>
#include <algorithm>

#include "gemm_common.h"
#include "launch.h"
#include "nvfp4_device.h"
#include "tile_schedule.h"

namespace nvfp4 {

// ---- kernel --------------------------------------------------------------
//
// Workgroup = NW waves side by side along N, each with the register budget
// of two waves per SIMD.  With four waves two workgroups share a compute unit
// (one wave of each per SIMD): while one workgroup sits in its prologue, a
// barrier or its VALU-heavy epilogue, the other keeps the matrix cores busy.
// With eight waves one workgroup fills the unit and each decoded A stage
// serves twice the columns.  The workgroup owns a BM x BN output tile of one group
// (BM = 32*WM rows, BN = NW*32*WN columns); each wave a BM x (32*WN) sub-tile
// held in accumulator registers (WM x WN v_mfma_f32_32x32x16_f16 tiles).
// K advances in stages of 128.
//   A (activations, shared by all waves) goes through two LDS buffers: each
//     thread decodes quarter rows of the stage (32 elements each) once,
//     straight from its global load, and stores the fp16 values in
//     MFMA-fragment order: for fragment m and substep s the 64 lanes' 16-byte
//     operands are one 1 KiB block (lane slots XOR-swizzled inside groups of
//     16), so both the writes and the per-substep reads are bank-conflict
//     free.  While the waves multiply stage i from one buffer, they decode
//     stage i+1 into the other.
//   B (weights) is private to each wave: every lane loads the packed codes
//     and E4M3 scales of its own column straight into registers one stage
//     ahead, and decodes them right before its MFMAs.
// K order: inside a 128 stage, lane half h covers elements [64h, 64h+64)
// and substep s takes [64h + 8s, 64h + 8s + 8); A and B use the same order,
// so the dot products are unchanged.
// The epilogue works on the accumulator registers in place: each lane holds
// one column of 16 rows per 32-row block, and for the SwiGLU tile the gate and
// up columns of one output column sit in the same lane.
#ifndef NVFP4_VPM
#define NVFP4_VPM 4
#endif

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2 };

// ---- tile schedule (cost model, tables: tile_schedule.h) -------------------
//
// Workgroups derive their tile from the device offsets (schedule_tile below)
// unless the launch carries a precomputed table.  Up to 256 groups the
// offsets are read once per workgroup; the grid is an upper bound and
// surplus workgroups exit.

// 256 consecutive groups, four per lane (group base + 64 i + lane)
struct GroupChunk {
  uint32_t cnt[4], cost[4], full[4];   // m-tiles, their cost, whole m-tiles
  int32_t start[4], end[4];            // row range of the group
};

template <int BM>
__device__ __forceinline__ void load_chunk(const int32_t* off, int G, uint32_t stages, int base,
                                           GroupChunk& c) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = base + 64 * i + lane;
    c.start[i] = g < G ? off[g] : 0;
    c.end[i] = g < G ? off[g + 1] : 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = (int64_t)c.end[i] - (int64_t)c.start[i];
    c.cnt[i] = 0; c.cost[i] = 0; c.full[i] = 0;
    if (n > 0) {
      const uint32_t f = (uint32_t)(n / BM), rem = (uint32_t)(n % BM);
      c.full[i] = f;
      c.cnt[i] = f + (rem ? 1u : 0u);
      c.cost[i] = f * tile_cost(BM / 32, stages) + (rem ? tile_cost((rem + 31) / 32, stages) : 0u);
    }
  }
}

// Finds workgroup bid's tile: its group *g, rows [*row0, *row1) and n-tile
// *nt (the same in every lane).  Returns false for a surplus workgroup.
// Up to 256 groups the offsets are read once and every step works on the
// lane-resident scans; beyond that each step streams the groups again.
template <int BM>
__device__ bool schedule_tile(const int32_t* off, int G, int64_t K, int64_t ntn, int64_t bid,
                              int* g_out, int64_t* row0, int64_t* row1, int64_t* nt) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t stages = (uint32_t)std::min<int64_t>(K / kKS, kCostMaxStages);
  const uint32_t full_cost = tile_cost(BM / 32, stages);
  const int x = (int)(bid % 8);
  const uint32_t pos = (uint32_t)(bid / 8);
  const uint32_t un = (uint32_t)ntn;
  // first m-tile of the group seen by this lane whose preceding cost reaches
  // t, given the group's scans (t <= ik)
  auto at = [&](uint32_t t, uint32_t ic, uint32_t ik, uint32_t cnt, uint32_t cost, uint32_t full) {
    const uint32_t ec = ic - cnt, ek = ik - cost;
    uint32_t j = t > ek ? (t - ek + full_cost - 1) / full_cost : 0u;
    if (j > full) j = cnt;                       // inside the partial tile: take the next one
    return ec + j;
  };
  auto first_lane = [](uint64_t hit) { return __ffsll((unsigned long long)hit) - 1; };
  uint32_t f0, f1, mt;
  if (G <= 256) {
    GroupChunk c;
    load_chunk<BM>(off, G, stages, 0, c);
    const int cols = (G + kWave - 1) / kWave;
    uint32_t ic[4], ik[4], cc = 0, ck = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < cols) {
        ic[i] = wave_incl_sum_u32(c.cnt[i]) + cc;
        ik[i] = wave_incl_sum_u32(c.cost[i]) + ck;
        cc = (uint32_t)__builtin_amdgcn_readlane((int)ic[i], kWave - 1);
        ck = (uint32_t)__builtin_amdgcn_readlane((int)ik[i], kWave - 1);
      } else {
        ic[i] = cc; ik[i] = ck;
      }
    }
    const uint32_t tiles = cc, total = ck;
    // XCD x's m-tiles [f0, f1): the first m-tiles whose preceding tiles
    // cost at least x/8 and (x+1)/8 of the total
    auto find = [&](uint32_t t) {
      uint32_t r = tiles;
      bool got = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t hit = __ballot(i < cols && 64 * i + lane < G && ik[i] >= t);
        if (!got && hit) {
          r = (uint32_t)__shfl((int)at(t, ic[i], ik[i], c.cnt[i], c.cost[i], c.full[i]),
                               first_lane(hit), kWave);
          got = true;
        }
      }
      return r;
    };
    f0 = find((uint32_t)((uint64_t)total * x / 8));
    f1 = x == 7 ? tiles : find((uint32_t)((uint64_t)total * (x + 1) / 8));
    const uint32_t logical = f0 * un + pos;
    if (logical >= f1 * un) return false;
    mt = logical / un;
    *nt = logical - mt * un;
    bool got = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t hit = __ballot(i < cols && 64 * i + lane < G && ic[i] > mt);
      if (!got && hit) {
        const int src = first_lane(hit);
        const int32_t r0 = c.start[i] + (int32_t)(mt - (ic[i] - c.cnt[i])) * BM;
        const int32_t r1 = std::min<int32_t>(r0 + BM, c.end[i]);
        *g_out = 64 * i + src;
        *row0 = __shfl(r0, src, kWave);
        *row1 = __shfl(r1, src, kWave);
        got = true;
      }
    }
    return got;
  }
  // many groups: stream them for the totals, the range and the tile's group
  GroupChunk c;
  uint32_t tiles = 0, total = 0;
  for (int base = 0; base < G; base += 256) {
    load_chunk<BM>(off, G, stages, base, c);
    tiles += wave_sum_u32(c.cnt[0] + c.cnt[1] + c.cnt[2] + c.cnt[3]);
    total += wave_sum_u32(c.cost[0] + c.cost[1] + c.cost[2] + c.cost[3]);
  }
  const uint32_t t0 = (uint32_t)((uint64_t)total * x / 8), t1 = (uint32_t)((uint64_t)total * (x + 1) / 8);
  bool have0 = false, have1 = (x == 7);
  f0 = tiles; f1 = tiles;
  uint32_t carry_c = 0, carry_k = 0;
  for (int base = 0; base < G && !(have0 && have1); base += 256) {
    load_chunk<BM>(off, G, stages, base, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = base + 64 * i + lane < G;
      const uint32_t ic = wave_incl_sum_u32(c.cnt[i]) + carry_c;
      const uint32_t ik = wave_incl_sum_u32(c.cost[i]) + carry_k;
      if (!have0) {
        const uint64_t hit = __ballot(valid && ik >= t0);
        if (hit) {
          f0 = (uint32_t)__shfl((int)at(t0, ic, ik, c.cnt[i], c.cost[i], c.full[i]), first_lane(hit), kWave);
          have0 = true;
        }
      }
      if (!have1) {
        const uint64_t hit = __ballot(valid && ik >= t1);
        if (hit) {
          f1 = (uint32_t)__shfl((int)at(t1, ic, ik, c.cnt[i], c.cost[i], c.full[i]), first_lane(hit), kWave);
          have1 = true;
        }
      }
      carry_c = (uint32_t)__builtin_amdgcn_readlane((int)ic, kWave - 1);
      carry_k = (uint32_t)__builtin_amdgcn_readlane((int)ik, kWave - 1);
    }
  }
  const uint32_t logical = f0 * un + pos;
  if (logical >= f1 * un) return false;
  mt = logical / un;
  *nt = logical - mt * un;
  carry_c = 0;
  for (int base = 0; base < G; base += 256) {
    load_chunk<BM>(off, G, stages, base, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ic = wave_incl_sum_u32(c.cnt[i]) + carry_c;
      const uint64_t hit = __ballot(base + 64 * i + lane < G && ic > mt);
      if (hit) {
        const int src = first_lane(hit);
        const int32_t r0 = c.start[i] + (int32_t)(mt - (ic - c.cnt[i])) * BM;
        const int32_t r1 = std::min<int32_t>(r0 + BM, c.end[i]);
        *g_out = base + 64 * i + src;
        *row0 = __shfl(r0, src, kWave);
        *row1 = __shfl(r1, src, kWave);
        return true;
      }
      carry_c = (uint32_t)__builtin_amdgcn_readlane((int)ic, kWave - 1);
    }
  }
  return false;
}

// LDS of one workgroup: the double-buffered fp16 A stage, which the epilogue
// reuses as staging (SwiGLU: a [16][64] gate and result block per wave for
// the rare binary64 tail; bf16 output: a [32][36]-dword block per wave),
// followed by the tile's per-row factors, written by the prologue ([BM]
// floats s_ga*s_gb; SwiGLU also [BM] times the router weight and [BM] the
// router weight).
template <int WM, int NW, int EPI>
constexpr int gemm_rfac_offset() {
  constexpr int a_buf = 2 * WM * 8 * 64 * 16;
  constexpr int stage = EPI == EPI_SWIGLU ? NW * 2048 * 4 : EPI == EPI_BF16 ? NW * 32 * 36 * 4 : 0;
  return a_buf > stage ? a_buf : stage;
}
template <int WM, int NW, int EPI>
constexpr int gemm_lds_bytes() {
  return gemm_rfac_offset<WM, NW, EPI>() + (EPI == EPI_SWIGLU ? 3 : 1) * 32 * WM * 4;
}

// Waves per SIMD the register budget is sized for: the 128-row tile's 128
// accumulator registers need the 256-register budget of two waves; the
// 32-row tile fits 128 registers and runs four.
template <int WM>
constexpr int gemm_waves_per_simd() { return WM == 1 ? 4 : 2; }

template <int WM, int WN, int NW, int EPI>
__global__ __launch_bounds__(64 * NW, gemm_waves_per_simd<WM>()) void gemm_w4a4_kernel(GemmArgs a) {
  constexpr int BM = 32 * WM;
  constexpr int BN = 32 * WN * NW;
  constexpr int NT = 64 * NW;                       // threads
  constexpr int A_BYTES = WM * 8 * 64 * 16;         // fp16 A stage (fragment order)
  constexpr int A_UNITS = BM * 4;                   // quarter rows of 32 elements
  constexpr int APT = A_UNITS / NT;                 // A units per thread
  static_assert(APT >= 1 && A_UNITS % NT == 0, "A stage split across threads");
  static_assert(EPI != EPI_SWIGLU || WN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(gemm_lds_bytes<WM, NW, EPI>() <= 160 * 1024, "LDS of one workgroup");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t K = a.k;
  const int64_t N = a.n;

  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  int g;
  int64_t row0, row1, nt;
  if (a.tile_table) {                           // precomputed schedule: one 16-byte entry
    const int4 te = a.tile_table[blockIdx.x];
    if (te.x < 0) return;
    g = te.x; row0 = te.y; row1 = te.z; nt = te.w;
  } else if (!schedule_tile<BM>(a.offsets, a.num_groups, K, ntn, blockIdx.x, &g, &row0, &row1, &nt)) {
    return;
  }
  g = __builtin_amdgcn_readfirstlane(g);       // wave-uniform: scalar bases below
  row0 = uniform64(row0);
  row1 = uniform64(row1);

  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- B: this lane's column j = 32*WN*wave + 32n + l32 of the tile.
  // Addresses are a scalar base (the group's matrix) plus a 32-bit lane
  // offset; the launcher rejects groups of 4 GiB or more.  Row-major B keeps
  // a row's stage in 64 code bytes + 8 scale bytes; the tiled layout
  // (nvfp4_pack_weights) stores each (32-row block, stage) as the 64 lanes'
  // operands side by side, so every load of a wave is one contiguous span.
  const bool tiled = a.b_layout == 1;
  const uint8_t* b_cbase = a.b_codes + (int64_t)g * N * (K / 2);
  const uint8_t* b_sbase = a.b_scales + (int64_t)g * N * (K / 16);
  const int64_t b_cstage = tiled ? 2048 : 64;    // bytes between stages
  const int64_t b_sstage = tiled ? 256 : 8;
  const int64_t b_c1 = tiled ? 1024 : 16;        // codes of substeps 4-7
  uint32_t bco[WN], bso[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    int64_t c, cmax = N - 1;
    if (EPI == EPI_SWIGLU) {                     // gate | up pairing
      constexpr int HALF = WN / 2;
      const int64_t gate0 = nt * (BN / 2) + (int64_t)wave * 32 * HALF;
      c = (n < HALF) ? gate0 + 32 * n + l32 : a.inter + gate0 + 32 * (n - HALF) + l32;
      cmax = (n < HALF) ? a.inter - 1 : 2 * a.inter - 1;
    } else {
      c = nt * BN + (int64_t)wave * 32 * WN + 32 * n + l32;
    }
    const int64_t row = c < cmax ? c : cmax;     // B row inside the group
    if (tiled) {                                 // (clamped columns read some valid row)
      const int64_t tile0 = (row / 32) * (K / kKS);
      bco[n] = (uint32_t)(tile0 * 2048 + 16 * lane);
      bso[n] = (uint32_t)(tile0 * 256 + 4 * lane);
    } else {
      bco[n] = (uint32_t)(row * (K / 2) + 32 * half);
      bso[n] = (uint32_t)(row * (K / 16) + 4 * half);
    }
  }
  // one stage of the lane's B columns, reloaded in place a part at a time:
  // codes of substeps 0-3 (c0), 4-7 (c1) and the four block scales (s).  The
  // 128-row tile holds one such set; the 32-row tile, whose stages are short,
  // holds two and keeps the loads of the next two stages in flight.
  struct BSet {
    u32x4_t c0[WN], c1[WN];
    uint32_t s[WN];
  };
  auto b_load_c0 = [&](BSet& b, int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) b.c0[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + bco[n]);
  };
  auto b_load_c1 = [&](BSet& b, int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) b.c1[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + b_c1 + bco[n]);
  };
  auto b_load_s = [&](BSet& b, int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) b.s[n] = *reinterpret_cast<const uint32_t*>(b_sbase + st * b_sstage + bso[n]);
  };

  // 16-byte slot of MFMA lane l in an A fragment block of substeps 4sq..4sq+3:
  // flipping bits 2-3 keeps the slot inside its group of 16 (reads stay
  // conflict free) and spreads the writers of one row over four bank groups
  auto aslot = [](int l, int sq) { return l ^ (4 * (sq + 2 * (l >> 5))); };
  // ---- A: thread-owned quarter rows (32 elements = 16 code bytes + 2 scales).
  // Row r of the tile is A row row0 + r, or, gathering (a_row_src), token
  // row a_row_src[row0 + r] of the token-major quantized activations (a
  // padding row's -1 reads the all-zero row a_pad_row).
  const bool gather = a.a_row_src != nullptr;
  const uint8_t* a_cbase = gather ? a.a_codes : a.a_codes + row0 * (K / 2);
  const uint8_t* a_sbase = gather ? a.a_scales : a.a_scales + row0 * (K / 16);
  uint32_t a_src[APT], a_ssrc[APT];
  int a_dst[APT];
#pragma unroll
  for (int j = 0; j < APT; ++j) {
    const int u = tid + NT * j;
    const int r = u / 4, q = u % 4, h = q / 2;
    int64_t ar = r < row1 - row0 ? r : row1 - row0 - 1;   // row inside the tile
    if (gather) {
      const int32_t t = a.a_row_src[row0 + ar];
      ar = t >= 0 ? (int64_t)t : a.a_pad_row;
    }
    a_src[j] = (uint32_t)(ar * (K / 2) + 16 * q);
    a_ssrc[j] = (uint32_t)(ar * (K / 16) + 2 * q);
    // fragment r/32, lane (r%32) + 32h, substeps 4(q%2) .. 4(q%2)+3
    a_dst[j] = (((r / 32) * 8 + 4 * (q % 2)) * 64 + aslot((r % 32) + 32 * h, q % 2)) * 16;
  }
  u32x4_t araw[APT];
  uint32_t asc[APT];
  auto a_load_unit = [&](int j, int64_t st) {
    araw[j] = *reinterpret_cast<const u32x4_t*>(a_cbase + st * 64 + a_src[j]);
    asc[j] = *reinterpret_cast<const uint16_t*>(a_sbase + st * 8 + a_ssrc[j]);
  };
  auto a_load = [&](int64_t st) {
#pragma unroll
    for (int j = 0; j < APT; ++j) a_load_unit(j, st);
  };
  // decode chunk c (8 elements) of quarter row j into buffer buf
  auto a_decode_unit = [&](int j, int c, int buf) {
    uint8_t* sb = smem + buf * A_BYTES;
    const half2_t s2 = e4m3x2_to_half2(asc[j]);
    const _Float16 sc = (c < 2) ? s2[0] : s2[1];
    *reinterpret_cast<half8_t*>(sb + a_dst[j] + c * 1024) = decode8(araw[j][c], half2_t{sc, sc});
  };
  auto a_decode = [&](int c, int buf) {
#pragma unroll
    for (int j = 0; j < APT; ++j) a_decode_unit(j, c, buf);
  };
  // With two quarter rows per thread, the next stage's A is decoded one
  // chunk per substep (row 0 in substeps 0-3, row 1 in 4-7) and each row's
  // registers take the stage after that as soon as its last chunk is decoded;
  // otherwise all rows are decoded in substeps 4-7 and reloaded after the
  // stage.  Spreading keeps the decode arithmetic even across the substeps.
  constexpr bool A_SPREAD = APT == 2;

  float16_t acc[WM][WN];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int n = 0; n < WN; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

  // decoded B operands of the substep about to be multiplied (filled one
  // substep ahead, across the stage boundary too)
  half8_t fbc[WN];
  // the lane's B operands of substep s from the code registers and scales
  auto b_decode = [&](const BSet& b, int s, const half2_t (&bsc)[WN][2], half8_t (&fb)[WN]) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const uint32_t c = s < 4 ? b.c0[n][s] : b.c1[n][s - 4];
      const _Float16 sc = bsc[n][s / 4][(s / 2) % 2];
      fb[n] = decode8(c, half2_t{sc, sc});
    }
  };
  auto b_scales = [&](const BSet& b, half2_t (&bsc)[WN][2]) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      bsc[n][0] = e4m3x2_to_half2(b.s[n]);
      bsc[n][1] = e4m3x2_to_half2(b.s[n] >> 16);
    }
  };

  // multiplies stage buffer `buf` with the B operands of set `cb` for the
  // first MV 32-row blocks of the tile (the others are all padding).
  // Software pipelined by substep: while the MFMAs of substep s run, the
  // lane reads the A fragments and decodes the B operands of substep s+1 (at
  // s = 7: substep 0 of the next stage, from set `nb`), and substeps 4..7
  // decode the next stage's A (raw registers loaded one stage earlier) into
  // buffer `nxt`.  Set cb's code registers of substeps 0-3 / 4-7 and its
  // scales are reloaded with stage `bload` right after their last decode
  // (one set: nb is cb and bload the next stage; two sets: nb holds the next
  // stage and bload is the one after).  The loads are unconditional (the
  // last stages re-fetch the last one): with a branch around them the
  // compiler has to assume the short path and waits for the loads just
  // issued before the A decode.
  auto compute = [&](auto mv_c, int buf, int nxt, int64_t bload, int64_t aload, BSet& cb, BSet& nb) {
    constexpr int MV = decltype(mv_c)::value;
    constexpr int VPM = NVFP4_VPM;                 // VALU per MFMA slot
    const uint8_t* sb = smem + buf * A_BYTES;
    auto a_frag = [&](int m, int s) {
      return *reinterpret_cast<const half8_t*>(sb + ((m * 8 + s) * 64 + aslot(lane, s / 4)) * 16);
    };
    half2_t bsc[WN][2];
    b_scales(cb, bsc);
    b_load_s(cb, bload);
    half8_t fa[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) fa[m] = a_frag(m, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t fbn[WN];
      if (s < 7) {
        b_decode(cb, s + 1, bsc, fbn);
      } else {                       // substep 0 of the next stage
        half2_t bsn[WN][2];
        b_scales(nb, bsn);
        b_decode(nb, 0, bsn, fbn);
      }
      // fragment m's registers take fragment m of the next substep as soon
      // as its MFMAs are issued
#pragma unroll
      for (int m = 0; m < MV; ++m) {
#pragma unroll
        for (int n = 0; n < WN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[m], fbc[n], acc[m][n], 0, 0, 0);
        if (s < 7) fa[m] = a_frag(m, s + 1);
      }
      if constexpr (A_SPREAD) {
        a_decode_unit(s / 4, s % 4, nxt);
        if (s % 4 == 3) a_load_unit(s / 4, aload);
      } else if (s >= 4) {
        a_decode(s - 4, nxt);
      }
      if (s == 2) b_load_c0(cb, bload);  // substeps 0-3 decoded
      if (s == 6) b_load_c1(cb, bload);  // substeps 4-7 decoded
#pragma unroll
      for (int n = 0; n < WN; ++n) fbc[n] = fbn[n];
      // issue order: each MFMA followed by a share of the decode arithmetic,
      // which runs in the MFMA's shadow, and the fragment reads in between
#pragma unroll
      for (int m = 0; m < MV; ++m) {
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        }
        if (s < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop.  Stage it is multiplied from A buffer it&1; its B parts
  // are replaced by the next stage's as they are used.  The next stage's A
  // codes (in registers,
  // loaded one stage earlier) are decoded into the other buffer between the
  // MFMAs of substeps 4-7, after which the registers receive the A codes of
  // the stage after that.  The tail stages re-fetch the last stage's A and B
  // into registers that nothing reads: the loop stays branch-free.
  const int64_t nst = K / kKS;
  BSet bx, by;
  // the tile's per-row factors: loaded with the first stage, written to LDS
  // once its A has been decoded (the epilogue then starts without a load)
  float* rfac = reinterpret_cast<float*>(smem + gemm_rfac_offset<WM, NW, EPI>());
  float rf_sa = 0.0f, rf_p = 0.0f;
  const float sgb = a.b_gscale[g];
  auto prologue = [&]() {
    if (tid < BM) {
      const int64_t row = row0 + tid;
      const int64_t rr = row < row1 ? row : row1 - 1;
      if (gather) {                              // the token's outer scale
        const int32_t t = a.a_row_src[rr];
        rf_sa = t >= 0 ? a.a_gscale[t] : 0.0f;
      } else {
        rf_sa = a.a_gscale[rr];
      }
      if (EPI == EPI_SWIGLU) rf_p = a.row_prob[rr];
    }
    a_load(0);
    b_load_s(bx, 0);
    b_load_c0(bx, 0);
    if constexpr (A_SPREAD) {
      // the loads left in flight end in the loop's own order (A row 0 of
      // stage 1, B codes of substeps 4-7, A row 1), so the wait counts the
      // compiler derives at the loop head hold for both ways in
      {
        half2_t bsc[WN][2];
        b_scales(bx, bsc);
        b_decode(bx, 0, bsc, fbc);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) a_decode_unit(0, c, 0);
      a_load_unit(0, nst > 1 ? 1 : 0);
      b_load_c1(bx, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) a_decode_unit(1, c, 0);
      a_load_unit(1, nst > 1 ? 1 : 0);
    } else {
      b_load_c1(bx, 0);
      {
        half2_t bsc[WN][2];
        b_scales(bx, bsc);
        b_decode(bx, 0, bsc, fbc);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) a_decode(c, 0);
      a_load(nst > 1 ? 1 : 0);
    }
    if (tid < BM) {
      const float sc = rf_sa * sgb;               // C = ACC * s_ga * s_gb
      rfac[tid] = sc;
      if (EPI == EPI_SWIGLU) {
        rfac[BM + tid] = sc * rf_p;               // the up half, weighted
        rfac[2 * BM + tid] = rf_p;
      }
    }
    __syncthreads();
  };
  auto clamp_st = [&](int64_t st) { return st < nst ? st : nst - 1; };
  auto main_loop = [&](auto mv_c) {
    prologue();
    for (int64_t it = 0; it < nst; ++it) {
      const int cur = (int)(it & 1), nxt = cur ^ 1;
      compute(mv_c, cur, nxt, clamp_st(it + 1), clamp_st(it + 2), bx, bx);
      if constexpr (!A_SPREAD) a_load(clamp_st(it + 2));
      __syncthreads();
    }
  };
  // two B sets, an even number of stages: stages it (set x) and it+1 (set y)
  // per iteration, each set reloaded two stages ahead
  auto main_loop2 = [&](auto mv_c) {
    prologue();
    b_load_s(by, clamp_st(1));
    b_load_c0(by, clamp_st(1));
    b_load_c1(by, clamp_st(1));
    for (int64_t it = 0; it < nst; it += 2) {
      compute(mv_c, 0, 1, clamp_st(it + 2), clamp_st(it + 2), bx, by);
      if constexpr (!A_SPREAD) a_load(clamp_st(it + 2));
      __syncthreads();
      compute(mv_c, 1, 0, clamp_st(it + 3), clamp_st(it + 3), by, bx);
      if constexpr (!A_SPREAD) a_load(clamp_st(it + 3));
      __syncthreads();
    }
  };
  // 32-row blocks of the tile that hold at least one valid row; the tile's
  // last rows are padding when the group ends inside it.
  const int mv = __builtin_amdgcn_readfirstlane((int)std::min<int64_t>(WM, (row1 - row0 + 31) / 32));
  static_assert(WM <= 4, "main loop instances");
  if constexpr (WM == 1) {
    if (nst % 2 == 0) main_loop2(std::integral_constant<int, 1>{});
    else main_loop(std::integral_constant<int, 1>{});
  } else switch (mv) {
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (WM >= 2) main_loop(std::integral_constant<int, 2 <= WM ? 2 : 1>{}); break;
    case 3: if constexpr (WM >= 3) main_loop(std::integral_constant<int, 3 <= WM ? 3 : 1>{}); break;
    default: main_loop(std::integral_constant<int, WM>{}); break;
  }

  // ---- epilogue straight from the accumulators: acc[m][n][r] holds
  // C[32m + 8(r/4) + 4h + r%4][32n + l32] of this wave's tile (h = lane/32,
  // l32 = lane%32).  The per-row factors go through LDS once (after the
  // loop's last barrier nothing reads the A buffers).  For 16-bit outputs
  // neighbouring lanes swap one value per row pair, so that each lane
  // stores two adjacent columns of one row as one dword.
  const bool odd = (lane & 1) != 0;
  // the row (inside the tile) of accumulator element r of 32-row block m
  auto trow = [&](int m, int r) { return 32 * m + 8 * (r / 4) + 4 * half + (r % 4); };
  // Stores address rows from a per-lane base row plus a compile-time offset
  // times a uniform row pitch.  Paired 16-bit stores: lane row
  // row0 + 4h + (lane & 1), offset 32m + 8(t/2) + 2(t%2) for pair t of
  // block m; single-column stores: lane row row0 + 4h, offset trow - 4h.
  const int64_t prow = row0 + 4 * half + (odd ? 1 : 0);
  const int plim = (int)(row1 - prow);           // pair offsets below this are real rows
  auto poff = [](int m, int t) { return 32 * m + 8 * (t / 2) + 2 * (t % 2); };
  // stores dwords v[t] at p + poff(m, t) * pitch, all of them when block m
  // is whole, else those on real rows
  auto store_pairs = [&](uint32_t* p, int64_t pitch, int m, const uint32_t (&v)[8]) {
    if (row0 + 32 * (m + 1) <= row1) {
#pragma unroll
      for (int t = 0; t < 8; ++t) p[poff(m, t) * pitch] = v[t];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (poff(m, t) < plim) p[poff(m, t) * pitch] = v[t];
    }
  };
  // pairs lanes 2i and 2i+1: of the rows of elements (r0, r0 + 1) the even
  // lane keeps the first and the odd lane the second, both as the bf16 pair
  // (column 2i, column 2i+1)
  auto pair_bf16 = [&](float v0, float v1) {
    const float give = odd ? v0 : v1;
    const float got = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, give), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    return odd ? pack_bf16x2(got, v1) : pack_bf16x2(v0, got);
  };
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    if (m >= mv) continue;
    float sv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(rfac + 32 * m + 8 * q + 4 * half);
      sv[4 * q] = t.x; sv[4 * q + 1] = t.y; sv[4 * q + 2] = t.z; sv[4 * q + 3] = t.w;
    }
    if (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const int64_t I = a.inter;
      const int64_t gate0 = nt * (BN / 2) + (int64_t)wave * 32 * HALF;
      float spv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(rfac + BM + 32 * m + 8 * q + 4 * half);
        spv[4 * q] = t.x; spv[4 * q + 1] = t.y; spv[4 * q + 2] = t.z; spv[4 * q + 3] = t.w;
      }
      uint32_t rmax[8];                          // |D| maxima of this lane's rows (bf16 bits)
#pragma unroll
      for (int t = 0; t < 8; ++t) rmax[t] = 0;
#pragma unroll
      for (int n = 0; n < HALF; ++n) {
        if (gate0 + 32 * n >= I) break;          // inter % 64 == 0: 32-column blocks are whole
        float dv[16];
        float gmin = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float gv = acc[m][n][r] * sv[r];
          dv[r] = swiglu_fast(gv, acc[m][HALF + n][r] * spv[r]);
          gmin = fminf(gmin, gv);
        }
        if (gmin < -80.0f) {
          // rare: the binary64 tail, in one copy (a loop over the 16
          // elements staged in this wave's part of the free A buffers)
          float* tg = reinterpret_cast<float*>(smem) + wave * 2048;  // [16][64] gate, then [16][64] result
#pragma unroll
          for (int r = 0; r < 16; ++r) tg[r * 64 + lane] = acc[m][n][r] * sv[r];
          float* tu = tg + 1024;
#pragma unroll
          for (int r = 0; r < 16; ++r) tu[r * 64 + lane] = acc[m][HALF + n][r] * sv[r];
#pragma unroll 1
          for (int r = 0; r < 16; ++r) {
            const float gv = tg[r * 64 + lane];
            if (gv < -80.0f) tu[r * 64 + lane] = swiglu_tail(gv, tu[r * 64 + lane], rfac[2 * BM + trow(m, r)]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (tg[r * 64 + lane] < -80.0f) dv[r] = tu[r * 64 + lane];
        }
        const int64_t colp = gate0 + 32 * n + (l32 & ~1);
        uint32_t pk[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pk[t] = pair_bf16(dv[2 * t], dv[2 * t + 1]);
          const uint32_t mag = pk[t] & 0x7FFF7FFFu;
          const uint32_t m16 = (mag & 0xFFFFu) > (mag >> 16) ? (mag & 0xFFFFu) : (mag >> 16);
          rmax[t] = rmax[t] > m16 ? rmax[t] : m16;
        }
        store_pairs(reinterpret_cast<uint32_t*>(a.d_out + prow * I + colp), I / 2, m, pk);
        if (a.c_out) {
          const int64_t cg = gate0 + 32 * n + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = row0 + trow(m, r);
            if (row < row1) {
              a.c_out[row * 2 * I + cg] = acc[m][n][r] * sv[r];
              a.c_out[row * 2 * I + I + cg] = acc[m][HALF + n][r] * sv[r];
            }
          }
        }
      }
      // row maxima over the wave's columns: the 16 lanes of one parity in a
      // lane half share rows; three halving exchanges (lane bits 4, 3, 2)
      // leave lane bits (4,3,2) = t's bits, a last one over bit 1 completes it
      const int b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1;
      auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
      uint32_t v4[4], v2[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t give = b4 ? rmax[j] : rmax[4 + j];
        const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)give, 0x401F);   // lane ^ 16
        v4[j] = umax(b4 ? rmax[4 + j] : rmax[j], got);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t give = b3 ? v4[j] : v4[2 + j];
        const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)give, 0x201F);   // lane ^ 8
        v2[j] = umax(b3 ? v4[2 + j] : v4[j], got);
      }
      uint32_t mx;
      {
        const uint32_t give = b2 ? v2[0] : v2[1];
        const uint32_t got = (uint32_t)__builtin_amdgcn_ds_swizzle((int)give, 0x101F);     // lane ^ 4
        mx = umax(b2 ? v2[1] : v2[0], got);
      }
      mx = umax(mx, (uint32_t)__builtin_amdgcn_ds_swizzle((int)mx, 0x081F));               // lane ^ 2
      const int t = 4 * b4 + 2 * b3 + b2;
      const int rr = 2 * t + (odd ? 1 : 0);
      const int64_t row = row0 + 32 * m + 8 * (rr / 4) + 4 * half + (rr % 4);
      if (((lane >> 1) & 1) == 0 && row < row1 && mx != 0u)
        atomicMax(reinterpret_cast<uint32_t*>(a.amax) + row, mx << 16);
    } else {
      // bf16: the wave's 32 x 32*WN block is staged in LDS (one dword per
      // column pair) and stored as 16-byte pieces, 8 lanes per row
      uint32_t* stage = reinterpret_cast<uint32_t*>(smem) + wave * (32 * 36);
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const int64_t col0 = nt * BN + (int64_t)wave * 32 * WN + 32 * n;
        if (col0 >= N) break;                    // N % 32 == 0: 32-column blocks are whole
        if (EPI == EPI_F32) {
          const int64_t srow = row0 + 4 * half;
          float* o = static_cast<float*>(a.out) + srow * N + col0 + l32;
          const int slim = (int)(row1 - srow);
          const bool whole = row0 + 32 * (m + 1) <= row1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = trow(m, r) - 4 * half;
            if (whole || off < slim) o[off * N] = acc[m][n][r] * sv[r];
          }
        } else {
          uint32_t pk[8];
#pragma unroll
          for (int t = 0; t < 8; ++t)
            pk[t] = pair_bf16(acc[m][n][2 * t] * sv[2 * t], acc[m][n][2 * t + 1] * sv[2 * t + 1]);
          // the pairs go to this wave's [32][72] bf16 staging block (row
          // pitch 144 bytes), to leave as 16-byte row pieces below
#pragma unroll
          for (int t = 0; t < 8; ++t)
            stage[(poff(0, t) + 4 * half + (odd ? 1 : 0)) * 36 + 16 * n + (l32 >> 1)] = pk[t];
        }
      }
      if (EPI == EPI_BF16) {
        static_assert(WN == 2, "the staged block is 64 columns wide");
        const int64_t colw = nt * BN + (int64_t)wave * 32 * WN;   // the wave's first column
        if (colw < N) {
          const int sr = lane >> 3, sc = lane & 7;               // 8 rows x 8 pieces of 16 bytes
          // N % 32 == 0: the wave's second 32-column block may lie past N
          // (its staging was not written), a piece never straddles it
          const bool col_ok = colw + 8 * sc < N;
          uint16_t* o = static_cast<uint16_t*>(a.out) + (row0 + 32 * m) * N + colw + 8 * sc;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = 8 * q + sr;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + r * 36 + 4 * sc);
            if (col_ok && row0 + 32 * m + r < row1) *reinterpret_cast<uint4*>(o + (int64_t)r * N) = v;
          }
        }
      }
    }
  }
}

// ---- B layout transfer ---------------------------------------------------
//
// Row-major B ([G*N rows, K/2 code bytes], [G*N, K/16] scales) -> the tiled
// layout read above.  Tile t = (g*(N/32) + rb) * (K/128) + st holds rows
// 32rb..32rb+31 of group g over K stage st:
//   codes  t*2048 + c*1024 + 16*L : row 32rb + L%32, code bytes
//          [64st + 32(L/32) + 16c, +16)            (c = 0, 1; L = 0..63)
//   scales t*256 + 4*L            : row 32rb + L%32, scale bytes [8st + 4(L/32), +4)
// One thread per 16-byte code piece; the c == 0 threads also move the scales.
__global__ __launch_bounds__(256) void pack_b_kernel(const uint8_t* codes, const uint8_t* scales,
                                                     int64_t rows, int64_t k, uint8_t* pcodes,
                                                     uint8_t* pscales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nst = k / kKS;
  if (i >= (rows / 32) * nst * 128) return;
  const int64_t t = i / 128;
  const int piece = (int)(i % 128), c = piece / 64, L = piece % 64;
  const int64_t rb = t / nst, st = t % nst;
  const int64_t row = rb * 32 + L % 32;
  const u32x4_t v =
      *reinterpret_cast<const u32x4_t*>(codes + row * (k / 2) + 64 * st + 32 * (L / 32) + 16 * c);
  *reinterpret_cast<u32x4_t*>(pcodes + t * 2048 + c * 1024 + 16 * L) = v;
  if (c == 0)
    *reinterpret_cast<uint32_t*>(pscales + t * 256 + 4 * L) =
        *reinterpret_cast<const uint32_t*>(scales + row * (k / 16) + 8 * st + 4 * (L / 32));
}

hipError_t launch_pack_b(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                         uint8_t* pcodes, uint8_t* pscales, hipStream_t s) {
  const int64_t n = (rows / 32) * (k / kKS) * 128;
  if (n == 0) return hipSuccess;
  pack_b_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(codes, scales, rows, k, pcodes, pscales);
  return hipGetLastError();
}

// ---- launchers -------------------------------------------------------------

// Grid of one launch: BM-row tiles, ntn n-tiles per m-tile, and the
// workgroup positions the XCD ranges need.
struct TileCfg {
  int bm;
  int64_t ntn, blocks;
};

template <int WM, int WN, int NW, int EPI>
static TileCfg tile_cfg(const GemmArgs& a) {
  constexpr int BM = 32 * WM, BN = 32 * WN * NW;
  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (a.n + BN - 1) / BN;
  // upper bound on the m-tiles of all groups: sum ceil(n_g/BM) <= cap/BM + G.
  // An XCD's range costs at most a 1/8 share of the total plus one m-tile,
  // and an m-tile costs between tile_cost(1) and tile_cost(WM), which bounds
  // its m-tiles; the grid gives every XCD that many positions.
  const int64_t mtiles = (a.rows_cap + BM - 1) / BM + a.num_groups;
  const int64_t st = std::min<int64_t>(a.k / kKS, kCostMaxStages);
  const int64_t cmax = kCostFixed + st * (kCostStage + WM), cmin = kCostFixed + st * (kCostStage + 1);
  const int64_t per_xcd = (cmax * (mtiles + 8) + 8 * cmin - 1) / (8 * cmin) + 1;
  return TileCfg{BM, ntn, 8 * per_xcd * ntn};
}

template <int WM, int WN, int NW, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int64_t blocks = tile_cfg<WM, WN, NW, EPI>(a).blocks;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.n * a.k / 2 > 0xFFFFFFFFll) return hipErrorInvalidValue;   // 32-bit lane offsets into a group
  constexpr size_t lds = (size_t)gemm_lds_bytes<WM, NW, EPI>();
  gemm_w4a4_kernel<WM, WN, NW, EPI><<<(unsigned)blocks, 64 * NW, lds, s>>>(a);
  return hipGetLastError();
}

// Tiles: MFMA blocks per wave (M, N) and waves per workgroup (along N).  The
// 128 x 256 tile serves groups of many rows, two workgroups per CU.  FC1
// (the SwiGLU epilogue; K = hidden size, 16 stages at 2048) takes the
// 128 x 512 tile, one workgroup per CU: it gains more from decoding each A
// stage for twice the columns than it loses without a second workgroup to
// cover prologue and epilogue.  The plain GEMMs keep 128 x 256: FC2's short
// K (the intermediate size, 6 stages at 768) loses on the wider tile, and
// for dense shapes the outcome depends on how the tiles fill the last round
// of the grid.  When the groups average at
// most kSmallTileRows rows (decode-sized batches: a few rows per expert) the
// 128-row tile would multiply one 32-row block and leave the weight stream
// at two workgroups per CU; the 32 x 128 tile runs four waves per SIMD, so
// twice as many weight loads are in flight.
#ifndef NVFP4_GEMM_TILE
#define NVFP4_GEMM_TILE 4, 2, 4
#endif
#ifndef NVFP4_GEMM_TILE_FC1
#define NVFP4_GEMM_TILE_FC1 4, 2, 8
#endif
#define NVFP4_GEMM_TILE_SMALL 1, 2, 2
#ifndef NVFP4_SMALL_TILE_ROWS
#define NVFP4_SMALL_TILE_ROWS 32
#endif
constexpr int64_t kSmallTileRows = NVFP4_SMALL_TILE_ROWS;

bool gemm_uses_small_tile(int64_t rows_cap, int64_t num_groups) {
  return rows_cap <= kSmallTileRows * num_groups;
}

hipError_t launch_gemm_plain(const GemmArgs& a, hipStream_t s) {
  if (gemm_uses_small_tile(a.rows_cap, a.num_groups)) {
    if (a.out_dtype == 0) return launch_cfg<NVFP4_GEMM_TILE_SMALL, EPI_F32>(a, s);
    return launch_cfg<NVFP4_GEMM_TILE_SMALL, EPI_BF16>(a, s);
  }
  if (a.out_dtype == 0) return launch_cfg<NVFP4_GEMM_TILE, EPI_F32>(a, s);
  return launch_cfg<NVFP4_GEMM_TILE, EPI_BF16>(a, s);
}

hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s) {
  if (gemm_uses_small_tile(a.rows_cap, a.num_groups))
    return launch_cfg<NVFP4_GEMM_TILE_SMALL, EPI_SWIGLU>(a, s);
  return launch_cfg<NVFP4_GEMM_TILE_FC1, EPI_SWIGLU>(a, s);
}

// the configuration launch_gemm_plain / launch_gemm_swiglu pick
static TileCfg launch_tile_cfg(const GemmArgs& a, bool swiglu) {
  const bool small = gemm_uses_small_tile(a.rows_cap, a.num_groups);
  if (swiglu)
    return small ? tile_cfg<NVFP4_GEMM_TILE_SMALL, EPI_SWIGLU>(a) : tile_cfg<NVFP4_GEMM_TILE_FC1, EPI_SWIGLU>(a);
  return small ? tile_cfg<NVFP4_GEMM_TILE_SMALL, EPI_BF16>(a) : tile_cfg<NVFP4_GEMM_TILE, EPI_BF16>(a);
}

int64_t gemm_grid_blocks(const GemmArgs& a, bool swiglu) {
  const int64_t b = launch_tile_cfg(a, swiglu).blocks;
  return b > 0 ? b : 0;
}

TileTableSpec gemm_mtile_table_spec(int64_t rows_cap, int32_t num_groups, int64_t k, int4* table) {
  GemmArgs g{};
  g.rows_cap = rows_cap; g.num_groups = num_groups; g.k = k;
  g.n = 32 * 2 * 8;                               // one 512-column tile: ntn = 1
  const TileCfg c = tile_cfg<4, 2, 8, EPI_F32>(g);
  TileTableSpec t{};
  t.table = table; t.bm = c.bm; t.k = k; t.ntn = 1; t.blocks = c.blocks > 0 ? c.blocks : 0;
  return t;
}

TileTableSpec gemm_tile_table_spec(const GemmArgs& a, bool swiglu, int4* table) {
  const TileCfg c = launch_tile_cfg(a, swiglu);
  TileTableSpec t{};
  t.table = table; t.bm = c.bm; t.k = a.k; t.ntn = c.ntn; t.blocks = c.blocks > 0 ? c.blocks : 0;
  return t;
}

}  // namespace nvfp4
