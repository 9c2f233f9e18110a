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
// device offsets: every workgroup derives its (group, m-tile) from a
// wave-wide scan of the per-group tile counts, so the host never reads them;
// surplus workgroups exit.
#include <type_traits>
#include <algorithm>

#include "launch.h"
#include "nvfp4_device.h"

namespace nvfp4 {

// ---- operand decode ------------------------------------------------------

// Two E4M3 bytes (bits 0-7 and 8-15 of s) -> their values as two fp16.
// Shifting a byte left by 7 places its exponent and mantissa in the fp16
// fields (bias 15 instead of 7; E4M3 subnormals land on fp16 subnormals);
// multiplying by 2^8 restores the value exactly.
__device__ __forceinline__ half2_t e4m3x2_to_half2(uint32_t s) {
  uint32_t v = ((s & 0x7Fu) << 7) | ((s & 0x7F00u) << 15);
  half2_t h;
  __builtin_memcpy(&h, &v, 4);
  const half2_t k256 = {(_Float16)256.0f, (_Float16)256.0f};
  return h * k256;
}

// 8 FP4 codes (one dword, element 2i in the low nibble of byte i) times the
// block scale -> 8 fp16 values, exactly.
__device__ __forceinline__ half8_t decode8(uint32_t c, half2_t sb) {
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
  h0 = h0 * sb; h1 = h1 * sb; h2 = h2 * sb; h3 = h3 * sb;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// ---- tile -> group map ---------------------------------------------------

// Finds the group owning global m-tile `mt` (m-tiles are numbered group by
// group, ceil(rows_g / BM) per group).  Returns false if mt is past the end.
__device__ __forceinline__ bool locate_mtile(const int32_t* off, int G, int BM, int64_t mt,
                                             int* g_out, int64_t* row0, int64_t* row1) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t carry = 0;
  for (int base = 0; base < G; base += kWave) {
    const int g = base + lane;
    int64_t cnt = 0;
    if (g < G) {
      const int64_t n = (int64_t)off[g + 1] - (int64_t)off[g];
      cnt = n > 0 ? (n + BM - 1) / BM : 0;
    }
    int64_t incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int64_t y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int64_t start = carry + incl - cnt;
    const bool mine = (g < G) && (mt >= start) && (mt < start + cnt);
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int gg = __shfl(g, src, kWave);
      const int64_t st = __shfl(start, src, kWave);
      *g_out = gg;
      *row0 = (int64_t)off[gg] + (mt - st) * BM;
      const int64_t end = off[gg + 1];
      *row1 = (*row0 + BM < end) ? *row0 + BM : end;
      return true;
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
  return false;
}

// ---- kernel --------------------------------------------------------------
//
// Workgroup = NW waves side by side along N, sized so that two workgroups
// share a compute unit (one wave of each per SIMD): while one workgroup sits
// in its prologue, a barrier or its VALU-heavy epilogue, the other keeps the
// matrix cores busy.  The workgroup owns a BM x BN output tile of one group
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
// The epilogue goes through LDS, 16 rows at a time, so that each lane
// finishes contiguous columns of one output row.
constexpr int kKS = 128;          // K per stage

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2 };

// Number of BM-row tiles over all groups (the same value in every lane).
__device__ __forceinline__ int64_t count_mtiles(const int32_t* off, int G, int BM) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t total = 0;
  for (int base = 0; base < G; base += kWave) {
    const int g = base + lane;
    int64_t cnt = 0;
    if (g < G) {
      const int64_t n = (int64_t)off[g + 1] - (int64_t)off[g];
      cnt = n > 0 ? (n + BM - 1) / BM : 0;
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) cnt += __shfl_xor(cnt, o, kWave);
    total += cnt;
  }
  return total;
}

// Workgroups are dealt to the 8 XCDs round robin (workgroup b runs on XCD
// b % 8).  Of the n real tiles (counted on the device; the grid is an upper
// bound), XCD x takes an equal contiguous range: consecutive tiles share A
// rows and, inside an expert, B rows, which then stay in that XCD's L2.
// Returns false for the surplus workgroups.
__device__ __forceinline__ bool xcd_remap(int64_t bid, int64_t n, int64_t* logical) {
  const int64_t x = bid % 8, pos = bid / 8, q = n / 8, r = n % 8;
  if (pos >= ((x < r) ? q + 1 : q)) return false;
  *logical = (x < r) ? x * (q + 1) + pos : r * (q + 1) + (x - r) * q + pos;
  return true;
}

// SwiGLU weighted by the router probability, in binary32; below g = -80
// binary32 exp(-g) overflows while g e^g u p may still be a normal bf16, so
// that rare tail is evaluated in binary64.
__device__ __noinline__ float swiglu_tail(float g, float u, float p) {
  const double eg = exp((double)g);
  return (float)(((double)g * eg / (1.0 + eg)) * (double)u * (double)p);
}

// silu(g) * up, with the router weight already folded into `up` (a few
// binary32 roundings; D is checked to one bf16 ulp and the hardware
// reciprocal, about 1 ulp of binary32, is far inside that)
__device__ __forceinline__ float swiglu_fast(float g, float up) {
  const float silu = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return silu * up;
}

// two binary32 -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t b = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int WM, int WN, int NW, int EPI>
__global__ __launch_bounds__(64 * NW, 2) void gemm_w4a4_kernel(GemmArgs a) {
  constexpr int BM = 32 * WM;
  constexpr int BN = 32 * WN * NW;
  constexpr int NT = 64 * NW;                       // threads
  constexpr int A_BYTES = WM * 8 * 64 * 16;         // fp16 A stage (fragment order)
  constexpr int A_UNITS = BM * 4;                   // quarter rows of 32 elements
  constexpr int APT = A_UNITS / NT;                 // A units per thread
  constexpr int LD = 32 * WN + 4;                   // fp32 words per epilogue LDS row
  static_assert(A_UNITS % NT == 0, "A stage split across threads");
  static_assert(EPI != EPI_SWIGLU || WN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(LD % 64 == 4, "epilogue rows on rotating banks");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t K = a.k;
  const int64_t N = a.n;

  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  int64_t logical;
  if (!xcd_remap(blockIdx.x, count_mtiles(a.offsets, a.num_groups, BM) * ntn, &logical)) return;
  const int64_t mt = logical / ntn;
  const int64_t nt = logical % ntn;
  int g;
  int64_t row0, row1;
  if (!locate_mtile(a.offsets, a.num_groups, BM, mt, &g, &row0, &row1)) return;
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
  // codes of substeps 0-3 (bc0), 4-7 (bc1) and the four block scales (bs)
  u32x4_t bc0[WN], bc1[WN];
  uint32_t bs[WN];
  auto b_load_c0 = [&](int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) bc0[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + bco[n]);
  };
  auto b_load_c1 = [&](int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) bc1[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + b_c1 + bco[n]);
  };
  auto b_load_s = [&](int64_t st) {
#pragma unroll
    for (int n = 0; n < WN; ++n) bs[n] = *reinterpret_cast<const uint32_t*>(b_sbase + st * b_sstage + bso[n]);
  };

  // 16-byte slot of MFMA lane l in an A fragment block of substeps 4sq..4sq+3:
  // flipping bits 2-3 keeps the slot inside its group of 16 (reads stay
  // conflict free) and spreads the writers of one row over four bank groups
  auto aslot = [](int l, int sq) { return l ^ (4 * (sq + 2 * (l >> 5))); };
  // ---- A: thread-owned quarter rows (32 elements = 16 code bytes + 2 scales)
  const uint8_t* a_cbase = a.a_codes + row0 * (K / 2);
  const uint8_t* a_sbase = a.a_scales + row0 * (K / 16);
  uint32_t a_src[APT], a_ssrc[APT];
  int a_dst[APT];
#pragma unroll
  for (int j = 0; j < APT; ++j) {
    const int u = tid + NT * j;
    const int r = u / 4, q = u % 4, h = q / 2;
    const int64_t ar = r < row1 - row0 ? r : row1 - row0 - 1;   // row inside the tile
    a_src[j] = (uint32_t)(ar * (K / 2) + 16 * q);
    a_ssrc[j] = (uint32_t)(ar * (K / 16) + 2 * q);
    // fragment r/32, lane (r%32) + 32h, substeps 4(q%2) .. 4(q%2)+3
    a_dst[j] = (((r / 32) * 8 + 4 * (q % 2)) * 64 + aslot((r % 32) + 32 * h, q % 2)) * 16;
  }
  u32x4_t araw[APT];
  uint32_t asc[APT];
  auto a_load = [&](int64_t st) {
#pragma unroll
    for (int j = 0; j < APT; ++j) {
      araw[j] = *reinterpret_cast<const u32x4_t*>(a_cbase + st * 64 + a_src[j]);
      asc[j] = *reinterpret_cast<const uint16_t*>(a_sbase + st * 8 + a_ssrc[j]);
    }
  };
  // decode chunk c (8 elements) of the thread's quarter rows into buffer buf
  auto a_decode = [&](int c, int buf) {
    uint8_t* sb = smem + buf * A_BYTES;
#pragma unroll
    for (int j = 0; j < APT; ++j) {
      const half2_t s2 = e4m3x2_to_half2(asc[j]);
      const _Float16 sc = (c < 2) ? s2[0] : s2[1];
      *reinterpret_cast<half8_t*>(sb + a_dst[j] + c * 1024) = decode8(araw[j][c], half2_t{sc, sc});
    }
  };

  float16_t acc[WM][WN];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int n = 0; n < WN; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

  // multiplies stage buffer `buf` with the B registers for the first MV
  // 32-row blocks of the tile (the others are all padding); substeps 4..7
  // also decode the next stage's A (raw registers loaded one stage earlier)
  // into buffer `nxt`.  Each part of the B registers is reloaded with stage
  // `bnext` as soon as it has been decoded.  The loads are unconditional
  // (the last stage re-fetches itself): with a branch around them the
  // compiler has to assume the short path and waits for the loads just
  // issued before the A decode.
  auto compute = [&](auto mv_c, int buf, int nxt, int64_t bnext) {
    constexpr int MV = decltype(mv_c)::value;
    const uint8_t* sb = smem + buf * A_BYTES;
    half2_t bsc[WN][2];
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      bsc[n][0] = e4m3x2_to_half2(bs[n]);
      bsc[n][1] = e4m3x2_to_half2(bs[n] >> 16);
    }
    b_load_s(bnext);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t fa[MV], fb[WN];
#pragma unroll
      for (int m = 0; m < MV; ++m)
        fa[m] = *reinterpret_cast<const half8_t*>(sb + ((m * 8 + s) * 64 + aslot(lane, s / 4)) * 16);
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const uint32_t c = s < 4 ? bc0[n][s] : bc1[n][s - 4];
        const _Float16 sc = bsc[n][s / 4][(s / 2) % 2];
        fb[n] = decode8(c, half2_t{sc, sc});
      }
      // the scheduler would sink these loads to the end of the stage, where
      // the next stage waits on them at once: keep them here
      if (s == 3) { b_load_c0(bnext); __builtin_amdgcn_sched_barrier(0); }
      if (s == 7) { b_load_c1(bnext); __builtin_amdgcn_sched_barrier(0); }
#pragma unroll
      for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int n = 0; n < WN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[m], fb[n], acc[m][n], 0, 0, 0);
      if (s >= 4) a_decode(s - 4, nxt);
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
  auto main_loop = [&](auto mv_c) {
    a_load(0);
    b_load_s(0);
    b_load_c0(0);
    b_load_c1(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) a_decode(c, 0);
    a_load(nst > 1 ? 1 : 0);
    __syncthreads();
    for (int64_t it = 0; it < nst; ++it) {
      const int cur = (int)(it & 1), nxt = cur ^ 1;
      const int64_t st1 = it + 1 < nst ? it + 1 : nst - 1;
      const int64_t st2 = it + 2 < nst ? it + 2 : nst - 1;
      compute(mv_c, cur, nxt, st1);
      a_load(st2);
      __syncthreads();
    }
  };
  // 32-row blocks of the tile that hold at least one valid row; the tile's
  // last rows are padding when the group ends inside it.
  const int mv = __builtin_amdgcn_readfirstlane((int)std::min<int64_t>(WM, (row1 - row0 + 31) / 32));
  static_assert(WM <= 4, "main loop instances");
  switch (mv) {
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (WM >= 2) main_loop(std::integral_constant<int, 2 <= WM ? 2 : 1>{}); break;
    case 3: if constexpr (WM >= 3) main_loop(std::integral_constant<int, 3 <= WM ? 3 : 1>{}); break;
    default: main_loop(std::integral_constant<int, WM>{}); break;
  }

  // ---- epilogue through LDS, 16 rows at a time (each wave its own region,
  // after the loop's last barrier nothing reads the A buffers).
  // acc[m][n][r] is C[32m + 8(r/4) + 4(lane/32) + r%4][32n + lane%32] of
  // this wave's tile; rows 16hh.. 16hh+15 come from r in [8hh, 8hh+8).
  float* ep = reinterpret_cast<float*>(smem) + wave * 16 * LD;
  const float sgb = a.b_gscale[g];
  const int er = lane & 15;                     // row of the 16 this lane finishes
  const int eq = lane >> 4;                     // which quarter of the columns
#pragma unroll
  for (int m = 0; m < WM; ++m) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (m < mv) {
#pragma unroll
        for (int n = 0; n < WN; ++n)
#pragma unroll
          for (int r = 8 * hh; r < 8 * hh + 8; ++r)
            ep[(8 * (r / 4 - 2 * hh) + 4 * half + (r % 4)) * LD + 32 * n + l32] = acc[m][n][r];
      }
      __syncthreads();                           // the rows are in LDS
      const int64_t row = row0 + 32 * m + 16 * hh + er;
      const bool rv = row < row1;
      const int64_t rr = rv ? row : row1 - 1;
      const float sga = a.a_gscale[rr];
      const float* src = ep + er * LD;
      if (EPI == EPI_SWIGLU) {
        constexpr int GC = 16 * WN;              // gate columns of this wave
        constexpr int PL = GC / 4;               // gate columns per lane
        const int64_t I = a.inter;
        const int64_t gate0 = nt * (BN / 2) + (int64_t)wave * GC;
        const float p = a.row_prob[rr];
        const float s = sga * sgb;               // C = ACC * s_ga * s_gb
        const float sp = s * p;                  // the up half, weighted
        u16x2_t mx2 = {0, 0};
        if (rv && gate0 < I) {
#pragma unroll
          for (int c8 = 0; c8 < PL; c8 += 8) {
            const int c = eq * PL + c8;          // column inside the gate half
            float gv[8], dv[8];
            float gmin = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              gv[i] = src[c + i] * s;
              dv[i] = swiglu_fast(gv[i], src[GC + c + i] * sp);
              gmin = fminf(gmin, gv[i]);
            }
            if (gmin < -80.0f) {
#pragma unroll
              for (int i = 0; i < 8; ++i)
                if (gv[i] < -80.0f) dv[i] = swiglu_tail(gv[i], src[GC + c + i] * s, p);
            }
            uint32_t packed[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              packed[i] = pack_bf16x2(dv[2 * i], dv[2 * i + 1]);
              const uint32_t mag = packed[i] & 0x7FFF7FFFu;
              u16x2_t v;
              __builtin_memcpy(&v, &mag, 4);
              mx2 = __builtin_elementwise_max(mx2, v);
            }
            const int64_t col = gate0 + c;
            *reinterpret_cast<uint4*>(a.d_out + rr * I + col) =
                make_uint4(packed[0], packed[1], packed[2], packed[3]);
            if (a.c_out) {
              float* cg = a.c_out + rr * 2 * I + col;
              float* cu = cg + I;
              float uv[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) uv[i] = src[GC + c + i] * s;
              *reinterpret_cast<float4*>(cg) = make_float4(gv[0], gv[1], gv[2], gv[3]);
              *reinterpret_cast<float4*>(cg + 4) = make_float4(gv[4], gv[5], gv[6], gv[7]);
              *reinterpret_cast<float4*>(cu) = make_float4(uv[0], uv[1], uv[2], uv[3]);
              *reinterpret_cast<float4*>(cu + 4) = make_float4(uv[4], uv[5], uv[6], uv[7]);
            }
          }
        }
        uint32_t mx = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
        // the row's maximum over the wave's four column quarters
        uint32_t other = (uint32_t)__shfl_xor((int)mx, 16, kWave);
        mx = mx > other ? mx : other;
        other = (uint32_t)__shfl_xor((int)mx, 32, kWave);
        mx = mx > other ? mx : other;
        if (rv && eq == 0 && mx != 0u)
          atomicMax(reinterpret_cast<uint32_t*>(a.amax) + row, mx << 16);
      } else {
        constexpr int PL = 8 * WN;               // columns per lane
        const float s = sga * sgb;               // out = ACC * s_ga * s_gb
        const int64_t col0 = nt * BN + (int64_t)wave * 32 * WN + eq * PL;
        if (rv) {
#pragma unroll
          for (int c8 = 0; c8 < PL; c8 += 8) {
            const int64_t col = col0 + c8;
            if (col >= N) break;                 // N % 32 == 0: 8-column runs are whole
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = src[eq * PL + c8 + i] * s;
            if (EPI == EPI_F32) {
              float* o = static_cast<float*>(a.out) + rr * N + col;
              *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
              *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
            } else {
              uint16_t* o = static_cast<uint16_t*>(a.out) + rr * N + col;
              *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                        pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
            }
          }
        }
      }
      __syncthreads();                           // rows consumed before they are overwritten
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

template <int WM, int WN, int NW, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 32 * WM, BN = 32 * WN * NW;
  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (a.n + BN - 1) / BN;
  // upper bound on the m-tiles of all groups: sum ceil(n_g/BM) <= cap/BM + G
  const int64_t mtiles = (a.rows_cap + BM - 1) / BM + a.num_groups;
  const int64_t blocks = mtiles * ntn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.n * a.k / 2 > 0xFFFFFFFFll) return hipErrorInvalidValue;   // 32-bit lane offsets into a group
  size_t lds = (size_t)2 * WM * 8 * 64 * 16;
  const size_t epi = (size_t)NW * 16 * (32 * WN + 4) * 4;
  if (epi > lds) lds = epi;
  gemm_w4a4_kernel<WM, WN, NW, EPI><<<(unsigned)blocks, 64 * NW, lds, s>>>(a);
  return hipGetLastError();
}

// Tile: MFMA blocks per wave (M, N) and waves per workgroup (along N).
#ifndef NVFP4_GEMM_TILE
#define NVFP4_GEMM_TILE 4, 2, 4
#endif
#ifndef NVFP4_GEMM_TILE_FC1
#define NVFP4_GEMM_TILE_FC1 NVFP4_GEMM_TILE
#endif

hipError_t launch_gemm_plain(const GemmArgs& a, hipStream_t s) {
  if (a.out_dtype == 0) return launch_cfg<NVFP4_GEMM_TILE, EPI_F32>(a, s);
  return launch_cfg<NVFP4_GEMM_TILE, EPI_BF16>(a, s);
}

hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s) {
  return launch_cfg<NVFP4_GEMM_TILE_FC1, EPI_SWIGLU>(a, s);
}

}  // namespace nvfp4
