// backward.hip -- the expert layer's backward pass on gfx950: BF16 GEMMs on
// BF16 operands under the straight-through approximation of the miniTE
// summary (§4.2, its default learning path: the saved original BF16
// activations and weights).  With dequantized operands it is the dequantized
// backward of "The 4-bitter Lesson" ("Improving Gradient Stability").
//
// One bf16 grouped GEMM kernel computes all four products.  In every one the
// B operand is a row-major matrix whose rows run along K ("K-major"); A has
// K contiguous in the dgrads and is K-major in the wgrads:
//   FC2 dgrad  dD [R, I]  = dYr [R, H] . W2[e] [H, I]     A: dy rows via row_src
//              -> bf16 rows, then the SwiGLU backward (its own kernel below)
//              -> dC [R, 2I] bf16 and the rows' router-weight gradients
//   FC1 dgrad  dXr[R, H]  = dC [R, 2I] . W1[e] [2I, H]    -> bf16 rows
//   FC2 wgrad  dW2[e] [H, I]  = sum over e's rows r of dYr[r]^T D[r]
//   FC1 wgrad  dW1[e] [2I, H] = sum over e's rows r of dC[r]^T x[row_src[r]]
// The dgrads group output rows by expert (a tile table, cost-balanced over
// the 8 XCDs); the wgrads group K (the expert's rows) and write one fp32
// matrix per expert.  Padding rows (row_src < 0) read as zeros.
//
// Tile 256 x 256, eight waves of 128 x 64 (4 x 2 v_mfma_f32_32x32x16_bf16
// blocks, two waves per SIMD), K-stage 32.  Both operands go from HBM
// straight into a four-slot LDS ring (buffer loads with the LDS destination,
// 16 bytes per lane): three stages are in flight while the matrix cores run
// the fourth.  Every global load is unconditional: masked lanes take an
// offset past the buffer and read zeros, so no branch makes the compiler
// drain the loads in flight.  K-major tiles are read from LDS with
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column of
// the 4 x 16 block the group reads (two of them give a lane the 8
// consecutive k the matrix core takes); K-contiguous tiles are read 16 bytes
// per lane.
// Output: the dgrads run their MFMAs with the operands swapped, so that a
// lane holds four consecutive columns of one row and stores them as one
// 8-byte bf16 piece; the wgrads keep one column per lane, so that each fp32
// store writes whole 128-byte row segments, addressed by a uniform row
// offset.
// The dgrads take their tiles from a table (cost-balanced over the 8 XCDs);
// the wgrads take experts heaviest first (an order the table kernel writes),
// so the experts with the most rows start first and the light ones fill in
// behind them.
#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"
#include "nvfp4_device.h"
#include "tile_schedule.h"

namespace nvfp4 {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NSTAGES = 4;                    // LDS ring: stages s .. s + 3 in flight
constexpr int REGION = 16384;                 // one operand's stage (256 x 32 bf16)
constexpr int STAGE_BYTES = 2 * REGION;       // A | B
constexpr int LDS_BYTES = NSTAGES * STAGE_BYTES;   // 131072

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// LDS tiles are unpadded and XOR-swizzled in 16-byte chunks, because a
// direct-to-LDS load writes one contiguous KiB per wave instruction:
//   K-major [32 k][256 columns] (512-byte rows): chunk c of row r at c ^ 4 (r % 4)
//   K-contiguous [256 rows][32 k] (64-byte rows): chunk c of row r at c ^ (r / 4) % 4
// The four rows of a transposing read and the eight rows of a 16-byte
// fragment read then fall on distinct banks.
__device__ __forceinline__ int swz_km(int r, int c) { return c ^ (4 * (r & 3)); }
__device__ __forceinline__ int swz_kc(int r, int c) { return c ^ ((r >> 2) & 3); }

// The matrix-core operand of a K-major tile: lane l receives column
// c0 + l % 32, rows k0 + 8 (l / 32) + 0..7 (two transposing reads; each lane
// of a 16-lane group receives one column of the 4 x 16 block the group reads).
__device__ __forceinline__ bf16x8_t frag_km(const uint16_t* s, int c0, int k0, int lane) {
  const int r = k0 + (lane >> 5) * 8 + ((lane & 15) >> 2);
  const int col = c0 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int off = 8 * swz_km(r, col >> 3) + (col & 7);     // rows r and r + 4 share it
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s + r * 256 + off));
  const bf16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s + (r + 4) * 256 + off));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The operand of a K-contiguous tile: lane l receives row r0 + l % 32,
// k = k0 + 8 (l / 32) + 0..7.
__device__ __forceinline__ bf16x8_t frag_kc(const uint16_t* s, int r0, int k0, int lane) {
  const int r = r0 + (lane & 31);
  const int c = (k0 >> 3) + (lane >> 5);
  return *reinterpret_cast<const bf16x8_t*>(s + r * 32 + 8 * swz_kc(r, c));
}

__device__ __forceinline__ u32x4_t bl16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ float bl4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

}  // namespace

// The kernel.  BWD_DGRAD_*: workgroup b takes tile table entry b (group,
// rows [r0, r1), n-tile).  BWD_WGRAD: tile b of (expert in the order table,
// m-tile, n-tile); GATHER 1 / 2: A / B rows along K are read through row_map.
// NW waves, each a 128 x (2 BN / NW) block (4 x 2 blocks of 32 x 32 for eight).
template <int MODE, int GATHER, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_gemm_kernel(BwdGemmArgs a) {
  // the LDS ring: one array per slot, so that the compiler sees that a load
  // into one slot does not write the slot being read (else it waits for
  // every load in flight before each read)
  __shared__ __align__(16) uint8_t S0[STAGE_BYTES];
  __shared__ __align__(16) uint8_t S1[STAGE_BYTES];
  __shared__ __align__(16) uint8_t S2[STAGE_BYTES];
  __shared__ __align__(16) uint8_t S3[STAGE_BYTES];
  constexpr bool WG = MODE == BWD_WGRAD;
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  constexpr int WNC = 2 * BN / NW;            // columns of a wave (2 waves along M)
  constexpr int JB = WNC / 32;                // its 32-column blocks
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int g, nt;
  int64_t m0, mlim, n0, k0, k1;
  if constexpr (WG) {
    const int64_t mtn = (a.m + BM - 1) / BM, ntn = (a.n + BN - 1) / BN;
    const int64_t per = mtn * ntn;
    const int64_t t = blockIdx.x;
    if (t >= (int64_t)a.num_groups * per) return;
    g = a.order[t / per];
    const int64_t q = t % per;
    m0 = (q / ntn) * BM;
    nt = (int)(q % ntn);
    mlim = a.m;
    k0 = a.offsets[g];
    k1 = a.offsets[g + 1];
  } else {
    const int4 e = a.tiles[blockIdx.x];
    if (e.x < 0) return;
    g = e.x;
    m0 = e.y;
    mlim = e.z;
    nt = e.w;
    k0 = 0;
    k1 = a.k;
  }
  n0 = (int64_t)nt * BN;
  g = __builtin_amdgcn_readfirstlane(g);
  const uint16_t* Ab = a.a.p;
  const uint16_t* Bb = a.b.p + (WG ? 0 : (int64_t)g * a.b.group_stride);

  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(Ab, a.a.bytes);
  const __amdgpu_buffer_rsrc_t br = buffer_rsrc(Bb, a.b.bytes);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t nst = (k1 - k0 + BK - 1) / BK;           // K stages

  // ---- direct-to-LDS loads.  A stage is 32 wave instructions of one KiB
  // (16 for A, 16 for B); wave w issues instructions w + NW q.  Lane L of an
  // instruction writes LDS bytes 16 L of its KiB, so it loads the global
  // chunk that the swizzle puts there.
  constexpr int QN = 16 / NW;                   // instructions per operand and wave
  // K-major (B; A in the wgrads): instruction i holds rows 2i and 2i + 1 of
  // the stage; the lane's chunk is the same for all of its instructions.
  const int km_half = lane >> 5;
  const int km_chunk = (lane & 31) ^ (4 * ((2 * wave_u + km_half) & 3));
  const int64_t bcol = n0 + 8 * km_chunk, acol = m0 + 8 * km_chunk;
  const bool bcol_ok = bcol < a.n, acol_ok = acol < mlim;
  auto km_row = [&](int q) { return 2 * (wave_u + NW * q) + km_half; };
  // K-contiguous A (dgrads): instruction i holds rows 16 i .. 16 i + 15, the
  // lane row 16 i + L / 4; its rows (and their gather) are fixed for the tile.
  const int kc_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t aoff[QN];
  if constexpr (!WG) {
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int64_t r = m0 + 16 * (wave_u + NW * q) + (lane >> 2);
      bool ok = r < mlim;
      int64_t src = r;
      if (ok && a.a.row_map) {
        const int32_t t = a.a.row_map[r];
        ok = t >= 0;
        if (a.a.gather) src = t;
      }
      aoff[q] = ok ? (uint32_t)((src * a.a.ld + 8 * kc_chunk) * 2) : kNone;
    }
  }
  auto slot_ptr = [&](auto u_c) -> uint8_t* {
    constexpr int U = decltype(u_c)::value;
    if constexpr (U == 0) return S0;
    else if constexpr (U == 1) return S1;
    else if constexpr (U == 2) return S2;
    else return S3;
  };
  // the gathered rows of stage st (clamped to the group's last row; rows past
  // it are masked where the loads use them)
  auto load_idx = [&](int64_t st, int32_t (&ix)[QN]) {
    if constexpr (GATHER != 0) {
      const int32_t* map = GATHER == 1 ? a.a.row_map : a.b.row_map;
      const int64_t kk = k0 + st * BK;
#pragma unroll
      for (int q = 0; q < QN; ++q) ix[q] = map[std::min<int64_t>(kk + km_row(q), k1 - 1)];
    }
  };
  // Per-lane offsets of stage 0 for the K-major operands that are not
  // gathered, and the number of stages whose row (k0 + km_row + BK st) lies
  // below k1: a stage adds BK rows, a uniform scalar step passed as the
  // load's soffset, so the per-stage lane work is one compare and a select.
  const uint32_t lda2 = (uint32_t)(a.a.ld * 2), ldb2 = (uint32_t)(a.b.ld * 2);
  uint32_t am0[QN], bm0[QN];
  int32_t kthr[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int64_t r0 = k0 + km_row(q);
    kthr[q] = (int32_t)((k1 - r0 + BK - 1) / BK);
    am0[q] = WG && GATHER != 1 && acol_ok && r0 < k1 ? (uint32_t)((r0 * a.a.ld + acol) * 2) : kNone;
    bm0[q] = GATHER != 2 && bcol_ok && r0 < k1 ? (uint32_t)((r0 * a.b.ld + bcol) * 2) : kNone;
  }
  // stage st into ring slot U = st % 4; stages past the last read nothing
  // and write zeros (the loads stay unconditional, so every wait below
  // counts the same instructions).  An offset of kNone plus the scalar step
  // (below 2^31) stays past the resource.
  auto dma = [&](auto u_c, int64_t st, const int32_t (&ix)[QN]) {
    uint8_t* sbase = slot_ptr(u_c);
    const bool live = st < nst;
    const int32_t st32 = (int32_t)st;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int i = wave_u + NW * q;
      uint32_t vo, so;
      if constexpr (!WG) {                     // K-contiguous rows: + BK elements a stage
        vo = live ? aoff[q] : kNone;
        so = live ? (uint32_t)(st * BK * 2) : 0u;
      } else if constexpr (GATHER == 1) {
        const bool ok = live && st32 < kthr[q] && ix[q] >= 0 && acol_ok;
        vo = ((uint32_t)ix[q] * lda2 + (uint32_t)(acol * 2)) | (ok ? 0u : kNone);
        so = 0u;
      } else {
        vo = live && st32 < kthr[q] ? am0[q] : kNone;
        so = live ? (uint32_t)st * (uint32_t)BK * lda2 : 0u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_t*)(sbase + i * 1024), 16, (int)vo,
                                               (int)__builtin_amdgcn_readfirstlane(so), 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      const int i = wave_u + NW * q;
      uint32_t vo, so;
      if constexpr (GATHER == 2) {
        const bool ok = live && st32 < kthr[q] && ix[q] >= 0 && bcol_ok;
        vo = ((uint32_t)ix[q] * ldb2 + (uint32_t)(bcol * 2)) | (ok ? 0u : kNone);
        so = 0u;
      } else {
        vo = live && st32 < kthr[q] ? bm0[q] : kNone;
        so = live ? (uint32_t)st * (uint32_t)BK * ldb2 : 0u;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void_t*)(sbase + REGION + i * 1024), 16,
                                               (int)vo, (int)__builtin_amdgcn_readfirstlane(so), 0, 0);
    }
  };

  float16_t acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave % 2, wn = wave / 2;               // the wave's 128 x WNC block
  // 32-row blocks wholly past the tile's rows take no matrix work (the count
  // is uniform in the wave: each count has its own instance of the loop)
  const int64_t vrows = mlim - (m0 + wm * 128);
  const int nvb = __builtin_amdgcn_readfirstlane(
      vrows <= 0 ? 0 : (vrows >= 128 ? 4 : (int)((vrows + 31) / 32)));
  // one stage of the first NVB row blocks: every fragment of both 16-k steps
  // is read before the first MFMA, so the reads' latency runs under the
  // MFMAs (the counter retires them in order)
  auto compute = [&](auto u_c, auto nvb_c) {
    constexpr int NVB = decltype(nvb_c)::value;
    constexpr int NA = NVB > 0 ? NVB : 1;
    const uint16_t* la = reinterpret_cast<const uint16_t*>(slot_ptr(u_c));
    const uint16_t* lb = reinterpret_cast<const uint16_t*>(slot_ptr(u_c) + REGION);
    bf16x8_t fb[BK / 16][JB], fa[BK / 16][NA];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
      for (int j = 0; j < JB; ++j) fb[kk][j] = frag_km(lb, wn * WNC + j * 32, kk * 16, lane);
#pragma unroll
      for (int i = 0; i < NVB; ++i)
        fa[kk][i] = WG ? frag_km(la, wm * 128 + i * 32, kk * 16, lane)
                       : frag_kc(la, wm * 128 + i * 32, kk * 16, lane);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < NVB; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
          acc[i][j] = WG ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0)
                         : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);
  };

  // ---- main loop: stages st + 1 .. st + 3 are in flight into the ring while
  // the matrix cores run stage st.  Iteration st waits, synchronises, reads
  // the rows of stage st + 5 (gathered operands), issues the loads of stage
  // st + 3, then multiplies stage st.  Its wait lets the wave's last 2D + 2X
  // memory instructions stay outstanding (D loads per stage, X row-index
  // loads): exactly those issued after stage st's loads.  The row indices
  // are read two stages before they are used, so that waiting for them never
  // waits for a stage still in flight (the counter is in order).  The
  // barrier carries no memory fence (a fence would wait for every load in
  // flight); a stage's LDS reads are all consumed by MFMAs before a wave
  // reaches the next barrier, after which its slot is reloaded.  The loop is
  // unrolled by the ring's four slots; stages past the last only wait,
  // synchronise and issue their (empty) loads.
  constexpr int D = 2 * QN, X = GATHER != 0 ? QN : 0;
  constexpr int WAIT_N = 2 * D + 2 * X;
  static_assert(WAIT_N < 64, "vmcnt range");
  constexpr int WAIT_IMM = (WAIT_N & 15) | ((WAIT_N >> 4) << 14) | (7 << 4) | (15 << 8);
  constexpr int WAIT_ALL = (7 << 4) | (15 << 8);          // vmcnt(0)
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  int32_t ix0[QN], ix1[QN], ix2[QN], ix3[QN];              // rows of stages = 0, 1, 2, 3 mod 4
  auto ixs = [&](auto u_c) -> int32_t (&)[QN] {
    constexpr int U = decltype(u_c)::value;
    if constexpr (U == 0) return ix0;
    else if constexpr (U == 1) return ix1;
    else if constexpr (U == 2) return ix2;
    else return ix3;
  };
  auto step = [&](auto u_c, auto nvb_c, int64_t st) {
    constexpr int U = decltype(u_c)::value;
    using UN = std::integral_constant<int, (U + 3) & 3>;   // slot of stage st + 3
    using UI = std::integral_constant<int, (U + 1) & 3>;   // index set of stage st + 5
    __builtin_amdgcn_s_waitcnt(WAIT_IMM);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if constexpr (GATHER != 0) load_idx(st + 5, ixs(UI{}));
    dma(UN{}, st + 3, ixs(UN{}));
    if (st < nst) compute(u_c, nvb_c);
  };
  auto run = [&](auto nvb_c) {
    if constexpr (GATHER != 0) {
      load_idx(0, ix0);
      load_idx(1, ix1);
      load_idx(2, ix2);
    }
    dma(C0{}, 0, ix0);
    if constexpr (GATHER != 0) load_idx(3, ix3);
    dma(C1{}, 1, ix1);
    if constexpr (GATHER != 0) load_idx(4, ix0);
    dma(C2{}, 2, ix2);
    for (int64_t st = 0; st < nst; st += 4) {
      step(C0{}, nvb_c, st);
      step(C1{}, nvb_c, st + 1);
      step(C2{}, nvb_c, st + 2);
      step(C3{}, nvb_c, st + 3);
    }
  };
  // every wave runs the same loads and barriers; only its matrix work
  // depends on its valid row blocks
  if (nst > 0) {
    switch (nvb) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      default: run(std::integral_constant<int, 4>{}); break;
    }
  }
  __builtin_amdgcn_s_waitcnt(WAIT_ALL);                   // no load into LDS outlives the loop
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // ---- epilogue.  N is a multiple of 128, so a 32-column block is wholly
  // inside or outside; so is a 32-row block of a wgrad (M too is a multiple
  // of 128).
  const int h = lane >> 5, l32 = lane & 31;
  if constexpr (MODE == BWD_WGRAD) {
    // acc[i][j][r] is row 8 (r / 4) + 4 h + r % 4 of the 32 x 32 block (i, j)
    // and column l32: each store writes 128 contiguous bytes of two rows.
    // The row's offset is uniform (the store's scalar offset), the lane's
    // column and its 4 h rows are its vector offset.
    const int64_t mn = a.m * a.n;
    const __amdgpu_buffer_rsrc_t orr = buffer_rsrc(a.out_f32 + (int64_t)g * mn, (uint32_t)(mn * 4));
    const uint32_t n4 = (uint32_t)a.n * 4u;
    const uint32_t vo = (uint32_t)(4 * h) * n4 + (uint32_t)(wn * WNC + l32) * 4u;
    // the wave's first row and column, uniform (m < 2^15, n < 2^15)
    const uint32_t rw = __builtin_amdgcn_readfirstlane((uint32_t)(m0 + (wave_u % 2) * 128));
    const uint32_t cw = __builtin_amdgcn_readfirstlane((uint32_t)(n0 + (wave_u / 2) * WNC));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rw + i * 32 >= (uint32_t)a.m) continue;
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        if (cw + j * 32 >= (uint32_t)a.n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), orr, (int)(vo + j * 128),
                                                (int)((rw + i * 32 + 8 * (r / 4) + (r % 4)) * n4 + 4 * n0), 0);
      }
    }
  } else {
    // The dgrads' MFMAs take the B fragment as their first operand (both
    // operands share one register layout), so acc[i][j] holds the block
    // transposed: acc[i][j][4 q + c] is row l32 and column 8 q + 4 h + c.  A
    // lane stores four consecutive columns of one row per q (8 bytes of bf16,
    // 16 of fp32) from one row pointer per row block.
    const int64_t c0 = n0 + wn * WNC + 4 * h;
    auto store = [&](auto f32_c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + wm * 128 + i * 32 + l32;
        if (row >= mlim) continue;
        uint16_t* o = a.out_bf16 + row * a.n + c0;
        float* of = a.out_f32 + row * a.n + c0;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          if (n0 + wn * WNC + j * 32 >= a.n) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                               acc[i][j][4 * q + 3]};
            *reinterpret_cast<u32x2_t*>(o + j * 32 + 8 * q) =
                (u32x2_t){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            if constexpr (decltype(f32_c)::value) *reinterpret_cast<f32x4_t*>(of + j * 32 + 8 * q) = v;
          }
        }
      }
    };
    if (a.out_f32) store(std::true_type{});
    else store(std::false_type{});
  }
}

// SwiGLU backward, one wave per routed row r < rows_end, from the FC2
// dgrad rows dD (bf16), the forward's FC1 output C = [g | u] (fp32) and the
// row's router weight p:
//   dC[r] = bf16([dD u p silu'(g) | dD silu(g) p])
//   dp[r] = sum over i of dD_i silu(g_i) u_i
// with silu(g) = g s, s = 1 / (1 + e^-g), silu'(g) = s (1 + g (1 - s));
// padding rows (row_src < 0) get zeros.  Lane l takes columns 8 l .. 8 l + 7
// of every 512 (16-byte dD and dC accesses, 32-byte C accesses); dp sums the
// lane's columns in order, then a fixed butterfly (deterministic).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* dD, const float* C,
                                                         const int32_t* row_src,
                                                         const float* row_prob,
                                                         const int32_t* rows_end, int64_t cap,
                                                         int64_t I, uint16_t* dC, float* dp) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (r >= cap || r >= (int64_t)*rows_end) return;
  const bool routed = row_src[r] >= 0;
  const float p = routed ? row_prob[r] : 0.0f;
  float part = 0.0f;
  for (int64_t c = (int64_t)lane * 8; c < I; c += kWave * 8) {
    const u32x4_t dv = *reinterpret_cast<const u32x4_t*>(dD + r * I + c);
    const float4* gp = reinterpret_cast<const float4*>(C + r * 2 * I + c);
    const float4* up = reinterpret_cast<const float4*>(C + r * 2 * I + I + c);
    const float4 g0 = gp[0], g1 = gp[1], u0 = up[0], u1 = up[1];
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float dg[8], du[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = dv[e / 2];
      const float d = __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
      const float sg = 1.0f / (1.0f + __expf(-g[e]));
      const float silu = g[e] * sg;
      const float dsilu = sg * (1.0f + g[e] * (1.0f - sg));
      dg[e] = routed ? d * u[e] * p * dsilu : 0.0f;
      du[e] = routed ? d * silu * p : 0.0f;
      part += routed ? d * silu * u[e] : 0.0f;
    }
    u32x4_t og, ou;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      og[q] = pack_bf16x2(dg[2 * q], dg[2 * q + 1]);
      ou[q] = pack_bf16x2(du[2 * q], du[2 * q + 1]);
    }
    *reinterpret_cast<u32x4_t*>(dC + r * 2 * I + c) = og;
    *reinterpret_cast<u32x4_t*>(dC + r * 2 * I + I + c) = ou;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
  if (lane == 0) dp[r] = part;
}

// dprob[t, j] = dp of the entry's row (0 for entries not routed)
__global__ __launch_bounds__(256) void bwd_entry_grad_kernel(const float* dp,
                                                             const int32_t* dst_row, int64_t n,
                                                             float* dprob) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t d = dst_row[i];
  dprob[i] = d >= 0 ? dp[d] : 0.0f;
}

// The two dgrad tile tables (workgroups 0 and 1) and the wgrads' expert
// order (workgroup 2): experts by descending row count, ties by id.
__global__ __launch_bounds__(256) void bwd_tables_kernel(const int32_t* offsets, int32_t G,
                                                         TileTableSpec t0, TileTableSpec t1,
                                                         int32_t* order) {
  __shared__ TileTableLds s;
  if (blockIdx.x < 2) {
    build_tile_table<BM>(offsets, G, blockIdx.x == 0 ? t0 : t1, threadIdx.x, 256, s);
    return;
  }
  for (int e = threadIdx.x; e <= G; e += 256) s.off[e] = offsets[e];
  __syncthreads();
  for (int e = threadIdx.x; e < G; e += 256) {
    const int32_t c = s.off[e + 1] - s.off[e];
    int rank = 0;
    for (int f = 0; f < G; ++f) {
      const int32_t cf = s.off[f + 1] - s.off[f];
      rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
    }
    order[rank] = e;
  }
}

int bwd_lds_bytes() { return LDS_BYTES; }

// The dgrads' tile cost model: a tile of v valid 32-row blocks and S stages
// costs kBwdCostFixed + S (kCostStage + v).  Measured on the Qwen3-shaped
// layer, a 256-row tile with one valid block takes about half the time of a
// full one (the weight stream, the transposing reads of B and the epilogue do
// not shrink with its rows), which this fixed term reproduces; the forward
// GEMM's smaller one left the XCD with the light experts finishing last.
#ifndef NVFP4_BWD_COST_FIXED
#define NVFP4_BWD_COST_FIXED 60
#endif
constexpr uint32_t kBwdCostFixed = NVFP4_BWD_COST_FIXED;

// Grid of a dgrad launch: every XCD's cost-balanced range of m-tiles (the
// bound of the forward GEMM's schedule, for 256-row tiles) times the n-tiles.
TileTableSpec bwd_dgrad_table_spec(int64_t rows_cap, int32_t num_groups, int64_t k, int64_t n,
                                   int4* table) {
  const int64_t ntn = (n + BN - 1) / BN;
  const int64_t mtiles = (rows_cap + BM - 1) / BM + num_groups;
  const int64_t st = std::min<int64_t>(k / kKS, kCostMaxStages);
  const int64_t cmax = kBwdCostFixed + st * (kCostStage + BM / 32);
  const int64_t cmin = kBwdCostFixed + st * (kCostStage + 1);
  const int64_t per_xcd = (cmax * (mtiles + 8) + 8 * cmin - 1) / (8 * cmin) + 1;
  TileTableSpec t{};
  t.table = table; t.bm = BM; t.k = k; t.ntn = ntn; t.blocks = 8 * per_xcd * ntn;
  t.fixed = kBwdCostFixed;
  return t;
}

int64_t bwd_wgrad_blocks(int32_t num_groups, int64_t m, int64_t n) {
  return (int64_t)num_groups * ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
}

hipError_t launch_bwd_tables(const int32_t* offsets, int32_t G, const TileTableSpec& t0,
                             const TileTableSpec& t1, int32_t* order, hipStream_t s) {
  bwd_tables_kernel<<<3, 256, 0, s>>>(offsets, G, t0, t1, order);
  return hipGetLastError();
}

// The wgrads gather one operand along K: A (dy rows, FC2) or B (x rows, FC1).
#ifndef NVFP4_BWD_WAVES
#define NVFP4_BWD_WAVES 8
#endif
constexpr int kBwdWaves = NVFP4_BWD_WAVES;

hipError_t launch_bwd_gemm(int mode, const BwdGemmArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const unsigned nb = (unsigned)blocks;
  constexpr int T = 64 * kBwdWaves;
  if (mode == BWD_DGRAD_ROWS) {
    bwd_gemm_kernel<BWD_DGRAD_ROWS, 0, kBwdWaves><<<nb, T, 0, s>>>(a);
  } else if (mode == BWD_WGRAD) {
    if ((a.a.row_map && a.b.row_map) || !a.order) return hipErrorInvalidValue;
    if (a.a.row_map) bwd_gemm_kernel<BWD_WGRAD, 1, kBwdWaves><<<nb, T, 0, s>>>(a);
    else if (a.b.row_map) bwd_gemm_kernel<BWD_WGRAD, 2, kBwdWaves><<<nb, T, 0, s>>>(a);
    else bwd_gemm_kernel<BWD_WGRAD, 0, kBwdWaves><<<nb, T, 0, s>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* dD, const float* C, const int32_t* row_src,
                             const float* row_prob, const int32_t* rows_end, int64_t cap,
                             int64_t inter, uint16_t* dC, float* dp, hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  swiglu_bwd_kernel<<<(unsigned)((cap + 3) / 4), 256, 0, s>>>(dD, C, row_src, row_prob, rows_end,
                                                            cap, inter, dC, dp);
  return hipGetLastError();
}

hipError_t launch_bwd_entry_grad(const float* dp, const int32_t* dst_row, int64_t n,
                                 float* dprob, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  bwd_entry_grad_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dp, dst_row, n, dprob);
  return hipGetLastError();
}

}  // namespace nvfp4
