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
//              with the SwiGLU backward in its epilogue -> dC [R, 2I] bf16
//              and per-row partial sums of the router-weight gradient
//   FC1 dgrad  dXr[R, H]  = dC [R, 2I] . W1[e] [2I, H]    -> bf16 rows
//   FC2 wgrad  dW2[e] [H, I]  = sum over e's rows r of dYr[r]^T D[r]
//   FC1 wgrad  dW1[e] [2I, H] = sum over e's rows r of dC[r]^T x[row_src[r]]
// The dgrads group output rows by expert (a tile table, cost-balanced over
// the 8 XCDs); the wgrads group K (the expert's rows) and write one fp32
// matrix per expert.  Padding rows (row_src < 0) read as zeros.
//
// Tile 128 x 256, four waves of 64 x 128 (2 x 4 v_mfma_f32_32x32x16_bf16
// blocks), K-stage 64, both operands double-buffered in LDS: the next
// stage's global loads are in flight while the matrix cores run the current
// one.  K-major operands are transposed on their way into LDS (two k-rows
// per thread, packed into one dword per column), so every fragment read is
// one 16-byte LDS load of 8 consecutive k.  The LDS row pitch of 72 bf16
// (36 dwords) keeps both the transposing stores (32 lanes on consecutive
// dwords of one row, the other 32 lanes 8 rows further, 32 banks apart) and
// the 16-byte fragment reads free of bank conflicts.
#include <algorithm>

#include "gemm_common.h"
#include "launch.h"
#include "nvfp4_device.h"
#include "tile_schedule.h"

namespace nvfp4 {

namespace {

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int LDSP = BK + 8;                          // LDS row pitch (bf16)
constexpr int A_BYTES = BM * LDSP * 2, B_BYTES = BN * LDSP * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;            // 110592

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

}  // namespace

// The kernel. BWD_DGRAD_*: workgroup b takes tile table entry b (group,
// rows [r0, r1), n-tile); BWD_WGRAD: tile b of the XCD-contiguous order
// over (group, m-tile, n-tile).
template <int MODE>
__global__ __launch_bounds__(256, 1) void bwd_gemm_kernel(BwdGemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool KMA = MODE == BWD_WGRAD;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int g;
  int64_t m0, mlim, n0, k0, k1;
  int nt;
  if constexpr (MODE == BWD_WGRAD) {
    const int64_t mtn = (a.m + BM - 1) / BM, ntn = (a.n + BN - 1) / BN;
    const int64_t total = (int64_t)a.num_groups * mtn * ntn;
    const int64_t per = (total + 7) / 8;
    const int64_t logical = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
    if (logical >= total) return;
    g = (int)(logical / (mtn * ntn));
    const int64_t t = logical % (mtn * ntn);
    m0 = (t / ntn) * BM;
    nt = (int)(t % ntn);
    n0 = (int64_t)nt * BN;
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
    n0 = (int64_t)nt * BN;
    k0 = 0;
    k1 = a.k;
  }
  g = __builtin_amdgcn_readfirstlane(g);
  const uint16_t* Ab = a.a.p;
  const uint16_t* Bb = a.b.p + (MODE == BWD_WGRAD ? 0 : (int64_t)g * a.b.group_stride);
  const int64_t nlim = a.n;

  auto sA = [&](int buf) { return reinterpret_cast<uint16_t*>(smem + buf * STAGE_BYTES); };
  auto sB = [&](int buf) {
    return reinterpret_cast<uint16_t*>(smem + buf * STAGE_BYTES + A_BYTES);
  };

  // ---- K-contiguous A (dgrads): piece i = tid + 256 j (j < 4) is row i / 8,
  // k (i % 8) * 8 of the stage; the rows (and their gather) are fixed.
  int64_t arow[4];
  bool aok[4];
  if constexpr (!KMA) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid + 256 * j;
      const int64_t r = m0 + i / 8;
      bool ok = r < mlim;
      int64_t src = r;
      if (ok && a.a.row_map) {
        const int32_t t = a.a.row_map[r];
        ok = t >= 0;
        if (a.a.gather) src = t;
      }
      aok[j] = ok;
      arow[j] = src * a.a.ld + (i % 8) * 8;
    }
  }
  // ---- K-major operand: pair piece i = tid + 256 j is k-rows 2 (i % 32) and
  // 2 (i % 32) + 1 of the stage, columns c0 + (i / 32) * 8 .. + 7.
  auto load_km = [&](const BwdOperand& op, const uint16_t* base, int64_t c0, int64_t clim,
                     int64_t kk, u32x4_t* v, int np) {
    for (int j = 0; j < np; ++j) {
      const int i = tid + 256 * j;
      const int64_t c = c0 + (i / 32) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t kr = kk + 2 * (i % 32) + h;
        bool ok = kr < k1 && c < clim;
        int64_t src = kr;
        if (ok && op.row_map) {
          const int32_t t = op.row_map[kr];
          ok = t >= 0;
          if (op.gather) src = t;
        }
        v[2 * j + h] = ok ? *reinterpret_cast<const u32x4_t*>(base + src * op.ld + c)
                          : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_km = [&](uint16_t* s, const u32x4_t* v, int np) {
    for (int j = 0; j < np; ++j) {
      const int i = tid + 256 * j;
      const int kl = 2 * (i % 32), cl = (i / 32) * 8;
      const u32x4_t lo = v[2 * j], hi = v[2 * j + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = lo[e / 2], w1 = hi[e / 2];
        const uint32_t x0 = (e & 1) ? (w0 >> 16) : (w0 & 0xFFFFu);
        const uint32_t x1 = (e & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16);
        *reinterpret_cast<uint32_t*>(s + (cl + e) * LDSP + kl) = x0 | x1;
      }
    }
  };

  constexpr int NPA = KMA ? 2 : 4;      // A: pair pieces (K-major) or 16-byte pieces
  constexpr int NPB = 4;                // B: pair pieces (256 columns)
  u32x4_t va[KMA ? 2 * NPA : NPA], vb[2 * NPB];
  auto load_stage = [&](int64_t kk) {
    if constexpr (KMA) {
      load_km(a.a, Ab, m0, mlim, kk, va, NPA);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        va[j] = aok[j] && kk + ((tid + 256 * j) % 8) * 8 < k1
                    ? *reinterpret_cast<const u32x4_t*>(Ab + arow[j] + kk)
                    : u32x4_t{0u, 0u, 0u, 0u};
    }
    load_km(a.b, Bb, n0, nlim, kk, vb, NPB);
  };
  auto store_stage = [&](int buf) {
    if constexpr (KMA) {
      store_km(sA(buf), va, NPA);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = tid + 256 * j;
        *reinterpret_cast<u32x4_t*>(sA(buf) + (i / 8) * LDSP + (i % 8) * 8) = va[j];
      }
    }
    store_km(sB(buf), vb, NPB);
  };

  float16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave / 2, wn = wave % 2;               // the wave's 64 x 128 quadrant
  // 32-row blocks wholly past the tile's rows take no matrix work
  const bool mv0 = m0 + wm * 64 < mlim, mv1 = m0 + wm * 64 + 32 < mlim;
  const int64_t nst = (k1 - k0 + BK - 1) / BK;
  if (nst > 0) {
    load_stage(k0);
    store_stage(0);
  }
  __syncthreads();
  for (int64_t s = 0; s < nst; ++s) {
    const int cur = (int)(s & 1);
    const bool more = s + 1 < nst;
    if (more) load_stage(k0 + (s + 1) * BK);
    const uint16_t* la = sA(cur);
    const uint16_t* lb = sB(cur);
    if (mv0) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8_t fb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = wn * 128 + j * 32 + (lane & 31);
          fb[j] = *reinterpret_cast<const bf16x8_t*>(lb + col * LDSP + kk * 16 + 8 * (lane >> 5));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (i == 1 && !mv1) break;
          const int row = wm * 64 + i * 32 + (lane & 31);
          const bf16x8_t fa =
              *reinterpret_cast<const bf16x8_t*>(la + row * LDSP + kk * 16 + 8 * (lane >> 5));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: acc[i][j][r] is row 8 (r / 4) + 4 h + r % 4 of the 32 x 32
  // block (i, j) of the wave, column l32 (h = lane / 32, l32 = lane % 32)
  const int h = lane >> 5, l32 = lane & 31;
  auto row_of = [&](int i, int r) -> int { return wm * 64 + i * 32 + 8 * (r / 4) + 4 * h + (r % 4); };
  auto col_of = [&](int j) -> int64_t { return n0 + wn * 128 + j * 32 + l32; };

  if constexpr (MODE == BWD_WGRAD) {
    float* out = a.out_f32 + (int64_t)g * a.m * a.n;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = col_of(j);
        if (col >= a.n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + row_of(i, r);
          if (row < mlim) out[row * a.n + col] = acc[i][j][r];
        }
      }
  } else if constexpr (MODE == BWD_DGRAD_ROWS) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = col_of(j);
        if (col >= a.n) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + row_of(i, r);
          if (row >= mlim) continue;
          a.out_bf16[row * a.n + col] = f32_to_bf16(acc[i][j][r]);
          if (a.out_f32) a.out_f32[row * a.n + col] = acc[i][j][r];
        }
      }
  } else {
    // SwiGLU backward.  a.n = I; C is [rows, 2I] fp32 (gate | up); the rows'
    // router weights and whether they are routed go through LDS once.
    float* sp = reinterpret_cast<float*>(smem);          // [128] router weight
    int32_t* sok = reinterpret_cast<int32_t*>(sp + BM);  // [128] routed (not padding)
    float* sdp = sp + 2 * BM;                            // [2][128] the waves' row sums
    if (tid < BM) {
      const int64_t r = m0 + tid;
      const bool routed = r < mlim && a.row_src[r] >= 0;
      sp[tid] = routed ? a.row_prob[r] : 0.0f;
      sok[tid] = routed ? 1 : 0;
    }
    __syncthreads();
    const int64_t I = a.n;
    float part[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[i][r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = col_of(j);
        if (col >= I) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = row_of(i, r);
          const int64_t row = m0 + lr;
          if (row >= mlim) continue;
          const float pw = sp[lr];
          const float d = acc[i][j][r];
          float dg = 0.0f, du = 0.0f;
          if (sok[lr]) {
            const float gt = a.c[row * 2 * I + col], up = a.c[row * 2 * I + I + col];
            const float sg = 1.0f / (1.0f + __expf(-gt));
            const float silu = gt * sg;
            const float dsilu = sg * (1.0f + gt * (1.0f - sg));
            dg = d * up * pw * dsilu;
            du = d * silu * pw;
            part[i][r] += d * silu * up;
          }
          a.out_bf16[row * 2 * I + col] = f32_to_bf16(dg);
          a.out_bf16[row * 2 * I + I + col] = f32_to_bf16(du);
          if (a.out_f32) a.out_f32[row * I + col] = d;
        }
      }
    // row sums over the wave's 128 columns: the 32 lanes of one half, then the
    // two waves of the row in wn order (a fixed order: deterministic)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = part[i][r];
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
        if (l32 == 0) sdp[wn * BM + row_of(i, r)] = v;
      }
    __syncthreads();
    if (tid < BM) {
      const int64_t row = m0 + tid;
      if (row < mlim) a.dp_part[row * a.dp_ld + nt] = sdp[tid] + sdp[BM + tid];
    }
  }
}

// dprob[t, j] = sum over the n-tiles of the partial sums of the entry's row
// (0 for entries not routed); dp_rows (nullable) receives the rows' sums.
__global__ __launch_bounds__(256) void bwd_entry_grad_kernel(const float* dp_part, int32_t dp_ld,
                                                             const int32_t* dst_row, int64_t n,
                                                             float* dprob, const int32_t* rows_end,
                                                             int64_t cap, float* dp_rows) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    const int32_t d = dst_row[i];
    float s = 0.0f;
    if (d >= 0)
      for (int q = 0; q < dp_ld; ++q) s += dp_part[(int64_t)d * dp_ld + q];
    dprob[i] = s;
  }
  if (dp_rows && i < cap && i < (int64_t)*rows_end) {
    float s = 0.0f;
    for (int q = 0; q < dp_ld; ++q) s += dp_part[i * dp_ld + q];
    dp_rows[i] = s;
  }
}

// The two dgrad tile tables: workgroup 0 writes t0, workgroup 1 t1.
__global__ __launch_bounds__(256) void bwd_tables_kernel(const int32_t* offsets, int32_t G,
                                                         TileTableSpec t0, TileTableSpec t1) {
  __shared__ TileTableLds s;
  build_tile_table<128>(offsets, G, blockIdx.x == 0 ? t0 : t1, threadIdx.x, 256, s);
}

int bwd_lds_bytes() { return LDS_BYTES; }

// Grid of a dgrad launch: every XCD's cost-balanced range of m-tiles (the
// bound of the forward GEMM's 128-row tiles) times the n-tiles.
TileTableSpec bwd_dgrad_table_spec(int64_t rows_cap, int32_t num_groups, int64_t k, int64_t n,
                                   int4* table) {
  const int64_t ntn = (n + BN - 1) / BN;
  const int64_t mtiles = (rows_cap + BM - 1) / BM + num_groups;
  const int64_t st = std::min<int64_t>(k / kKS, kCostMaxStages);
  const int64_t cmax = kCostFixed + st * (kCostStage + BM / 32), cmin = kCostFixed + st * (kCostStage + 1);
  const int64_t per_xcd = (cmax * (mtiles + 8) + 8 * cmin - 1) / (8 * cmin) + 1;
  TileTableSpec t{};
  t.table = table; t.bm = BM; t.k = k; t.ntn = ntn; t.blocks = 8 * per_xcd * ntn;
  return t;
}

int64_t bwd_wgrad_blocks(int32_t num_groups, int64_t m, int64_t n) {
  const int64_t total = (int64_t)num_groups * ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  return 8 * ((total + 7) / 8);
}

int64_t bwd_n_tiles(int64_t n) { return (n + BN - 1) / BN; }

hipError_t launch_bwd_tables(const int32_t* offsets, int32_t G, const TileTableSpec& t0,
                             const TileTableSpec& t1, hipStream_t s) {
  bwd_tables_kernel<<<2, 256, 0, s>>>(offsets, G, t0, t1);
  return hipGetLastError();
}

hipError_t launch_bwd_gemm(int mode, const BwdGemmArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (mode) {
    case BWD_DGRAD_SWIGLU:
      bwd_gemm_kernel<BWD_DGRAD_SWIGLU><<<(unsigned)blocks, 256, LDS_BYTES, s>>>(a);
      break;
    case BWD_DGRAD_ROWS:
      bwd_gemm_kernel<BWD_DGRAD_ROWS><<<(unsigned)blocks, 256, LDS_BYTES, s>>>(a);
      break;
    case BWD_WGRAD:
      bwd_gemm_kernel<BWD_WGRAD><<<(unsigned)blocks, 256, LDS_BYTES, s>>>(a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_entry_grad(const float* dp_part, int32_t dp_ld, const int32_t* dst_row,
                                 int64_t n, float* dprob, const int32_t* rows_end, int64_t cap,
                                 float* dp_rows, hipStream_t s) {
  const int64_t m = std::max<int64_t>(n, dp_rows ? cap : 0);
  if (m <= 0) return hipSuccess;
  bwd_entry_grad_kernel<<<(unsigned)((m + 255) / 256), 256, 0, s>>>(dp_part, dp_ld, dst_row, n,
                                                                  dprob, rows_end, cap, dp_rows);
  return hipGetLastError();
}

}  // namespace nvfp4
