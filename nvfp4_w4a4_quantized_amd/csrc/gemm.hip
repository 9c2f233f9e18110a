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
// the epilogue (miniTE §5.4 "ACC x alpha_a[m] (x alpha_b[n])"; miniTE summary
// §4.2 "FP32 epilogue rescaling").
//
// Structure.  A workgroup owns a BM x BN output tile of one group; each wave
// a (32*WM) x (32*WN) sub-tile kept in accumulator registers.  Every lane
// loads its own operand fragments straight from global memory (16 bytes of
// codes and 2 scale bytes per fragment per 64-deep K step), prefetching the
// next K step while decoding and multiplying the current one.  The K order
// inside a 64-step is permuted identically for A and B (lane half g takes
// elements [32g, 32g+32)), which leaves the sum unchanged and gives each lane
// contiguous bytes.  Group boundaries come from the device offsets: every
// workgroup derives its (group, m-tile) from a wave-wide scan of the per-group
// tile counts, so the host never reads them; surplus workgroups exit.
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

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2 };

template <int WM, int WN, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_w4a4_kernel(GemmArgs a) {
  constexpr int BM = 32 * WM * WGM;
  constexpr int BN = 32 * WN * WGN;          // B rows (output columns) per tile
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t K = a.k;
  const int64_t N = a.n;

  // output-column tiles: plain -> N / BN; SwiGLU -> inter / (BN/2) gate|up pairs
  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  const int64_t mt = (int64_t)blockIdx.x / ntn;
  const int64_t nt = (int64_t)blockIdx.x % ntn;
  int g;
  int64_t row0, row1;
  if (!locate_mtile(a.offsets, a.num_groups, BM, mt, &g, &row0, &row1)) return;

  // ---- operand rows of this lane
  const int half = lane >> 5;                // K half of the 64-step
  const int l32 = lane & 31;
  int64_t arow[WM];
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    int64_t r = row0 + wm * 32 * WM + m * 32 + l32;
    arow[m] = r < row1 ? r : row1 - 1;        // clamp (results discarded)
  }
  int64_t bcol[WN];                           // output column of each n-block (lane)
  int64_t brow[WN];                           // B row inside the group
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    int64_t c;
    if (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const int64_t gate0 = nt * (BN / 2) + wn * 32 * HALF;
      c = (n < HALF) ? gate0 + 32 * n + l32 : a.inter + gate0 + 32 * (n - HALF) + l32;
      bcol[n] = c;
      const int64_t cmax = (n < HALF) ? a.inter - 1 : 2 * a.inter - 1;
      brow[n] = c < cmax ? c : cmax;
    } else {
      c = nt * BN + wn * 32 * WN + 32 * n + l32;
      bcol[n] = c;
      brow[n] = c < N ? c : N - 1;
    }
  }
  const uint8_t* ac_ptr[WM];
  const uint8_t* as_ptr[WM];
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    ac_ptr[m] = a.a_codes + arow[m] * (K / 2) + 16 * half;
    as_ptr[m] = a.a_scales + arow[m] * (K / 16) + 2 * half;
  }
  const uint8_t* bc_ptr[WN];
  const uint8_t* bs_ptr[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    const int64_t r = (int64_t)g * N + brow[n];
    bc_ptr[n] = a.b_codes + r * (K / 2) + 16 * half;
    bs_ptr[n] = a.b_scales + r * (K / 16) + 2 * half;
  }

  float16_t acc[WM][WN];
#pragma unroll
  for (int m = 0; m < WM; ++m)
#pragma unroll
    for (int n = 0; n < WN; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;

  const int64_t nk = K / 64;
  uint4 ca[WM], cb[WN];
  uint32_t sa[WM], sbv[WN];
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    ca[m] = *reinterpret_cast<const uint4*>(ac_ptr[m]);
    sa[m] = *reinterpret_cast<const uint16_t*>(as_ptr[m]);
  }
#pragma unroll
  for (int n = 0; n < WN; ++n) {
    cb[n] = *reinterpret_cast<const uint4*>(bc_ptr[n]);
    sbv[n] = *reinterpret_cast<const uint16_t*>(bs_ptr[n]);
  }

  for (int64_t kt = 0; kt < nk; ++kt) {
    uint4 na[WM], nb[WN];
    uint32_t nsa[WM], nsb[WN];
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int m = 0; m < WM; ++m) {
        na[m] = *reinterpret_cast<const uint4*>(ac_ptr[m] + (kt + 1) * 32);
        nsa[m] = *reinterpret_cast<const uint16_t*>(as_ptr[m] + (kt + 1) * 4);
      }
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        nb[n] = *reinterpret_cast<const uint4*>(bc_ptr[n] + (kt + 1) * 32);
        nsb[n] = *reinterpret_cast<const uint16_t*>(bs_ptr[n] + (kt + 1) * 4);
      }
    }
    half2_t sah[WM], sbh[WN];
#pragma unroll
    for (int m = 0; m < WM; ++m) sah[m] = e4m3x2_to_half2(sa[m]);
#pragma unroll
    for (int n = 0; n < WN; ++n) sbh[n] = e4m3x2_to_half2(sbv[n]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t fa[WM], fb[WN];
#pragma unroll
      for (int m = 0; m < WM; ++m) {
        const uint32_t c = s == 0 ? ca[m].x : s == 1 ? ca[m].y : s == 2 ? ca[m].z : ca[m].w;
        const half2_t sc = (s < 2) ? half2_t{sah[m][0], sah[m][0]} : half2_t{sah[m][1], sah[m][1]};
        fa[m] = decode8(c, sc);
      }
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const uint32_t c = s == 0 ? cb[n].x : s == 1 ? cb[n].y : s == 2 ? cb[n].z : cb[n].w;
        const half2_t sc = (s < 2) ? half2_t{sbh[n][0], sbh[n][0]} : half2_t{sbh[n][1], sbh[n][1]};
        fb[n] = decode8(c, sc);
      }
#pragma unroll
      for (int m = 0; m < WM; ++m)
#pragma unroll
        for (int n = 0; n < WN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[m], fb[n], acc[m][n], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int m = 0; m < WM; ++m) { ca[m] = na[m]; sa[m] = nsa[m]; }
#pragma unroll
      for (int n = 0; n < WN; ++n) { cb[n] = nb[n]; sbv[n] = nsb[n]; }
    }
  }

  // ---- epilogue: acc[m][n][r] is C[row, col] with
  //   row = 32m + 8(r/4) + 4(lane/32) + r%4,  col = 32n + lane%32
  const float sgb = a.b_gscale[g];
  const int64_t wrow0 = row0 + wm * 32 * WM;
  if (EPI != EPI_SWIGLU) {
#pragma unroll
    for (int m = 0; m < WM; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = wrow0 + 32 * m + 8 * (r / 4) + 4 * half + (r % 4);
        if (row >= row1) continue;
        const float sga = a.a_gscale[row];
#pragma unroll
        for (int n = 0; n < WN; ++n) {
          const int64_t col = bcol[n];
          if (col >= N) continue;
          const float v = (acc[m][n][r] * sga) * sgb;
          if (EPI == EPI_F32)
            static_cast<float*>(a.out)[row * N + col] = v;
          else
            static_cast<uint16_t*>(a.out)[row * N + col] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  } else {
    constexpr int HALF = WN / 2;
    const int64_t I = a.inter;
#pragma unroll
    for (int m = 0; m < WM; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = wrow0 + 32 * m + 8 * (r / 4) + 4 * half + (r % 4);
        const bool rv = row < row1;
        const int64_t rr = rv ? row : row1 - 1;
        const float sga = a.a_gscale[rr];
        const float p = a.row_prob[rr];
        uint32_t mx = 0u;
#pragma unroll
        for (int n = 0; n < HALF; ++n) {
          const int64_t col = bcol[n];                  // gate column (< inter if valid)
          const bool cv = rv && col < I;
          const float gv = (acc[m][n][r] * sga) * sgb;
          const float uv = (acc[m][n + HALF][r] * sga) * sgb;
          float dv;
          if (gv >= -80.0f) {
            const float silu = gv / (1.0f + __expf(-gv));
            dv = (silu * uv) * p;
          } else {
            // exp(-g) overflows binary32 below g = -88.7 while g e^g u p can
            // still be a normal bf16: evaluate this rare tail in binary64.
            const double eg = exp((double)gv);
            dv = (float)(((double)gv * eg / (1.0 + eg)) * (double)uv * (double)p);
          }
          const uint32_t db = f32_to_bf16_bits(dv);
          if (cv) {
            a.d_out[rr * I + col] = (uint16_t)db;
            if (a.c_out) {
              a.c_out[rr * 2 * I + col] = gv;
              a.c_out[rr * 2 * I + I + col] = uv;
            }
            const uint32_t mag = db & 0x7FFFu;
            mx = mx > mag ? mx : mag;
          }
        }
        // max over the 32 lanes that hold this row (same lane half)
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) {
          uint32_t y = (uint32_t)__shfl_xor((int)mx, o, kWave);
          mx = mx > y ? mx : y;
        }
        if (rv && l32 == 0 && mx != 0u)
          atomicMax(reinterpret_cast<uint32_t*>(a.amax) + row, mx << 16);
      }
    }
  }
}

// ---- launchers -------------------------------------------------------------

template <int WM, int WN, int WGM, int WGN, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = 32 * WM * WGM, BN = 32 * WN * WGN;
  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (a.n + BN - 1) / BN;
  // upper bound on the m-tiles of all groups: sum ceil(n_g/BM) <= cap/BM + G
  const int64_t mtiles = (a.rows_cap + BM - 1) / BM + a.num_groups;
  const int64_t blocks = mtiles * ntn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  gemm_w4a4_kernel<WM, WN, WGM, WGN, EPI><<<(unsigned)blocks, 64 * WGM * WGN, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_plain(const GemmArgs& a, hipStream_t s) {
  if (a.out_dtype == 0) return launch_cfg<4, 2, 1, 4, EPI_F32>(a, s);
  return launch_cfg<4, 2, 1, 4, EPI_BF16>(a, s);
}

hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s) {
  return launch_cfg<4, 2, 1, 4, EPI_SWIGLU>(a, s);
}

}  // namespace nvfp4
