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
// Workgroup = NW waves side by side along N.  The workgroup owns a BM x BN
// output tile of one group (BM = 32*WM rows, BN = NW*32*WN columns); each
// wave a BM x (32*WN) sub-tile held in accumulator registers
// (WM x WN v_mfma_f32_32x32x16_f16 tiles).  K advances in stages of 128 with
// two LDS buffers: while the waves multiply stage i, they fill stage i+1.
//   A (activations, shared by all waves): each thread decodes a quarter row
//     of the stage (32 elements) once, straight from its global load, and
//     stores the fp16 values in MFMA-fragment order: for fragment m and
//     substep s the 64 lanes' 16-byte operands are one 1 KiB block (lane
//     slots XOR-swizzled inside groups of 16), so both the writes and the
//     per-substep reads are bank-conflict free.
//   B (weights, distinct per wave): copied packed by global->LDS loads (64
//     code bytes per row in swizzled 16-byte slots, the 8 scale bytes in a
//     separate array) and decoded by each wave into registers right before
//     its MFMAs.
// K order: inside a 128 stage, lane half h covers elements [64h, 64h+64)
// and substep s takes [64h + 8s, 64h + 8s + 8); A and B use the same order,
// so the dot products are unchanged.
// The epilogue goes through LDS, one 32-row block at a time, so that each
// lane writes contiguous bytes of one output row.
constexpr int kKS = 128;          // K per stage
constexpr int kRowB = 80;         // LDS bytes per staged B row
constexpr int kEpiLd = 136;       // fp32 words per epilogue LDS row (128 + pad)

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_SWIGLU = 2 };

// Workgroups are dealt to the 8 XCDs round robin; renumber them so that each
// XCD walks a contiguous range of tiles (consecutive tiles share A rows and,
// inside an expert, B rows, which then stay in that XCD's L2).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n) {
  const int64_t x = bid % 8, pos = bid / 8, q = n / 8, r = n % 8;
  return (x < r) ? x * (q + 1) + pos : r * (q + 1) + (x - r) * q + pos;
}

// SwiGLU weighted by the router probability, in binary32; below g = -80
// binary32 exp(-g) overflows while g e^g u p may still be a normal bf16, so
// that rare tail is evaluated in binary64.
__device__ __noinline__ float swiglu_tail(float g, float u, float p) {
  const double eg = exp((double)g);
  return (float)(((double)g * eg / (1.0 + eg)) * (double)u * (double)p);
}

__device__ __forceinline__ float swiglu_weighted(float g, float u, float p) {
  if (g >= -80.0f) {
    // D is checked to one bf16 ulp; the hardware reciprocal (about 1 ulp of
    // binary32) is far inside that.
    const float silu = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
    return (silu * u) * p;
  }
  return swiglu_tail(g, u, p);
}

template <int WM, int WN, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_w4a4_kernel(GemmArgs a) {
  constexpr int NW = WGM * WGN;                     // waves: WGM along M x WGN along N
  constexpr int BM = 32 * WM * WGM;
  constexpr int BN = 32 * WN * WGN;
  constexpr int NT = 64 * NW;                       // threads
  constexpr int A_BYTES = (BM / 32) * 8 * 64 * 16;  // fp16 A stage (fragment order)
  constexpr int BC_BYTES = BN * 64;                 // packed B codes (swizzled rows)
  constexpr int BS_BYTES = BN * 8;                  // B block scales
  constexpr int STAGE = A_BYTES + BC_BYTES + BS_BYTES;
  constexpr int A_UNITS = BM * 4;                   // quarter rows of 32 elements
  constexpr int APT = (A_UNITS + NT - 1) / NT;      // A units per thread
  constexpr bool A_FULL = (A_UNITS % NT) == 0;      // every thread owns APT units
  constexpr int BC_INSTR = BN / 16 / NW;            // 1 KiB code loads per wave
  constexpr int BS_INSTR = BN / 32 / NW;            // 256-byte scale loads per wave
  static_assert(EPI != EPI_SWIGLU || WN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(BC_INSTR * 16 * NW == BN && BS_INSTR * 32 * NW == BN, "B tile split across waves");
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t K = a.k;
  const int64_t N = a.n;

  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  const int64_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = logical / ntn;
  const int64_t nt = logical % ntn;
  int g;
  int64_t row0, row1;
  if (!locate_mtile(a.offsets, a.num_groups, BM, mt, &g, &row0, &row1)) return;

  // output column of B-tile row j (gate|up pairing for SwiGLU)
  auto b_col = [&](int j) -> int64_t {
    const int w = j / (32 * WN), n = (j / 32) % WN, c = j % 32;
    if (EPI == EPI_SWIGLU) {
      constexpr int HALF = WN / 2;
      const int64_t gate0 = nt * (BN / 2) + (int64_t)w * 32 * HALF;
      return (n < HALF) ? gate0 + 32 * n + c : a.inter + gate0 + 32 * (n - HALF) + c;
    }
    return nt * BN + (int64_t)w * 32 * WN + 32 * n + c;
  };
  auto b_src_row = [&](int j) -> int64_t {     // B row inside the [G*N, K] matrix
    int64_t c = b_col(j);
    int64_t cmax = N - 1;
    if (EPI == EPI_SWIGLU) cmax = (((j / 32) % WN) < WN / 2) ? a.inter - 1 : 2 * a.inter - 1;
    return (int64_t)g * N + (c < cmax ? c : cmax);
  };
  // 16-byte slot of part p in staged B row r: XOR swizzle keeps the fragment
  // reads (32 consecutive rows, one part) on distinct LDS banks
  auto bslot = [](int r, int p) { return p ^ ((r >> 2) & 3); };

  // 16-byte slot of MFMA lane l in an A fragment block of substeps 4sq..4sq+3:
  // flipping bits 2-3 keeps the slot inside its group of 16 (reads stay
  // conflict free) and spreads the writers of one row over four bank groups
  auto aslot = [](int l, int sq) { return l ^ (4 * (sq + 2 * (l >> 5))); };
  // ---- A: thread-owned quarter rows (32 elements = 16 code bytes + 2 scales)
  int64_t a_src[APT], a_ssrc[APT];
  int a_dst[APT];
  bool a_ok[APT];
#pragma unroll
  for (int j = 0; j < APT; ++j) {
    const int u = tid + NT * j;
    a_ok[j] = u < A_UNITS;
    const int r = a_ok[j] ? u / 4 : 0, q = u % 4, h = q / 2;
    int64_t ar = row0 + r;
    ar = ar < row1 ? ar : row1 - 1;
    a_src[j] = ar * (K / 2) + 16 * q;
    a_ssrc[j] = ar * (K / 16) + 2 * q;
    // fragment r/32, lane (r%32) + 32h, substeps 4(q%2) .. 4(q%2)+3; the
    // lane slot is XOR-swizzled (aslot) so that the four threads of one row
    // write to distinct banks
    a_dst[j] = (((r / 32) * 8 + 4 * (q % 2)) * 64 + aslot((r % 32) + 32 * h, q % 2)) * 16;
  }
  // ---- B: global -> LDS copies issued by every wave (no registers involved)
  int64_t bc_src[BC_INSTR], bs_src[BS_INSTR];
#pragma unroll
  for (int j = 0; j < BC_INSTR; ++j) {
    const int c = wave + NW * j;                 // 16-row chunk: 1 KiB of LDS
    const int r = c * 16 + lane / 4, q = lane % 4;
    bc_src[j] = b_src_row(r) * (K / 2) + 16 * bslot(r, q);
  }
#pragma unroll
  for (int j = 0; j < BS_INSTR; ++j) {
    const int c = wave + NW * j;                 // 32-row chunk: 256 bytes of LDS
    const int r = c * 32 + lane / 2;
    bs_src[j] = b_src_row(r) * (K / 16) + 4 * (lane % 2);
  }
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  typedef __attribute__((address_space(1))) void* gbl_ptr_t;
  auto b_issue = [&](int64_t st, int buf) {
    uint8_t* sb = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < BC_INSTR; ++j) {
      const int c = wave + NW * j;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(a.b_codes + bc_src[j] + st * 64),
                                       (lds_ptr_t)(sb + A_BYTES + c * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < BS_INSTR; ++j) {
      const int c = wave + NW * j;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(a.b_scales + bs_src[j] + st * 8),
                                       (lds_ptr_t)(sb + A_BYTES + BC_BYTES + c * 256), 4, 0, 0);
    }
  };
  u32x4_t araw[APT];
  uint32_t asc[APT];
  auto a_load = [&](int64_t st) {
#pragma unroll
    for (int j = 0; j < APT; ++j)
      if (A_FULL || a_ok[j]) {
        araw[j] = *reinterpret_cast<const u32x4_t*>(a.a_codes + a_src[j] + st * 64);
        asc[j] = *reinterpret_cast<const uint16_t*>(a.a_scales + a_ssrc[j] + st * 8);
      }
  };
  // decode chunk c (8 elements) of the thread's quarter rows into buffer buf
  auto a_decode = [&](int c, int buf) {
    uint8_t* sb = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < APT; ++j)
      if (A_FULL || a_ok[j]) {
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

  const int half = lane >> 5;
  const int l32 = lane & 31;
  int b_row[WN];
#pragma unroll
  for (int n = 0; n < WN; ++n) b_row[n] = wn * 32 * WN + 32 * n + l32;

  // multiplies stage buffer `buf` for the first MV 32-row blocks of the
  // wave's rows (the others are all padding); substeps 4..7 also decode the
  // next stage's A (raw registers loaded at the start of the stage) into
  // buffer `nxt`
  auto compute = [&](auto mv_c, int buf, int nxt) {
    constexpr int MV = decltype(mv_c)::value;
    const uint8_t* sb = smem + buf * STAGE;
    u32x4_t rb0[WN], rb1[WN];
    half2_t bsc[WN][2];
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int r = b_row[n];
      rb0[n] = *reinterpret_cast<const u32x4_t*>(sb + A_BYTES + r * 64 + 16 * bslot(r, 2 * half));
      rb1[n] = *reinterpret_cast<const u32x4_t*>(sb + A_BYTES + r * 64 + 16 * bslot(r, 2 * half + 1));
      const uint32_t sw = *reinterpret_cast<const uint32_t*>(sb + A_BYTES + BC_BYTES + r * 8 + 4 * half);
      bsc[n][0] = e4m3x2_to_half2(sw);
      bsc[n][1] = e4m3x2_to_half2(sw >> 16);
    }
    // software pipeline: the operands of substep s+1 (A fragments from LDS,
    // B decoded in registers) are produced while the MFMAs of substep s run
    auto load_a = [&](half8_t (&fa)[WM], int s) {
#pragma unroll
      for (int m = 0; m < MV; ++m)
        fa[m] = *reinterpret_cast<const half8_t*>(sb + (((wm * WM + m) * 8 + s) * 64 + aslot(lane, s / 4)) * 16);
    };
    auto decode_b = [&](half8_t (&fb)[WN], int s) {
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const uint32_t c = s < 4 ? rb0[n][s] : rb1[n][s - 4];
        const _Float16 sc = bsc[n][s / 4][(s / 2) % 2];
        fb[n] = decode8(c, half2_t{sc, sc});
      }
    };
    half8_t fa0[WM], fa1[WM], fb0[WN], fb1[WN];
    load_a(fa0, 0);
    decode_b(fb0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t (&fa)[WM] = (s & 1) ? fa1 : fa0;
      half8_t (&fb)[WN] = (s & 1) ? fb1 : fb0;
      half8_t (&fan)[WM] = (s & 1) ? fa0 : fa1;
      half8_t (&fbn)[WN] = (s & 1) ? fb0 : fb1;
      if (s < 7) load_a(fan, s + 1);
#pragma unroll
      for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int n = 0; n < WN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[m], fb[n], acc[m][n], 0, 0, 0);
      if (s < 7) decode_b(fbn, s + 1);
      if (s >= 4) a_decode(s - 4, nxt);
    }
  };

  // ---- main loop.  Stage it is multiplied from buffer it&1.  At the start
  // of the stage the next stage's B is requested straight into the other
  // buffer; the next stage's A codes (already in registers, loaded one stage
  // earlier) are decoded into it between the MFMAs of substeps 4-7, after
  // which the registers receive the A codes of the stage after that.  Vector
  // memory loads complete in issue order, so waiting until only the A loads
  // (issued last) may be outstanding guarantees the B copy has landed before
  // the barrier.  The tail stages re-fetch the last stage into the idle
  // buffer, which nothing reads: the loop stays branch-free.
  constexpr int A_LOADS = 2 * APT;              // VMEM ops issued by a_load
  static_assert(A_LOADS <= 15, "vmcnt immediate");
  const int64_t nst = K / kKS;
  auto main_loop = [&](auto mv_c) {
    a_load(0);
    b_issue(0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) a_decode(c, 0);
    a_load(nst > 1 ? 1 : 0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | A_LOADS); // vmcnt(A_LOADS): B of stage 0 is in LDS
    __syncthreads();
    for (int64_t it = 0; it < nst; ++it) {
      const int cur = (int)(it & 1), nxt = cur ^ 1;
      const int64_t st1 = it + 1 < nst ? it + 1 : it;
      const int64_t st2 = it + 2 < nst ? it + 2 : nst - 1;
      b_issue(st1, nxt);
      compute(mv_c, cur, nxt);
      a_load(st2);
      __builtin_amdgcn_s_waitcnt(0x0F70 | A_LOADS);
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0) before LDS is reused
  };
  // 32-row blocks of this wave's rows that hold at least one valid row; the
  // tile's last rows are padding when the group ends inside it.  The count is
  // the same for every wave of a row of waves, so barriers stay uniform.
  const int mv = __builtin_amdgcn_readfirstlane((int)std::min<int64_t>(
      WM, std::max<int64_t>(0, (row1 - row0 - 32 * WM * wm + 31) / 32)));
  static_assert(WM <= 4, "main loop instances");
  switch (mv) {
    case 0: break;
    case 1: main_loop(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (WM >= 2) main_loop(std::integral_constant<int, 2 <= WM ? 2 : 1>{}); break;
    case 3: if constexpr (WM >= 3) main_loop(std::integral_constant<int, 3 <= WM ? 3 : 1>{}); break;
    default: main_loop(std::integral_constant<int, WM>{}); break;
  }

  // ---- epilogue through LDS, one 32-row block at a time.  acc[m][n][r] is
  // C[32m + 8(r/4) + 4(lane/32) + r%4][32n + lane%32] of this wave's tile.
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * kEpiLd;
  const float sgb = a.b_gscale[g];
  const int er = lane >> 1;                     // row of the block this lane finishes
  const int eh = lane & 1;                      // which half of the columns
#pragma unroll
  for (int m = 0; m < WM; ++m) {
    if (m < mv) {
#pragma unroll
      for (int n = 0; n < WN; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(8 * (r / 4) + 4 * half + (r % 4)) * kEpiLd + 32 * n + l32] = acc[m][n][r];
    }
    __syncthreads();                             // the block is in LDS (every wave loops WM times)
    const int64_t row = row0 + 32 * (wm * WM + m) + er;
    const bool rv = row < row1;
    const int64_t rr = rv ? row : row1 - 1;
    const float sga = a.a_gscale[rr];
    const float* src = ep + er * kEpiLd;
    if (EPI == EPI_SWIGLU) {
      constexpr int GC = 32 * WN / 2;            // gate columns of this wave
      const int64_t I = a.inter;
      const int64_t gate0 = nt * (BN / 2) + (int64_t)wn * GC;
      const float p = a.row_prob[rr];
      uint32_t mx = 0u;
      if (rv && gate0 < I) {
#pragma unroll
        for (int c8 = 0; c8 < GC / 2; c8 += 8) {
          const int c = eh * (GC / 2) + c8;      // column inside the gate half
          uint32_t packed[4];
          float gv[8], uv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            gv[i] = (src[c + i] * sga) * sgb;
            uv[i] = (src[GC + c + i] * sga) * sgb;
          }
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const uint32_t d0 = f32_to_bf16_bits(swiglu_weighted(gv[i], uv[i], p));
            const uint32_t d1 = f32_to_bf16_bits(swiglu_weighted(gv[i + 1], uv[i + 1], p));
            packed[i / 2] = d0 | (d1 << 16);
            const uint32_t m0 = d0 & 0x7FFFu, m1 = d1 & 0x7FFFu;
            mx = mx > m0 ? mx : m0;
            mx = mx > m1 ? mx : m1;
          }
          const int64_t col = gate0 + c;
          *reinterpret_cast<uint4*>(a.d_out + rr * I + col) =
              make_uint4(packed[0], packed[1], packed[2], packed[3]);
          if (a.c_out) {
            float* cg = a.c_out + rr * 2 * I + col;
            float* cu = cg + I;
            *reinterpret_cast<float4*>(cg) = make_float4(gv[0], gv[1], gv[2], gv[3]);
            *reinterpret_cast<float4*>(cg + 4) = make_float4(gv[4], gv[5], gv[6], gv[7]);
            *reinterpret_cast<float4*>(cu) = make_float4(uv[0], uv[1], uv[2], uv[3]);
            *reinterpret_cast<float4*>(cu + 4) = make_float4(uv[4], uv[5], uv[6], uv[7]);
          }
        }
      }
      const uint32_t other = (uint32_t)__shfl_xor((int)mx, 1, kWave);
      mx = mx > other ? mx : other;
      if (rv && eh == 0 && mx != 0u)
        atomicMax(reinterpret_cast<uint32_t*>(a.amax) + row, mx << 16);
    } else {
      constexpr int WC = 32 * WN;                // columns of this wave
      const int64_t col0 = nt * BN + (int64_t)wn * WC + eh * (WC / 2);
      if (rv) {
#pragma unroll
        for (int c8 = 0; c8 < WC / 2; c8 += 8) {
          const int64_t col = col0 + c8;
          if (col >= N) break;                   // N % 32 == 0: 8-column runs are whole
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = (src[eh * (WC / 2) + c8 + i] * sga) * sgb;
          if (EPI == EPI_F32) {
            float* o = static_cast<float*>(a.out) + rr * N + col;
            *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
          } else {
            uint16_t* o = static_cast<uint16_t*>(a.out) + rr * N + col;
            *reinterpret_cast<uint4*>(o) = make_uint4(
                f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16),
                f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16),
                f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16));
          }
        }
      }
    }
    __syncthreads();                             // block consumed before it is overwritten
  }
}

// ---- launchers -------------------------------------------------------------

template <int WM, int WN, int WGM, int WGN, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int NW = WGM * WGN, BM = 32 * WM * WGM, BN = 32 * WN * WGN;
  const int64_t ntn = (EPI == EPI_SWIGLU) ? (a.inter + BN / 2 - 1) / (BN / 2) : (a.n + BN - 1) / BN;
  // upper bound on the m-tiles of all groups: sum ceil(n_g/BM) <= cap/BM + G
  const int64_t mtiles = (a.rows_cap + BM - 1) / BM + a.num_groups;
  const int64_t blocks = mtiles * ntn;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t stage = (size_t)(BM / 32) * 8 * 64 * 16 + (size_t)BN * (64 + 8);
  size_t lds = 2 * stage;
  const size_t epi = (size_t)NW * 32 * kEpiLd * 4;
  if (epi > lds) lds = epi;
  gemm_w4a4_kernel<WM, WN, WGM, WGN, EPI><<<(unsigned)blocks, 64 * NW, lds, s>>>(a);
  return hipGetLastError();
}

// Tile: MFMA blocks per wave (M, N) and waves per workgroup (M, N).
#ifndef NVFP4_GEMM_TILE
#define NVFP4_GEMM_TILE 4, 2, 1, 8
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
