// single_pass.hip -- the expert layer's FC1 -> weighted SwiGLU -> NVFP4
// quantize -> FC2 in one kernel, with online amax compensation (miniTE
// Technical Report §5.6, "Exploring Single-Pass Fusion").
//
// One workgroup owns a 128-row block of one expert (8 waves, one workgroup per
// compute unit) and never writes the intermediate activation or its
// quantization to memory:
//   FC1, slice by slice: for each 256-column slice i of the intermediate
//     dimension it runs FC1 over K = hidden for the slice's gate and up
//     columns (the grouped GEMM's 128 x 512 tile, A gathered from the
//     token-major quantized rows), applies the router-weighted SwiGLU, rounds
//     to bf16 and stages the slice P_i in LDS.  Four threads per row then take
//     the slice's row maximum, update the row's running amax gamax, set
//     gs_i = gamax / 2688 and encode the slice's 16-blocks with gs_i into an
//     LDS copy of the row block's FC2 input (codes, E4M3 scales, and gs_i per
//     row and slice).
//   FC2: for each 512-column slab of the output it runs FC2 over K = inter
//     with A decoded from that LDS copy.  The accumulators hold
//     sum_i (q s_b)(q s_b) in the units of the current slice's gs: entering
//     slice i they are multiplied by gs_{i-1} / gs_i (the page's
//     O = O * (gs_prev / gs) + dO_i), and the epilogue applies
//     gs_last * gs_W2.  Slices with gs_i = 0 (a row all zero so far)
//     contribute nothing and leave O at zero.
// The K-tile of the online scale is the FC1 slice, 256 intermediate columns
// (two FC2 K-stages); the last slice may be narrower.  The operand decode
// and the matrix-core usage are those of the grouped GEMM (gemm.hip): exact
// fp16 operands, v_mfma_f32_32x32x16_f16, fp32 accumulation.
#include <type_traits>

#include "gemm_common.h"
#include "launch.h"
#include "nvfp4_device.h"
#include "tile_schedule.h"

namespace nvfp4 {

namespace {

constexpr int WM = 4, WN = 2, NW = 8;              // 128 x 512 tile, 8 waves
constexpr int BM = 32 * WM;                        // rows per workgroup
constexpr int BN = 32 * WN * NW;                   // 512 columns per FC1 / FC2 tile
constexpr int NT = 64 * NW;                        // threads
constexpr int SLICE = BN / 2;                      // intermediate columns per slice
constexpr int A_BYTES = WM * 8 * 64 * 16;          // fp16 A stage in fragment order

// LDS carve (bytes) for intermediate size I
struct SpLds {
  int a_buf;       // 2 * A_BYTES: A stages; the bf16 slice staging; FC2 output staging
  int a2c, a2s;    // [BM][I/2] codes, [BM][I/16] scales of the FC2 input
  int gs;          // [nslices][BM] float: gs_i per row
  int ratio;       // [nslices][BM] float: gs_{i-1} / gs_i (0 when gs_i == 0)
  int gam;         // [BM] float: running amax
  int rfac;        // [3][BM] float: s_ga*s_gb, that times the router weight, the router weight
  int bytes;
};

__host__ __device__ constexpr int round16(int v) { return (v + 15) / 16 * 16; }

__host__ __device__ inline SpLds sp_lds(int64_t I) {
  SpLds L{};
  const int ns = (int)((I + SLICE - 1) / SLICE);
  int o = 0;
  L.a_buf = o; o += 2 * A_BYTES;
  L.a2c = o; o += round16(BM * (int)(I / 2));
  L.a2s = o; o += round16(BM * (int)(I / 16));
  L.gs = o; o += round16(ns * BM * 4);
  L.ratio = o; o += round16(ns * BM * 4);
  L.gam = o; o += BM * 4;
  L.rfac = o; o += 3 * BM * 4;
  L.bytes = o;
  return L;
}

}  // namespace

extern __shared__ __align__(16) uint8_t sp_smem[];

// One FC1 slice (PHASE 0) or one FC2 slab (PHASE 1) of the workgroup's
// m-tile.  Each is a function of its own: its registers are allocated
// apart from the others', and nothing of one slice stays live across the
// next slice's main loop.  MV: the m-tile's 32-row blocks that hold a valid
// row; the blocks past them (all padding) take no matrix work, SwiGLU,
// quantization or stores.
template <int PHASE, int MV>
__device__ __noinline__ void sp_body(const SinglePassArgs& a, int idx) {
  uint8_t* smem = sp_smem;
  const int4 te = a.tile_table[blockIdx.x];
  const int g = __builtin_amdgcn_readfirstlane(te.x);
  const int64_t row0 = uniform64(te.y), row1 = uniform64(te.z);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t H = a.hidden, I = a.inter;
  const int nslices = (int)((I + SLICE - 1) / SLICE);
  const SpLds L = sp_lds(I);
  float* gs_l = reinterpret_cast<float*>(smem + L.gs);
  float* ratio_l = reinterpret_cast<float*>(smem + L.ratio);
  float* gam_l = reinterpret_cast<float*>(smem + L.gam);
  float* rfac = reinterpret_cast<float*>(smem + L.rfac);
  uint8_t* a2c_l = smem + L.a2c;
  uint8_t* a2s_l = smem + L.a2s;
  const int64_t nrow = row1 - row0;                // valid rows of the block

  // 16-byte slot of MFMA lane l in an A fragment block of substeps 4sq..4sq+3
  auto aslot = [](int l, int sq) { return l ^ (4 * (sq + 2 * (l >> 5))); };
  // A: thread tid owns quarter row u = tid (row r = tid/4, quarter q = tid%4)
  const int ar = tid / 4, aq = tid % 4, ah = aq / 2;
  const int a_dst = (((ar / 32) * 8 + 4 * (aq % 2)) * 64 + aslot((ar % 32) + 32 * ah, aq % 2)) * 16;
  // FC1's A row: the token row of routed row row0 + ar (clamped into the
  // block; a padding row reads the all-zero row)
  uint32_t a1_src, a1_ssrc;
  {
    const int64_t rr = row0 + (ar < nrow ? ar : nrow - 1);
    const int32_t t = a.a_row_src[rr];
    const int64_t tok = t >= 0 ? (int64_t)t : a.a_pad_row;
    a1_src = (uint32_t)(tok * (H / 2) + 16 * aq);
    a1_ssrc = (uint32_t)(tok * (H / 16) + 2 * aq);
  }
  u32x4_t araw;
  uint32_t asc;
  auto a_decode = [&](int c, int buf) {            // chunk c (8 elements) into stage buffer buf
    uint8_t* sb = smem + L.a_buf + buf * A_BYTES;
    const half2_t s2 = e4m3x2_to_half2(asc);
    const _Float16 sc = (c < 2) ? s2[0] : s2[1];
    *reinterpret_cast<half8_t*>(sb + a_dst + c * 1024) = decode8(araw[c], half2_t{sc, sc});
  };

  float16_t acc[WM][WN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int m = 0; m < WM; ++m)
#pragma unroll
      for (int n = 0; n < WN; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.0f;
  };

  // B: the lane's column (row of the weight matrix) per n; one stage of codes
  // (substeps 0-3, 4-7) and scales, reloaded in place as they are decoded
  struct BSet {
    u32x4_t c0[WN], c1[WN];
    uint32_t s[WN];
  };
  BSet bx;
  half8_t fbc[WN];
  auto b_scales = [&](const BSet& b, half2_t (&bsc)[WN][2]) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      bsc[n][0] = e4m3x2_to_half2(b.s[n]);
      bsc[n][1] = e4m3x2_to_half2(b.s[n] >> 16);
    }
  };
  auto b_decode = [&](const BSet& b, int s, const half2_t (&bsc)[WN][2], half8_t (&fb)[WN]) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const uint32_t c = s < 4 ? b.c0[n][s] : b.c1[n][s - 4];
      const _Float16 sc = bsc[n][s / 4][(s / 2) % 2];
      fb[n] = decode8(c, half2_t{sc, sc});
    }
  };

  // One GEMM pass over K (nst stages of 128) into acc.  A_FROM_LDS: A is the
  // FC2 input in LDS, else FC1's gathered token rows.  B: matrix base
  // (codes, scales) of the group, tiled or row-major, lane offsets bco/bso.
  // at_stage(st) runs before the MFMAs of stage st (the online rescale).
  auto gemm_pass = [&](auto a_from_lds, int64_t K, const uint8_t* b_cbase, const uint8_t* b_sbase,
                       bool tiled, const uint32_t (&bco)[WN], const uint32_t (&bso)[WN],
                       auto at_stage) {
    constexpr bool ALDS = decltype(a_from_lds)::value;
    const int64_t nst = K / kKS;
    const int64_t b_cstage = tiled ? 2048 : 64, b_sstage = tiled ? 256 : 8, b_c1 = tiled ? 1024 : 16;
    auto a_load = [&](int64_t st) {
      if constexpr (ALDS) {
        araw = *reinterpret_cast<const u32x4_t*>(a2c_l + ar * (I / 2) + st * 64 + 16 * aq);
        asc = *reinterpret_cast<const uint16_t*>(a2s_l + ar * (I / 16) + st * 8 + 2 * aq);
      } else {
        araw = *reinterpret_cast<const u32x4_t*>(a.a_codes + st * 64 + a1_src);
        asc = *reinterpret_cast<const uint16_t*>(a.a_scales + st * 8 + a1_ssrc);
      }
    };
    auto b_load_c0 = [&](int64_t st) {
#pragma unroll
      for (int n = 0; n < WN; ++n) bx.c0[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + bco[n]);
    };
    auto b_load_c1 = [&](int64_t st) {
#pragma unroll
      for (int n = 0; n < WN; ++n) bx.c1[n] = *reinterpret_cast<const u32x4_t*>(b_cbase + st * b_cstage + b_c1 + bco[n]);
    };
    auto b_load_s = [&](int64_t st) {
#pragma unroll
      for (int n = 0; n < WN; ++n) bx.s[n] = *reinterpret_cast<const uint32_t*>(b_sbase + st * b_sstage + bso[n]);
    };
    auto clamp_st = [&](int64_t st) { return st < nst ? st : nst - 1; };
    // prologue: stage 0's A decoded into buffer 0, B codes and scales of
    // stage 0 in registers, the first B operands decoded, A of stage 1 loading
    a_load(0);
    b_load_s(0);
    b_load_c0(0);
    b_load_c1(0);
    {
      half2_t bsc[WN][2];
      b_scales(bx, bsc);
      b_decode(bx, 0, bsc, fbc);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) a_decode(c, 0);
    a_load(clamp_st(1));
    __syncthreads();
    for (int64_t it = 0; it < nst; ++it) {
      const int cur = (int)(it & 1), nxt = cur ^ 1;
      at_stage(it);
      const uint8_t* sb = smem + L.a_buf + cur * A_BYTES;
      auto a_frag = [&](int m, int s) {
        return *reinterpret_cast<const half8_t*>(sb + ((m * 8 + s) * 64 + aslot(lane, s / 4)) * 16);
      };
      half2_t bsc[WN][2];
      b_scales(bx, bsc);
      b_load_s(clamp_st(it + 1));
      half8_t fa[WM];
#pragma unroll
      for (int m = 0; m < MV; ++m) fa[m] = a_frag(m, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        half8_t fbn[WN];
        if (s < 7) {
          b_decode(bx, s + 1, bsc, fbn);
        } else {                                   // substep 0 of the next stage
          half2_t bsn[WN][2];
          b_scales(bx, bsn);
          b_decode(bx, 0, bsn, fbn);
        }
#pragma unroll
        for (int m = 0; m < MV; ++m) {
#pragma unroll
          for (int n = 0; n < WN; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[m], fbc[n], acc[m][n], 0, 0, 0);
          if (s < 7) fa[m] = a_frag(m, s + 1);
        }
        if (s >= 4) a_decode(s - 4, nxt);
        if (s == 2) b_load_c0(clamp_st(it + 1));
        if (s == 6) b_load_c1(clamp_st(it + 1));
#pragma unroll
        for (int n = 0; n < WN; ++n) fbc[n] = fbn[n];
#pragma unroll
        for (int m = 0; m < MV; ++m) {
#pragma unroll
          for (int n = 0; n < WN; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
          if (s < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      a_load(clamp_st(it + 2));
      __syncthreads();
    }
  };

  // the row (inside the block) of accumulator element r of 32-row block m
  auto trow = [&](int m, int r) { return 32 * m + 8 * (r / 4) + 4 * half + (r % 4); };
  // lane offsets of B columns (matrix rows) c[n], clamped to `rows` - 1
  auto b_offsets = [&](const int64_t (&c)[WN], int64_t rows, int64_t K, bool tiled,
                       uint32_t (&bco)[WN], uint32_t (&bso)[WN]) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
      const int64_t row = c[n] < rows ? c[n] : rows - 1;
      if (tiled) {
        const int64_t tile0 = (row / 32) * (K / kKS);
        bco[n] = (uint32_t)(tile0 * 2048 + 16 * lane);
        bso[n] = (uint32_t)(tile0 * 256 + 4 * lane);
      } else {
        bco[n] = (uint32_t)(row * (K / 2) + 32 * half);
        bso[n] = (uint32_t)(row * (K / 16) + 4 * half);
      }
    }
  };
  auto no_hook = [](int64_t) {};

  // ---------------- FC1, slice by slice, quantized into LDS ----------------
  const bool tiled1 = a.w1_layout == 1;
  const uint8_t* w1c = a.w1_codes + (int64_t)g * 2 * I * (H / 2);
  const uint8_t* w1s = a.w1_scales + (int64_t)g * 2 * I * (H / 16);
  uint16_t* stage16 = reinterpret_cast<uint16_t*>(smem + L.a_buf);   // [BM][SLICE] bf16
  if constexpr (PHASE == 0) {
    const int sl = idx;
    const int64_t j0 = (int64_t)sl * SLICE + (int64_t)wave * 32;    // this wave's gate columns
    const bool wave_live = j0 < I;                 // inter % 64 == 0: whole 32-column blocks
    int64_t cols[WN] = {j0 + l32, I + j0 + l32};  // gate, up
    uint32_t bco[WN], bso[WN];
    b_offsets(cols, 2 * I, H, tiled1, bco, bso);
    zero_acc();
    gemm_pass(std::false_type{}, H, w1c, w1s, tiled1, bco, bso, no_hook);
    // weighted SwiGLU of the slice -> bf16 staging [row][column in slice]
    if (wave_live) {
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        float sv[16], spv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *reinterpret_cast<const float4*>(rfac + 32 * m + 8 * q + 4 * half);
          sv[4 * q] = t.x; sv[4 * q + 1] = t.y; sv[4 * q + 2] = t.z; sv[4 * q + 3] = t.w;
          const float4 u = *reinterpret_cast<const float4*>(rfac + BM + 32 * m + 8 * q + 4 * half);
          spv[4 * q] = u.x; spv[4 * q + 1] = u.y; spv[4 * q + 2] = u.z; spv[4 * q + 3] = u.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = trow(m, r);
          const float gv = acc[m][0][r] * sv[r];
          float dv = swiglu_fast(gv, acc[m][1][r] * spv[r]);
          if (gv < -80.0f) dv = swiglu_tail_f32(gv, acc[m][1][r] * sv[r], rfac[2 * BM + row]);
          const uint16_t d16 = (uint16_t)(pack_bf16x2(dv, 0.0f) & 0xFFFFu);
          stage16[row * SLICE + wave * 32 + l32] = d16;
          const int64_t grow = row0 + row;
          if (grow < row1) {
            if (a.c_out) {
              a.c_out[grow * 2 * I + j0 + l32] = gv;
              a.c_out[grow * 2 * I + I + j0 + l32] = acc[m][1][r] * sv[r];
            }
            if (a.p_out) a.p_out[grow * I + j0 + l32] = d16;
          }
        }
      }
    }
    __syncthreads();
    // quantize the slice: four threads per row, each 1/4 of its 16-blocks;
    // the row's slice maximum by two lane exchanges, then gamax, gs_i (rows
    // of the valid blocks only; a wave's rows share one block)
    if ((tid >> 2) < 32 * MV) {
      const int r = tid >> 2, qd = tid & 3;
      const int64_t width = I - (int64_t)sl * SLICE < SLICE ? I - (int64_t)sl * SLICE : SLICE;
      const int nbq = (int)(width / 64);           // blocks per thread (width % 128 == 0: 2 or 4)
      uint32_t w[4][8];
      uint32_t mloc = 0u;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        if (bi < nbq) {
          const uint16_t* src = stage16 + r * SLICE + (qd * nbq + bi) * 16;
          const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(src);
          const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(src + 8);
          w[bi][0] = v0.x; w[bi][1] = v0.y; w[bi][2] = v0.z; w[bi][3] = v0.w;
          w[bi][4] = v1.x; w[bi][5] = v1.y; w[bi][6] = v1.z; w[bi][7] = v1.w;
          const uint32_t mb = bf16_absmax_bits(w[bi]);
          mloc = mloc > mb ? mloc : mb;
        }
      }
      // lanes 4r .. 4r+3 hold one row: max over the quad
      uint32_t mx = mloc;
      uint32_t o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)mx, 0x041F);   // lane ^ 1
      mx = mx > o ? mx : o;
      o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)mx, 0x081F);            // lane ^ 2
      mx = mx > o ? mx : o;
      const float smax = __uint_as_float(mx << 16);
      const float gam_prev = gam_l[r];
      const float gam = smax > gam_prev ? smax : gam_prev;   // running row amax
      const float gs = gam / 2688.0f;                         // gs = gamax / 2688
      if (qd == 0) {
        gam_l[r] = gam;
        gs_l[sl * BM + r] = gs;
        const float prev = sl > 0 ? gs_l[(sl - 1) * BM + r] : 0.0f;
        ratio_l[sl * BM + r] = gs != 0.0f ? prev / gs : 0.0f;  // O *= gs_prev / gs
        const int64_t grow = row0 + r;
        if (a.gs_out && grow < row1) a.gs_out[grow * nslices + sl] = gs;
      }
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        if (bi < nbq) {
          uint32_t sb;
          const uint2 c = quantize_block16(w[bi], gs, 0, &sb);
          const int64_t blk = ((int64_t)sl * SLICE) / 16 + qd * nbq + bi;   // block within the row
          *reinterpret_cast<uint2*>(a2c_l + r * (I / 2) + blk * 8) = c;
          a2s_l[r * (I / 16) + blk] = (uint8_t)sb;
          const int64_t grow = row0 + r;
          if (grow < row1) {
            if (a.a2c_out) *reinterpret_cast<uint2*>(a.a2c_out + grow * (I / 2) + blk * 8) = c;
            if (a.a2s_out) a.a2s_out[grow * (I / 16) + blk] = (uint8_t)sb;
          }
        }
      }
    }
    __syncthreads();
    return;
  }

  // ---------------- FC2 from the LDS copy, slab by slab ----------------
  const bool tiled2 = a.w2_layout == 1;
  const uint8_t* w2c = a.w2_codes + (int64_t)g * H * (I / 2);
  const uint8_t* w2s = a.w2_scales + (int64_t)g * H * (I / 16);
  const float sgw2 = a.w2_gscale[g];
  const bool odd = (lane & 1) != 0;
  {
    const int sb2 = idx;
    const int64_t col0 = (int64_t)sb2 * BN + (int64_t)wave * 32 * WN;   // this wave's first column
    int64_t cols[WN] = {col0 + l32, col0 + 32 + l32};
    uint32_t bco[WN], bso[WN];
    b_offsets(cols, H, I, tiled2, bco, bso);
    zero_acc();
    // entering slice i (stage 2i, i >= 1): O *= gs_{i-1} / gs_i per row
    auto rescale = [&](int64_t st) {
      if (st == 0 || (st * kKS) % SLICE != 0) return;
      const int sl = (int)(st * kKS / SLICE);
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        float rv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *reinterpret_cast<const float4*>(ratio_l + sl * BM + 32 * m + 8 * q + 4 * half);
          rv[4 * q] = t.x; rv[4 * q + 1] = t.y; rv[4 * q + 2] = t.z; rv[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int n = 0; n < WN; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][n][r] *= rv[r];
      }
    };
    gemm_pass(std::true_type{}, I, w2c, w2s, tiled2, bco, bso, rescale);
    // epilogue: Y = O * gs_last * gs_W2
#pragma unroll
    for (int m = 0; m < MV; ++m) {
      float fv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t = *reinterpret_cast<const float4*>(gs_l + (nslices - 1) * BM + 32 * m + 8 * q + 4 * half);
        fv[4 * q] = t.x * sgw2; fv[4 * q + 1] = t.y * sgw2; fv[4 * q + 2] = t.z * sgw2; fv[4 * q + 3] = t.w * sgw2;
      }
#pragma unroll
      for (int n = 0; n < WN; ++n) {
        const int64_t c = col0 + 32 * n + l32;
        if (col0 + 32 * n >= H) continue;          // H % 128 == 0: 32-column blocks are whole
        if (a.y_f32) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t grow = row0 + trow(m, r);
            if (grow < row1) a.y_f32[grow * H + c] = acc[m][n][r] * fv[r];
          }
        } else {
          // neighbouring lanes swap one value per row pair, so each lane
          // stores two adjacent columns of one row as one dword
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float v0 = acc[m][n][2 * t] * fv[2 * t], v1 = acc[m][n][2 * t + 1] * fv[2 * t + 1];
            const float give = odd ? v0 : v1;
            const float got = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                0, __builtin_bit_cast(int, give), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
            const uint32_t pk = odd ? pack_bf16x2(got, v1) : pack_bf16x2(v0, got);
            const int rr = 2 * t + (odd ? 1 : 0);
            const int64_t grow = row0 + 32 * m + 8 * (rr / 4) + 4 * half + (rr % 4);
            if (grow < row1)
              *reinterpret_cast<uint32_t*>(a.y_bf16 + grow * H + col0 + 32 * n + (l32 & ~1)) = pk;
          }
        }
      }
    }
    __syncthreads();                               // the A buffers are reused by the next slab
  }
}

__global__ __launch_bounds__(NT, 1) void single_pass_kernel(SinglePassArgs a) {
  const int4 te = a.tile_table[blockIdx.x];
  if (te.x < 0) return;
  const int tid = threadIdx.x;
  const SpLds L = sp_lds(a.inter);
  // per-row factors of FC1's epilogue; running amax 0 (read after the first
  // main loop's barriers)
  if (tid < BM) {
    const int64_t row0 = te.y, nrow = (int64_t)te.z - te.y;
    const int64_t rr = row0 + (tid < nrow ? tid : nrow - 1);
    const int32_t tk = a.a_row_src[rr];               // the row's token (-1: padding)
    const float sa = (tk >= 0 ? a.a_gscale[tk] : 0.0f) * a.w1_gscale[te.x];
    const float p = a.row_prob[rr];
    float* rfac = reinterpret_cast<float*>(sp_smem + L.rfac);
    rfac[tid] = sa;
    rfac[BM + tid] = sa * p;
    rfac[2 * BM + tid] = p;
    reinterpret_cast<float*>(sp_smem + L.gam)[tid] = 0.0f;
  }
  const int nslices = (int)((a.inter + SLICE - 1) / SLICE);
  const int nslabs = (int)((a.hidden + BN - 1) / BN);
  auto run = [&](auto mv_c) {
    constexpr int MV = decltype(mv_c)::value;
    for (int sl = 0; sl < nslices; ++sl) sp_body<0, MV>(a, sl);
    for (int sb = 0; sb < nslabs; ++sb) sp_body<1, MV>(a, sb);
  };
  const int64_t nrow = (int64_t)te.z - te.y;     // 1 .. BM valid rows
  switch (__builtin_amdgcn_readfirstlane((int)((nrow + 31) / 32))) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, WM>{}); break;
  }
}

// The 128-row blocks in cost-balanced XCD ranges, as for FC1, except that an
// XCD's last, partial round of blocks is cut into 64-row halves when that
// fits its 32 compute units (the kernel takes any row range up to 128 rows,
// and a half with at most two valid 32-row blocks costs about two thirds of a
// whole block): one workgroup per CU runs blocks of a few hundred
// microseconds, so the last round decides the launch.
constexpr uint32_t kXcdCUs = 32;

TileTableSpec single_pass_table_spec(int64_t rows_cap, int32_t num_groups, int64_t hidden,
                                     int4* table) {
  TileTableSpec t = gemm_mtile_table_spec(rows_cap, num_groups, hidden, table);
  t.split_tail = kXcdCUs;
  if (t.blocks > 0) t.blocks += 8 * (kXcdCUs / 2);
  return t;
}

int single_pass_lds_bytes(int64_t inter) { return sp_lds(inter).bytes; }

hipError_t launch_single_pass(const SinglePassArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  const int lds = sp_lds(a.inter).bytes;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  single_pass_kernel<<<(unsigned)blocks, NT, lds, s>>>(a);
  return hipGetLastError();
}

}  // namespace nvfp4
