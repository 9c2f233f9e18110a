// quantize.hip -- NVFP4 quantization of bf16 rows on gfx950.
//
// One wavefront per row.  Lane l owns the 16-element blocks l, l+64, ...
// (BPL blocks), so each load instruction of the wave reads a contiguous
// 2 KiB span (coalesced), and the row stays in registers between the amax
// reduction and the encoding.  The row amax is a wave-wide max of the |bf16|
// bit patterns; the per-token outer scale is s_g = amax / 2688 (miniTE
// Technical Report §5.6), or amax / 1536 under Four-Over-Six.  Group (per-expert) scales take an atomic max of
// the row amaxes first (order independent, so deterministic).
#include "launch.h"
#include "nvfp4_device.h"

namespace nvfp4 {

int blocks_per_lane(int64_t k) {
  int64_t nb = (k + 15) / 16;
  int64_t per = (nb + kWave - 1) / kWave;
  if (per <= 1) return 1;
  if (per <= 2) return 2;
  if (per <= 4) return 4;
  if (per <= 8) return 8;
  if (per <= 16) return 16;
  return 0;
}

// Loads the lane's blocks of one bf16 row (zeros for blocks past the row end)
// and returns the lane's max |x| as bits of a bf16 magnitude.
template <int BPL>
__device__ __forceinline__ uint32_t load_row_blocks(const uint16_t* row, int nblocks, int lane,
                                                    uint32_t (&w)[BPL][8]) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + kWave * i;
    if (b < nblocks) {
      const uint16_t* p = row + (int64_t)b * 16;
      u32x4_t u0 = load_stream16(p);
      u32x4_t u1 = load_stream16(p + 8);
      w[i][0] = u0.x; w[i][1] = u0.y; w[i][2] = u0.z; w[i][3] = u0.w;
      w[i][4] = u1.x; w[i][5] = u1.y; w[i][6] = u1.z; w[i][7] = u1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[i][j] = 0u;
    }
    const uint32_t mi = bf16_absmax_bits(w[i]);
    m = m > mi ? m : mi;
  }
  return m;
}

// Group of `row` given non-decreasing offsets (the last g with off[g] <= row).
__device__ __forceinline__ int find_group(const int32_t* off, int num_groups, int64_t row) {
  int lo = 0, hi = num_groups - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if ((int64_t)off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int BPL>
__global__ __launch_bounds__(256, BPL <= 2 ? 8 : 1) void quantize_rows_kernel(QuantRowsArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (row >= a.rows) return;
  const int nblocks = (int)(a.k / 16);
  const uint16_t* xr = a.x + row * a.ld_x;
  uint32_t w[BPL][8];
  uint32_t mbits = load_row_blocks<BPL>(xr, nblocks, lane, w);
  float amax;
  if (a.amax_kind == 0) {
    amax = __uint_as_float(wave_max_u32(mbits) << 16);
  } else if (a.amax_kind == 1) {
    amax = a.amax_in[row];
  } else if (a.amax_kind == 3) {
    amax = a.amax_in[0];
  } else {
    int g = find_group(a.group_offsets, a.num_groups, row);
    amax = a.amax_in[g];
  }
  const float s_g = outer_scale(amax, a.block_rule);
  uint8_t* crow = a.codes + row * (a.k / 2);
  uint8_t* srow = a.scales + row * (a.k / 16);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + kWave * i;
    if (b < nblocks) {
      uint32_t sb;
      uint2 c = quantize_block16(w[i], s_g, a.block_rule, &sb);
      *reinterpret_cast<uint2*>(crow + (int64_t)b * 8) = c;
      srow[b] = (uint8_t)sb;
    }
  }
  if (a.amax_kind != 2 && lane == 0) a.gscale[row] = s_g;
}

// Outer scale given per row (amax kind 1) or per group (kind 2): one thread
// per 16-element block, consecutive threads on consecutive blocks of a row
// (32-byte reads and 8-byte writes side by side), so short rows leave no
// lane idle and no reduction is needed.  Rows * blocks < 2^32.
__global__ __launch_bounds__(256) void quantize_blocks_kernel(QuantRowsArgs a) {
  const uint32_t nb = (uint32_t)(a.k / 16);
  const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  const uint64_t total = (uint64_t)a.rows * nb;
  const uint32_t row = (uint32_t)(i < total ? i : total - 1) / nb;
  int g = 0;
  if (a.amax_kind == 2) {
    // a wave's rows are consecutive: one uniform search from its first row,
    // then lanes past a group boundary step forward
    g = find_group(a.group_offsets, a.num_groups, (int64_t)__builtin_amdgcn_readfirstlane(row));
    while (g + 1 < a.num_groups && (int64_t)a.group_offsets[g + 1] <= (int64_t)row) ++g;
  }
  if (i >= total) return;
  const uint32_t b = (uint32_t)i - row * nb;
  const float amax = a.amax_kind == 1 ? a.amax_in[row] : a.amax_in[a.amax_kind == 3 ? 0 : g];
  const float s_g = outer_scale(amax, a.block_rule);
  const uint16_t* p = a.x + (int64_t)row * a.ld_x + (int64_t)b * 16;
  const u32x4_t u0 = load_stream16(p);
  const u32x4_t u1 = load_stream16(p + 8);
  const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
  uint32_t sb;
  const uint2 c = quantize_block16(w, s_g, a.block_rule, &sb);
  *reinterpret_cast<uint2*>(a.codes + (int64_t)row * (a.k / 2) + (int64_t)b * 8) = c;
  a.scales[(int64_t)row * (a.k / 16) + b] = (uint8_t)sb;
  if ((a.amax_kind == 1 || a.amax_kind == 3) && b == 0) a.gscale[row] = s_g;
}

// 16x16 two-dimensional blocks (per-group outer scale from amax_in): each
// lane owns one tile (16 rows of a group x one 16-element block column),
// finds its maximum, then encodes the 16 rows with it; the scale byte is
// stored in each of the tile's rows.  Consecutive lanes take consecutive
// block columns, so every load and store of a wave is contiguous.
__global__ __launch_bounds__(256) void quantize_tiles2d_kernel(QuantRowsArgs a) {
  const int64_t nb = a.k / 16;
  const int64_t per_rt = (nb + kWave - 1) / kWave * kWave;   // lanes per 16-row tile row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rt = gid / per_rt, b = gid % per_rt;
  if (rt >= a.rows / 16 || b >= nb) return;
  const int64_t r0 = rt * 16;
  const float s_g = outer_scale(a.amax_in[find_group(a.group_offsets, a.num_groups, r0)], 0);
  auto load = [&](int r, uint32_t (&w)[8]) {
    const uint16_t* p = a.x + (r0 + r) * a.ld_x + b * 16;
    const u32x4_t u0 = load_stream16(p);
    const u32x4_t u1 = load_stream16(p + 8);
    w[0] = u0.x; w[1] = u0.y; w[2] = u0.z; w[3] = u0.w;
    w[4] = u1.x; w[5] = u1.y; w[6] = u1.z; w[7] = u1.w;
  };
  // the whole tile stays in registers (one pass over HBM): a second read of
  // the rows no longer hits L2 once the other waves' tiles have gone through
  uint32_t w[16][8];
#pragma unroll
  for (int r = 0; r < 16; ++r) load(r, w[r]);
  uint32_t tbits = 0u;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t m = bf16_absmax_bits(w[r]);
    tbits = tbits > m ? tbits : m;
  }
  const float tmax = __uint_as_float(tbits << 16);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    uint32_t sb;
    const uint2 c = quantize_block16_tile(w[r], tmax, s_g, &sb);
    *reinterpret_cast<uint2*>(a.codes + (r0 + r) * (a.k / 2) + b * 8) = c;
    a.scales[(r0 + r) * (a.k / 16) + b] = (uint8_t)sb;
  }
}

hipError_t launch_quantize_tiles2d(const QuantRowsArgs& a, hipStream_t s) {
  const int64_t nb = a.k / 16;
  const int64_t threads = (a.rows / 16) * ((nb + kWave - 1) / kWave * kWave);
  if (threads == 0) return hipSuccess;
  quantize_tiles2d_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Group amax: each wave takes kAmaxRows consecutive rows, keeps a per-lane
// running maximum while the rows stay in one group, and publishes it with one
// atomic max when the group changes or its rows end.  (One atomic per row
// serialised on the group's single word: about 0.6 us each.)
constexpr int kAmaxRows = 64;

template <int BPL>
__global__ __launch_bounds__(256) void group_amax_kernel(const uint16_t* x, int64_t k, int64_t ld_x,
                                                         const int32_t* off, int32_t num_groups,
                                                         uint32_t* amax_bits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int64_t last = off[num_groups];
  const int64_t r0 = (int64_t)off[0] + wid * kAmaxRows;
  if (r0 >= last) return;
  const int64_t r1 = r0 + kAmaxRows < last ? r0 + kAmaxRows : last;
  const int nblocks = (int)(k / 16);
  int g = find_group(off, num_groups, r0);
  int64_t gend = off[g + 1];
  uint32_t m = 0u;
  auto flush = [&]() {
    const uint32_t mx = wave_max_u32(m);
    if (lane == 0 && mx != 0u) atomicMax(amax_bits + g, mx << 16);
    m = 0u;
  };
  for (int64_t r = r0; r < r1; ++r) {
    while (r >= gend) {                          // next non-empty group (uniform)
      flush();
      ++g;
      gend = off[g + 1];
    }
    uint32_t w[BPL][8];
    const uint32_t mi = load_row_blocks<BPL>(x + r * ld_x, nblocks, lane, w);
    m = m > mi ? m : mi;
  }
  flush();
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void group_finalize_kernel(const float* amax, float* gscale, int32_t n, int rule) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) gscale[i] = outer_scale(amax[i], rule);
}

hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  const int64_t total = a.rows * (a.k / 16);
  if (a.amax_kind != 0 && total < 0xFFFFFFFFll) {
    quantize_blocks_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.rows + 3) / 4)), block(256);
  switch (blocks_per_lane(a.k)) {
    case 1: quantize_rows_kernel<1><<<grid, block, 0, s>>>(a); break;
    case 2: quantize_rows_kernel<2><<<grid, block, 0, s>>>(a); break;
    case 4: quantize_rows_kernel<4><<<grid, block, 0, s>>>(a); break;
    case 8: quantize_rows_kernel<8><<<grid, block, 0, s>>>(a); break;
    case 16: quantize_rows_kernel<16><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_group_amax(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                             const int32_t* off, int32_t num_groups, uint32_t* amax_bits,
                             hipStream_t s) {
  fill_u32_kernel<<<(num_groups + 255) / 256, 256, 0, s>>>(amax_bits, num_groups, 0u);
  if (rows == 0) return hipGetLastError();
  // the group rows lie inside [0, rows): an upper bound on the waves needed
  const int64_t waves = (rows + kAmaxRows - 1) / kAmaxRows;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  switch (blocks_per_lane(k)) {
    case 1: group_amax_kernel<1><<<grid, block, 0, s>>>(x, k, ld_x, off, num_groups, amax_bits); break;
    case 2: group_amax_kernel<2><<<grid, block, 0, s>>>(x, k, ld_x, off, num_groups, amax_bits); break;
    case 4: group_amax_kernel<4><<<grid, block, 0, s>>>(x, k, ld_x, off, num_groups, amax_bits); break;
    case 8: group_amax_kernel<8><<<grid, block, 0, s>>>(x, k, ld_x, off, num_groups, amax_bits); break;
    case 16: group_amax_kernel<16><<<grid, block, 0, s>>>(x, k, ld_x, off, num_groups, amax_bits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The tensor's amax for one outer scale per tensor: bounds = {0, rows} for
// the group reduction over all rows.
__global__ void tensor_bounds_kernel(int32_t* bounds, int32_t rows) {
  if (threadIdx.x == 0) { bounds[0] = 0; bounds[1] = rows; }
}

hipError_t launch_tensor_amax(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                              int32_t* bounds, uint32_t* amax_bits, hipStream_t s) {
  tensor_bounds_kernel<<<1, 64, 0, s>>>(bounds, (int32_t)rows);
  return launch_group_amax(x, rows, k, ld_x, bounds, 1, amax_bits, s);
}

// out[0] = max of amax_rows[r] over r < min(cap, *rows_end) (0 if none): one
// workgroup, each thread a strided share, then a fixed-order reduction.
__global__ __launch_bounds__(1024) void rows_amax_kernel(const float* amax_rows,
                                                         const int32_t* rows_end, int64_t cap,
                                                         float* out) {
  __shared__ uint32_t wm[16];
  const int64_t n = cap < (int64_t)*rows_end ? cap : (int64_t)*rows_end;
  uint32_t m = 0u;
  for (int64_t r = threadIdx.x; r < n; r += 1024) {
    const uint32_t v = __float_as_uint(amax_rows[r]);   // amax >= 0: bits order as values
    m = m > v ? m : v;
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & (kWave - 1)) == 0) wm[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int i = 0; i < 16; ++i) t = t > wm[i] ? t : wm[i];
    out[0] = __uint_as_float(t);
  }
}

hipError_t launch_rows_amax(const float* amax_rows, const int32_t* rows_end, int64_t cap,
                            float* out, hipStream_t s) {
  rows_amax_kernel<<<1, 1024, 0, s>>>(amax_rows, rows_end, cap, out);
  return hipGetLastError();
}

hipError_t launch_group_finalize(const float* amax, float* gscale, int32_t n, int rule,
                                 hipStream_t s) {
  group_finalize_kernel<<<(n + 255) / 256, 256, 0, s>>>(amax, gscale, n, rule);
  return hipGetLastError();
}

}  // namespace nvfp4
