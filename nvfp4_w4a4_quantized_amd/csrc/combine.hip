// combine.hip -- unpermute the expert outputs back to token order:
// y[t, :] = bf16(sum_j Y[dst_row[t, j], :]), j ascending, fp32 accumulation.
// The router weight was applied before FC2 (miniTE Technical Report §5.4:
// the activated gate/up product is multiplied by the routing probability),
// so this is a plain sum.  One workgroup per
// token; each thread owns 8 consecutive columns (16-byte loads and stores).
// The fixed j order makes the result bitwise reproducible.
#include "launch.h"
#include "nvfp4_device.h"

namespace nvfp4 {

// The 8 values of one row piece (16 bytes of bf16 or 32 bytes of fp32).
template <int DTYPE>
struct RowPiece {
  uint4 v[DTYPE == 0 ? 2 : 1];
};

template <int DTYPE>
__device__ __forceinline__ RowPiece<DTYPE> load_piece(const void* y_rows, int64_t r, int64_t H,
                                                      int64_t c) {
  RowPiece<DTYPE> p;
  if (DTYPE == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const float*>(y_rows) + r * H + c);
    p.v[0] = q[0];
    p.v[DTYPE == 0 ? 1 : 0] = q[1];
  } else {
    p.v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y_rows) + r * H + c);
  }
  return p;
}

template <int DTYPE>
__device__ __forceinline__ void add_piece(float (&s)[8], const RowPiece<DTYPE>& p) {
  if (DTYPE == 0) {
    const uint4 a = p.v[0], b = p.v[DTYPE == 0 ? 1 : 0];
    s[0] += __uint_as_float(a.x); s[1] += __uint_as_float(a.y);
    s[2] += __uint_as_float(a.z); s[3] += __uint_as_float(a.w);
    s[4] += __uint_as_float(b.x); s[5] += __uint_as_float(b.y);
    s[6] += __uint_as_float(b.z); s[7] += __uint_as_float(b.w);
  } else {
    const uint4 u = p.v[0];
    s[0] += bf16_lo(u.x); s[1] += bf16_hi(u.x);
    s[2] += bf16_lo(u.y); s[3] += bf16_hi(u.y);
    s[4] += bf16_lo(u.z); s[5] += bf16_hi(u.z);
    s[6] += bf16_lo(u.w); s[7] += bf16_hi(u.w);
  }
}

// KMAX > 0 (topk <= KMAX): the token's row indices are read first and all
// its row pieces are requested before the first add, so a token costs one
// memory latency instead of topk of them; the adds keep the j order.
template <int DTYPE, int KMAX>   // DTYPE 0: fp32 rows, 1: bf16 rows
__global__ __launch_bounds__(256) void combine_kernel(const void* y_rows, const int32_t* dst,
                                                      int64_t tokens, int32_t topk, int64_t H,
                                                      uint16_t* y) {
  const int64_t t = blockIdx.x;
  if (t >= tokens) return;
  int32_t rows[KMAX > 0 ? KMAX : 1];
  if constexpr (KMAX > 0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rows[j] = j < topk ? dst[t * topk + j] : -1;
  }
  for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += (int64_t)blockDim.x * 8) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (KMAX > 0) {
      RowPiece<DTYPE> p[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (rows[j] >= 0) p[j] = load_piece<DTYPE>(y_rows, rows[j], H, c);
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (rows[j] >= 0) add_piece<DTYPE>(s, p[j]);
    } else {
      for (int j = 0; j < topk; ++j) {
        const int32_t r = dst[t * topk + j];
        if (r < 0) continue;
        add_piece<DTYPE>(s, load_piece<DTYPE>(y_rows, r, H, c));
      }
    }
    uint4 o;
    o.x = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
    o.y = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
    o.z = f32_to_bf16_bits(s[4]) | (f32_to_bf16_bits(s[5]) << 16);
    o.w = f32_to_bf16_bits(s[6]) | (f32_to_bf16_bits(s[7]) << 16);
    *reinterpret_cast<uint4*>(y + t * H + c) = o;
  }
}

hipError_t launch_combine(const void* y_rows, int dtype, const int32_t* dst, int64_t tokens,
                          int32_t topk, int64_t hidden, uint16_t* y, hipStream_t s) {
  if (tokens == 0) return hipSuccess;
  int threads = (int)((hidden / 8 + 63) / 64 * 64);
  if (threads > 256) threads = 256;
  if (threads < 64) threads = 64;
  const int kmax = topk <= 8 ? 8 : (topk <= 16 ? 16 : 0);
#define NVFP4_COMBINE(D, KM) \
  combine_kernel<D, KM><<<(unsigned)tokens, threads, 0, s>>>(y_rows, dst, tokens, topk, hidden, y)
  switch (dtype * 100 + kmax) {
    case 8: NVFP4_COMBINE(0, 8); break;
    case 16: NVFP4_COMBINE(0, 16); break;
    case 0: NVFP4_COMBINE(0, 0); break;
    case 108: NVFP4_COMBINE(1, 8); break;
    case 116: NVFP4_COMBINE(1, 16); break;
    default: NVFP4_COMBINE(1, 0); break;
  }
#undef NVFP4_COMBINE
  return hipGetLastError();
}

}  // namespace nvfp4
