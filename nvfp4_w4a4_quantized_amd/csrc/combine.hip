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

template <int DTYPE>   // 0: fp32 rows, 1: bf16 rows
__global__ __launch_bounds__(256) void combine_kernel(const void* y_rows, const int32_t* dst,
                                                      int64_t tokens, int32_t topk, int64_t H,
                                                      uint16_t* y) {
  const int64_t t = blockIdx.x;
  if (t >= tokens) return;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < H; c += (int64_t)blockDim.x * 8) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < topk; ++j) {
      const int32_t r = dst[t * topk + j];
      if (r < 0) continue;
      if (DTYPE == 0) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(y_rows) + (int64_t)r * H + c);
        float4 u0 = p[0], u1 = p[1];
        s[0] += u0.x; s[1] += u0.y; s[2] += u0.z; s[3] += u0.w;
        s[4] += u1.x; s[5] += u1.y; s[6] += u1.z; s[7] += u1.w;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(y_rows) + (int64_t)r * H + c);
        s[0] += bf16_lo(u.x); s[1] += bf16_hi(u.x);
        s[2] += bf16_lo(u.y); s[3] += bf16_hi(u.y);
        s[4] += bf16_lo(u.z); s[5] += bf16_hi(u.z);
        s[6] += bf16_lo(u.w); s[7] += bf16_hi(u.w);
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
  if (dtype == 0)
    combine_kernel<0><<<(unsigned)tokens, threads, 0, s>>>(y_rows, dst, tokens, topk, hidden, y);
  else
    combine_kernel<1><<<(unsigned)tokens, threads, 0, s>>>(y_rows, dst, tokens, topk, hidden, y);
  return hipGetLastError();
}

}  // namespace nvfp4
