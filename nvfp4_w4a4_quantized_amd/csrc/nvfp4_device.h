// nvfp4_device.h -- gfx950 device helpers for the NVFP4 W4A4 path: bf16
// unpacking, the E4M3 block-scale codec, the per-block E2M1 encoder and
// wavefront reductions.
//
// Format (miniTE Technical Report §2.2, §5.1, §5.6; The 4-bitter Lesson,
// "Four-Over-Six"): x^ = q * s_b * s_g, q on the E2M1 grid
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, s_b an E4M3 scale per 16 elements along K,
// s_g = amax / 2688 in FP32.  Every quantizer step is one IEEE binary32
// operation with round-to-nearest-even; the library is built with
// -ffp-contract=off and correctly rounded fp32 division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ u32x4_t load_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Largest |bf16| bit pattern (0..0x7FFF) among N dwords of packed bf16
// pairs: packed unsigned 16-bit maxima of the magnitudes (for non-negative
// values the bit patterns order like the values).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
template <int N>
__device__ __forceinline__ uint32_t bf16_absmax_bits(const uint32_t (&w)[N]) {
  u16x2_t m = {0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t a = w[i] & 0x7FFF7FFFu;
    u16x2_t v;
    __builtin_memcpy(&v, &a, 4);
    m = __builtin_elementwise_max(m, v);
  }
  return m[0] > m[1] ? (uint32_t)m[0] : (uint32_t)m[1];
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// E4M3 (OCP, bias 7) byte of a non-negative binary32 value, round to nearest
// even, values >= 448 saturate to 0x7E.  Written on the binary32 bit pattern:
// below 2^-6 the E4M3 step is 2^-9, so the byte is rint(v * 2^9) (exact
// scaling); above, the byte keeps 3 mantissa bits of v with RNE on the 20
// dropped bits, the carry moving into the exponent.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  if (!(v < 448.0f)) return 0x7Eu;
  if (v < 0.015625f) return (uint32_t)__builtin_rintf(v * 512.0f);
  uint32_t b = __float_as_uint(v);
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
}

// Value of a non-negative E4M3 byte as binary32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0u) return (float)m * 0.001953125f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Wave-wide maximum of a non-negative value held as raw bits (monotonic for
// non-negative floats).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

// Encodes 16 consecutive elements (one block) given the block's decode step
// d = s_b * s_g.  The grid decision is taken on the correctly rounded
// binary32 quotient r = fl(x / d), rounded to E2M1 with ties to the even code
// and saturation at 6 by the gfx950 FP4 conversion (scale 1.0).
//
// Fast path: r' = fl(x * fl(1/d)) differs from x/d by less than 2^-22.9
// relative (two roundings of 2^-24 each, 1/d normal because
// 2^-126 <= d < 2^126).  The E2M1 decision of r' and of fl(x/d) can differ
// only where x/d lies within that distance of a rounding threshold
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, i.e. 4*|r| an integer).  Elements
// whose 4*|r'| is within 2^-16 of an integer in [1, 23] (a band about 50x
// wider than the error) need the IEEE division; when a block holds one, the
// whole block is recomputed that way (for the other elements both quotients
// give the same code), and so is every block with d < 2^-126.  d == 0 (s_b
// underflowed or s_g == 0) gives r = x * 0 = +-0: magnitude 0, sign kept.
template <int SEL>
__device__ __forceinline__ uint32_t pack_fp4_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

__device__ __forceinline__ uint2 encode_block16(const float (&x)[16], float d) {
  const bool full_div = (d != 0.0f) && (d < 1.17549435e-38f);
  const float inv = (d == 0.0f) ? 0.0f : 1.0f / d;
  float r[16];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    r[i] = x[i] * inv;
    const float f = __builtin_fabsf(r[i]) * 4.0f;
    near |= (f >= 0.5f) && (f < 23.5f) &&
            (__builtin_fabsf(f - __builtin_rintf(f)) < 1.52587890625e-05f);
  }
  if (full_div || near) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = x[i] / d;
  }
  uint32_t w0 = pack_fp4_pair<0>(0u, r[0], r[1]);
  w0 = pack_fp4_pair<1>(w0, r[2], r[3]);
  w0 = pack_fp4_pair<2>(w0, r[4], r[5]);
  w0 = pack_fp4_pair<3>(w0, r[6], r[7]);
  uint32_t w1 = pack_fp4_pair<0>(0u, r[8], r[9]);
  w1 = pack_fp4_pair<1>(w1, r[10], r[11]);
  w1 = pack_fp4_pair<2>(w1, r[12], r[13]);
  w1 = pack_fp4_pair<3>(w1, r[14], r[15]);
  return make_uint2(w0, w1);
}

// Quantizes one 16-element block of bf16 values (two uint4 words = 8 dwords,
// element 2i in the low half of dword i) with outer scale s_g.  Returns the
// 8 code bytes; *scale receives the E4M3 byte.
//   s_b = E4M3(fl(bmax / fl(6 * s_g))) (0 when s_g == 0), d = fl(s_b * s_g).
__device__ __forceinline__ uint2 quantize_block16(const uint32_t (&w)[8], float s_g,
                                                  uint32_t* scale) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  const float bmax = __uint_as_float(bf16_absmax_bits(w) << 16);
  uint32_t sb = 0u;
  if (s_g != 0.0f) {
    const float t = 6.0f * s_g;
    sb = e4m3_encode(bmax / t);
  }
  *scale = sb;
  const float d = e4m3_value(sb) * s_g;
  return encode_block16(x, d);
}

}  // namespace nvfp4
