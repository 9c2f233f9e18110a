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

// Buffer-resource loads: an offset at or past the resource's size reads as
// zero without a memory access, so a masked element needs no branch (a
// branch around a load makes the compiler wait, where the paths join, for
// every load in flight).  Resources stay below 2^31 bytes (the launchers
// check), and kNone lies past every one.
constexpr uint32_t kNone = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void_t;

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

// Wave-wide inclusive scans through DPP lane moves (no LDS round trips):
// shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the row broadcasts
// of lane 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3).  Every
// lane of the wave must be active.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v, Op op) {
  const int lane = threadIdx.x & (kWave - 1);
  const int rl = lane & 15;
  uint32_t t;
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  if (rl >= 1) v = op(t, v);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  if (rl >= 2) v = op(t, v);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  if (rl >= 4) v = op(t, v);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  if (rl >= 8) v = op(t, v);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x142, 0xf, 0xf, false);   // row_bcast:15
  if ((lane & 31) >= 16) v = op(t, v);
  t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x143, 0xf, 0xf, false);   // row_bcast:31
  if (lane >= 32) v = op(t, v);
  return v;
}

// Wave-wide maximum of a non-negative value held as raw bits (monotonic for
// non-negative floats), the same in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = wave_incl_scan_dpp(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// Encodes 16 consecutive elements (one block) given the block's decode step
// d = s_b * s_g.  The grid decision is taken on the correctly rounded
// binary32 quotient r = fl(x / d), rounded to E2M1 with ties to the even code
// and saturation at 6 by the gfx950 FP4 conversion (scale 1.0).
//
// Fast path: with inv = fl(1/d) (1/d normal because 2^-126 <= d < 2^126),
// lo = fl(x * fl(inv * (1 - 2^-20))) and hi = fl(x * fl(inv * (1 + 2^-20)))
// bracket both x/d and fl(x/d) strictly: each carries at most three binary32
// roundings (relative error below 3.1 * 2^-24), far inside the 2^-20 offset,
// and fl(x/d) itself is within 2^-24 of x/d.  E2M1 rounding is monotonic, so
// when lo and hi get the same code, every value between them, fl(x/d)
// included, gets that code.  An element pair whose two codes differ (a
// quotient near a rounding threshold) is recomputed with the IEEE division,
// and every block with d < 2^-126 recomputes all 16 quotients.  d == 0
// (s_b underflowed or s_g == 0) gives r = x * 0 = +-0: magnitude 0, sign
// kept.  Overflowing products (huge x/d) saturate to code 7 on both sides.
template <int SEL>
__device__ __forceinline__ uint32_t pack_fp4_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

__device__ __forceinline__ uint2 pack_fp4_block(const float (&r)[16]) {
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

__device__ __forceinline__ uint2 encode_block16(const float (&x)[16], float d) {
  const bool full_div = (d != 0.0f) && (d < 1.17549435e-38f);
  // inv = 1/d within one ulp (v_rcp_f32, a normal input): with the 2^-20
  // offsets the products still bracket fl(x/d) strictly (total relative
  // error below 2^-23 + 3 * 2^-24 < 2^-21)
  const float inv = (d == 0.0f) ? 0.0f : __builtin_amdgcn_rcpf(d);
  const float inv_lo = inv * 0.99999904632568359375f;   // 1 - 2^-20
  const float inv_hi = inv * 1.00000095367431640625f;   // 1 + 2^-20
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x[i] * inv_lo;
  const uint2 lo = pack_fp4_block(r);
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = x[i] * inv_hi;
  const uint2 hi = pack_fp4_block(r);
  if (full_div) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = x[i] / d;
    return pack_fp4_block(r);
  }
  // Only the element pairs whose two codes differ take the IEEE division.
  // With bf16 inputs and scales that are short binary fractions, quotients
  // at or within an ulp of a rounding threshold are not rare (a few per
  // thousand elements, most of them exact ties), so a per-block fallback
  // would run in most waves; per pair it runs where a lane needs it.
  uint2 out = lo;
  const uint32_t dx = lo.x ^ hi.x, dy = lo.y ^ hi.y;
  if ((dx | dy) != 0u) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t dw = j < 4 ? dx : dy;
      if ((dw >> (8 * (j % 4))) & 0xFFu) {
        const float r0 = x[2 * j] / d, r1 = x[2 * j + 1] / d;
        switch (j) {
          case 0: out.x = pack_fp4_pair<0>(out.x, r0, r1); break;
          case 1: out.x = pack_fp4_pair<1>(out.x, r0, r1); break;
          case 2: out.x = pack_fp4_pair<2>(out.x, r0, r1); break;
          case 3: out.x = pack_fp4_pair<3>(out.x, r0, r1); break;
          case 4: out.y = pack_fp4_pair<0>(out.y, r0, r1); break;
          case 5: out.y = pack_fp4_pair<1>(out.y, r0, r1); break;
          case 6: out.y = pack_fp4_pair<2>(out.y, r0, r1); break;
          default: out.y = pack_fp4_pair<3>(out.y, r0, r1); break;
        }
      }
    }
  }
  return out;
}

// Block rules: 0 maps every block maximum to the largest E2M1 value 6.  1 and
// 2 are Four-Over-Six (The 4-bitter Lesson, "Four-Over-Six for RL Weights
// and Activations"): each block is quantized with its maximum mapped to 6
// and to 4 and keeps the candidate with the smaller block error (1: sum of
// squares, 2: sum of absolute values, both in binary32 over the 16 elements
// in order); ties keep 6.  The page's formula names an FP8 maximum for this
// mode without giving it; 256 keeps the 4-candidate's scale (1.5x, at most
// 384) inside E4M3, so the outer scale is amax / (6 * 256).
__device__ __forceinline__ float outer_scale(float amax, int rule) {
  return rule == 0 ? amax / 2688.0f : amax / 1536.0f;
}

// e4m3_encode(fl(num / den)) for num >= 0 (or NaN/inf), den > 0, without the
// IEEE division in the common case.  q = fl(num * rcp(den)) lies within a
// few ulp of fl(num / den) when den is normal.  Above 2^-6 the E4M3 byte is
// the round-to-nearest-even of q's top 3 mantissa bits (values from 432 up
// all give 0x7E), so two quotients a few ulp apart can only get different
// bytes when a midpoint between E4M3 neighbours (dropped 20 bits = 0x80000)
// lies between them; within 16 ulp of one, in the E4M3 subnormal range, or
// for a subnormal den, the IEEE quotient decides.
__device__ __forceinline__ uint32_t e4m3_of_quotient(float num, float den) {
  if (num == 0.0f) return 0u;
  const float q = num * __builtin_amdgcn_rcpf(den);
  const uint32_t dropped = __float_as_uint(q) & 0xFFFFFu;
  const bool near_mid = dropped - 0x7FFF0u <= 0x20u;
  if (near_mid || q < 0.0157f || den < 1.17549435e-38f) return e4m3_encode(num / den);
  return e4m3_encode(q);
}

// E4M3 byte of the block scale mapping bmax to `top`, and the decode step.
__device__ __forceinline__ uint32_t block_scale(float bmax, float s_g, float top, float* d) {
  uint32_t sb = 0u;
  if (s_g != 0.0f) sb = e4m3_of_quotient(bmax, top * s_g);
  *d = e4m3_value(sb) * s_g;
  return sb;
}

// Block error of codes c (two dwords, element 2i in the low nibble of byte
// i) with scale byte sb: sum over i of e^2 (rule 1) or |e| (rule 2),
// e = x_i - fl((q_i * s_b) * s_g), accumulated in order in binary32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <int SEL>
__device__ __forceinline__ f32x2_t fp4_pair_value(uint32_t w) {   // codes of byte SEL
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ float block_error(const float (&x)[16], uint2 c, uint32_t sb, float s_g,
                                             int rule) {
  const float s_b = e4m3_value(sb);
  f32x2_t q[8];
  q[0] = fp4_pair_value<0>(c.x); q[1] = fp4_pair_value<1>(c.x);
  q[2] = fp4_pair_value<2>(c.x); q[3] = fp4_pair_value<3>(c.x);
  q[4] = fp4_pair_value<0>(c.y); q[5] = fp4_pair_value<1>(c.y);
  q[6] = fp4_pair_value<2>(c.y); q[7] = fp4_pair_value<3>(c.y);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = (q[i / 2][i % 2] * s_b) * s_g;   // q * s_b is exact
    const float e = x[i] - v;
    acc = acc + (rule == 1 ? e * e : __builtin_fabsf(e));
  }
  return acc;
}

// One 16-element block (8 dwords of bf16 pairs) scaled by a given maximum:
// the 16x16 tile maximum of two-dimensional weight blocks (standard rule).
__device__ __forceinline__ uint2 quantize_block16_tile(const uint32_t (&w)[8], float tmax, float s_g,
                                                       uint32_t* scale) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  float d;
  *scale = block_scale(tmax, s_g, 6.0f, &d);
  return encode_block16(x, d);
}

// Quantizes one 16-element block of bf16 values (two uint4 words = 8 dwords,
// element 2i in the low half of dword i) with outer scale s_g under a block
// rule.  Returns the 8 code bytes; *scale receives the E4M3 byte.
//   s_b = E4M3(fl(bmax / fl(top * s_g))) (0 when s_g == 0), d = fl(s_b * s_g).
__device__ __forceinline__ uint2 quantize_block16(const uint32_t (&w)[8], float s_g, int rule,
                                                  uint32_t* scale) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  const float bmax = __uint_as_float(bf16_absmax_bits(w) << 16);
  float d6;
  const uint32_t sb6 = block_scale(bmax, s_g, 6.0f, &d6);
  const uint2 c6 = encode_block16(x, d6);
  if (rule == 0) {
    *scale = sb6;
    return c6;
  }
  float d4;
  const uint32_t sb4 = block_scale(bmax, s_g, 4.0f, &d4);
  const uint2 c4 = encode_block16(x, d4);
  const bool four = block_error(x, c4, sb4, s_g, rule) < block_error(x, c6, sb6, s_g, rule);
  *scale = four ? sb4 : sb6;
  return four ? c4 : c6;
}

}  // namespace nvfp4
