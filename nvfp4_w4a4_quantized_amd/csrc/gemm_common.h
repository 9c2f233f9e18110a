// gemm_common.h -- pieces shared by the grouped GEMM (gemm.hip) and the
// single-pass FC1 -> FC2 kernel (single_pass.hip): the exact NVFP4 -> fp16
// operand decode and the epilogue arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// SwiGLU weighted by the router probability, in binary32; below g = -80
// binary32 exp(-g) overflows while g e^g u p may still be a normal bf16, so
// that rare tail is evaluated in binary64.
__device__ __forceinline__ float swiglu_tail(float g, float u, float p) {
  const double eg = exp((double)g);
  return (float)(((double)g * eg / (1.0 + eg)) * (double)u * (double)p);
}

// The same tail in binary32 for g < -80, without a call or binary64: there
// e^g < 2^-115, so e^g / (1 + e^g) rounds to e^g and the result is
// sign(g u p) * exp(g + ln|g| + ln|u| + ln|p|), whose logarithm stays in
// range while e^g alone would underflow.  The hardware exponential flushes
// subnormal results, so it is evaluated 64 binades up (+64 ln 2) and the
// exact multiply by 2^-64 rounds the result into the subnormals.  The
// relative error (a few binary32 roundings of terms below ~150 in magnitude,
// then exp) is below 1e-4, far inside one bf16 ulp.
__device__ __forceinline__ float swiglu_tail_f32(float g, float u, float p) {
  const float lm = g + __logf(__builtin_fabsf(g)) + __logf(__builtin_fabsf(u)) +
                   __logf(__builtin_fabsf(p));
  const float v = __expf(lm + 44.3614195558365f) * 5.42101086242752217e-20f;   // 2^-64
  return __builtin_copysignf(v, g * u * p);
}

// silu(g) * up, with the router weight already folded into `up` (a few
// binary32 roundings; D is checked to one bf16 ulp and the hardware
// reciprocal, about 1 ulp of binary32, is far inside that)
__device__ __forceinline__ float swiglu_fast(float g, float up) {
  const float silu = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
  return silu * up;
}

// two binary32 -> two bf16 (round to nearest even) in one dword
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t b = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &b, 4);
  return u;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace nvfp4
