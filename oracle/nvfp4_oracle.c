/*
 * nvfp4_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the
 * header for who may use it and for the page citations).
 *
 * Written for readability against the definitions, not for speed: codecs are
 * nearest-value searches over the enumerated grids, the GEMM is a triple loop
 * over decoded fp64 operands.  OpenMP only splits independent rows; it never
 * changes an arithmetic order.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* O1: encodings                                                            */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes by index ([4BIT] "Four-Over-Six" prints this grid). */
static const double kE2M1Grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(unsigned code) {
  double mag = kE2M1Grid[code & 7u];
  return (code & 8u) ? -mag : mag;
}

unsigned orc_e2m1_encode(float r) {
  unsigned sign = signbit(r) ? 8u : 0u;
  double a = fabs((double)r);
  /* saturate: the largest magnitude is 6 (no Inf/NaN in E2M1) */
  if (!(a < 6.0)) return sign | 7u;
  /* nearest grid value; on an exact tie keep the even index */
  unsigned best = 0;
  double best_dist = fabs(a - kE2M1Grid[0]);
  for (unsigned i = 1; i < 8; ++i) {
    double dist = fabs(a - kE2M1Grid[i]); /* exact: a has 24 bits, grid 3 */
    if (dist < best_dist || (dist == best_dist && (i % 2u) == 0u && (best % 2u) != 0u)) {
      best = i;
      best_dist = dist;
    }
  }
  return sign | best;
}

double orc_e4m3_value(unsigned byte) {
  unsigned s = (byte >> 7) & 1u;
  unsigned e = (byte >> 3) & 15u;
  unsigned m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;           /* the only NaN pattern */
  if (e == 0u) v = ldexp((double)m, -9);          /* subnormal: m * 2^-9 */
  else v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

unsigned orc_e4m3_encode(float v) {
  double a = (double)v;
  /* the non-negative finite bytes 0x00..0x7E have increasing values */
  unsigned best = 0;
  double best_dist = fabs(a - orc_e4m3_value(0));
  for (unsigned b = 1; b <= 0x7Eu; ++b) {
    double dist = fabs(a - orc_e4m3_value(b));   /* exact in fp64 */
    if (dist < best_dist || (dist == best_dist && (b % 2u) == 0u)) {
      best = b;
      best_dist = dist;
    }
  }
  return best; /* values above 448 are nearest to 448 = 0x7E: saturation */
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

uint16_t orc_f64_to_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
  /* The bf16 truncation of the nearest binary32 value is within one bf16 step
   * of v, so the nearest bf16 is that value or one of its two neighbours.
   * Compare exact fp64 distances; ties go to the even bf16 pattern. */
  float f = (float)v;
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t mid = (uint16_t)(bits >> 16);
  uint16_t best = mid;
  double best_dist = INFINITY;
  for (int delta = -1; delta <= 1; ++delta) {
    uint16_t c = (uint16_t)(mid + delta);
    if ((c & 0x7F80u) == 0x7F80u) continue;            /* Inf / NaN patterns */
    if ((c & 0x8000u) != (mid & 0x8000u)) continue;    /* wrapped across zero */
    double dist = fabs((double)orc_bf16_to_f32(c) - v);
    if (dist < best_dist || (dist == best_dist && (c & 1u) == 0u)) {
      best = c;
      best_dist = dist;
    }
  }
  return best;
}

/* ------------------------------------------------------------------------ */
/* O2-O4: NVFP4 quantization                                                */
/* ------------------------------------------------------------------------ */

float orc_row_amax(const uint16_t* x, int64_t k) {
  float amax = 0.0f;
  for (int64_t i = 0; i < k; ++i) {
    float a = fabsf(orc_bf16_to_f32(x[i]));
    if (a > amax) amax = a;
  }
  return amax;
}

/* One block's E4M3 scale byte and its 16 codes, with the block maximum
 * mapped to the E2M1 value `top` (6 for the standard rule; 4 for the second
 * Four-Over-Six candidate). */
static unsigned quantize_block_bmax(const uint16_t* blk, float bmax, float s_g, float top,
                                   unsigned codes16[16]);

static unsigned quantize_block(const uint16_t* blk, float s_g, float top, unsigned codes16[16]) {
  float bmax = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float a = fabsf(orc_bf16_to_f32(blk[i]));
    if (a > bmax) bmax = a;
  }
  return quantize_block_bmax(blk, bmax, s_g, top, codes16);
}

/* The same with the scaling maximum given (the 2D tile maximum for 16x16
 * weight blocks). */
static unsigned quantize_block_bmax(const uint16_t* blk, float bmax, float s_g, float top,
                                   unsigned codes16[16]) {
  /* block scale: maps the block maximum to `top` */
  unsigned sb_byte = 0;
  if (s_g != 0.0f) {
    float t = top * s_g;
    float q = bmax / t;
    sb_byte = orc_e4m3_encode(q);
  }
  float s_b = (float)orc_e4m3_value(sb_byte);  /* exact in binary32 */
  float d = s_b * s_g;                          /* per-block decode step */
  for (int i = 0; i < 16; ++i) {
    float xv = orc_bf16_to_f32(blk[i]);
    unsigned code;
    if (d == 0.0f) {
      code = signbit(xv) ? 8u : 0u;             /* underflowed block */
    } else {
      float r = xv / d;                         /* IEEE binary32 division */
      code = orc_e2m1_encode(r);
      if (signbit(xv)) code |= 8u; else code &= 7u;
    }
    codes16[i] = code;
  }
  return sb_byte;
}

/* Packs a block's codes: element 2j in the low nibble of byte j. */
static void pack_block(int64_t b, const unsigned codes16[16], uint8_t* codes) {
  for (int i = 0; i < 16; ++i) {
    int64_t e = b * 16 + i;
    unsigned code = codes16[i];
    codes[e / 2] |= (uint8_t)((e % 2) ? (code << 4) : code);
  }
}

float orc_quantize_row_with_amax(const uint16_t* x, int64_t k, float amax,
                                 uint8_t* codes, uint8_t* scales) {
  /* outer (second-level) scale: [miniTE] §5.6 divides the amax by 2688 */
  float s_g = amax / 2688.0f;
  memset(codes, 0, (size_t)(k / 2));
  for (int64_t b = 0; b < k / 16; ++b) {
    unsigned c[16];
    /* the block maximum maps to the largest E2M1 value, 6 */
    scales[b] = (uint8_t)quantize_block(x + b * 16, s_g, 6.0f, c);
    pack_block(b, c, codes);
  }
  return s_g;
}

/* Block error of a candidate: the values q * s_b * s_g against x, summed
 * left to right in binary32 (metric 1: squares, 2: absolute values). */
static float block_error(const uint16_t* blk, const unsigned codes16[16], unsigned sb_byte,
                         float s_g, int metric) {
  float s_b = (float)orc_e4m3_value(sb_byte);
  float acc = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float xv = orc_bf16_to_f32(blk[i]);
    float qs = (float)(orc_e2m1_value(codes16[i]) * (double)s_b);  /* exact */
    float v = qs * s_g;
    float e = xv - v;
    float term = (metric == 1) ? e * e : fabsf(e);
    acc = acc + term;
  }
  return acc;
}

float orc_quantize_row_rule(const uint16_t* x, int64_t k, float amax, int rule,
                            uint8_t* codes, uint8_t* scales) {
  if (rule == 0) return orc_quantize_row_with_amax(x, k, amax, codes, scales);
  /* 4/6: the outer scale leaves room for blocks mapped to 4, whose scale is
   * 1.5x that of the same block mapped to 6: s_g = amax / (6 * 256) */
  float s_g = amax / 1536.0f;
  memset(codes, 0, (size_t)(k / 2));
  for (int64_t b = 0; b < k / 16; ++b) {
    const uint16_t* blk = x + b * 16;
    unsigned c6[16], c4[16];
    unsigned sb6 = quantize_block(blk, s_g, 6.0f, c6);
    unsigned sb4 = quantize_block(blk, s_g, 4.0f, c4);
    float e6 = block_error(blk, c6, sb6, s_g, rule);
    float e4 = block_error(blk, c4, sb4, s_g, rule);
    /* the reduced range only where it lowers the block error; ties keep 6 */
    int four = e4 < e6;
    scales[b] = (uint8_t)(four ? sb4 : sb6);
    pack_block(b, four ? c4 : c6, codes);
  }
  return s_g;
}

float orc_outer_scale(float amax, int rule) {
  return rule == 0 ? amax / 2688.0f : amax / 1536.0f;
}

int orc_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                 int domain, const int32_t* group_offsets, int32_t num_groups,
                 const float* amax_in,
                 uint8_t* codes, uint8_t* scales, float* gscale) {
  return orc_quantize_rule(x, rows, k, ld_x, domain, group_offsets, num_groups, amax_in, 0,
                           codes, scales, gscale);
}

/* max |x| over rows [r0, r1) */
static float group_amax(const uint16_t* x, int64_t ld_x, int64_t k, int64_t r0, int64_t r1) {
  float amax = 0.0f;
  for (int64_t r = r0; r < r1; ++r) {
    float a = orc_row_amax(x + r * ld_x, k);
    if (a > amax) amax = a;
  }
  return amax;
}

int orc_quantize_rule(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                      int domain, const int32_t* group_offsets, int32_t num_groups,
                      const float* amax_in, int rule,
                      uint8_t* codes, uint8_t* scales, float* gscale) {
  if (rows < 0 || k < 0 || k % 16 != 0 || ld_x < k) return 1;
  if (rule < 0 || rule > 2) return 1;
  if (domain == 0) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      const uint16_t* xr = x + r * ld_x;
      float amax = amax_in ? amax_in[r] : orc_row_amax(xr, k);
      gscale[r] = orc_quantize_row_rule(xr, k, amax, rule, codes + r * (k / 2), scales + r * (k / 16));
    }
    return 0;
  }
  if (domain == 1) {
    if (!group_offsets || num_groups < 0) return 1;
    for (int32_t g = 0; g < num_groups; ++g) {
      int64_t r0 = group_offsets[g], r1 = group_offsets[g + 1];
      if (r0 < 0 || r1 < r0 || r1 > rows) return 1;
      float amax = amax_in ? amax_in[g] : group_amax(x, ld_x, k, r0, r1);
#pragma omp parallel for schedule(static)
      for (int64_t r = r0; r < r1; ++r)
        (void)orc_quantize_row_rule(x + r * ld_x, k, amax, rule, codes + r * (k / 2),
                                    scales + r * (k / 16));
      gscale[g] = orc_outer_scale(amax, rule); /* the s_g every row of the group used */
    }
    return 0;
  }
  if (domain == 2) {
    /* per-group outer scale with 16x16 blocks: 16 consecutive rows of a group
     * and 16 consecutive elements share one E4M3 scale, set by the tile
     * maximum ([miniTE] §2.2 and App. D2 compare one- and two-dimensional
     * block scaling of weights without giving the block shape).  Reading: the tile's
     * maximum maps to 6 exactly as a 1D block's would, every element is
     * encoded with the tile's decode step, and the scale byte is stored in
     * each of the tile's rows so that [rows, k/16] keeps its meaning. */
    if (!group_offsets || num_groups < 0 || rule != 0) return 1;
    for (int32_t g = 0; g < num_groups; ++g) {
      int64_t r0 = group_offsets[g], r1 = group_offsets[g + 1];
      if (r0 < 0 || r1 < r0 || r1 > rows || (r1 - r0) % 16 != 0) return 1;
      float amax = amax_in ? amax_in[g] : group_amax(x, ld_x, k, r0, r1);
      float s_g = orc_outer_scale(amax, 0);
      for (int64_t t0 = r0; t0 < r1; t0 += 16) {
        for (int64_t r = t0; r < t0 + 16; ++r) memset(codes + r * (k / 2), 0, (size_t)(k / 2));
        for (int64_t b = 0; b < k / 16; ++b) {
          float tmax = 0.0f;
          for (int64_t r = t0; r < t0 + 16; ++r) {
            float a = orc_row_amax(x + r * ld_x + b * 16, 16);
            if (a > tmax) tmax = a;
          }
          for (int64_t r = t0; r < t0 + 16; ++r) {
            unsigned c[16];
            scales[r * (k / 16) + b] =
                (uint8_t)quantize_block_bmax(x + r * ld_x + b * 16, tmax, s_g, 6.0f, c);
            pack_block(b, c, codes + r * (k / 2));
          }
        }
      }
      gscale[g] = s_g;
    }
    return 0;
  }
  return 1;
}

void orc_dequantize_row(const uint8_t* codes, const uint8_t* scales, float gscale,
                        int64_t k, double* out) {
  for (int64_t e = 0; e < k; ++e) {
    unsigned byte = codes[e / 2];
    unsigned code = (e % 2) ? (byte >> 4) : (byte & 15u);
    out[e] = orc_e2m1_value(code) * orc_e4m3_value(scales[e / 16]) * (double)gscale;
  }
}

/* ------------------------------------------------------------------------ */
/* O6: routing                                                              */
/* ------------------------------------------------------------------------ */

int64_t orc_rows_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t align) {
  return tokens * (int64_t)topk + (int64_t)num_experts * (int64_t)(align - 1);
}

int orc_route(const int32_t* topk_idx, const float* topk_prob, int64_t tokens,
              int32_t topk, int32_t num_experts, int32_t align,
              int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || align < 1) return 1;
  int64_t* counts = (int64_t*)calloc((size_t)num_experts, sizeof(int64_t));
  if (!counts) return 1;
  int64_t n_entries = tokens * topk;
  for (int64_t i = 0; i < n_entries; ++i) {
    int32_t e = topk_idx[i];
    if (e >= 0 && e < num_experts) counts[e] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < num_experts; ++e) {
    int64_t padded = (counts[e] + align - 1) / align * align;
    offsets[e + 1] = (int32_t)(offsets[e] + padded);
  }
  /* stable placement: walk entries in flattened order, fill each expert's
   * segment front to back */
  int64_t* fill = (int64_t*)calloc((size_t)num_experts, sizeof(int64_t));
  if (!fill) { free(counts); return 1; }
  for (int64_t i = 0; i < n_entries; ++i) {
    int32_t e = topk_idx[i];
    if (e < 0 || e >= num_experts) { dst_row[i] = -1; continue; }
    int64_t r = offsets[e] + fill[e];
    fill[e] += 1;
    dst_row[i] = (int32_t)r;
    row_src[r] = (int32_t)(i / topk);
    row_prob[r] = topk_prob[i];
  }
  /* padding rows */
  for (int32_t e = 0; e < num_experts; ++e) {
    for (int64_t r = offsets[e] + counts[e]; r < offsets[e + 1]; ++r) {
      row_src[r] = -1;
      row_prob[r] = 0.0f;
    }
  }
  free(fill);
  free(counts);
  return 0;
}

int orc_moe_permute(const uint16_t* x, int64_t tokens, int64_t hidden,
                    const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                    int32_t num_experts, int32_t align,
                    int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                    uint8_t* codes, uint8_t* scales, float* gscale) {
  return orc_moe_permute_rule(x, tokens, hidden, topk_idx, topk_prob, topk, num_experts, align,
                              0, offsets, dst_row, row_src, row_prob, codes, scales, gscale);
}

int orc_moe_permute_rule(const uint16_t* x, int64_t tokens, int64_t hidden,
                         const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                         int32_t num_experts, int32_t align, int rule,
                         int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                         uint8_t* codes, uint8_t* scales, float* gscale) {
  if (hidden < 0 || hidden % 16 != 0 || rule < 0 || rule > 2) return 1;
  int st = orc_route(topk_idx, topk_prob, tokens, topk, num_experts, align,
                     offsets, dst_row, row_src, row_prob);
  if (st != 0 || !x) return st;
  int64_t rows = offsets[num_experts];
  /* quantize each routed row from its source token (per-token scale: every
   * copy of a token is identical because the amax domain is the row) */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* c = codes + r * (hidden / 2);
    uint8_t* s = scales + r * (hidden / 16);
    int32_t t = row_src[r];
    if (t < 0) {
      memset(c, 0, (size_t)(hidden / 2));
      memset(s, 0, (size_t)(hidden / 16));
      gscale[r] = 0.0f;
      continue;
    }
    const uint16_t* xr = x + (int64_t)t * hidden;
    gscale[r] = orc_quantize_row_rule(xr, hidden, orc_row_amax(xr, hidden), rule, c, s);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O7: grouped GEMM                                                         */
/* ------------------------------------------------------------------------ */

static int32_t group_of_row(const int32_t* offsets, int32_t num_groups, int64_t r) {
  for (int32_t g = 0; g < num_groups; ++g)
    if (r >= offsets[g] && r < offsets[g + 1]) return g;
  return -1;
}

/* fp64 dot product of one A row with one B row, plus the absolute sum. */
static void dot_row(const double* a, const double* b, int64_t k, double* sum, double* abs_sum) {
  double s = 0.0, as = 0.0;
  for (int64_t i = 0; i < k; ++i) {
    double p = a[i] * b[i]; /* exact: each operand has <= 6 significant bits */
    s += p;
    as += fabs(p);
  }
  *sum = s;
  *abs_sum = as;
}

int orc_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                     const int32_t* offsets, int32_t num_groups, int64_t n, int64_t k,
                     float* out, double* bound) {
  if (num_groups < 0 || n < 0 || k < 0 || k % 16 != 0) return 1;
  for (int32_t g = 0; g < num_groups; ++g) {
    int64_t r0 = offsets[g], r1 = offsets[g + 1];
    if (r1 < r0) return 1;
    if (r1 == r0) continue;
    /* decode the group's B once: q_b * s_b (outer scale applied at the end) */
    double* bdec = (double*)malloc(sizeof(double) * (size_t)(n * k));
    if (!bdec) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
      orc_dequantize_row(b_codes + ((int64_t)g * n + j) * (k / 2),
                         b_scales + ((int64_t)g * n + j) * (k / 16), 1.0f, k, bdec + j * k);
    double sgb = (double)b_gscale[g];
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = r0; r < r1; ++r) {
      double* adec = (double*)malloc(sizeof(double) * (size_t)k);
      orc_dequantize_row(a_codes + r * (k / 2), a_scales + r * (k / 16), 1.0f, k, adec);
      double sga = (double)a_gscale[r];
      for (int64_t j = 0; j < n; ++j) {
        double s, as;
        dot_row(adec, bdec + j * k, k, &s, &as);
        out[r * n + j] = (float)(s * sga * sgb);
        if (bound) bound[r * n + j] = as * fabs(sga * sgb);
      }
      free(adec);
    }
    free(bdec);
  }
  return 0;
}

int orc_grouped_gemm_at(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                        const int32_t* offsets, int32_t num_groups, int64_t n, int64_t k,
                        const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out, double* bound) {
  if (num_groups < 0 || n < 0 || k < 0 || k % 16 != 0) return 1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < count; ++i) {
    int64_t r = rows[i], j = cols[i];
    int32_t g = group_of_row(offsets, num_groups, r);
    if (g < 0 || j < 0 || j >= n) {
      out[i] = 0.0f;
      if (bound) bound[i] = 0.0;
      continue;
    }
    double* adec = (double*)malloc(sizeof(double) * (size_t)k);
    double* bdec = (double*)malloc(sizeof(double) * (size_t)k);
    orc_dequantize_row(a_codes + r * (k / 2), a_scales + r * (k / 16), 1.0f, k, adec);
    orc_dequantize_row(b_codes + ((int64_t)g * n + j) * (k / 2),
                       b_scales + ((int64_t)g * n + j) * (k / 16), 1.0f, k, bdec);
    double s, as;
    dot_row(adec, bdec, k, &s, &as);
    double sc = (double)a_gscale[r] * (double)b_gscale[g];
    out[i] = (float)(s * sc);
    if (bound) bound[i] = as * fabs(sc);
    free(adec);
    free(bdec);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O8: weighted SwiGLU + row amax                                           */
/* ------------------------------------------------------------------------ */

void orc_swiglu(const float* c, const float* prob, int64_t rows, int64_t inter,
                uint16_t* d, float* amax) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float m = 0.0f;
    for (int64_t j = 0; j < inter; ++j) {
      double g = (double)c[r * 2 * inter + j];
      double u = (double)c[r * 2 * inter + inter + j];
      double silu = g / (1.0 + exp(-g));
      uint16_t h = orc_f64_to_bf16(silu * u * (double)prob[r]);
      d[r * inter + j] = h;
      float a = fabsf(orc_bf16_to_f32(h));
      if (a > m) m = a;
    }
    amax[r] = m;
  }
}

/* ------------------------------------------------------------------------ */
/* O11: combine                                                             */
/* ------------------------------------------------------------------------ */

void orc_combine(const float* y_rows, const int32_t* dst_row, int64_t tokens,
                 int32_t topk, int64_t hidden, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t h = 0; h < hidden; ++h) {
      double s = 0.0;
      for (int32_t j = 0; j < topk; ++j) {
        int32_t r = dst_row[t * topk + j];
        if (r >= 0) s += (double)y_rows[(int64_t)r * hidden + h];
      }
      y[t * hidden + h] = orc_f64_to_bf16(s);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Whole layer                                                              */
/* ------------------------------------------------------------------------ */

static double now_seconds(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

int orc_moe_forward(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                    const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                    int32_t num_experts, int32_t align,
                    const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_gscale,
                    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gscale,
                    const orc_moe_buffers* b, uint16_t* y, double* stage_seconds) {
  return orc_moe_forward_rule(x, tokens, hidden, inter, topk_idx, topk_prob, topk, num_experts,
                              align, 0, w1_codes, w1_scales, w1_gscale, w2_codes, w2_scales,
                              w2_gscale, b, y, stage_seconds);
}

int orc_moe_forward_rule(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                         const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                         int32_t num_experts, int32_t align, int act_rule,
                         const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_gscale,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gscale,
                         const orc_moe_buffers* b, uint16_t* y, double* stage_seconds) {
  if (!b || hidden % 16 != 0 || inter % 16 != 0) return 1;
  double t0 = now_seconds();
  int st = orc_moe_permute_rule(x, tokens, hidden, topk_idx, topk_prob, topk, num_experts, align,
                                act_rule, b->offsets, b->dst_row, b->row_src, b->row_prob,
                                b->a1_codes, b->a1_scales, b->a1_gscale);
  if (st) return st;
  int64_t rows = b->offsets[num_experts];
  double t1 = now_seconds();
  st = orc_grouped_gemm(b->a1_codes, b->a1_scales, b->a1_gscale, w1_codes, w1_scales, w1_gscale,
                        b->offsets, num_experts, 2 * inter, hidden, b->c_fc1, NULL);
  if (st) return st;
  double t2 = now_seconds();
  orc_swiglu(b->c_fc1, b->row_prob, rows, inter, b->d, b->amax_d);
  double t3 = now_seconds();
  /* FC2 input: requantize D with the amax produced alongside it ([miniTE] §5.3) */
  st = orc_quantize_rule(b->d, rows, inter, inter, 0, NULL, 0, b->amax_d, act_rule,
                         b->a2_codes, b->a2_scales, b->a2_gscale);
  if (st) return st;
  double t4 = now_seconds();
  st = orc_grouped_gemm(b->a2_codes, b->a2_scales, b->a2_gscale, w2_codes, w2_scales, w2_gscale,
                        b->offsets, num_experts, hidden, inter, b->y_rows, NULL);
  if (st) return st;
  double t5 = now_seconds();
  orc_combine(b->y_rows, b->dst_row, tokens, topk, hidden, y);
  double t6 = now_seconds();
  if (stage_seconds) {
    stage_seconds[0] = t1 - t0; stage_seconds[1] = t2 - t1; stage_seconds[2] = t3 - t2;
    stage_seconds[3] = t4 - t3; stage_seconds[4] = t5 - t4; stage_seconds[5] = t6 - t5;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O12: single-pass FC1 -> SwiGLU -> quantize -> FC2 ([miniTE] §5.6)         */
/* ------------------------------------------------------------------------ */

int orc_online_quantize(const uint16_t* p, int64_t rows, int64_t inter, int64_t tile,
                        uint8_t* codes, uint8_t* scales, float* gs) {
  if (rows < 0 || inter < 16 || inter % 16 != 0 || tile < 16 || tile % 16 != 0) return 1;
  const int64_t ntiles = (inter + tile - 1) / tile;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* pr = p + r * inter;
    uint8_t* cr = codes + r * (inter / 2);
    memset(cr, 0, (size_t)(inter / 2));
    float gamax = 0.0f;                               /* running row amax */
    for (int64_t i = 0; i < ntiles; ++i) {
      const int64_t c0 = i * tile, c1 = (c0 + tile < inter) ? c0 + tile : inter;
      float rowmax = orc_row_amax(pr + c0, c1 - c0);  /* max |P_i| */
      if (rowmax > gamax) gamax = rowmax;
      float s = gamax / 2688.0f;                      /* gs = gamax / 2688 */
      for (int64_t b = c0 / 16; b < c1 / 16; ++b) {
        unsigned c[16];
        scales[r * (inter / 16) + b] = (uint8_t)quantize_block(pr + b * 16, s, 6.0f, c);
        pack_block(b, c, cr);
      }
      gs[r * ntiles + i] = s;
    }
  }
  return 0;
}

int orc_single_pass_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gs,
                         int64_t tile, const uint8_t* b_codes, const uint8_t* b_scales,
                         const float* b_gscale, const int32_t* offsets, int32_t num_groups,
                         int64_t n, int64_t k, float* out, double* bound) {
  if (num_groups < 0 || n < 0 || k < 16 || k % 16 != 0 || tile < 16 || tile % 16 != 0) return 1;
  const int64_t ntiles = (k + tile - 1) / tile;
  for (int32_t g = 0; g < num_groups; ++g) {
    int64_t r0 = offsets[g], r1 = offsets[g + 1];
    if (r1 < r0) return 1;
    if (r1 == r0) continue;
    /* q_b * s_b of the group's rows (its outer scale applied at the end) */
    double* bdec = (double*)malloc(sizeof(double) * (size_t)(n * k));
    if (!bdec) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
      orc_dequantize_row(b_codes + ((int64_t)g * n + j) * (k / 2),
                         b_scales + ((int64_t)g * n + j) * (k / 16), 1.0f, k, bdec + j * k);
    const double sgw = (double)b_gscale[g];
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = r0; r < r1; ++r) {
      /* q_a * s_a: block scales included, the tiles' gs excluded */
      double* adec = (double*)malloc(sizeof(double) * (size_t)k);
      orc_dequantize_row(a_codes + r * (k / 2), a_scales + r * (k / 16), 1.0f, k, adec);
      const float* gsr = gs + r * ntiles;
      for (int64_t j = 0; j < n; ++j) {
        const double* bj = bdec + j * k;
        double o = 0.0, gs_prev = 0.0, babs = 0.0;
        for (int64_t i = 0; i < ntiles; ++i) {
          const int64_t c0 = i * tile, c1 = (c0 + tile < k) ? c0 + tile : k;
          const double gsi = (double)gsr[i];
          if (gsi == 0.0) continue;                   /* gamax = 0: contributes zero */
          double d_o = 0.0, d_abs = 0.0;
          for (int64_t kk = c0; kk < c1; ++kk) {
            double prod = adec[kk] * bj[kk];          /* exact: <= 6 significant bits each */
            d_o += prod;
            d_abs += fabs(prod);
          }
          o = o * (gs_prev / gsi) + d_o;              /* O = O * (gs_prev / gs) + dO_i */
          gs_prev = gsi;
          babs += d_abs * gsi;
        }
        out[r * n + j] = (float)(o * gs_prev * sgw);  /* Y = O * gs_prev * gs_W2 */
        if (bound) bound[r * n + j] = babs * fabs(sgw);
      }
      free(adec);
    }
    free(bdec);
  }
  return 0;
}

int orc_moe_forward_single_pass(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                                const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                                int32_t num_experts, int32_t align, int64_t tile,
                                const uint8_t* w1_codes, const uint8_t* w1_scales,
                                const float* w1_gscale, const uint8_t* w2_codes,
                                const uint8_t* w2_scales, const float* w2_gscale,
                                const orc_moe_buffers* b, float* gs_tiles, uint16_t* y,
                                double* stage_seconds) {
  if (!b || !gs_tiles || hidden % 16 != 0 || inter % 16 != 0) return 1;
  double t0 = now_seconds();
  int st = orc_moe_permute_rule(x, tokens, hidden, topk_idx, topk_prob, topk, num_experts, align,
                                0, b->offsets, b->dst_row, b->row_src, b->row_prob,
                                b->a1_codes, b->a1_scales, b->a1_gscale);
  if (st) return st;
  int64_t rows = b->offsets[num_experts];
  double t1 = now_seconds();
  st = orc_grouped_gemm(b->a1_codes, b->a1_scales, b->a1_gscale, w1_codes, w1_scales, w1_gscale,
                        b->offsets, num_experts, 2 * inter, hidden, b->c_fc1, NULL);
  if (st) return st;
  double t2 = now_seconds();
  orc_swiglu(b->c_fc1, b->row_prob, rows, inter, b->d, b->amax_d);   /* P = D */
  double t3 = now_seconds();
  st = orc_online_quantize(b->d, rows, inter, tile, b->a2_codes, b->a2_scales, gs_tiles);
  if (st) return st;
  double t4 = now_seconds();
  st = orc_single_pass_gemm(b->a2_codes, b->a2_scales, gs_tiles, tile, w2_codes, w2_scales,
                            w2_gscale, b->offsets, num_experts, hidden, inter, b->y_rows, NULL);
  if (st) return st;
  double t5 = now_seconds();
  orc_combine(b->y_rows, b->dst_row, tokens, topk, hidden, y);
  double t6 = now_seconds();
  if (stage_seconds) {
    stage_seconds[0] = t1 - t0; stage_seconds[1] = t2 - t1; stage_seconds[2] = t3 - t2;
    stage_seconds[3] = t4 - t3; stage_seconds[4] = t5 - t4; stage_seconds[5] = t6 - t5;
  }
  return 0;
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
