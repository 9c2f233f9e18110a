/*
 * nvfp4_oracle.h -- plain, slow CPU oracle for the per-token NVFP4 W4A4 MoE
 * expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library defines the expected results that
 * the HIP path is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant generator with the HIP library, and the HIP library never
 * calls it.
 *
 * Sources (cited by page title and section; the pages are
 *   [miniTE]   "miniTE Technical Report: Stable and Efficient Reinforcement
 *              Learning with Native NVFP4" (infix.io/research/miniTE)
 *   [miniTE-S] "miniTE: Diagnosing and Bridging the Execution Gap in Native
 *              NVFP4 Reinforcement Learning", source-linked summary
 *              (paperlayer.ai/abs/2610.23928v1)
 *   [TRIAGE]   "TRIAGE: Direction-Aware Mismatch Stabilization of Native NVFP4
 *              Reinforcement Learning"
 *   [4BIT]     "The 4-bitter Lesson" (humans& blog mirror)
 *
 * Arithmetic.  Quantizer decisions are taken in IEEE binary32 with
 * round-to-nearest-even, one operation at a time (build flags: -O2
 * -fno-fast-math -ffp-contract=off, x86-64 SSE, denormals preserved), because
 * [4BIT] "Four-Over-Six" describes the quantizer's scale arithmetic as scalar
 * FP32.  GEMM sums are exact-product fp64.  Every function states the reading
 * it takes where the pages are silent or garbled.
 *
 * Status codes: 0 ok, 1 invalid argument.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- O1: element and scale encodings --------------------------------- */

/* E2M1 value of a 4-bit code: bit 3 = sign, bits 2..0 index the grid
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} printed in [4BIT] "Four-Over-Six" and named in
 * [miniTE] §2.2.  Returns the signed value (−0.0 for code 8). */
double orc_e2m1_value(unsigned code);

/* Nearest E2M1 magnitude index (0..7) to |r|; ties go to the even index
 * (round-to-nearest-even on the grid); |r| >= 6 saturates to index 7 (6.0).
 * Returns the full 4-bit code with the sign bit taken from signbit(r). */
unsigned orc_e2m1_encode(float r);

/* OCP E4M3FN value of a byte (bias 7, subnormals m*2^-9, 0x7F/0xFF NaN).
 * [miniTE] §2.2 and §5.1: an E4M3 scale per block of 16 elements. */
double orc_e4m3_value(unsigned byte);

/* Nearest non-negative finite E4M3 byte (0x00..0x7E) to v >= 0, ties to the
 * even mantissa, values above the largest finite value 448 saturate to 0x7E.
 * 448 = 2688 / 6 is implied by the divisor 2688 in [miniTE] §5.6. */
unsigned orc_e4m3_encode(float v);

/* bf16 <-> binary32 / binary64 helpers (bf16 = the top 16 bits of binary32). */
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f64_to_bf16(double v);   /* round-to-nearest-even, finite inputs */

/* ---- O2-O4: NVFP4 quantization of one row ----------------------------- */

/* Quantizes k bf16 values (k % 16 == 0) given the outer-scale amax:
 *   s_g = fl32(amax / 2688)                        [miniTE] §5.6 (outer amax over 2688)
 *   per 16-element block b (along k):
 *     bmax = max |x| over the block
 *     s_b  = 0                     if s_g == 0
 *          = E4M3(fl32(bmax / fl32(6 * s_g)))       otherwise
 *     d    = fl32(s_b * s_g)                         decode x^ = q * s_b * s_g
 *     code = sign(x) | 0           if d == 0  (underflow, never NaN/Inf)
 *          = E2M1(fl32(x / d))     otherwise
 * Codes are packed two per byte, element 2j in the low nibble of byte j;
 * scales are one byte per block.  Writes k/2 code bytes, k/16 scale bytes.
 * Returns s_g. */
float orc_quantize_row_with_amax(const uint16_t* x, int64_t k, float amax,
                                 uint8_t* codes, uint8_t* scales);

/* Four-Over-Six ([4BIT] "Four-Over-Six for RL Weights and Activations"):
 * every block is quantized twice, with its maximum mapped to the E2M1 value
 * 6 and to 4, and keeps the candidate with the smaller block error; ties keep
 * 6.  rule 1 measures the error as a sum of squares, rule 2 as a sum of
 * absolute values (the page allows either).  Readings of the pages (their formula
 * names an FP8 maximum E4M3_4OVER6_MAXVAL without giving it):
 *   s_g   = fl32(amax / 1536), 1536 = 6 * 256: the FP8 maximum is lowered to
 *           256 so that the 4-candidate's block scale (1.5x the 6-candidate's,
 *           at most 384) stays inside E4M3;
 *   candidate c in {6, 4}: s_b = E4M3(fl32(bmax / fl32(c * s_g))),
 *           d = fl32(s_b * s_g), codes E2M1(fl32(x / d)) as in rule 0;
 *   error = sum over the 16 elements, in order, of e^2 (rule 1) or |e|
 *           (rule 2), e = fl32(x - fl32((q * s_b) * s_g)), in binary32 (the
 *           page's reference candidate: code value times block scale times
 *           amax over E2M1_MAXVAL * E4M3_4OVER6_MAXVAL, errors summed in
 *           FP32);
 *   the 4-candidate is kept only if its error is strictly smaller.
 * rule 0 is orc_quantize_row_with_amax.  Returns s_g. */
float orc_quantize_row_rule(const uint16_t* x, int64_t k, float amax, int rule,
                            uint8_t* codes, uint8_t* scales);

/* The outer scale of a domain with maximum amax under a rule:
 * amax / 2688 (rule 0) or amax / 1536 (rules 1, 2). */
float orc_outer_scale(float amax, int rule);

/* Row amax = max |x| over k bf16 values (exact). */
float orc_row_amax(const uint16_t* x, int64_t k);

/* Quantizes a bf16 matrix x [rows, ld_x] (first k columns used).
 *   domain 0: one outer scale per row (per-token activations:
 *             [miniTE] §2.3, §5.1; [4BIT] "Baseline recipe").
 *   domain 1: one outer scale per group of rows [off[g], off[g+1])
 *             (per-expert weights: [miniTE] §2.2 lets the recipe pick a tensor,
 *             expert or row domain; [4BIT] "Baseline recipe": one FP32 scale
 *             per weight tensor).
 *   domain 2: as domain 1, with 16x16 blocks: 16 consecutive rows of a group
 *             times 16 consecutive elements share one scale, set by the tile
 *             maximum; every group's row count must be a multiple of 16
 *             (2D weight quantization: [miniTE] §2.2, App. D2); rule 0 only.
 * amax_in (nullable): [rows] (domain 0) or [num_groups] (domain 1) amax values
 * used as given instead of the reduction ([miniTE] §5.3 amax reuse).
 * Outputs: codes [rows, k/2], scales [rows, k/16], gscale [rows] or
 * [num_groups]. */
int orc_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                 int domain, const int32_t* group_offsets, int32_t num_groups,
                 const float* amax_in,
                 uint8_t* codes, uint8_t* scales, float* gscale);
/* orc_quantize with a block rule (0 standard, 1 4/6 MSE, 2 4/6 MAE). */
int orc_quantize_rule(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                      int domain, const int32_t* group_offsets, int32_t num_groups,
                      const float* amax_in, int rule,
                      uint8_t* codes, uint8_t* scales, float* gscale);

/* O5: x^ = q * s_b * s_g in fp64 for one quantized row. */
void orc_dequantize_row(const uint8_t* codes, const uint8_t* scales, float gscale,
                        int64_t k, double* out);

/* ---- O6: routing permutation ------------------------------------------ */

/* Rows capacity: tokens*topk + num_experts*(align-1). */
int64_t orc_rows_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t align);

/* Contiguous expert-major layout with offsets ([miniTE] §5.2; [miniTE-S]
 * §4.3).  Entries (t, j) with expert id outside [0, E) are not routed
 * (dst_row = -1).  counts[e] = #entries with id e; offsets[e+1] = offsets[e]
 * + roundup(counts[e], align).  Inside an expert, rows are in ascending order
 * of the flattened entry index t*topk + j (ascending token when a token picks
 * an expert at most once).  Padding rows get row_src = -1, row_prob = 0. */
int orc_route(const int32_t* topk_idx, const float* topk_prob, int64_t tokens,
              int32_t topk, int32_t num_experts, int32_t align,
              int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob);

/* O6 + O2-O4: routing plus per-token quantization scattered to the routed rows
 * ([miniTE] §5.3: amax collected during the permutation, quantization reuses
 * it).  Each routed row r = dst_row[t, j] holds token t quantized with its own
 * row amax; padding rows hold zero codes, zero scales and s_g = 0.  Rows at or
 * beyond offsets[E] are not written.  x may be NULL (metadata only). */
int orc_moe_permute(const uint16_t* x, int64_t tokens, int64_t hidden,
                    const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                    int32_t num_experts, int32_t align,
                    int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                    uint8_t* codes, uint8_t* scales, float* gscale);
/* orc_moe_permute quantizing with a block rule (see orc_quantize_row_rule). */
int orc_moe_permute_rule(const uint16_t* x, int64_t tokens, int64_t hidden,
                         const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                         int32_t num_experts, int32_t align, int rule,
                         int32_t* offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                         uint8_t* codes, uint8_t* scales, float* gscale);

/* ---- O7: W4A4 grouped GEMM -------------------------------------------- */

/* For each group g, every row r in [off[g], off[g+1]) and every n < N:
 *   S = sum_k (q_a s_a)(q_b s_b)     exact products, fp64 accumulation
 *   out[r, n] = fl32(S * s_ga[r] * s_gb[g])   (fp64, rounded once)
 *   bound[r, n] = sum_k |a_k b_k| with fully dequantized operands.
 * A: codes [rows, K/2], scales [rows, K/16], gscale [rows].
 * B: codes [G, N, K/2], scales [G, N, K/16], gscale [G]  ("block-scaled
 * GEMM" with the FP32 outer scales applied in the epilogue: [miniTE] §5.4).
 * Rows outside [off[0], off[G]) are not written.  bound may be NULL. */
int orc_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                     const int32_t* offsets, int32_t num_groups, int64_t n, int64_t k,
                     float* out, double* bound);

/* Same definition evaluated at the listed (row, col) pairs only.  Rows that
 * fall in no group give 0. */
int orc_grouped_gemm_at(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                        const int32_t* offsets, int32_t num_groups, int64_t n, int64_t k,
                        const int64_t* rows, const int64_t* cols, int64_t count,
                        float* out, double* bound);

/* ---- O8: router-weighted SwiGLU and its row amax ---------------------- */

/* C [rows, 2I] fp32 holds the gate half then the up half ([miniTE] §5.4):
 *   D[r, j] = bf16(silu(C[r, j]) * C[r, I + j] * prob[r]),  j < I,
 * evaluated in fp64 and rounded once to bf16 ([miniTE] §5.4: the activation
 * output is weighted by the routing probability; §5.3 the weighted SwiGLU
 * output is exactly the FC2 quantizer input).  amax[r] = max_j |D[r, j]|
 * over the bf16 values. */
void orc_swiglu(const float* c, const float* prob, int64_t rows, int64_t inter,
                uint16_t* d, float* amax);

/* ---- O11: combine (unpermute) ----------------------------------------- */

/* y[t, :] = bf16(sum_j Y[dst_row[t, j], :]) in fp64, j ascending; entries
 * with dst_row < 0 contribute nothing.  The router weight is already inside
 * D, so this is a plain sum ([miniTE] §5.4). */
void orc_combine(const float* y_rows, const int32_t* dst_row, int64_t tokens,
                 int32_t topk, int64_t hidden, uint16_t* y);

/* ---- Whole layer (O6 -> O11) ------------------------------------------ */

/* Runs route + quantize-permute, FC1, SwiGLU, requantize (amax reuse), FC2
 * and combine with the definitions above.  Intermediates are written to the
 * non-NULL pointers in `inter_out` order:
 *   a1 codes/scales/gscale, C fp32 [R_cap, 2I], D bf16 [R_cap, I], amaxD,
 *   a2 codes/scales/gscale, Y fp32 [R_cap, H].
 * Weights are pre-quantized NVFP4 (per-expert outer scales).  Returns the
 * wall time of each stage in seconds in stage_seconds[6] when non-NULL:
 * route+quantize, FC1, SwiGLU, requantize, FC2, combine. */
typedef struct {
  uint8_t* a1_codes; uint8_t* a1_scales; float* a1_gscale;
  float* c_fc1; uint16_t* d; float* amax_d;
  uint8_t* a2_codes; uint8_t* a2_scales; float* a2_gscale;
  float* y_rows;
  int32_t* offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
} orc_moe_buffers;

int orc_moe_forward(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                    const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                    int32_t num_experts, int32_t align,
                    const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_gscale,
                    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gscale,
                    const orc_moe_buffers* buf, uint16_t* y, double* stage_seconds);
/* orc_moe_forward with a block rule for both activation quantizations (the
 * routed tokens and the requantized D); the weights come pre-quantized. */
int orc_moe_forward_rule(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                         const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                         int32_t num_experts, int32_t align, int act_rule,
                         const uint8_t* w1_codes, const uint8_t* w1_scales, const float* w1_gscale,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gscale,
                         const orc_moe_buffers* buf, uint16_t* y, double* stage_seconds);

/* ---- O12: single-pass FC1 -> SwiGLU -> quantize -> FC2 ---------------- */
/* [miniTE] §5.6 "Exploring Single-Pass Fusion": FC2 consumes the activation
 * in K-tiles before the row's full amax is known.  A running row amax over
 * the tiles seen so far sets each tile's outer scale, and the FC2 partial
 * sum is converted to the new scale whenever that scale grows.  The codes
 * therefore differ from the two-pass quantization by design.
 *
 * Readings (the page gives the steps, not the sizes):
 *   - the activation tile P_i is the weighted SwiGLU of O8 rounded to bf16,
 *     i.e. columns [i*tile, min((i+1)*tile, inter)) of the two-pass D, so
 *     that a row whose maximum lies in its first tile quantizes exactly as
 *     in the two-pass path;
 *   - gs_i = fl32(gamax_i / 2688) with gamax_i = max(|P_0..P_i|), and the
 *     tile's blocks are encoded by O3/O4 with s_g = gs_i;
 *   - "If gamax = 0 ... skip": a tile with gs_i == 0 adds nothing (its
 *     scales are 0 and its codes carry only the sign, as O4 gives);
 *   - tile (the K-tile width) is a parameter, a multiple of 16; the last
 *     tile may be narrower. */

/* O12a: per row of P (bf16 [rows, inter]), tile by tile in ascending order:
 * gamax = max(gamax, max|P_i|), gs_i = gamax / 2688, then E4M3 scales and
 * E2M1 codes of the tile's 16-blocks with s_g = gs_i.  codes [rows,
 * inter/2], scales [rows, inter/16], gs [rows, ntiles] with ntiles =
 * ceil(inter / tile).  Status 1 on bad sizes. */
int orc_online_quantize(const uint16_t* p, int64_t rows, int64_t inter, int64_t tile,
                        uint8_t* codes, uint8_t* scales, float* gs);

/* O12b: the FC2 of online-quantized rows.  For row r of group g and column
 * n, with O = 0 and gs_prev = 0, for every tile i with gs_i > 0 in order:
 *   dO_i = sum over the tile's k of (q_a s_a)[r, k] (q_b s_b)[g, n, k]
 *          (exact fp64: block scales included, gs excluded),
 *   O = O * (gs_prev / gs_i) + dO_i,  gs_prev = gs_i;
 * then out[r, n] = fl32(O * gs_prev * s_gb[g]) (0 when every gs_i is 0).
 * bound (nullable) = sum_k |a_k b_k| over the fully dequantized operands
 * (a_k scaled by the gs of its tile).  Rows outside the groups untouched. */
int orc_single_pass_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* gs,
                         int64_t tile, const uint8_t* b_codes, const uint8_t* b_scales,
                         const float* b_gscale, const int32_t* offsets, int32_t num_groups,
                         int64_t n, int64_t k, float* out, double* bound);

/* The whole layer with O12 in place of O9 + O10: route + quantize-permute,
 * FC1, SwiGLU (D = P), online quantize, single-pass FC2, combine.  Buffers
 * as orc_moe_forward (a2_gscale and amax_d unused) plus gs_tiles
 * [R_cap, ceil(inter / tile)]; stage_seconds as orc_moe_forward (the
 * requantize stage is the online quantize). */
int orc_moe_forward_single_pass(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                                const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                                int32_t num_experts, int32_t align, int64_t tile,
                                const uint8_t* w1_codes, const uint8_t* w1_scales,
                                const float* w1_gscale, const uint8_t* w2_codes,
                                const uint8_t* w2_scales, const float* w2_gscale,
                                const orc_moe_buffers* buf, float* gs_tiles, uint16_t* y,
                                double* stage_seconds);

/* Sets the number of OpenMP threads of the following calls (n > 0); the
 * arithmetic and its order do not depend on it. */
void orc_set_num_threads(int n);

/* Number of OpenMP threads the oracle uses (1 when built without OpenMP). */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
