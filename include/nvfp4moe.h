/*
 * nvfp4moe.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 MoE expert path.
 *
 * The path: per-token NVFP4 quantization of activations fused with the MoE
 * routing permutation, a W4A4 grouped GEMM over every expert's FC1 (gate|up)
 * and FC2 (down) projections, and a router-weighted SwiGLU whose bf16 output
 * and row amax feed the FC2 requantization.
 *
 * Sources, cited by page title and section:
 *   [miniTE]   "miniTE Technical Report: Stable and Efficient Reinforcement
 *              Learning with Native NVFP4"
 *   [miniTE-S] "miniTE: Diagnosing and Bridging the Execution Gap in Native
 *              NVFP4 Reinforcement Learning" (source-linked summary)
 *   [4BIT]     "The 4-bitter Lesson"
 *
 * NVFP4 format ([miniTE] §2.2, §5.1; [4BIT] "Baseline recipe",
 * "Four-Over-Six"): a value is x^ = q * s_b * s_g with q an E2M1 code on the
 * grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (bit 3 = sign), s_b an OCP E4M3 scale
 * shared by 16 consecutive elements along K, and s_g an FP32 outer scale:
 * one per token (row) for activations, one per expert matrix for weights.
 * Quantization (bit-exact contract):
 *   s_g  = fl32(amax / 2688)                               ([miniTE] §5.6)
 *   s_b  = E4M3_rne_satfinite(fl32(bmax / fl32(6 * s_g))), 0 when s_g == 0
 *   d    = fl32(s_b * s_g); code = sign(x) | E2M1_rne_satfinite(fl32(x / d)),
 *          magnitude 0 when d == 0
 * with IEEE binary32 round-to-nearest-even at every step.
 *
 * Layouts (all row-major, K contiguous):
 *   codes        uint8 [rows, k/2]   element 2j in the low nibble of byte j
 *   block_scales uint8 [rows, k/16]  E4M3 bytes (bias 7, max 0x7E = 448)
 *   global scale float [rows] (per row) or [groups] (per group)
 *   bf16 tensors travel as uint16_t bit patterns.
 * Weight matrices are [G, N, K] (one [N, K] matrix per expert, K contiguous):
 *   codes [G, N, K/2], block scales [G, N, K/16], outer scales [G].
 *
 * Ownership and execution: every pointer argument is a DEVICE pointer unless
 * stated otherwise, owned by the caller; the library allocates no device or
 * host memory on these calls.  All calls are asynchronous on `stream`
 * (a hipStream_t passed as void*, NULL = the null stream): the host returns
 * after enqueueing the kernels, with no host<->device synchronisation, and
 * nothing is read back to the host.  Calls that share a workspace must be
 * ordered by the caller.  No C++ exception crosses this interface.
 *
 * Errors: arguments are validated on the host before any HIP call; a failed
 * check returns NVFP4_INVALID_ARGUMENT (or NVFP4_UNSUPPORTED for shapes the
 * kernels do not handle) and enqueues nothing.  Launch failures return
 * NVFP4_HIP_ERROR.  Data-dependent preconditions (finite inputs, expert ids
 * of one token distinct) are the caller's contract; expert ids outside
 * [0, num_experts) are legal and mean "not routed".  A library built with
 * NVFP4_DEBUG_CHECKS defined (libnvfp4moe_debug.so) checks them on the device
 * in moe_permute and moe_expert_forward and reports what it found in the
 * precondition word (below); a violated precondition never faults, in either
 * build, it only makes the affected outputs meaningless.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK 0
#define NVFP4_INVALID_ARGUMENT 1
#define NVFP4_UNSUPPORTED 2
#define NVFP4_HIP_ERROR 3
#define NVFP4_WORKSPACE_TOO_SMALL 4
#define NVFP4_SCRATCH_LIMIT 5

/* Block rules of the quantizer (see nvfp4_quantize). */
#define NVFP4_BLOCK_RULE_SIX 0
#define NVFP4_BLOCK_RULE_4OVER6_MSE 1
#define NVFP4_BLOCK_RULE_4OVER6_MAE 2

/* Human-readable name of a status code (static storage, never NULL). */
const char* nvfp4_status_string(int status);

/* ------------------------------------------------------------------------
 * Precondition word (debug build).  [miniTE] §4.5 (strict layout checks and
 * a deterministic mode to make failures attributable).
 * The first uint32 (byte offset 0) of the workspace of moe_permute and of
 * moe_expert_forward is reserved in every build.  In a build with
 * NVFP4_DEBUG_CHECKS, each call clears it on its stream before its first
 * kernel and its routing kernels OR into it:
 *   NVFP4_PRECONDITION_DUPLICATE_EXPERT  a token names one expert id in
 *                                        [0, num_experts) more than once
 *   NVFP4_PRECONDITION_NONFINITE_INPUT   an activation x is Inf or NaN
 *   NVFP4_PRECONDITION_NONFINITE_PROB    a router weight is Inf or NaN
 * The word is valid once the call's work on the stream has completed; the
 * caller reads it with an ordinary device-to-host copy.  Outputs for clean
 * inputs are bit-identical to the release build's.  In the release build the
 * word is left untouched.
 * nvfp4_debug_checks() returns 1 in a build with NVFP4_DEBUG_CHECKS, else 0.
 * ---------------------------------------------------------------------- */
#define NVFP4_PRECONDITION_DUPLICATE_EXPERT 0x1u
#define NVFP4_PRECONDITION_NONFINITE_INPUT 0x2u
#define NVFP4_PRECONDITION_NONFINITE_PROB 0x4u
int nvfp4_debug_checks(void);

/* ------------------------------------------------------------------------
 * nvfp4_quantize -- NVFP4 quantization of a bf16 matrix.
 * [miniTE] §2.2 (two-level scaling; the recipe chooses the outer-scale
 * domain), §5.1 (per-token outer scale), §5.3 (amax reuse); [4BIT] "Baseline
 * recipe" (per-token activation scale, one FP32 scale per weight tensor).
 *
 *   x            bf16 [rows, ld_x], first k columns used; k % 16 == 0,
 *                ld_x >= k, ld_x % 8 == 0, 16-byte aligned
 *   scale_domain 0: one outer scale per row (activations);
 *                1: one outer scale per group of rows
 *                   [group_offsets[g], group_offsets[g+1]) (expert weights;
 *                   one group over all rows is the per-tensor scale);
 *                2: as 1, with 16x16 two-dimensional blocks ([miniTE] §2.2,
 *                   App. D2 "2D weight quantization"): 16 consecutive rows
 *                   of a group and 16 consecutive elements share one E4M3
 *                   scale set by the tile maximum, stored in each of the
 *                   tile's rows (block_scales keeps its [rows, k/16] shape,
 *                   so the GEMM reads it unchanged).  rows % 16 == 0 and
 *                   block_rule 0, else NVFP4_UNSUPPORTED; every group's row
 *                   count must be a multiple of 16 (caller contract).
 *   group_offsets int32 [num_groups + 1], non-decreasing, within [0, rows]
 *                (domain 1 only; device pointer)
 *   amax_in      nullable float [rows] (domain 0) or [num_groups] (domain 1):
 *                use these amax values instead of reducing |x|
 *   block_rule   NVFP4_BLOCK_RULE_*: 0 maps every block maximum to the E2M1
 *                value 6 (s_g = amax / 2688); 1 and 2 are Four-Over-Six
 *                ([4BIT] "Four-Over-Six for RL Weights and Activations"):
 *                s_g = amax / 1536 (the FP8 maximum of this mode read as 256,
 *                so a block mapped to 4 keeps a finite E4M3 scale), and each
 *                block keeps the candidate with its maximum mapped to 4 only
 *                where that lowers the block error: 1 = sum of squares, 2 =
 *                sum of absolute values of x - q*s_b*s_g, in binary32 over
 *                the 16 elements in order; ties keep 6.
 *   codes        out uint8 [rows, k/2];  block_scales out uint8 [rows, k/16]
 *   global_scales out float [rows] (domain 0) or [num_groups] (domain 1);
 *                in domain 1 without amax_in it also serves as the scratch
 *                for the group amax reduction (no other memory is used).
 * Limits: 1 <= k <= 16384; rows, num_groups < 2^31.
 * ---------------------------------------------------------------------- */
int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                   int scale_domain, const int32_t* group_offsets, int32_t num_groups,
                   const float* amax_in, int block_rule,
                   uint8_t* codes, uint8_t* block_scales, float* global_scales,
                   void* stream);

/* ------------------------------------------------------------------------
 * MoE routing permutation fused with per-token quantization.
 * [miniTE] §5.2 (contiguous buffers with expert offsets, device-side metadata,
 * zero-token experts and padding in the same grouped path), §5.3 (row amax
 * collected during the permutation and reused by the quantizer);
 * [miniTE-S] §4.3.
 *
 * Layout of the routed rows: expert-major; expert e owns rows
 * [expert_offsets[e], expert_offsets[e+1]) whose length is its entry count
 * rounded up to `align`.  Inside an expert, rows follow ascending flattened
 * entry index t*topk + j (ascending token).  Row r of entry (t, j) holds
 * token t quantized with its own per-token scale; dst_row[t*topk + j] = r,
 * row_src[r] = t, row_prob[r] = topk_prob[t*topk + j].  Padding rows have
 * row_src = -1, row_prob = 0, zero codes, zero scales and s_g = 0.  Entries
 * with an expert id outside [0, num_experts) get dst_row = -1.  Rows at or
 * beyond expert_offsets[num_experts] are not written.
 *
 *   x            nullable bf16 [tokens, hidden]: NULL computes the metadata only
 *   topk_idx     int32 [tokens, topk];  topk_prob float [tokens, topk]
 *   align        power of two in [1, 256]
 *   block_rule   the quantizer's block rule (see nvfp4_quantize)
 *   expert_offsets out int32 [num_experts + 1]
 *   dst_row      out int32 [tokens, topk]
 *   row_src, row_prob  out [moe_rows_capacity(...)]
 *   codes, block_scales, global_scales  out [capacity, hidden/2],
 *                [capacity, hidden/16], [capacity] (unused when x is NULL)
 *   workspace    device scratch of moe_permute_workspace_size() bytes,
 *                16-byte aligned; its first uint32 is the precondition word
 * Limits: 1 <= topk <= num_experts <= 1024; hidden % 16 == 0,
 * hidden <= 16384; tokens * topk + num_experts * align < 2^31.
 * ---------------------------------------------------------------------- */
int64_t moe_rows_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t align);
size_t moe_permute_workspace_size(int64_t tokens, int32_t topk, int32_t num_experts);
int moe_permute(const uint16_t* x, int64_t tokens, int64_t hidden,
                const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                int32_t num_experts, int32_t align, int32_t block_rule,
                int32_t* expert_offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                uint8_t* codes, uint8_t* block_scales, float* global_scales,
                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs and results as moe_permute,
 * without the workspace: the routing scratch is a static device array of
 * NVFP4_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up on the first call on a
 * device).  The call allocates nothing, host or device.  The caller still
 * passes every input and output buffer.
 *   Limit: moe_permute_workspace_size(tokens, topk, num_experts) <=
 *   NVFP4_NOALLOC_SCRATCH_BYTES (e.g. 128 experts up to 261,000 tokens, 1024
 *   experts up to 32,700 tokens), else NVFP4_SCRATCH_LIMIT before any HIP
 *   call.
 *   All calls on one GPU share that GPU's array: calls that overlap on one
 *   GPU (different streams, or threads without ordering) race and give
 *   undefined results.  Calls ordered on one stream are safe; nothing from
 *   an earlier call is read.  In a build with NVFP4_DEBUG_CHECKS the
 *   precondition word is written to the array, out of the caller's reach.
 * ---------------------------------------------------------------------- */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int moe_permute_noalloc(const uint16_t* x, int64_t tokens, int64_t hidden,
                        const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                        int32_t num_experts, int32_t align, int32_t block_rule,
                        int32_t* expert_offsets, int32_t* dst_row, int32_t* row_src,
                        float* row_prob, uint8_t* codes, uint8_t* block_scales,
                        float* global_scales, void* stream);

/* ------------------------------------------------------------------------
 * w4a4_grouped_gemm -- one grouped call over all experts.
 * [miniTE] §5.2 (dense grouped GEMM fed by contiguous buffers and device
 * offsets), §5.4 (block-scaled GEMM; ACC * alpha_a[m] * alpha_b in an FP32
 * epilogue); [miniTE-S] §4.2 (FP32 epilogue rescaling).
 *
 * For each group g and row r in [group_offsets[g], group_offsets[g+1]):
 *   out[r, n] = s_ga[r] * s_gb[g] * sum_k (q_a s_a)[r, k] * (q_b s_b)[g, n, k]
 * Operands are decoded exactly to fp16 (q * s_b has at most 6 significant
 * bits), multiplied on the fp16 matrix cores and accumulated in fp32.
 * Accuracy: |out - exact| <= 2^-10 * sum_k |a_k b_k| + 1e-6 (fp32 output).
 *
 *   a_*          A rows: codes [rows_cap, k/2], scales [rows_cap, k/16],
 *                outer scales [rows_cap]
 *   b_*          B: codes [G, n, k/2], scales [G, n, k/16], outer scales [G]
 *   b_layout     0: B codes and scales row-major as above; 1: the same bytes
 *                rearranged by nvfp4_pack_weights (faster loads)
 *   group_offsets int32 [num_groups + 1] on the device, non-decreasing,
 *                group_offsets[0] >= 0, group_offsets[G] <= rows_cap; empty
 *                groups are legal; the host never reads it
 *   out_dtype    0: float32, 1: bf16 (round-to-nearest-even)
 *   out          [rows_cap, n], 16-byte aligned; rows outside [off[0], off[G])
 *                are not written
 * Limits: k % 128 == 0, k <= 16384; n % 32 == 0; 1 <= num_groups <= 1024;
 * one group's B codes (n * k / 2 bytes) below 4 GiB (NVFP4_UNSUPPORTED).
 * ---------------------------------------------------------------------- */
int w4a4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                      int64_t rows_cap,
                      const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                      const int32_t* group_offsets, int32_t num_groups, int64_t n, int64_t k,
                      int b_layout, int out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * w4a4_grouped_gemm_swiglu -- FC1 with the fused router-weighted SwiGLU
 * epilogue and the row amax of its output.
 * [miniTE] §5.3 (weighted SwiGLU with row amax: the statistic of exactly the
 * tensor FC2 quantizes), §5.4 (the pre-activation output is the gate half
 * followed by the up half; the activation output is weighted by the routing
 * probability; its amax is reduced in the same epilogue).
 *
 * B holds the fused [G, 2*inter, k] gate|up weights (gate = rows [0, inter)).
 * For every routed row r and j < inter, with C the grouped GEMM above:
 *   D[r, j]  = bf16(silu(C[r, j]) * C[r, inter + j] * row_prob[r])
 *   amax[r]  = max_j |D[r, j]|   (over the bf16 values; bit-exact)
 *   c_out    nullable float [rows_cap, 2*inter]: also store C
 * amax must be zero-filled by the caller for the rows of the call (the
 * kernel takes an order-independent maximum into it).
 * Limits: as w4a4_grouped_gemm, with inter % 64 == 0.
 * ---------------------------------------------------------------------- */
int w4a4_grouped_gemm_swiglu(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             int64_t rows_cap,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_gscale,
                             const int32_t* group_offsets, int32_t num_groups, int64_t inter,
                             int64_t k, int b_layout, const float* row_prob,
                             uint16_t* d_out, float* amax, float* c_out, void* stream);

/* ------------------------------------------------------------------------
 * nvfp4_pack_weights -- scale-layout transfer for static weights: rearranges
 * row-major NVFP4 B (codes [G, n, k/2], scales [G, n, k/16]) into the tiled
 * layout the grouped GEMM reads with whole-wavefront contiguous loads
 * (b_layout 1).  [miniTE] §5.4 (scale-layout transfer ahead of the GEMM).
 * A pure byte permutation into buffers of the same sizes (outer scales are
 * unchanged).  Tile t = (g*(n/32) + rb)*(k/128) + st covers rows
 * 32rb..32rb+31 of group g and K stage st (128 elements):
 *   packed_codes[t*2048 + c*1024 + 16*L + i]
 *       = codes[g, 32rb + L%32, 64st + 32(L/32) + 16c + i]   c < 2, L < 64, i < 16
 *   packed_scales[t*256 + 4*L + i]
 *       = scales[g, 32rb + L%32, 8st + 4(L/32) + i]           L < 64, i < 4
 * Outputs must not overlap the inputs.  Limits: n % 32 == 0, k % 128 == 0,
 * k <= 16384.
 * ---------------------------------------------------------------------- */
int nvfp4_pack_weights(const uint8_t* codes, const uint8_t* scales, int32_t num_groups,
                       int64_t n, int64_t k, uint8_t* packed_codes, uint8_t* packed_scales,
                       void* stream);

/* ------------------------------------------------------------------------
 * moe_combine -- unpermute: y[t, :] = bf16(sum_j Y[dst_row[t, j], :]) with a
 * fixed j order and fp32 accumulation; entries with dst_row < 0 add nothing.
 * The router weight is already inside D ([miniTE] §5.4), so this is a plain
 * sum.  y_rows_dtype 0: float32 rows, 1: bf16 rows.  hidden % 8 == 0.
 * ---------------------------------------------------------------------- */
int moe_combine(const void* y_rows, int y_rows_dtype, const int32_t* dst_row,
                int64_t tokens, int32_t topk, int64_t hidden, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_forward -- the whole expert layer in one call:
 *   routing + per-token quantization -> FC1 grouped GEMM + SwiGLU + amax ->
 *   requantize D with that amax -> FC2 grouped GEMM -> moe_combine.
 * [miniTE] §5.2-§5.4 (the fused FC1 and FC2 flows).
 * The routed rows equal moe_permute's bit for bit, but the layer does not
 * write them: each token is quantized once into a token-major row and FC1
 * reads routed row r from token row_src[r] (the permutation is applied by
 * the GEMM's operand loads).
 *
 *   x            bf16 [tokens, hidden];  y out bf16 [tokens, hidden]
 *   w1           NVFP4 gate|up weights [E, 2*inter, hidden] (+ scales, [E])
 *   act_block_rule  block rule of both activation quantizations (the routed
 *                tokens and the requantized D); the weights carry whatever
 *                rule they were quantized with ([4BIT] "Four-Over-Six ...":
 *                weights, activations or both)
 *   act_scale_domain  outer scale of both activation quantizations
 *                ([miniTE] §2.3, §5.1): 0 = one per token / routed row (the
 *                per-token recipe); 1 = one per tensor: x quantized with
 *                s_g = amax(x) / 2688 for every token (nvfp4_quantize domain 1
 *                with one group), D with the maximum of amax_d over the routed
 *                rows; a1_gscale and a2_gscale then hold that value per row
 *   w2           NVFP4 down weights    [E, hidden, inter]
 *                (each row-major or tiled, per its layout member)
 *   workspace    moe_expert_forward_workspace_size() bytes, 256-byte aligned;
 *                its first uint32 is the precondition word
 *   debug        nullable: every non-NULL member receives that intermediate
 *                (in place of the workspace copy); fc1_out, y_rows_f32,
 *                a1_codes and a1_scales are only produced when requested
 *                (y_rows_f32 switches the FC2 output to fp32; a1_codes and
 *                a1_scales, given together, receive the permuted routed
 *                rows of moe_permute's layout, copied from the token rows)
 *   stage_events nullable array of 6 hipEvent_t (as void*), recorded on
 *                `stream` before route, FC1, requantize, FC2, combine and
 *                after combine (profiling; see nvfp4_event_*).
 * Limits: hidden % 128 == 0, inter % 128 == 0, hidden, inter <= 16384,
 * (tokens + 1) * hidden / 2 < 2^32, plus the limits of moe_permute.
 * ---------------------------------------------------------------------- */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  int32_t layout;                 /* b_layout of w4a4_grouped_gemm: 0 or 1 */
} nvfp4_weights;

typedef struct {
  int32_t* expert_offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
  uint8_t* a1_codes; uint8_t* a1_scales; float* a1_gscale;
  float* fc1_out;                 /* [cap, 2*inter] fp32, optional */
  uint16_t* d;                    /* [cap, inter] bf16 */
  float* amax_d;                  /* [cap] */
  uint8_t* a2_codes; uint8_t* a2_scales; float* a2_gscale;
  uint16_t* y_rows;               /* [cap, hidden] bf16 FC2 output */
  float* y_rows_f32;              /* [cap, hidden] fp32 FC2 output, optional */
} nvfp4_moe_intermediates;

size_t moe_expert_forward_workspace_size(int64_t tokens, int64_t hidden, int64_t inter,
                                         int32_t topk, int32_t num_experts, int32_t align);
int moe_expert_forward(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                       const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                       int32_t num_experts, int32_t align, int32_t act_block_rule,
                       int32_t act_scale_domain,
                       const nvfp4_weights* w1, const nvfp4_weights* w2, uint16_t* y,
                       void* workspace, size_t workspace_bytes,
                       const nvfp4_moe_intermediates* debug, void* const* stage_events,
                       void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_forward_single_pass -- the expert layer with FC1 -> weighted
 * SwiGLU -> NVFP4 quantize -> FC2 fused into one kernel by online amax
 * compensation ([miniTE] §5.6 "Exploring Single-Pass Fusion").  The
 * intermediate activation and its quantization never leave the chip.
 *
 * Routing, the per-token quantization and FC1 are those of
 * moe_expert_forward.  Per routed row r, the intermediate dimension is taken
 * in tiles of 256 columns, i = 0, 1, ... (the last may be narrower):
 *   P_i     = bf16(silu(gate) * up * row_prob[r]) of the tile's columns,
 *   gamax_i = max(gamax_{i-1}, max |P_i|), gamax_{-1} = 0,
 *   gs_i    = fl32(gamax_i / 2688),
 *   the tile's 16-blocks encoded as in nvfp4_quantize with s_g = gs_i,
 *   O       = O * (gs_{i-1} / gs_i) + sum over the tile's k of
 *             (q_a s_a)(q_w s_w)   (tiles with gs_i = 0 add nothing),
 *   Y[r, n] = O * gs_last * s_gw2[e], then the combine.
 * A row whose maximum lies in its first tile quantizes exactly as in the
 * two-pass layer; other rows' earlier tiles use smaller scales, so their
 * codes differ from the two-pass codes by design.
 *
 *   arguments as moe_expert_forward (act_block_rule: the standard rule only)
 *   debug        nullable: every non-NULL member receives that intermediate
 *                (valid rows only); y_rows_f32 switches the FC2 rows to fp32;
 *                a1_codes and a1_scales are given together
 *   stage_events nullable array of 4 hipEvent_t (as void*), recorded before
 *                the routing, before the fused kernel, before the combine and
 *                after it
 * Limits: as moe_expert_forward, and inter <= 1152 (the row block's
 * quantized FC2 input, 128 rows x inter * 9/16 bytes, is held on chip beside
 * the 64 KiB of operand stages).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t* expert_offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
  uint8_t* a1_codes; uint8_t* a1_scales; float* a1_gscale;
  float* fc1_out;                 /* [cap, 2*inter] fp32 FC1 pre-activation */
  uint16_t* p;                    /* [cap, inter] bf16 weighted SwiGLU (the tiles P_i) */
  uint8_t* a2_codes;              /* [cap, inter/2] the online-quantized FC2 input */
  uint8_t* a2_scales;             /* [cap, inter/16] */
  float* gs_tiles;                /* [cap, ceil(inter/256)] gs_i per row and tile */
  uint16_t* y_rows;               /* [cap, hidden] bf16 FC2 rows */
  float* y_rows_f32;              /* [cap, hidden] fp32 FC2 rows */
} nvfp4_single_pass_intermediates;

size_t moe_expert_forward_single_pass_workspace_size(int64_t tokens, int64_t hidden,
                                                     int64_t inter, int32_t topk,
                                                     int32_t num_experts, int32_t align);
int moe_expert_forward_single_pass(const uint16_t* x, int64_t tokens, int64_t hidden,
                                   int64_t inter, const int32_t* topk_idx,
                                   const float* topk_prob, int32_t topk, int32_t num_experts,
                                   int32_t align, const nvfp4_weights* w1,
                                   const nvfp4_weights* w2, uint16_t* y, void* workspace,
                                   size_t workspace_bytes,
                                   const nvfp4_single_pass_intermediates* debug,
                                   void* const* stage_events, void* stream);

/* ------------------------------------------------------------------------
 * moe_expert_backward -- gradients of the expert layer under the
 * straight-through approximation: the forward's quantizers count as the
 * identity and every gradient is a BF16 GEMM (bf16 operands, fp32
 * accumulation) on BF16 operands.  [miniTE] §4.2 (the default learning path
 * saves the original BF16 activations and weights and skips backward
 * quantization); [4BIT] "Improving Gradient Stability" (the same GEMMs on
 * the dequantized operands: pass bf16 DQ(Q(.)) as x, d, w1, w2).
 *
 * With routed row r of expert e (rows [expert_offsets[e],
 * expert_offsets[e+1])), token t = row_src[r], p = row_prob[r], and the
 * forward's FC1 output C[r] = [g | u] (gate columns [0, inter)):
 *   dYr[r] = dy[t]                          (0 for padding rows, t < 0)
 *   dD[r]  = bf16(dYr[r] . W2[e])
 *   dC[r]  = bf16([dD u p silu'(g) | dD silu(g) p]),  silu(g) = g sigmoid(g),
 *            silu'(g) = s (1 + g (1 - s)), s = sigmoid(g), in fp32 from the
 *            bf16 dD; 0 for padding rows
 *   dp[r]  = sum over i of dD[r, i] silu(g_i) u_i          (fp32)
 *   dXr[r] = bf16(dC[r] . W1[e])
 *   dx[t]  = bf16(sum over j of dXr[dst_row[t, j]])   (j ascending, fp32 sums)
 *   dW2[e] = sum over e's rows of dYr[r]^T d[r]        fp32 [E, hidden, inter]
 *   dW1[e] = sum over e's rows of dC[r]^T x[t]         fp32 [E, 2*inter, hidden]
 *   dprob[t, j] = dp[dst_row[t, j]]  (0 for entries not routed)
 * The GEMMs accumulate in fp32 in an order of their own, the same on every
 * call; dp sums in a fixed order (all outputs are bitwise reproducible).
 *
 *   dy       bf16 [tokens, hidden]   the gradient of y
 *   x        bf16 [tokens, hidden]   FC1's input operand
 *   rows_cap capacity of the routed-row arrays (moe_rows_capacity of the
 *            forward's call); expert_offsets[num_experts] <= rows_cap
 *   fc1_out  fp32 [rows_cap, 2*inter]  the forward's FC1 output C
 *            (nvfp4_moe_intermediates.fc1_out)
 *   d        bf16 [rows_cap, inter]  FC2's input operand (the forward's D;
 *            its padding rows must be finite, the forward writes zeros)
 *   expert_offsets [num_experts+1], row_src, row_prob [rows_cap],
 *   dst_row [tokens, topk]: the forward's routing (nvfp4_moe_intermediates)
 *   w1       bf16 [E, 2*inter, hidden];  w2 bf16 [E, hidden, inter]
 *   dx       out bf16 [tokens, hidden];  dprob out fp32 [tokens, topk]
 *   dw1, dw2 out fp32, every expert written (zeros for experts with no rows)
 *   workspace moe_expert_backward_workspace_size() bytes, 256-byte aligned
 *   debug    nullable: dd, dc, dp_rows and dx_rows replace the workspace
 *            copies; dx_rows_f32 (fp32 [rows_cap, hidden], the FC1 dgrad
 *            before its bf16 rounding) is only written when given
 *   stage_events nullable array of 8 hipEvent_t (as void*), recorded before
 *            the tile tables, FC2 dgrad, the SwiGLU backward, FC1 dgrad, the
 *            dx / dprob reductions, FC2 wgrad, FC1 wgrad and after them (the
 *            order the stages run in)
 * bf16 arrays, fc1_out, dw1, dw2 and dx_rows_f32 16-byte aligned, the others
 * 4-byte aligned; rows are read only inside [0, expert_offsets[num_experts]).
 * Limits: hidden % 128 == 0, inter % 128 == 0, hidden, inter <= 16384,
 * num_experts <= 1024, rows_cap < 2^31, and below 2^31 bytes each: dy (and
 * x), fc1_out, one expert's w1 (NVFP4_UNSUPPORTED otherwise).
 * Errors: NVFP4_INVALID_ARGUMENT / NVFP4_UNSUPPORTED before any HIP call;
 * NVFP4_WORKSPACE_TOO_SMALL; NVFP4_HIP_ERROR if a launch fails.
 * ---------------------------------------------------------------------- */
typedef struct {
  uint16_t* dd;                   /* [rows_cap, inter] bf16 FC2 dgrad */
  uint16_t* dc;                   /* [rows_cap, 2*inter] bf16 SwiGLU input gradient */
  float* dp_rows;                 /* [rows_cap] router-weight gradient of each row */
  uint16_t* dx_rows;              /* [rows_cap, hidden] bf16 FC1 dgrad rows */
  float* dx_rows_f32;             /* [rows_cap, hidden] fp32 FC1 dgrad rows */
} nvfp4_moe_backward_intermediates;

size_t moe_expert_backward_workspace_size(int64_t rows_cap, int64_t hidden, int64_t inter,
                                          int32_t num_experts);
int moe_expert_backward(const uint16_t* dy, const uint16_t* x, int64_t tokens, int64_t hidden,
                        int64_t inter, int32_t topk, int32_t num_experts, int64_t rows_cap,
                        const float* fc1_out, const uint16_t* d, const int32_t* expert_offsets,
                        const int32_t* row_src, const float* row_prob, const int32_t* dst_row,
                        const uint16_t* w1, const uint16_t* w2, uint16_t* dx, float* dw1,
                        float* dw2, float* dprob, void* workspace, size_t workspace_bytes,
                        const nvfp4_moe_backward_intermediates* debug,
                        void* const* stage_events, void* stream);

/* ------------------------------------------------------------------------
 * Profiling helpers: thin wrappers over hipEventCreate / hipEventRecord /
 * hipEventElapsedTime / hipEventDestroy so a caller without HIP headers can
 * time the stages of moe_expert_forward on its stream.  (These allocate a
 * HIP event; they are not on the hot path.)
 * ---------------------------------------------------------------------- */
int nvfp4_event_create(void** event);
int nvfp4_event_record(void* event, void* stream);
int nvfp4_event_elapsed_ms(void* start, void* stop, float* ms);
int nvfp4_event_destroy(void* event);

#ifdef __cplusplus
}
#endif
#endif
