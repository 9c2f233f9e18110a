// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/nvfp4moe.h).  Every launcher
// enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "nvfp4moe.h"
#include "tile_schedule.h"

namespace nvfp4 {

// Blocks (16 elements) per lane needed for a row of k elements, rounded up to
// a supported power of two (1, 2, 4, 8, 16); 0 if k is too large.
int blocks_per_lane(int64_t k);

// ---- quantize.hip ----
// amax source of a row: reduce |x| (kind 0), amax_in[row] (kind 1),
// group_amax[group(row)] (kind 2, groups given by offsets), or amax_in[0]
// for every row (kind 3, one outer scale per tensor, written per row).
struct QuantRowsArgs {
  const uint16_t* x; int64_t rows; int64_t k; int64_t ld_x;
  int amax_kind; const float* amax_in; const int32_t* group_offsets; int32_t num_groups;
  uint8_t* codes; uint8_t* scales; float* gscale;  // gscale written for kinds 0, 1
  int block_rule;                                   // 0 standard, 1/2 Four-Over-Six (MSE/MAE)
};
hipError_t launch_quantize_rows(const QuantRowsArgs& a, hipStream_t s);
// 16x16 two-dimensional blocks, per-group scale from amax_in (rows % 16 == 0)
hipError_t launch_quantize_tiles2d(const QuantRowsArgs& a, hipStream_t s);
// Group amax: zero `amax_bits[num_groups]`, then atomic max of every row's amax.
hipError_t launch_group_amax(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                             const int32_t* group_offsets, int32_t num_groups,
                             uint32_t* amax_bits, hipStream_t s);
// amax over all rows of x into amax_bits[0] (float bits); bounds: int32[2] scratch.
hipError_t launch_tensor_amax(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x,
                              int32_t* bounds, uint32_t* amax_bits, hipStream_t s);
// out[0] = max of amax_rows[r] over r < min(cap, *rows_end).
hipError_t launch_rows_amax(const float* amax_rows, const int32_t* rows_end, int64_t cap,
                            float* out, hipStream_t s);
// gscale[g] = amax[g] / 2688 (in place allowed: amax may alias gscale).
hipError_t launch_group_finalize(const float* amax, float* gscale, int32_t num_groups,
                                 int rule, hipStream_t s);

// ---- route.hip ----
int64_t route_num_chunks(int64_t tokens);
size_t route_workspace_bytes(int64_t tokens, int32_t num_experts);
struct RouteArgs {
  const uint16_t* x; int64_t tokens; int64_t hidden;
  const int32_t* topk_idx; const float* topk_prob; int32_t topk; int32_t num_experts;
  int32_t align;
  int32_t* offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
  uint8_t* codes; uint8_t* scales; float* gscale;
  float* zero_per_row;  // nullable: rows [0, zero_rows) set to 0 (one coalesced fill)
  int64_t zero_rows;
  TileTableSpec tables[2];  // GEMM tile tables written from the offsets (num_tables of them)
  int32_t num_tables;
  void* workspace;      // route_workspace_bytes(); its first uint32 is the precondition word
  int32_t block_rule;   // 0 standard, 1/2 Four-Over-Six (MSE/MAE)
  uint32_t* error_word; // set by launch_route in a build with NVFP4_DEBUG_CHECKS
  // Gather mode (tok_codes non-NULL, with x): each token is quantized once
  // into token-major rows tok_codes [tokens + 1, hidden/2], tok_scales
  // [tokens + 1, hidden/16], tok_gscale [tokens]; row `tokens` is set to
  // zero codes and scales (the row padding rows read).  No routed-row copies
  // are written (codes / scales unused), gscale[r] receives the outer scale
  // of row r's token, and row_src must be given (the GEMM reads row r from
  // token row_src[r]).
  uint8_t* tok_codes; uint8_t* tok_scales; float* tok_gscale;
  uint8_t* entry_rank;  // gather mode: [tokens * topk] scratch (rank inside the chunk)
  const float* tok_amax; // nullable: one amax for every token (per-tensor outer scale)
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// Permuted rows r < *rows_end (device) copied from the token-major rows of
// gather mode (codes, scales and outer scale, each output nullable); padding
// rows (row_src < 0) get zeros.
hipError_t launch_gather_rows(const uint8_t* tok_codes, const uint8_t* tok_scales,
                              const float* tok_gscale, const int32_t* row_src,
                              const int32_t* rows_end, int64_t cap, int64_t hidden,
                              uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s);
// moe_permute's host-side argument checks (all but the workspace): an
// NVFP4_* status, NVFP4_OK when the call may proceed.  No HIP call.
int permute_args_status(const uint16_t* x, int64_t tokens, int64_t hidden,
                        const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                        int32_t num_experts, int32_t align, int32_t block_rule,
                        const int32_t* expert_offsets, const int32_t* dst_row,
                        const int32_t* row_src, const float* row_prob, const uint8_t* codes,
                        const uint8_t* block_scales, const float* global_scales);

// ---- gemm.hip ----
struct GemmArgs {
  const uint8_t* a_codes; const uint8_t* a_scales; const float* a_gscale;
  const uint8_t* b_codes; const uint8_t* b_scales; const float* b_gscale;
  const int32_t* offsets; int32_t num_groups;
  int64_t rows_cap;
  int64_t n;      // B rows per group (2*inter for the SwiGLU epilogue)
  int64_t k;
  int b_layout;   // 0 row-major B, 1 tiled (launch_pack_b)
  // plain epilogue
  int out_dtype; void* out;
  // SwiGLU epilogue
  const float* row_prob; uint16_t* d_out; float* amax; float* c_out; int64_t inter;
  // nullable: the launch's tile schedule, written beforehand by a kernel that
  // holds the offsets (one {group, row0, row1, n-tile} entry per workgroup,
  // group < 0 = none; see tile_schedule.h)
  const int4* tile_table;
  // nullable: A rows gathered from token-major codes / scales (row r reads
  // token a_row_src[r]; -1, a padding row, reads row a_pad_row, all zero, so
  // its products are +0 as in the permuted layout).  Gathering, a_gscale is
  // per token too: row r's outer scale is a_gscale[a_row_src[r]] (0 for a
  // padding row).  (a_pad_row + 1) * k / 2 < 2^32.
  const int32_t* a_row_src;
  int64_t a_pad_row;
};
hipError_t launch_gemm_plain(const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_swiglu(const GemmArgs& a, hipStream_t s);
// Workgroups of the launch that launch_gemm_plain / launch_gemm_swiglu make
// for these arguments (the entries of its tile table).
int64_t gemm_grid_blocks(const GemmArgs& a, bool swiglu);
// What a table builder needs to write that launch's table into `table`.
TileTableSpec gemm_tile_table_spec(const GemmArgs& a, bool swiglu, int4* table);
// Row-major B (rows % 32 == 0, k % 128 == 0) -> the tiled layout.
hipError_t launch_pack_b(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                         uint8_t* pcodes, uint8_t* pscales, hipStream_t s);

// One table entry per 128-row m-tile (BM = 128, one column tile), cost
// balanced over the XCDs like the GEMMs' (the single-pass kernel's grid).
TileTableSpec gemm_mtile_table_spec(int64_t rows_cap, int32_t num_groups, int64_t k, int4* table);

// ---- single_pass.hip ----
// FC1 -> weighted SwiGLU -> online-amax NVFP4 quantization -> FC2 in one
// kernel (one workgroup per 128-row m-tile of the tile table).
struct SinglePassArgs {
  const uint8_t* a_codes; const uint8_t* a_scales;   // token-major quantized activations
  const float* a_gscale;                             // [tokens] outer scale of each token
  const int32_t* a_row_src; int64_t a_pad_row;       // routed row -> token row; the zero row
  const float* row_prob;
  const uint8_t* w1_codes; const uint8_t* w1_scales; const float* w1_gscale; int w1_layout;
  const uint8_t* w2_codes; const uint8_t* w2_scales; const float* w2_gscale; int w2_layout;
  int64_t hidden, inter;
  const int4* tile_table;
  uint16_t* y_bf16;        // [rows_cap, hidden] FC2 rows (or:)
  float* y_f32;            // nullable: fp32 FC2 rows instead
  // nullable debug outputs (valid rows only)
  float* c_out;            // [rows_cap, 2 inter] FC1 pre-activation
  uint16_t* p_out;         // [rows_cap, inter] bf16 weighted SwiGLU
  uint8_t* a2c_out; uint8_t* a2s_out;   // [rows_cap, inter/2], [rows_cap, inter/16]
  float* gs_out;           // [rows_cap, ceil(inter / 256)] per-slice outer scales
};
TileTableSpec single_pass_table_spec(int64_t rows_cap, int32_t num_groups, int64_t hidden,
                                     int4* table);
int single_pass_lds_bytes(int64_t inter);
hipError_t launch_single_pass(const SinglePassArgs& a, int64_t blocks, hipStream_t s);

// ---- backward.hip ----
enum { BWD_DGRAD_ROWS = 1, BWD_WGRAD = 2 };

// One bf16 operand of a backward GEMM: row-major, `ld` elements per row; per
// group (the dgrads' B) at p + g * group_stride.  row_map (nullable) marks
// the rows: row r is read only if row_map[r] >= 0, and from row row_map[r]
// when `gather` is set (the wgrads always gather through it).
struct BwdOperand {
  const uint16_t* p;
  int64_t ld, group_stride;
  const int32_t* row_map;
  int32_t gather;
  uint32_t bytes;             // readable bytes from p (per group: from its base), < 2^31
};

struct BwdGemmArgs {
  BwdOperand a, b;
  const int32_t* offsets;     // [G + 1] rows of each group
  int32_t num_groups;
  int64_t m, n, k;            // wgrad: output [G, m, n]; dgrad: n columns, K = k
  const int4* tiles;          // dgrad tile table
  const int32_t* order;       // wgrad: experts, heaviest first
  float* out_f32;             // wgrad output; dgrad: optional fp32 copy
  uint16_t* out_bf16;         // dgrad output rows
};

int bwd_lds_bytes();
TileTableSpec bwd_dgrad_table_spec(int64_t rows_cap, int32_t num_groups, int64_t k, int64_t n,
                                   int4* table);
int64_t bwd_wgrad_blocks(int32_t num_groups, int64_t m, int64_t n);
hipError_t launch_bwd_tables(const int32_t* offsets, int32_t G, const TileTableSpec& t0,
                             const TileTableSpec& t1, int32_t* order, hipStream_t s);
hipError_t launch_bwd_gemm(int mode, const BwdGemmArgs& a, int64_t blocks, hipStream_t s);
hipError_t launch_swiglu_bwd(const uint16_t* dD, const float* C, const int32_t* row_src,
                             const float* row_prob, const int32_t* rows_end, int64_t cap,
                             int64_t inter, uint16_t* dC, float* dp, hipStream_t s);
hipError_t launch_bwd_entry_grad(const float* dp, const int32_t* dst_row, int64_t n,
                                 float* dprob, hipStream_t s);

// ---- combine.hip ----
hipError_t launch_combine(const void* y_rows, int y_rows_dtype, const int32_t* dst_row,
                          int64_t tokens, int32_t topk, int64_t hidden, uint16_t* y,
                          hipStream_t s);

}  // namespace nvfp4
