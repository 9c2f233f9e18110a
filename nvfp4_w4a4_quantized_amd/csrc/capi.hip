// capi.hip -- the C ABI declared in include/nvfp4moe.h: host-side argument
// validation (before any HIP call), workspace carving and kernel launches.
#include "nvfp4moe.h"

#include <hip/hip_runtime.h>

#include "launch.h"

using namespace nvfp4;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_HIP_ERROR; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool valid_align(int32_t align) {
  return align >= 1 && align <= 256 && (align & (align - 1)) == 0;
}

constexpr int64_t kMaxK = 16384;
constexpr int32_t kMaxExperts = 1024;

// Sequential carve of 256-byte aligned regions out of one workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += round_up(count * sizeof(T), 256);
    return p;
  }
};

struct MoeLayout {
  int32_t* route_ws_i; int32_t* offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
  uint8_t* tokc; uint8_t* toks; float* tokg;   // token-major quantized activations
  uint8_t* rank;                               // routing entries' ranks inside their chunk
  uint16_t* d; float* amax_d;
  uint8_t* a2c; uint8_t* a2s; float* a2g;
  uint16_t* y_rows;
  int4* tab1; int4* tab2;   // FC1 / FC2 tile tables
  int32_t* bounds;          // per-tensor activation scale: the reduction's row range
  float* tamax;             // per-tensor activation scale: amax of x [0], of D [1]
  size_t bytes;
};

// The FC1 / FC2 launch arguments that fix the grids (sizes only).
GemmArgs moe_gemm_shape(int64_t cap, int64_t H, int64_t I, int32_t E, bool fc1) {
  GemmArgs g{};
  g.num_groups = E; g.rows_cap = cap;
  g.n = fc1 ? 2 * I : H; g.k = fc1 ? H : I; g.inter = fc1 ? I : 0;
  return g;
}

MoeLayout carve_moe(void* ws, int64_t T, int64_t H, int64_t I, int32_t k, int32_t E, int32_t align) {
  const int64_t cap = moe_rows_capacity(T, k, E, align);
  Carver c(ws);
  MoeLayout L;
  L.route_ws_i = c.take<int32_t>(route_workspace_bytes(T, E) / 4);
  L.offsets = c.take<int32_t>(E + 1);
  L.dst_row = c.take<int32_t>((size_t)(T * k));
  L.row_src = c.take<int32_t>((size_t)cap);
  L.row_prob = c.take<float>((size_t)cap);
  L.tokc = c.take<uint8_t>((size_t)((T + 1) * H / 2));   // + the zero row padding rows read
  L.toks = c.take<uint8_t>((size_t)((T + 1) * H / 16));
  L.tokg = c.take<float>((size_t)T);
  L.rank = c.take<uint8_t>((size_t)(T * k));
  L.d = c.take<uint16_t>((size_t)(cap * I));
  L.amax_d = c.take<float>((size_t)cap);
  L.a2c = c.take<uint8_t>((size_t)(cap * I / 2));
  L.a2s = c.take<uint8_t>((size_t)(cap * I / 16));
  L.a2g = c.take<float>((size_t)cap);
  L.y_rows = c.take<uint16_t>((size_t)(cap * H));
  L.tab1 = c.take<int4>((size_t)gemm_grid_blocks(moe_gemm_shape(cap, H, I, E, true), true));
  L.tab2 = c.take<int4>((size_t)gemm_grid_blocks(moe_gemm_shape(cap, H, I, E, false), false));
  L.bounds = c.take<int32_t>(2);
  L.tamax = c.take<float>(2);
  L.bytes = c.used;
  return L;
}

// Workspace of the single-pass layer: routing, token rows, per-row maps and
// scales, the FC2 rows and the fused kernel's tile table.
struct SpLayout {
  int32_t* route_ws_i; int32_t* offsets; int32_t* dst_row; int32_t* row_src; float* row_prob;
  uint8_t* tokc; uint8_t* toks; float* tokg; uint8_t* rank;
  uint16_t* y_rows;
  int4* tab;
  int64_t blocks;
  size_t bytes;
};

SpLayout carve_single_pass(void* ws, int64_t T, int64_t H, int64_t I, int32_t k, int32_t E,
                           int32_t align) {
  const int64_t cap = moe_rows_capacity(T, k, E, align);
  Carver c(ws);
  SpLayout L;
  L.route_ws_i = c.take<int32_t>(route_workspace_bytes(T, E) / 4);
  L.offsets = c.take<int32_t>(E + 1);
  L.dst_row = c.take<int32_t>((size_t)(T * k));
  L.row_src = c.take<int32_t>((size_t)cap);
  L.row_prob = c.take<float>((size_t)cap);
  L.tokc = c.take<uint8_t>((size_t)((T + 1) * H / 2));
  L.toks = c.take<uint8_t>((size_t)((T + 1) * H / 16));
  L.tokg = c.take<float>((size_t)T);
  L.rank = c.take<uint8_t>((size_t)(T * k));
  L.y_rows = c.take<uint16_t>((size_t)(cap * H));
  L.blocks = single_pass_table_spec(cap, E, H, nullptr).blocks;
  L.tab = c.take<int4>((size_t)L.blocks);
  L.bytes = c.used;
  return L;
}

// Workspace of the backward: the two dgrad tile tables, the wgrads' expert
// order, dD, dC, the rows' router-weight gradients and the FC1 dgrad rows.
struct BwdLayout {
  int4* tab2; int4* tab1;   // FC2 / FC1 dgrad tile tables
  int64_t blocks2, blocks1;
  int32_t* order;
  uint16_t* dd; uint16_t* dc; float* dp; uint16_t* dxr;
  size_t bytes;
};

BwdLayout carve_backward(void* ws, int64_t cap, int64_t H, int64_t I, int32_t E) {
  Carver c(ws);
  BwdLayout L;
  L.blocks2 = bwd_dgrad_table_spec(cap, E, H, I, nullptr).blocks;
  L.blocks1 = bwd_dgrad_table_spec(cap, E, 2 * I, H, nullptr).blocks;
  L.tab2 = c.take<int4>((size_t)L.blocks2);
  L.tab1 = c.take<int4>((size_t)L.blocks1);
  L.order = c.take<int32_t>((size_t)E);
  L.dd = c.take<uint16_t>((size_t)(cap * I));
  L.dc = c.take<uint16_t>((size_t)(cap * 2 * I));
  L.dp = c.take<float>((size_t)cap);
  L.dxr = c.take<uint16_t>((size_t)(cap * H));
  L.bytes = c.used;
  return L;
}

bool route_args_ok(int64_t tokens, int32_t topk, int32_t num_experts, int32_t align) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || num_experts > kMaxExperts) return false;
  if (topk > num_experts || !valid_align(align)) return false;
  const int64_t cap = (int64_t)tokens * topk + (int64_t)num_experts * align;
  return cap < 0x7FFFFFFFLL;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_INVALID_ARGUMENT: return "invalid argument";
    case NVFP4_UNSUPPORTED: return "unsupported shape";
    case NVFP4_HIP_ERROR: return "HIP launch/runtime error";
    case NVFP4_WORKSPACE_TOO_SMALL: return "workspace too small";
    case NVFP4_SCRATCH_LIMIT: return "exceeds the static scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

int nvfp4_debug_checks(void) {
#ifdef NVFP4_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld_x, int scale_domain,
                   const int32_t* group_offsets, int32_t num_groups, const float* amax_in,
                   int block_rule, uint8_t* codes, uint8_t* block_scales, float* global_scales,
                   void* stream) {
  if (block_rule < 0 || block_rule > 2) return NVFP4_INVALID_ARGUMENT;
  if (rows < 0 || rows >= 0x7FFFFFFFLL || k < 16 || k % 16 != 0 || ld_x < k || ld_x % 8 != 0)
    return NVFP4_INVALID_ARGUMENT;
  if (k > kMaxK) return NVFP4_UNSUPPORTED;
  if (!x || !codes || !block_scales || !global_scales) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(global_scales, 4))
    return NVFP4_INVALID_ARGUMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  QuantRowsArgs a{x, rows, k, ld_x, 0, amax_in, group_offsets, num_groups,
                  codes, block_scales, global_scales, block_rule};
  if (scale_domain == 0) {
    a.amax_kind = amax_in ? 1 : 0;
    return hip_status(launch_quantize_rows(a, s));
  }
  if (scale_domain != 1 && scale_domain != 2) return NVFP4_INVALID_ARGUMENT;
  if (!group_offsets || num_groups < 1 || num_groups >= 0x7FFFFFFF) return NVFP4_INVALID_ARGUMENT;
  if (scale_domain == 2 && (rows % 16 != 0 || block_rule != 0)) return NVFP4_UNSUPPORTED;
  // group amax: reduce into global_scales (as bits) unless given
  const float* amax_src = amax_in;
  if (!amax_src) {
    hipError_t e = launch_group_amax(x, rows, k, ld_x, group_offsets, num_groups,
                                     reinterpret_cast<uint32_t*>(global_scales), s);
    if (e != hipSuccess) return NVFP4_HIP_ERROR;
    amax_src = global_scales;
  }
  a.amax_kind = 2;
  a.amax_in = amax_src;
  hipError_t e = scale_domain == 2 ? launch_quantize_tiles2d(a, s) : launch_quantize_rows(a, s);
  if (e != hipSuccess) return NVFP4_HIP_ERROR;
  return hip_status(launch_group_finalize(amax_src, global_scales, num_groups, block_rule, s));
}

int64_t moe_rows_capacity(int64_t tokens, int32_t topk, int32_t num_experts, int32_t align) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || align < 1) return 0;
  return tokens * (int64_t)topk + (int64_t)num_experts * (int64_t)(align - 1);
}

size_t moe_permute_workspace_size(int64_t tokens, int32_t topk, int32_t num_experts) {
  (void)topk;
  if (tokens < 0 || num_experts < 1) return 0;
  return route_workspace_bytes(tokens, num_experts);
}

}  // extern "C"

// moe_permute's host-side checks of everything but the workspace.
int nvfp4::permute_args_status(const uint16_t* x, int64_t tokens, int64_t hidden,
                               const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                               int32_t num_experts, int32_t align, int32_t block_rule,
                               const int32_t* expert_offsets, const int32_t* dst_row,
                               const int32_t* row_src, const float* row_prob, const uint8_t* codes,
                               const uint8_t* block_scales, const float* global_scales) {
  if (!route_args_ok(tokens, topk, num_experts, align)) return NVFP4_INVALID_ARGUMENT;
  if (block_rule < 0 || block_rule > 2) return NVFP4_INVALID_ARGUMENT;
  if (!expert_offsets || !row_src || !row_prob) return NVFP4_INVALID_ARGUMENT;
  if (tokens > 0 && (!topk_idx || !topk_prob || !dst_row)) return NVFP4_INVALID_ARGUMENT;
  if (x) {
    if (hidden < 16 || hidden % 16 != 0) return NVFP4_INVALID_ARGUMENT;
    if (hidden > kMaxK) return NVFP4_UNSUPPORTED;
    if (!codes || !block_scales || !global_scales) return NVFP4_INVALID_ARGUMENT;
    if (!aligned(x, 16) || !aligned(codes, 8)) return NVFP4_INVALID_ARGUMENT;
  }
  return NVFP4_OK;
}

extern "C" {

int moe_permute(const uint16_t* x, int64_t tokens, int64_t hidden, const int32_t* topk_idx,
                const float* topk_prob, int32_t topk, int32_t num_experts, int32_t align,
                int32_t block_rule, int32_t* expert_offsets, int32_t* dst_row, int32_t* row_src, float* row_prob,
                uint8_t* codes, uint8_t* block_scales, float* global_scales, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int st = permute_args_status(x, tokens, hidden, topk_idx, topk_prob, topk, num_experts,
                                     align, block_rule, expert_offsets, dst_row, row_src, row_prob,
                                     codes, block_scales, global_scales);
  if (st != NVFP4_OK) return st;
  if (!workspace || !aligned(workspace, 16)) return NVFP4_INVALID_ARGUMENT;
  if (workspace_bytes < route_workspace_bytes(tokens, num_experts)) return NVFP4_WORKSPACE_TOO_SMALL;
  RouteArgs a{};
  a.x = x; a.tokens = tokens; a.hidden = x ? hidden : 0;
  a.topk_idx = topk_idx; a.topk_prob = topk_prob; a.topk = topk;
  a.num_experts = num_experts; a.align = align;
  a.offsets = expert_offsets; a.dst_row = dst_row; a.row_src = row_src; a.row_prob = row_prob;
  a.codes = codes; a.scales = block_scales; a.gscale = global_scales;
  a.workspace = workspace; a.block_rule = block_rule;
  return hip_status(launch_route(a, static_cast<hipStream_t>(stream)));
}

static int gemm_args_ok(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        int64_t rows_cap, const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_gscale, const int32_t* group_offsets, int32_t num_groups,
                        int64_t k) {
  if (!a_codes || !a_scales || !a_gscale || !b_codes || !b_scales || !b_gscale || !group_offsets)
    return NVFP4_INVALID_ARGUMENT;
  if (rows_cap < 0 || rows_cap >= 0x7FFFFFFFLL || num_groups < 1 || num_groups > kMaxExperts)
    return NVFP4_INVALID_ARGUMENT;
  if (k < 16 || k % 16 != 0) return NVFP4_INVALID_ARGUMENT;
  if (k % 128 != 0 || k > kMaxK) return NVFP4_UNSUPPORTED;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4))
    return NVFP4_INVALID_ARGUMENT;
  return NVFP4_OK;
}

int w4a4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                      int64_t rows_cap, const uint8_t* b_codes, const uint8_t* b_scales,
                      const float* b_gscale, const int32_t* group_offsets, int32_t num_groups,
                      int64_t n, int64_t k, int b_layout, int out_dtype, void* out,
                      void* stream) {
  int st = gemm_args_ok(a_codes, a_scales, a_gscale, rows_cap, b_codes, b_scales, b_gscale,
                        group_offsets, num_groups, k);
  if (st != NVFP4_OK) return st;
  if (!out || (out_dtype != 0 && out_dtype != 1) || !aligned(out, 16)) return NVFP4_INVALID_ARGUMENT;
  if (b_layout != 0 && b_layout != 1) return NVFP4_INVALID_ARGUMENT;
  if (n < 32 || n % 32 != 0) return NVFP4_UNSUPPORTED;
  if ((int64_t)num_groups * n >= 0x7FFFFFFFLL) return NVFP4_INVALID_ARGUMENT;
  if (n * (k / 2) > 0xFFFFFFFFLL) return NVFP4_UNSUPPORTED;   // 32-bit offsets inside a group
  GemmArgs a{};
  a.a_codes = a_codes; a.a_scales = a_scales; a.a_gscale = a_gscale;
  a.b_codes = b_codes; a.b_scales = b_scales; a.b_gscale = b_gscale;
  a.offsets = group_offsets; a.num_groups = num_groups; a.rows_cap = rows_cap;
  a.n = n; a.k = k; a.b_layout = b_layout; a.out_dtype = out_dtype; a.out = out;
  return hip_status(launch_gemm_plain(a, static_cast<hipStream_t>(stream)));
}

int w4a4_grouped_gemm_swiglu(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                             int64_t rows_cap, const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_gscale, const int32_t* group_offsets,
                             int32_t num_groups, int64_t inter, int64_t k, int b_layout,
                             const float* row_prob,
                             uint16_t* d_out, float* amax, float* c_out, void* stream) {
  int st = gemm_args_ok(a_codes, a_scales, a_gscale, rows_cap, b_codes, b_scales, b_gscale,
                        group_offsets, num_groups, k);
  if (st != NVFP4_OK) return st;
  if (!row_prob || !d_out || !amax) return NVFP4_INVALID_ARGUMENT;
  if (b_layout != 0 && b_layout != 1) return NVFP4_INVALID_ARGUMENT;
  if (inter < 64 || inter % 64 != 0) return NVFP4_UNSUPPORTED;
  if ((int64_t)num_groups * 2 * inter >= 0x7FFFFFFFLL) return NVFP4_INVALID_ARGUMENT;
  if (2 * inter * (k / 2) > 0xFFFFFFFFLL) return NVFP4_UNSUPPORTED;   // 32-bit offsets inside a group
  GemmArgs a{};
  a.a_codes = a_codes; a.a_scales = a_scales; a.a_gscale = a_gscale;
  a.b_codes = b_codes; a.b_scales = b_scales; a.b_gscale = b_gscale;
  a.offsets = group_offsets; a.num_groups = num_groups; a.rows_cap = rows_cap;
  a.n = 2 * inter; a.k = k; a.inter = inter; a.b_layout = b_layout;
  a.row_prob = row_prob; a.d_out = d_out; a.amax = amax; a.c_out = c_out;
  return hip_status(launch_gemm_swiglu(a, static_cast<hipStream_t>(stream)));
}

int moe_combine(const void* y_rows, int y_rows_dtype, const int32_t* dst_row, int64_t tokens,
                int32_t topk, int64_t hidden, uint16_t* y, void* stream) {
  if (tokens < 0 || topk < 1 || hidden < 8 || hidden % 8 != 0) return NVFP4_INVALID_ARGUMENT;
  if (y_rows_dtype != 0 && y_rows_dtype != 1) return NVFP4_INVALID_ARGUMENT;
  if (tokens > 0 && (!y_rows || !dst_row || !y)) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(y_rows, 16) || !aligned(y, 16)) return NVFP4_INVALID_ARGUMENT;
  return hip_status(launch_combine(y_rows, y_rows_dtype, dst_row, tokens, topk, hidden, y,
                                   static_cast<hipStream_t>(stream)));
}

size_t moe_expert_forward_workspace_size(int64_t tokens, int64_t hidden, int64_t inter,
                                         int32_t topk, int32_t num_experts, int32_t align) {
  if (!route_args_ok(tokens, topk, num_experts, align) || hidden < 0 || inter < 0) return 0;
  return carve_moe(nullptr, tokens, hidden, inter, topk, num_experts, align).bytes;
}

int moe_expert_forward(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t inter,
                       const int32_t* topk_idx, const float* topk_prob, int32_t topk,
                       int32_t num_experts, int32_t align, int32_t act_block_rule,
                       int32_t act_scale_domain, const nvfp4_weights* w1,
                       const nvfp4_weights* w2, uint16_t* y, void* workspace,
                       size_t workspace_bytes, const nvfp4_moe_intermediates* debug,
                       void* const* stage_events, void* stream) {
  if (!route_args_ok(tokens, topk, num_experts, align)) return NVFP4_INVALID_ARGUMENT;
  if (act_block_rule < 0 || act_block_rule > 2) return NVFP4_INVALID_ARGUMENT;
  if (act_scale_domain != 0 && act_scale_domain != 1) return NVFP4_INVALID_ARGUMENT;
  if (hidden < 128 || hidden % 128 != 0 || inter < 128 || inter % 128 != 0)
    return NVFP4_UNSUPPORTED;
  if (hidden > kMaxK || inter > kMaxK) return NVFP4_UNSUPPORTED;
  if (!w1 || !w2 || !w1->codes || !w1->scales || !w1->gscale || !w2->codes || !w2->scales ||
      !w2->gscale || !workspace)
    return NVFP4_INVALID_ARGUMENT;
  if ((w1->layout != 0 && w1->layout != 1) || (w2->layout != 0 && w2->layout != 1))
    return NVFP4_INVALID_ARGUMENT;
  if (tokens > 0 && (!x || !y || !topk_idx || !topk_prob)) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(workspace, 256) || (x && !aligned(x, 16)) || (y && !aligned(y, 16)) ||
      !aligned(w1->codes, 16) || !aligned(w2->codes, 16) || !aligned(w1->scales, 4) ||
      !aligned(w2->scales, 4))
    return NVFP4_INVALID_ARGUMENT;
  if ((int64_t)num_experts * 2 * inter >= 0x7FFFFFFFLL ||
      (int64_t)num_experts * hidden >= 0x7FFFFFFFLL)
    return NVFP4_INVALID_ARGUMENT;
  if ((tokens + 1) * (hidden / 2) > 0xFFFFFFFFLL) return NVFP4_UNSUPPORTED;   // 32-bit row offsets
  MoeLayout L = carve_moe(workspace, tokens, hidden, inter, topk, num_experts, align);
  if (workspace_bytes < L.bytes) return NVFP4_WORKSPACE_TOO_SMALL;
  float* c_out = nullptr;
  float* y_f32 = nullptr;
  if (debug) {
    if (debug->expert_offsets) L.offsets = debug->expert_offsets;
    if (debug->dst_row) L.dst_row = debug->dst_row;
    if (debug->row_src) L.row_src = debug->row_src;
    if (debug->row_prob) L.row_prob = debug->row_prob;
    if ((debug->a1_codes != nullptr) != (debug->a1_scales != nullptr)) return NVFP4_INVALID_ARGUMENT;
    if (debug->d) L.d = debug->d;
    if (debug->amax_d) L.amax_d = debug->amax_d;
    if (debug->a2_codes) L.a2c = debug->a2_codes;
    if (debug->a2_scales) L.a2s = debug->a2_scales;
    if (debug->a2_gscale) L.a2g = debug->a2_gscale;
    if (debug->y_rows) L.y_rows = debug->y_rows;
    c_out = debug->fc1_out;
    y_f32 = debug->y_rows_f32;
    const void* ptrs16[] = {debug->a1_codes, L.a2c, L.d, L.y_rows, y_f32};
    for (const void* p : ptrs16)
      if (p && !aligned(p, 16)) return NVFP4_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t cap = moe_rows_capacity(tokens, topk, num_experts, align);
  auto mark = [&](int i) -> hipError_t {
    if (!stage_events || !stage_events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s);
  };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return NVFP4_HIP_ERROR;
  GemmArgs g1{};
  g1.a_codes = L.tokc; g1.a_scales = L.toks; g1.a_gscale = L.tokg; g1.a_row_src = L.row_src;
  g1.a_pad_row = tokens;
  g1.b_codes = w1->codes; g1.b_scales = w1->scales; g1.b_gscale = w1->gscale;
  g1.offsets = L.offsets; g1.num_groups = num_experts; g1.rows_cap = cap;
  g1.n = 2 * inter; g1.k = hidden; g1.inter = inter; g1.b_layout = w1->layout;
  g1.row_prob = L.row_prob; g1.d_out = L.d; g1.amax = L.amax_d; g1.c_out = c_out;
  g1.tile_table = L.tab1;
  GemmArgs g2{};
  g2.a_codes = L.a2c; g2.a_scales = L.a2s; g2.a_gscale = L.a2g;
  g2.b_codes = w2->codes; g2.b_scales = w2->scales; g2.b_gscale = w2->gscale;
  g2.offsets = L.offsets; g2.num_groups = num_experts; g2.rows_cap = cap;
  g2.n = hidden; g2.k = inter; g2.b_layout = w2->layout;
  g2.out_dtype = y_f32 ? 0 : 1;
  g2.out = y_f32 ? static_cast<void*>(y_f32) : static_cast<void*>(L.y_rows);
  g2.tile_table = L.tab2;
  // a1 + a2: routing metadata and per-token quantization.  Each token is
  // quantized once into a token-major row; FC1 reads routed row r from token
  // row_src[r] (the permutation is applied by the GEMM's A loads, so no
  // routed copies are written).  The same launches clear amax_d over the
  // whole capacity (FC1 takes atomic maxima into it) and, while they hold
  // the offsets, write both GEMMs' tile tables.
  RouteArgs ra{};
  ra.x = x; ra.tokens = tokens; ra.hidden = hidden;
  ra.topk_idx = topk_idx; ra.topk_prob = topk_prob; ra.topk = topk;
  ra.num_experts = num_experts; ra.align = align;
  ra.offsets = L.offsets; ra.dst_row = L.dst_row;
  ra.row_src = L.row_src;
  ra.row_prob = L.row_prob; ra.gscale = nullptr;   // the GEMMs read tok_gscale through row_src
  ra.tok_codes = L.tokc; ra.tok_scales = L.toks; ra.tok_gscale = L.tokg; ra.entry_rank = L.rank;
  ra.zero_per_row = L.amax_d; ra.zero_rows = cap;
  ra.tables[0] = gemm_tile_table_spec(g1, true, L.tab1);
  ra.tables[1] = gemm_tile_table_spec(g2, false, L.tab2);
  ra.num_tables = 2;
  ra.workspace = L.route_ws_i; ra.block_rule = act_block_rule;
  if (act_scale_domain == 1 && tokens > 0) {
    // one outer scale for the whole x ([miniTE] §2.3 per-tensor scaling)
    if ((e = launch_tensor_amax(x, tokens, hidden, hidden, L.bounds,
                                reinterpret_cast<uint32_t*>(L.tamax), s)) != hipSuccess)
      return NVFP4_HIP_ERROR;
    ra.tok_amax = L.tamax;
  }
  if ((e = launch_route(ra, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if (debug) {   // the permuted rows and their outer scales, for inspection
    if ((e = launch_gather_rows(L.tokc, L.toks, L.tokg, L.row_src, L.offsets + num_experts, cap,
                                hidden, debug->a1_codes, debug->a1_scales, debug->a1_gscale,
                                s)) != hipSuccess)
      return NVFP4_HIP_ERROR;
  }
  if ((e = mark(1)) != hipSuccess) return NVFP4_HIP_ERROR;
  // a3 + a4: FC1 with the weighted SwiGLU epilogue and D's row amax
  if ((e = launch_gemm_swiglu(g1, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if ((e = mark(2)) != hipSuccess) return NVFP4_HIP_ERROR;
  // a5: requantize D reusing its amax (rows up to offsets[E] live on device:
  // quantize the whole capacity; rows past the end are ignored downstream)
  QuantRowsArgs q{L.d, cap, inter, inter, 1, L.amax_d, nullptr, 0, L.a2c, L.a2s, L.a2g,
                  act_block_rule};
  if (act_scale_domain == 1) {
    // one outer scale for all routed rows of D: the maximum of their amax
    if ((e = launch_rows_amax(L.amax_d, L.offsets + num_experts, cap, L.tamax + 1, s)) !=
        hipSuccess)
      return NVFP4_HIP_ERROR;
    q.amax_kind = 3;
    q.amax_in = L.tamax + 1;
  }
  if ((e = launch_quantize_rows(q, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if ((e = mark(3)) != hipSuccess) return NVFP4_HIP_ERROR;
  // a6: FC2
  if ((e = launch_gemm_plain(g2, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if ((e = mark(4)) != hipSuccess) return NVFP4_HIP_ERROR;
  // a7: combine
  if ((e = launch_combine(y_f32 ? static_cast<const void*>(y_f32) : L.y_rows, y_f32 ? 0 : 1,
                          L.dst_row, tokens, topk, hidden, y, s)) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if ((e = mark(5)) != hipSuccess) return NVFP4_HIP_ERROR;
  return NVFP4_OK;
}

size_t moe_expert_backward_workspace_size(int64_t rows_cap, int64_t hidden, int64_t inter,
                                          int32_t num_experts) {
  if (rows_cap < 0 || rows_cap >= 0x7FFFFFFFLL || hidden < 0 || inter < 0 || num_experts < 1 ||
      num_experts > kMaxExperts)
    return 0;
  return carve_backward(nullptr, rows_cap, hidden, inter, num_experts).bytes;
}

int moe_expert_backward(const uint16_t* dy, const uint16_t* x, int64_t tokens, int64_t hidden,
                        int64_t inter, int32_t topk, int32_t num_experts, int64_t rows_cap,
                        const float* fc1_out, const uint16_t* d, const int32_t* expert_offsets,
                        const int32_t* row_src, const float* row_prob, const int32_t* dst_row,
                        const uint16_t* w1, const uint16_t* w2, uint16_t* dx, float* dw1,
                        float* dw2, float* dprob, void* workspace, size_t workspace_bytes,
                        const nvfp4_moe_backward_intermediates* debug,
                        void* const* stage_events, void* stream) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || num_experts > kMaxExperts || topk > num_experts)
    return NVFP4_INVALID_ARGUMENT;
  if (rows_cap < 0 || rows_cap >= 0x7FFFFFFFLL || tokens * topk >= 0x7FFFFFFFLL)
    return NVFP4_INVALID_ARGUMENT;
  if (hidden < 128 || hidden % 128 != 0 || inter < 128 || inter % 128 != 0)
    return NVFP4_UNSUPPORTED;
  if (hidden > kMaxK || inter > kMaxK) return NVFP4_UNSUPPORTED;
  if (!w1 || !w2 || !dw1 || !dw2 || !expert_offsets || !workspace) return NVFP4_INVALID_ARGUMENT;
  if (rows_cap > 0 && (!fc1_out || !d || !row_src || !row_prob)) return NVFP4_INVALID_ARGUMENT;
  if (tokens > 0 && (!dy || !x || !dx || !dprob || !dst_row)) return NVFP4_INVALID_ARGUMENT;
  const void* a16[] = {dy, x, fc1_out, d, w1, w2, dx, dw1, dw2, workspace};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return NVFP4_INVALID_ARGUMENT;
  const void* a4[] = {dprob, row_src, row_prob, dst_row, expert_offsets};
  for (const void* p : a4)
    if (p && !aligned(p, 4)) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(workspace, 256)) return NVFP4_INVALID_ARGUMENT;
  // every operand the GEMMs read is addressed with 32-bit byte offsets
  const int64_t tok_bytes = tokens * hidden * 2, c_bytes = rows_cap * 2 * inter * 4;
  const int64_t dc_bytes = rows_cap * 2 * inter * 2, w_bytes = 2 * inter * hidden * 2;
  if (tok_bytes >= 0x80000000LL || c_bytes >= 0x80000000LL || dc_bytes >= 0x80000000LL ||
      w_bytes >= 0x80000000LL)
    return NVFP4_UNSUPPORTED;
  BwdLayout L = carve_backward(workspace, rows_cap, hidden, inter, num_experts);
  if (workspace_bytes < L.bytes) return NVFP4_WORKSPACE_TOO_SMALL;
  float* dxr_f32 = nullptr;
  if (debug) {
    if (debug->dd) L.dd = debug->dd;
    if (debug->dc) L.dc = debug->dc;
    if (debug->dp_rows) L.dp = debug->dp_rows;
    if (debug->dx_rows) L.dxr = debug->dx_rows;
    dxr_f32 = debug->dx_rows_f32;
    const void* p16[] = {L.dd, L.dc, L.dxr};
    for (const void* p : p16)
      if (!aligned(p, 16)) return NVFP4_INVALID_ARGUMENT;
    if (dxr_f32 && !aligned(dxr_f32, 16)) return NVFP4_INVALID_ARGUMENT;
    const void* p4[] = {L.dp};
    for (const void* p : p4)
      if (p && !aligned(p, 4)) return NVFP4_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    if (!stage_events || !stage_events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s);
  };
  if (mark(0) != hipSuccess) return NVFP4_HIP_ERROR;
  // the dgrads' tile tables from the device offsets
  const TileTableSpec t2 = bwd_dgrad_table_spec(rows_cap, num_experts, hidden, inter, L.tab2);
  const TileTableSpec t1 = bwd_dgrad_table_spec(rows_cap, num_experts, 2 * inter, hidden, L.tab1);
  if (launch_bwd_tables(expert_offsets, num_experts, t2, t1, L.order, s) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if (mark(1) != hipSuccess) return NVFP4_HIP_ERROR;
  // FC2 dgrad: dD = dYr W2[e] (bf16 rows), then the SwiGLU backward
  BwdGemmArgs f2{};
  f2.a = BwdOperand{dy, hidden, 0, row_src, 1, (uint32_t)tok_bytes};
  f2.b = BwdOperand{w2, inter, hidden * inter, nullptr, 0, (uint32_t)(hidden * inter * 2)};
  f2.offsets = expert_offsets; f2.num_groups = num_experts;
  f2.m = rows_cap; f2.n = inter; f2.k = hidden; f2.tiles = L.tab2;
  f2.out_bf16 = L.dd;
  if (launch_bwd_gemm(BWD_DGRAD_ROWS, f2, L.blocks2, s) != hipSuccess) return NVFP4_HIP_ERROR;
  if (mark(2) != hipSuccess) return NVFP4_HIP_ERROR;
  if (launch_swiglu_bwd(L.dd, fc1_out, row_src, row_prob, expert_offsets + num_experts, rows_cap,
                        inter, L.dc, L.dp, s) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if (mark(3) != hipSuccess) return NVFP4_HIP_ERROR;
  // The dgrads and the reductions first, the wgrads last: the FC1 dgrad and
  // the dx sum then read dC and dXr right after they were written, while
  // they are still in the last-level cache, rather than behind the wgrads'
  // 2.4 GB of weight-gradient stores (the dx sum ran at half speed there).
  // FC1 dgrad: dXr = dC W1[e] (bf16 rows)
  BwdGemmArgs f1{};
  f1.a = BwdOperand{L.dc, 2 * inter, 0, nullptr, 0, (uint32_t)dc_bytes};
  f1.b = BwdOperand{w1, hidden, 2 * inter * hidden, nullptr, 0, (uint32_t)w_bytes};
  f1.offsets = expert_offsets; f1.num_groups = num_experts;
  f1.m = rows_cap; f1.n = hidden; f1.k = 2 * inter; f1.tiles = L.tab1;
  f1.out_bf16 = L.dxr; f1.out_f32 = dxr_f32;
  if (launch_bwd_gemm(BWD_DGRAD_ROWS, f1, L.blocks1, s) != hipSuccess) return NVFP4_HIP_ERROR;
  if (mark(4) != hipSuccess) return NVFP4_HIP_ERROR;
  // dx: the sum of each token's rows; dprob: each entry's row sum
  if (launch_combine(L.dxr, 1, dst_row, tokens, topk, hidden, dx, s) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if (launch_bwd_entry_grad(L.dp, dst_row, tokens * topk, dprob, s) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if (mark(5) != hipSuccess) return NVFP4_HIP_ERROR;
  // FC2 wgrad: dW2[e] = dYr^T D over the expert's rows
  BwdGemmArgs w2g{};
  w2g.a = BwdOperand{dy, hidden, 0, row_src, 1, (uint32_t)tok_bytes};
  w2g.b = BwdOperand{d, inter, 0, nullptr, 0, (uint32_t)(dc_bytes / 2)};
  w2g.offsets = expert_offsets; w2g.num_groups = num_experts; w2g.order = L.order;
  w2g.m = hidden; w2g.n = inter; w2g.out_f32 = dw2;
  if (launch_bwd_gemm(BWD_WGRAD, w2g, bwd_wgrad_blocks(num_experts, hidden, inter), s) !=
      hipSuccess)
    return NVFP4_HIP_ERROR;
  if (mark(6) != hipSuccess) return NVFP4_HIP_ERROR;
  // FC1 wgrad: dW1[e] = dC^T X over the expert's rows
  BwdGemmArgs w1g{};
  w1g.a = BwdOperand{L.dc, 2 * inter, 0, nullptr, 0, (uint32_t)dc_bytes};
  w1g.b = BwdOperand{x, hidden, 0, row_src, 1, (uint32_t)tok_bytes};
  w1g.offsets = expert_offsets; w1g.num_groups = num_experts; w1g.order = L.order;
  w1g.m = 2 * inter; w1g.n = hidden; w1g.out_f32 = dw1;
  if (launch_bwd_gemm(BWD_WGRAD, w1g, bwd_wgrad_blocks(num_experts, 2 * inter, hidden), s) !=
      hipSuccess)
    return NVFP4_HIP_ERROR;
  if (mark(7) != hipSuccess) return NVFP4_HIP_ERROR;
  return NVFP4_OK;
}

int nvfp4_pack_weights(const uint8_t* codes, const uint8_t* scales, int32_t num_groups,
                       int64_t n, int64_t k, uint8_t* packed_codes, uint8_t* packed_scales,
                       void* stream) {
  if (!codes || !scales || !packed_codes || !packed_scales) return NVFP4_INVALID_ARGUMENT;
  if (num_groups < 1 || n < 0 || k < 0) return NVFP4_INVALID_ARGUMENT;
  if (n % 32 != 0 || k % 128 != 0 || k > kMaxK) return NVFP4_UNSUPPORTED;
  if ((int64_t)num_groups * n >= 0x7FFFFFFFLL) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(codes, 16) || !aligned(packed_codes, 16) || !aligned(scales, 4) ||
      !aligned(packed_scales, 4))
    return NVFP4_INVALID_ARGUMENT;
  return hip_status(launch_pack_b(codes, scales, (int64_t)num_groups * n, k, packed_codes,
                                  packed_scales, static_cast<hipStream_t>(stream)));
}

int nvfp4_event_create(void** event) {
  if (!event) return NVFP4_INVALID_ARGUMENT;
  hipEvent_t ev;
  if (hipEventCreate(&ev) != hipSuccess) return NVFP4_HIP_ERROR;
  *event = ev;
  return NVFP4_OK;
}

int nvfp4_event_record(void* event, void* stream) {
  if (!event) return NVFP4_INVALID_ARGUMENT;
  return hip_status(hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream)));
}

int nvfp4_event_elapsed_ms(void* start, void* stop, float* ms) {
  if (!start || !stop || !ms) return NVFP4_INVALID_ARGUMENT;
  return hip_status(hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)));
}

int nvfp4_event_destroy(void* event) {
  if (!event) return NVFP4_INVALID_ARGUMENT;
  return hip_status(hipEventDestroy(static_cast<hipEvent_t>(event)));
}

size_t moe_expert_forward_single_pass_workspace_size(int64_t tokens, int64_t hidden,
                                                     int64_t inter, int32_t topk,
                                                     int32_t num_experts, int32_t align) {
  if (!route_args_ok(tokens, topk, num_experts, align) || hidden < 0 || inter < 0) return 0;
  return carve_single_pass(nullptr, tokens, hidden, inter, topk, num_experts, align).bytes;
}

int moe_expert_forward_single_pass(const uint16_t* x, int64_t tokens, int64_t hidden,
                                   int64_t inter, const int32_t* topk_idx,
                                   const float* topk_prob, int32_t topk, int32_t num_experts,
                                   int32_t align, const nvfp4_weights* w1,
                                   const nvfp4_weights* w2, uint16_t* y, void* workspace,
                                   size_t workspace_bytes,
                                   const nvfp4_single_pass_intermediates* debug,
                                   void* const* stage_events, void* stream) {
  if (!route_args_ok(tokens, topk, num_experts, align)) return NVFP4_INVALID_ARGUMENT;
  if (hidden < 128 || hidden % 128 != 0 || inter < 128 || inter % 128 != 0)
    return NVFP4_UNSUPPORTED;
  if (hidden > kMaxK || inter > 1152) return NVFP4_UNSUPPORTED;   // on-chip FC2 input (LDS)
  if (!w1 || !w2 || !w1->codes || !w1->scales || !w1->gscale || !w2->codes || !w2->scales ||
      !w2->gscale || !workspace)
    return NVFP4_INVALID_ARGUMENT;
  if ((w1->layout != 0 && w1->layout != 1) || (w2->layout != 0 && w2->layout != 1))
    return NVFP4_INVALID_ARGUMENT;
  if (tokens > 0 && (!x || !y || !topk_idx || !topk_prob)) return NVFP4_INVALID_ARGUMENT;
  if (!aligned(workspace, 256) || (x && !aligned(x, 16)) || (y && !aligned(y, 16)) ||
      !aligned(w1->codes, 16) || !aligned(w2->codes, 16) || !aligned(w1->scales, 4) ||
      !aligned(w2->scales, 4))
    return NVFP4_INVALID_ARGUMENT;
  if ((int64_t)num_experts * 2 * inter >= 0x7FFFFFFFLL ||
      (int64_t)num_experts * hidden >= 0x7FFFFFFFLL)
    return NVFP4_INVALID_ARGUMENT;
  if ((tokens + 1) * (hidden / 2) > 0xFFFFFFFFLL) return NVFP4_UNSUPPORTED;
  if (2 * inter * (hidden / 2) > 0xFFFFFFFFLL || hidden * (inter / 2) > 0xFFFFFFFFLL)
    return NVFP4_UNSUPPORTED;
  SpLayout L = carve_single_pass(workspace, tokens, hidden, inter, topk, num_experts, align);
  if (workspace_bytes < L.bytes) return NVFP4_WORKSPACE_TOO_SMALL;
  const int64_t cap = moe_rows_capacity(tokens, topk, num_experts, align);
  float* y_f32 = nullptr;
  SinglePassArgs sp{};
  if (debug) {
    if ((debug->a1_codes != nullptr) != (debug->a1_scales != nullptr)) return NVFP4_INVALID_ARGUMENT;
    if (debug->expert_offsets) L.offsets = debug->expert_offsets;
    if (debug->dst_row) L.dst_row = debug->dst_row;
    if (debug->row_src) L.row_src = debug->row_src;
    if (debug->row_prob) L.row_prob = debug->row_prob;
    if (debug->y_rows) L.y_rows = debug->y_rows;
    y_f32 = debug->y_rows_f32;
    sp.c_out = debug->fc1_out; sp.p_out = debug->p;
    sp.a2c_out = debug->a2_codes; sp.a2s_out = debug->a2_scales; sp.gs_out = debug->gs_tiles;
    const void* ptrs16[] = {debug->a1_codes, L.y_rows, y_f32};
    for (const void* q : ptrs16)
      if (q && !aligned(q, 16)) return NVFP4_INVALID_ARGUMENT;
    if (debug->a2_codes && !aligned(debug->a2_codes, 8)) return NVFP4_INVALID_ARGUMENT;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    if (!stage_events || !stage_events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s);
  };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return NVFP4_HIP_ERROR;
  RouteArgs ra{};
  ra.x = x; ra.tokens = tokens; ra.hidden = hidden;
  ra.topk_idx = topk_idx; ra.topk_prob = topk_prob; ra.topk = topk;
  ra.num_experts = num_experts; ra.align = align;
  ra.offsets = L.offsets; ra.dst_row = L.dst_row; ra.row_src = L.row_src;
  ra.row_prob = L.row_prob; ra.gscale = nullptr;   // the kernel reads tok_gscale through row_src
  ra.tok_codes = L.tokc; ra.tok_scales = L.toks; ra.tok_gscale = L.tokg; ra.entry_rank = L.rank;
  ra.tables[0] = single_pass_table_spec(cap, num_experts, hidden, L.tab);
  ra.num_tables = 1;
  ra.workspace = L.route_ws_i; ra.block_rule = 0;
  if ((e = launch_route(ra, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if (debug) {
    if ((e = launch_gather_rows(L.tokc, L.toks, L.tokg, L.row_src, L.offsets + num_experts, cap,
                                hidden, debug->a1_codes, debug->a1_scales, debug->a1_gscale,
                                s)) != hipSuccess)
      return NVFP4_HIP_ERROR;
  }
  if ((e = mark(1)) != hipSuccess) return NVFP4_HIP_ERROR;
  sp.a_codes = L.tokc; sp.a_scales = L.toks; sp.a_gscale = L.tokg;
  sp.a_row_src = L.row_src; sp.a_pad_row = tokens; sp.row_prob = L.row_prob;
  sp.w1_codes = w1->codes; sp.w1_scales = w1->scales; sp.w1_gscale = w1->gscale;
  sp.w1_layout = w1->layout;
  sp.w2_codes = w2->codes; sp.w2_scales = w2->scales; sp.w2_gscale = w2->gscale;
  sp.w2_layout = w2->layout;
  sp.hidden = hidden; sp.inter = inter; sp.tile_table = L.tab;
  sp.y_bf16 = L.y_rows; sp.y_f32 = y_f32;
  if ((e = launch_single_pass(sp, L.blocks, s)) != hipSuccess) return NVFP4_HIP_ERROR;
  if ((e = mark(2)) != hipSuccess) return NVFP4_HIP_ERROR;
  if ((e = launch_combine(y_f32 ? static_cast<const void*>(y_f32) : L.y_rows, y_f32 ? 0 : 1,
                          L.dst_row, tokens, topk, hidden, y, s)) != hipSuccess)
    return NVFP4_HIP_ERROR;
  if ((e = mark(3)) != hipSuccess) return NVFP4_HIP_ERROR;
  return NVFP4_OK;
}

}  // extern "C"
