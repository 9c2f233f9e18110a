// noalloc.hip -- moe_permute for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the routing scratch lives in a file-scope device array instead
// of a caller workspace.
//
// The array is a host-side stand-in in host code: its device address is
// taken once per device with hipGetSymbolAddress (each GPU holds its own
// copy), and only that address is ever handed to kernels.  Every call on one
// GPU shares that GPU's array, so calls that overlap on one GPU race; the
// routing kernels write every scratch word they later read (histogram,
// chunk bases, counts), so nothing needs clearing between calls.
#include "nvfp4moe.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = NVFP4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on
// the first call on each device).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int moe_permute_noalloc(const uint16_t* x, int64_t tokens, int64_t hidden,
                                   const int32_t* topk_idx, const float* topk_prob,
                                   int32_t topk, int32_t num_experts, int32_t align,
                                   int32_t block_rule, int32_t* expert_offsets, int32_t* dst_row,
                                   int32_t* row_src, float* row_prob, uint8_t* codes,
                                   uint8_t* block_scales, float* global_scales, void* stream) {
  // every host-side check before the first HIP call
  const int st = nvfp4::permute_args_status(x, tokens, hidden, topk_idx, topk_prob, topk,
                                            num_experts, align, block_rule, expert_offsets,
                                            dst_row, row_src, row_prob, codes, block_scales,
                                            global_scales);
  if (st != NVFP4_OK) return st;
  if (moe_permute_workspace_size(tokens, topk, num_experts) > kScratchBytes)
    return NVFP4_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return NVFP4_HIP_ERROR;
  return moe_permute(x, tokens, hidden, topk_idx, topk_prob, topk, num_experts, align, block_rule,
                     expert_offsets, dst_row, row_src, row_prob, codes, block_scales,
                     global_scales, ws, kScratchBytes, stream);
}
