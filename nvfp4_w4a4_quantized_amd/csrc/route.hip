// route.hip -- MoE routing permutation fused with per-token NVFP4
// quantization (miniTE Technical Report §5.2: contiguous expert-major buffers
// with device-side offsets, zero-token experts and padding in the same path;
// §5.3: the row amax is collected while the token is being permuted and the
// quantizer reuses it).
//
// Three launches, no host synchronisation (one for small batches: see
// kSmallEntries below):
//   1. hist:    one wave per chunk of 64 tokens counts its entries per expert
//               (LDS histogram) -> hist[e][chunk] (expert-major).
//   2. scan:    one workgroup per 8 experts; each derives every expert's
//               total (a thread per expert sums its contiguous row of chunk
//               counts) and offsets[] (exclusive scan of the totals rounded
//               up to `align`), then writes base[e][chunk] = offsets[e] +
//               #entries of e in earlier chunks for its own experts with
//               wave scans along their rows.  It also clears the rows'
//               amax cells that FC1 accumulates into (one coalesced fill).
//   3. scatter: each wave takes TPW consecutive tokens of one chunk.  It
//               quantizes a token once (row amax, block scales, codes in
//               registers) while the next token's row is already loading, and
//               writes it to each of the token's k destination rows.  The
//               rank of token t inside expert e is base[e][chunk] + popcount
//               of the chunk's ballot mask of tokens choosing e below t: a
//               stable order (ascending token) without any order-dependent
//               atomics.  Extra waves (one per expert) fill the padding rows.
//
// The expert layer's gather mode (tok_codes set) quantizes each token once
// into a token-major row and writes only the row maps.  Two launches while
// the chunk-count matrix is small enough for every workgroup to read it
// whole (kFusedScanInts): the ranked histogram (route_hist_rank_kernel),
// then route_scan_entries_kernel (each workgroup repeats the scan's totals,
// then writes the entries, padding rows or tile tables; the others quantize
// the tokens).
// Larger matrices take three: histogram, scan + the quantization, entries.
#include "launch.h"
#include "nvfp4_device.h"

namespace nvfp4 {

constexpr int kChunk = 64;          // tokens per chunk = lanes of one wave
constexpr int kScanThreads = 256;

int64_t route_num_chunks(int64_t tokens) { return (tokens + kChunk - 1) / kChunk; }

// workspace: the precondition word (uint32, in a 256-byte slot of its own),
// hist[E][nchunks] int32, base[E][nchunks] int32, counts[E] int32 (each
// 256-byte aligned)
constexpr size_t kErrorSlot = 256;
static size_t route_matrix_bytes(int64_t tokens, int32_t num_experts) {
  const size_t m = (size_t)route_num_chunks(tokens) * (size_t)num_experts * 4u;
  return (m + 255u) & ~(size_t)255u;
}

size_t route_workspace_bytes(int64_t tokens, int32_t num_experts) {
  size_t counts = ((size_t)num_experts * 4u + 255u) & ~(size_t)255u;
  return kErrorSlot + 2 * route_matrix_bytes(tokens, num_experts) + counts;
}

#ifdef NVFP4_DEBUG_CHECKS
// Debug build: data preconditions checked on the device.  Each wave ORs the
// bits of what it found into the workspace's error word (cleared by the
// launch sequence first); nothing else changes, and a violated precondition
// stays fault-free (ranks of duplicated ids stay within the expert's counted
// rows, the quantizer has no value-dependent control flow).
__global__ void clear_word_kernel(uint32_t* word) {
  if (threadIdx.x == 0) *word = 0u;
}

__device__ __forceinline__ void report_bits(uint32_t* word, bool hit, uint32_t bit) {
  if (__ballot(hit) != 0ull && (threadIdx.x & (kWave - 1)) == 0) atomicOr(word, bit);
}

// bf16 pair with an exponent field of all ones (Inf or NaN)
__device__ __forceinline__ bool bf16_pair_nonfinite(uint32_t u) {
  return (u & 0x7F80u) == 0x7F80u || (u & 0x7F800000u) == 0x7F800000u;
}
#endif

// KMAX > 0 (topk <= KMAX): a lane's k expert ids are all requested before
// the first LDS add (a loop over a run-time count would wait for each load).
// Workgroup `wg` (256 threads) counts chunks 4*wg .. 4*wg+3, one per wave;
// lds holds 4*E counters.
template <int KMAX>
__device__ __forceinline__ void hist_chunks(const int32_t* idx, int64_t tokens, int32_t topk,
                                            int32_t E, int64_t nchunks, int32_t* hist,
                                            int64_t wg, int32_t* lds) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  int32_t* h = lds + wave * E;
  for (int e = lane; e < E; e += kWave) h[e] = 0;
  __syncthreads();
  const int64_t chunk = wg * 4 + wave;
  if (chunk < nchunks) {
    const int64_t t = chunk * kChunk + lane;
    if (t < tokens) {
      if constexpr (KMAX > 0) {
        int ids[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) ids[j] = j < topk ? idx[t * topk + j] : -1;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (ids[j] >= 0 && ids[j] < E) atomicAdd(h + ids[j], 1);
      } else {
        for (int j = 0; j < topk; ++j) {
          int e = idx[t * topk + j];
          if (e >= 0 && e < E) atomicAdd(h + e, 1);
        }
      }
    }
  }
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < E; e += kWave) hist[(int64_t)e * nchunks + chunk] = h[e];
}

// Gather mode's histogram: per chunk (one wave, lane = token) a 64-bit mask
// per expert of the chunk's tokens that chose it, built with LDS ORs.  The
// chunk's count for an expert is the mask's popcount, and an entry's stable
// rank among the chunk's entries of its expert (ascending token) is the
// popcount of the mask below its lane, written to rank[t*topk + j].  A token
// naming an expert twice counts once (both entries get one rank: a violated
// precondition stays inside the counted rows).  lds holds 4*E masks.
template <int KMAX>
__device__ __forceinline__ void hist_rank_chunks(const RouteArgs& a, int64_t nchunks,
                                                 int32_t* hist, uint8_t* rank, int64_t wg,
                                                 unsigned long long* lds) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int E = a.num_experts, k = a.topk;
  unsigned long long* m = lds + (size_t)wave * E;
  for (int e = lane; e < E; e += kWave) m[e] = 0ull;
  __syncthreads();
  const int64_t chunk = wg * 4 + wave;
  const int64_t t = chunk * kChunk + lane;
  const bool valid = chunk < nchunks && t < a.tokens;
  const unsigned long long bit = 1ull << lane, below = bit - 1ull;
  auto routed = [&](int e) { return e >= 0 && e < E; };
  if constexpr (KMAX > 0) {
    int ids[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ids[j] = (valid && j < k) ? a.topk_idx[t * k + j] : -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (routed(ids[j])) atomicOr(m + ids[j], bit);
#ifdef NVFP4_DEBUG_CHECKS
    bool dup = false;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
#pragma unroll
      for (int j = i + 1; j < KMAX; ++j) dup |= (routed(ids[i]) && ids[i] == ids[j]);
    report_bits(a.error_word, dup, NVFP4_PRECONDITION_DUPLICATE_EXPERT);
#endif
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (valid && j < k) rank[t * k + j] = routed(ids[j]) ? (uint8_t)__popcll(m[ids[j]] & below) : 0;
  } else {
    bool dup = false;
    if (valid)
      for (int j = 0; j < k; ++j) {
        const int e = a.topk_idx[t * k + j];
        if (!routed(e)) continue;
        atomicOr(m + e, bit);
#ifdef NVFP4_DEBUG_CHECKS
        for (int i = 0; i < j; ++i) dup |= (a.topk_idx[t * k + i] == e);
#endif
      }
#ifdef NVFP4_DEBUG_CHECKS
    report_bits(a.error_word, dup, NVFP4_PRECONDITION_DUPLICATE_EXPERT);
#endif
    (void)dup;
    __syncthreads();
    if (valid)
      for (int j = 0; j < k; ++j) {
        const int e = a.topk_idx[t * k + j];
        rank[t * k + j] = routed(e) ? (uint8_t)__popcll(m[e] & below) : 0;
      }
  }
  if (chunk < nchunks)
    for (int e = lane; e < E; e += kWave) hist[(int64_t)e * nchunks + chunk] = __popcll(m[e]);
}

template <int KMAX>
__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* idx, int64_t tokens,
                                                          int32_t topk, int32_t E,
                                                          int64_t nchunks, int32_t* hist) {
  extern __shared__ int32_t lds[];   // [4 waves][E]
  hist_chunks<KMAX>(idx, tokens, topk, E, nchunks, hist, blockIdx.x, lds);
}

__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v, int lane) {
  (void)lane;
  return (int32_t)wave_incl_scan_dpp((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ int32_t wave_sum_i32(int32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_scan_i32(v, 0), kWave - 1);
}

// Scan: one workgroup per kScanExperts experts.  Every workgroup derives all
// experts' offsets itself (thread e sums expert e's contiguous row of chunk
// counts, then a block scan of the padded totals), then writes the chunk
// bases of its own experts with wave scans along their rows; workgroup 0
// also publishes offsets[] and counts[].  Many small workgroups instead of
// one: the per-expert chains run in parallel.
constexpr int kScanExperts = 8;     // experts whose bases one workgroup writes
constexpr int kScanMaxE = 1024;     // experts per layer (4 per thread)
constexpr int kScanPer = kScanMaxE / kScanThreads;   // experts per thread in the totals
constexpr int kScanWaves = kScanThreads / kWave;

// Expert offsets from the totals tot[i] of experts tid + kScanThreads*i (a
// kScanThreads-thread block): off[e] = exclusive scan, in expert order, of
// the totals rounded up to `align`; off[E] = the padded row count.  The
// thread-major blocks are scanned per i across the workgroup, i in order.
// Ends with a barrier (off is then readable by every thread).
__device__ void block_expert_offsets(const int32_t (&tot)[kScanPer], int32_t E, int32_t align,
                                     int32_t* off, int32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int32_t carry = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    if (kScanThreads * i >= E) break;
    const int32_t pad = (tot[i] + align - 1) / align * align;
    const int32_t incl = wave_incl_scan_i32(pad, lane);
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int32_t before = carry, all = 0;
#pragma unroll
    for (int j = 0; j < kScanWaves; ++j) {
      const int32_t v = wsum[j];
      if (j < w) before += v;
      all += v;
    }
    const int e = tid + kScanThreads * i;
    if (e < E) off[e] = before + incl - pad;
    carry += all;
    __syncthreads();                               // wsum is rewritten next round
  }
  if (tid == 0) off[E] = carry;
  __syncthreads();
}

// zero[0, n) = 0 by workgroups [0, nblocks) of the grid (grid-stride,
// 16-byte stores where aligned)
__device__ __forceinline__ void grid_zero_fill(float* zero, int64_t n, int64_t nblocks) {
  if (!zero || (int64_t)blockIdx.x >= nblocks) return;
  const int64_t nt = nblocks * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = (reinterpret_cast<uintptr_t>(zero) & 15u) == 0 ? n / 4 : 0;
  for (int64_t i = i0; i < n4; i += nt) reinterpret_cast<float4*>(zero)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = 4 * n4 + i0; i < n; i += nt) zero[i] = 0.0f;
}

// The scan of workgroup blockIdx.x of scan_wgs (the kernels below).
__device__ void route_scan_body(const int32_t* hist, int32_t* base, int64_t nchunks, int32_t E,
                                int32_t align, int32_t* counts, int32_t* offsets, float* zero,
                                int64_t nzero, int64_t scan_wgs) {
  constexpr int NWAVES = kScanWaves;
  constexpr int PER = kScanPer;
  __shared__ int32_t off[kScanMaxE + 1];
  __shared__ int32_t wsum[NWAVES];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  grid_zero_fill(zero, nzero, scan_wgs);
  // expert totals: expert e = tid + kScanThreads*i, summed over its row
  int32_t tot[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + kScanThreads * i;
    int32_t t = 0;
    if (e < E) {
      const int32_t* row = hist + (int64_t)e * nchunks;
      int64_t c = 0;
      if ((nchunks & 3) == 0) {                    // rows are 16-byte aligned
        // eight 16-byte loads in flight per step, not one load per wait
        for (; c + 32 <= nchunks; c += 32) {
          int4 q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) q[u] = *reinterpret_cast<const int4*>(row + c + 4 * u);
#pragma unroll
          for (int u = 0; u < 8; ++u) t += q[u].x + q[u].y + q[u].z + q[u].w;
        }
        for (; c < nchunks; c += 4) {
          const int4 q = *reinterpret_cast<const int4*>(row + c);
          t += q.x + q.y + q.z + q.w;
        }
      }
      for (; c < nchunks; ++c) t += row[c];
    }
    tot[i] = t;
  }
  block_expert_offsets(tot, E, align, off, wsum);
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += kScanThreads) offsets[e] = off[e];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + kScanThreads * i;
      if (e < E) counts[e] = tot[i];
    }
  }
  // base[e][c] = offsets[e] + entries of e in chunks before c, for this
  // workgroup's experts (wave w takes experts e0 + w, e0 + w + NWAVES, ...)
  const int e0 = blockIdx.x * kScanExperts;
  for (int e = e0 + w; e < e0 + kScanExperts && e < E; e += NWAVES) {
    const int32_t* row = hist + (int64_t)e * nchunks;
    int32_t* brow = base + (int64_t)e * nchunks;
    int32_t run = off[e];
    for (int64_t c0 = 0; c0 < nchunks; c0 += kWave) {
      const int64_t c = c0 + lane;
      const int32_t x = c < nchunks ? row[c] : 0;
      const int32_t in = wave_incl_scan_i32(x, lane);
      if (c < nchunks) brow[c] = run + in - x;
      run += __builtin_amdgcn_readlane(in, kWave - 1);
    }
  }
}

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(const int32_t* hist, int32_t* base,
                                                                  int64_t nchunks, int32_t E,
                                                                  int32_t align, int32_t* counts,
                                                                  int32_t* offsets, float* zero,
                                                                  int64_t nzero) {
  route_scan_body(hist, base, nchunks, E, align, counts, offsets, zero, nzero, gridDim.x);
}

// tokens per scatter wave (a divisor of kChunk): two while the double-buffered
// row fits the register budget, one for the longest rows
constexpr int tokens_per_wave(int bpl) { return bpl <= 4 ? 2 : 1; }

template <int BPL>
__device__ __forceinline__ void load_token_row(const uint16_t* xr, int nblocks, int lane,
                                               uint32_t (&w)[BPL][8]) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + kWave * i;
    if (b < nblocks) {
      const uint16_t* p = xr + (int64_t)b * 16;
      const u32x4_t u0 = load_stream16(p);
      const u32x4_t u1 = load_stream16(p + 8);
      w[i][0] = u0.x; w[i][1] = u0.y; w[i][2] = u0.z; w[i][3] = u0.w;
      w[i][4] = u1.x; w[i][5] = u1.y; w[i][6] = u1.z; w[i][7] = u1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) w[i][j] = 0u;
    }
  }
}

// One token of the wave's TPW, quantized in registers (row amax, block
// scales, codes): the lane's blocks lane + 64 i.  amax_in (nullable): the
// tensor's amax, used instead of the row's (one outer scale per tensor).
template <int BPL>
__device__ __forceinline__ float quantize_token_regs(const uint32_t (&w)[BPL][8], int rule,
                                                     const float* amax_in, uint2 (&codes)[BPL],
                                                     uint32_t (&sbytes)[BPL]) {
  float amax;
  if (amax_in) {
    amax = *amax_in;
  } else {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint32_t mi = bf16_absmax_bits(w[i]);
      m = m > mi ? m : mi;
    }
    amax = __uint_as_float(wave_max_u32(m) << 16);
  }
  const float s_g = outer_scale(amax, rule);
#pragma unroll
  for (int i = 0; i < BPL; ++i) codes[i] = quantize_block16(w[i], s_g, rule, &sbytes[i]);
  return s_g;
}

// The quantized token into a row of `codes` / `scales` (all lanes).
template <int BPL>
__device__ __forceinline__ void store_token_row(uint8_t* cr, uint8_t* sr, int nblocks, int lane,
                                                const uint2 (&codes)[BPL],
                                                const uint32_t (&sbytes)[BPL]) {
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = lane + kWave * i;
    if (b < nblocks) {
      *reinterpret_cast<uint2*>(cr + (int64_t)b * 8) = codes[i];
      sr[b] = (uint8_t)sbytes[i];
    }
  }
}

// Gather mode: row `tokens` of the token-major rows, which padding rows
// read, set to zero codes and scales (by the wave of the last token).
__device__ __forceinline__ void zero_pad_row(const RouteArgs& a, int lane) {
  const int64_t H = a.hidden;
  uint8_t* cr = a.tok_codes + a.tokens * (H / 2);
  uint8_t* sr = a.tok_scales + a.tokens * (H / 16);
  for (int64_t i = 8 * lane; i < H / 2; i += 8 * kWave)
    *reinterpret_cast<uint2*>(cr + i) = make_uint2(0u, 0u);
  for (int64_t i = lane; i < H / 16; i += kWave) sr[i] = 0;
}

// Gather mode: token t quantized by one wave into its token-major row.
template <int BPL>
__device__ __forceinline__ void quantize_token_wave(const RouteArgs& a, int64_t t) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t H = a.hidden;
  const int nblocks = (int)(H / 16);
  uint32_t w[1][BPL][8];
  load_token_row<BPL>(a.x + t * H, nblocks, lane, w[0]);
#ifdef NVFP4_DEBUG_CHECKS
  {
    bool badx = false;
#pragma unroll
    for (int i = 0; i < BPL; ++i)
#pragma unroll
      for (int u = 0; u < 8; ++u) badx |= bf16_pair_nonfinite(w[0][i][u]);
    report_bits(a.error_word, badx, NVFP4_PRECONDITION_NONFINITE_INPUT);
  }
#endif
  uint2 codes[BPL];
  uint32_t sbytes[BPL];
  const float s_g = quantize_token_regs<BPL>(w[0], a.block_rule, a.tok_amax, codes, sbytes);
  store_token_row<BPL>(a.tok_codes + t * (H / 2), a.tok_scales + t * (H / 16), nblocks, lane,
                       codes, sbytes);
  if (lane == 0) a.tok_gscale[t] = s_g;
  if (t == a.tokens - 1) zero_pad_row(a, lane);
}

// Gather mode, first launch: each workgroup counts four chunks' entries per
// expert and ranks them inside their chunk (hist_rank_chunks).  The tokens
// are quantized in the next launch, beside the scan.
template <int KMAX>
__global__ __launch_bounds__(256) void route_hist_rank_kernel(RouteArgs a, int64_t nchunks,
                                                              int32_t* hist) {
  extern __shared__ unsigned long long lds64[];   // [4 waves][E]
  hist_rank_chunks<KMAX>(a, nchunks, hist, a.entry_rank, blockIdx.x, lds64);
}

// Gather mode, second launch: workgroups [0, scan_wgs) run the scan; the
// others quantize tokens [tq_begin, tokens), one per wave (the scan is a
// short latency-bound chain on a few workgroups).
template <int BPL>
__global__ __launch_bounds__(256) void route_scan_quant_kernel(RouteArgs a, const int32_t* hist,
                                                               int32_t* base, int32_t* counts,
                                                               int64_t nchunks, int64_t scan_wgs,
                                                               int64_t tq_begin) {
  if ((int64_t)blockIdx.x < scan_wgs) {
    route_scan_body(hist, base, nchunks, a.num_experts, a.align, counts, a.offsets,
                    a.zero_per_row, a.zero_rows, scan_wgs);
    return;
  }
  const int64_t t = tq_begin + ((int64_t)blockIdx.x - scan_wgs) * 4 + threadIdx.x / kWave;
  if (t < a.tokens) quantize_token_wave<BPL>(a, t);
}

// Small batches (SMALL: at most kSmallEntries routing entries) run the
// whole permutation in this one launch: every workgroup histograms all the
// expert ids in LDS, also counting those of the tokens before its own chunk
// (a workgroup's 4*TPW tokens lie in one chunk), derives the offsets with
// the block scan, and takes its chunk bases from LDS.  The redundant
// histograms (a few KiB of ids per workgroup) cost less than the two extra
// dependent launches.  Workgroup 0 publishes offsets[].
constexpr int64_t kSmallEntries = 4096;

// Workgroups at the front of the scatter grid that write the GEMMs' tile
// tables (RouteArgs::tables) from the offsets, while the other workgroups
// permute: the tables cost no launch.  First in the grid, they are
// dispatched first.
constexpr int kTableWorkgroups = 16;

template <int BPL, int KMAX, bool SMALL>
__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a, const int32_t* base,
                                                            const int32_t* counts,
                                                            int64_t token_waves, int64_t nchunks,
                                                            int64_t twg) {
  constexpr int TPW = tokens_per_wave(BPL);
  static_assert(kChunk % TPW == 0, "a wave's tokens share one chunk");
  static_assert(kChunk % (4 * TPW) == 0, "a workgroup's tokens share one chunk");
  static_assert(!SMALL || kScanThreads == 256, "the block scan runs on the 256 threads");
  const int lane = threadIdx.x & (kWave - 1);
  // workgroups [0, twg) write the tile tables, the others permute
  const bool table_wg = (int64_t)blockIdx.x < twg;        // uniform per workgroup
  const int64_t bx = table_wg ? 0 : (int64_t)blockIdx.x - twg;
  const int64_t wid = bx * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int k = a.topk, E = a.num_experts;
  const int64_t H = a.hidden;
  __shared__ TileTableLds tls;
  if constexpr (!SMALL) {
    if (table_wg) {                      // offsets come from the scan launch
      build_tile_tables(a.offsets, E, a.tables[0], a.tables[1], a.num_tables,
                        (int64_t)blockIdx.x * 256 + threadIdx.x, twg * 256, tls);
      return;
    }
  }
  const int64_t t0 = wid * TPW;                      // TPW consecutive tokens of one chunk
  const int nt = (wid < token_waves && !table_wg) ? (int)(a.tokens - t0 < TPW ? a.tokens - t0 : TPW) : 0;
  const int nblocks = (int)(H / 16);

  // Phase 1: every load of the wave is issued before any store (a store may
  // alias a later load as far as the compiler knows) and before the first
  // barrier (loads do not move across one): the tokens' rows, the chunk's
  // expert ids, the router weights of the lane's entries and, for small
  // batches, all the routing entries for the histogram.  The kernel then
  // waits for memory once.
  uint32_t w[TPW][BPL][8];
  if (a.x) {
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti)
      if (ti < nt) load_token_row<BPL>(a.x + (t0 + ti) * H, nblocks, lane, w[ti]);
  }
  const int64_t chunk = t0 / kChunk;
  const int64_t tl = chunk * kChunk + lane;          // token of this lane in the chunk
  const bool lane_valid = tl < a.tokens && nt > 0;
  int ids[KMAX > 0 ? KMAX : 1];                      // the expert ids of the lane's chunk token
  float prob_l[TPW];                                 // router weight of entry `lane` of token ti
  // the expert id of entry (lane / k, lane % k) of the wave's tokens
  int ent_e = -1;
  if constexpr (KMAX > 0) {
    if (lane < TPW * k && lane / k < nt) ent_e = a.topk_idx[t0 * k + lane];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ids[i] = (lane_valid && i < k) ? a.topk_idx[tl * k + i] : -1;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) prob_l[ti] = (ti < nt && lane < k) ? a.topk_prob[(t0 + ti) * k + lane] : 0.0f;
  }
  // gather mode after the first launch quantized the tokens: their outer
  // scales become the rows' (x is NULL here)
  float tok_sg[TPW];
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti)
    tok_sg[ti] = (!a.x && a.tok_gscale && ti < nt) ? a.tok_gscale[t0 + ti] : 0.0f;
  constexpr int kHistPer = SMALL ? (int)(kSmallEntries / 256) : 1;   // entries per thread
  int hist_ids[kHistPer];
  if constexpr (SMALL) {
    const int64_t nent = a.tokens * k;
#pragma unroll
    for (int u = 0; u < kHistPer; ++u) {
      const int64_t i = threadIdx.x + 256 * u;
      hist_ids[u] = i < nent ? a.topk_idx[i] : -1;
    }
  }

  // SMALL: per-expert entries (s_cnt), those before the chunk (s_bef, then
  // the chunk bases) and the offsets (s_off), all in LDS
  __shared__ int32_t s_cnt[SMALL ? kScanMaxE : 1], s_bef[SMALL ? kScanMaxE : 1];
  __shared__ int32_t s_off[SMALL ? kScanMaxE + 1 : 1], s_wsum[kScanWaves];
  if constexpr (SMALL) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) { s_cnt[e] = 0; s_bef[e] = 0; }
    __syncthreads();
    const int64_t c0 = (bx * 4 * TPW) / kChunk * kChunk;   // the chunk's first token
    const int64_t nbef = (c0 < a.tokens ? c0 : a.tokens) * k;
#pragma unroll
    for (int u = 0; u < kHistPer; ++u) {
      const int64_t i = tid + 256 * u;
      const int e = hist_ids[u];
      if (e >= 0 && e < E) {
        atomicAdd(s_cnt + e, 1);
        if (i < nbef) atomicAdd(s_bef + e, 1);
      }
    }
    __syncthreads();
    int32_t tot[kScanPer];
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int e = tid + 256 * i;
      tot[i] = e < E ? s_cnt[e] : 0;
    }
    block_expert_offsets(tot, E, a.align, s_off, s_wsum);
    for (int e = tid; e < E; e += 256) s_bef[e] += s_off[e];
    if (blockIdx.x == 0)
      for (int e = tid; e <= E; e += 256) a.offsets[e] = s_off[e];
    __syncthreads();
  }
  if constexpr (SMALL) {
    grid_zero_fill(a.zero_per_row, a.zero_rows, gridDim.x);
    if (table_wg) {                      // offsets from this workgroup's own histogram
      build_tile_tables(s_off, E, a.tables[0], a.tables[1], a.num_tables,
                        (int64_t)blockIdx.x * 256 + threadIdx.x, twg * 256, tls);
      return;
    }
  }
  auto chunk_base = [&](int e, int64_t chunk) -> int64_t {
    if constexpr (SMALL) return s_bef[e];
    else return base[(int64_t)e * nchunks + chunk];
  };

  if (wid >= token_waves) {
    // padding rows of expert e: [offsets[e] + counts[e], offsets[e+1])
    const int64_t e = wid - token_waves;
    if (e >= E) return;
    const int64_t r0 = SMALL ? (int64_t)s_off[e] + s_cnt[e] : (int64_t)a.offsets[e] + counts[e];
    const int64_t r1 = SMALL ? s_off[e + 1] : a.offsets[e + 1];
    for (int64_t r = r0; r < r1; ++r) {
      if (lane == 0) {
        if (a.row_src) a.row_src[r] = -1;
        a.row_prob[r] = 0.0f;
        if ((a.x || a.tok_gscale) && a.gscale) a.gscale[r] = 0.0f;
      }
      if (a.x && !a.tok_codes) {
        uint8_t* cr = a.codes + r * (H / 2);
        for (int64_t i = lane * 8; i < H / 2; i += kWave * 8)
          *reinterpret_cast<uint2*>(cr + i) = make_uint2(0u, 0u);
        uint8_t* sr = a.scales + r * (H / 16);
        for (int64_t i = lane; i < H / 16; i += kWave) sr[i] = 0;
      }
    }
    return;
  }
  // destination of entry j of token ti is held by lane j (lanes < k)
  int64_t dst_l[TPW];
  if constexpr (KMAX > 0) {
    // Lane L < TPW*k holds entry (L / k, L % k) of the wave's tokens: its
    // expert id (loaded in phase 1) and that expert's chunk base, one load
    // instruction for the whole wave.  The ballots then need no memory
    // traffic: every lane holds the k expert ids of its own chunk token.
    int64_t base_l = 0;
    if (ent_e >= 0 && ent_e < E) base_l = chunk_base(ent_e, chunk);
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      dst_l[ti] = -1;
      const int pos = (int)((t0 + ti) % kChunk);
      const uint64_t below_mask = pos == 0 ? 0ull : ((1ull << pos) - 1ull);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k && ti < nt) {
          const int src = ti * k + j;
          const int e = __builtin_amdgcn_readlane(ent_e, src);
          if (e >= 0 && e < E) {
            bool hit = false;
#pragma unroll
            for (int i = 0; i < KMAX; ++i) hit |= (ids[i] == e);
            const uint64_t mask = __ballot(hit);
            const int64_t b = (int64_t)__builtin_amdgcn_readlane((int)base_l, src);
            const int64_t d = b + __popcll(mask & below_mask);
            if (lane == j) dst_l[ti] = d;
          }
        }
      }
    }
  } else {
    // any k: the entries are resolved one by one in phase 2
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) dst_l[ti] = -1;
  }

#ifdef NVFP4_DEBUG_CHECKS
  {
    // one token naming an expert twice; a non-finite router weight; a
    // non-finite activation (all of the wave's tokens)
    bool dup = false, badp = false, badx = false;
    if constexpr (KMAX > 0) {
      if (lane_valid && tl >= t0 && tl < t0 + nt) {
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
#pragma unroll
          for (int j = i + 1; j < KMAX; ++j)
            dup |= (j < k && ids[i] >= 0 && ids[i] < E && ids[i] == ids[j]);
      }
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti) badp |= (ti < nt && lane < k && !__builtin_isfinite(prob_l[ti]));
    } else {
      for (int ti = 0; ti < nt; ++ti) {
        const int32_t* row = a.topk_idx + (t0 + ti) * k;
        for (int j = lane; j < k; j += kWave) {
          const int e = row[j];
          badp |= !__builtin_isfinite(a.topk_prob[(t0 + ti) * k + j]);
          if (e < 0 || e >= E) continue;
          for (int i = 0; i < j; ++i) dup |= (row[i] == e);
        }
      }
    }
    if (a.x) {
#pragma unroll
      for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
        for (int i = 0; i < BPL; ++i)
#pragma unroll
          for (int u = 0; u < 8; ++u) badx |= (ti < nt && bf16_pair_nonfinite(w[ti][i][u]));
    }
    report_bits(a.error_word, dup, NVFP4_PRECONDITION_DUPLICATE_EXPERT);
    report_bits(a.error_word, badp, NVFP4_PRECONDITION_NONFINITE_PROB);
    report_bits(a.error_word, badx, NVFP4_PRECONDITION_NONFINITE_INPUT);
  }
#endif

  // Phase 2: quantize each token once, then write its k rows and maps
#pragma unroll
  for (int ti = 0; ti < TPW; ++ti) {
    if (ti >= nt) break;
    const int64_t t = t0 + ti;
    uint2 codes[BPL];
    uint32_t sbytes[BPL];
    float s_g = tok_sg[ti];
    if (a.x) {
      s_g = quantize_token_regs<BPL>(w[ti], a.block_rule, a.tok_amax, codes, sbytes);
      // gather mode: the token's one quantized row (the GEMM reads it through
      // row_src); otherwise a copy per destination row below
      if (a.tok_codes) {
        store_token_row<BPL>(a.tok_codes + t * (H / 2), a.tok_scales + t * (H / 16), nblocks,
                             lane, codes, sbytes);
        if (lane == 0) a.tok_gscale[t] = s_g;
        if (t == a.tokens - 1) zero_pad_row(a, lane);
      }
    }
    // the quantized token into row dst (all lanes)
    auto store_row = [&](int64_t dst) {
      if (dst < 0 || !a.x || a.tok_codes) return;
      store_token_row<BPL>(a.codes + dst * (H / 2), a.scales + dst * (H / 16), nblocks, lane,
                           codes, sbytes);
    };
    // the maps of entry j (router weight p), by the lane that holds it
    auto store_meta = [&](int j, int64_t dst, float p) {
      a.dst_row[t * k + j] = (int32_t)dst;
      if (dst < 0) return;
      if (a.row_src) a.row_src[dst] = (int32_t)t;
      a.row_prob[dst] = p;
      if ((a.x || a.tok_gscale) && a.gscale) a.gscale[dst] = s_g;
    };
    if constexpr (KMAX > 0) {
      if (lane < k) store_meta(lane, dst_l[ti], prob_l[ti]);
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) store_row(__shfl(dst_l[ti], j, kWave));
    } else {
      const int pos = (int)(t % kChunk);
      const uint64_t below_mask = pos == 0 ? 0ull : ((1ull << pos) - 1ull);
      for (int j = 0; j < k; ++j) {
        const int e = a.topk_idx[t * k + j];
        int64_t dst = -1;
        if (e >= 0 && e < E) {
          bool hit = false;
          if (lane_valid)
            for (int i = 0; i < k; ++i) hit |= (a.topk_idx[tl * k + i] == e);
          const uint64_t mask = __ballot(hit);
          dst = chunk_base(e, chunk) + __popcll(mask & below_mask);
        }
        if (lane == 0) store_meta(j, dst, a.topk_prob[t * k + j]);
        store_row(dst);
      }
    }
  }
}

// Gather mode, third launch of the three-launch path.  Workgroups [0, twg)
// write the tile tables.  Then one thread per routing entry i = t*topk + j:
// its row is dst = base[e][chunk of t] + its rank inside the chunk, and it
// writes dst_row[i], row_src[dst] = t and row_prob[dst] (the GEMMs read a
// row's outer scale through row_src).  The last workgroups give one wave per expert for
// its padding rows [offsets[e] + counts[e], offsets[e+1]).
__global__ __launch_bounds__(256) void route_entries_kernel(RouteArgs a, const int32_t* base,
                                                            const int32_t* counts,
                                                            int64_t nchunks, int64_t entry_wgs,
                                                            int64_t twg) {
  __shared__ TileTableLds tls;
  if ((int64_t)blockIdx.x < twg) {
    // one table per workgroup: the first third of them write table 0 (FC1),
    // the rest table 1 (FC2, about twice the entries), side by side
    const int64_t w0 = a.num_tables > 1 ? twg / 3 : twg;
    const int64_t b = blockIdx.x;
    if (b < w0)
      build_tile_tables(a.offsets, a.num_experts, a.tables[0], a.tables[0], 1,
                        b * 256 + threadIdx.x, w0 * 256, tls);
    else
      build_tile_tables(a.offsets, a.num_experts, a.tables[1], a.tables[1], 1,
                        (b - w0) * 256 + threadIdx.x, (twg - w0) * 256, tls);
    return;
  }
  const int64_t bx = (int64_t)blockIdx.x - twg;
  const int E = a.num_experts, k = a.topk;
  if (bx < entry_wgs) {
    const int64_t i = bx * 256 + threadIdx.x;
    const bool live = i < a.tokens * k;
    const int64_t t = live ? i / k : 0;
    const int e = live ? a.topk_idx[i] : -1;
    const float p = live ? a.topk_prob[i] : 0.0f;
#ifdef NVFP4_DEBUG_CHECKS
    report_bits(a.error_word, live && !__builtin_isfinite(p), NVFP4_PRECONDITION_NONFINITE_PROB);
#endif
    if (!live) return;
    int64_t d = -1;
    if (e >= 0 && e < E) {
      d = (int64_t)base[(int64_t)e * nchunks + t / kChunk] + a.entry_rank[i];
      a.row_src[d] = (int32_t)t;
      a.row_prob[d] = p;
    }
    a.dst_row[i] = (int32_t)d;
    return;
  }
  const int64_t e = (bx - entry_wgs) * 4 + threadIdx.x / kWave;
  if (e >= E) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r1 = a.offsets[e + 1];
  for (int64_t r = (int64_t)a.offsets[e] + counts[e] + lane; r < r1; r += kWave) {
    a.row_src[r] = -1;
    a.row_prob[r] = 0.0f;
  }
}

// Gather mode, second and last launch of the two-launch path, taken when
// the chunk-count matrix hist (E x nchunks) is small enough for every
// workgroup to read it whole (kFusedScanInts): the scan, the entries and the
// tile tables in one launch.  Each workgroup derives the expert offsets
// itself: its threads sum contiguous stretches of the expert-major matrix
// into per-expert totals in LDS (entries of the workgroup's own chunk's
// predecessors in a second sum), then a block scan of the padded totals.
// Workgroups [0, twg) then write the tile tables; the next nchunks take one
// chunk each: entry i of token t (chunk c) choosing e goes to row
// off[e] + (entries of e in chunks before c) + its rank inside the chunk.
// Then one wave per expert for its padding rows; all of these clear a slice
// of the rows' amax cells first.  The workgroups past nroute quantize tokens
// [tq_begin, tokens): the entries no longer copy a token's outer scale (the
// GEMMs read it through row_src), so nothing in this launch waits for them.
constexpr int64_t kFusedScanInts = 32768;
constexpr int kEntryPreload = 4;    // entries per thread whose loads overlap the offsets

template <int BPL>
__global__ __launch_bounds__(256) void route_scan_entries_kernel(RouteArgs a, const int32_t* hist,
                                                                 int64_t nchunks, int64_t twg,
                                                                 int64_t nroute, int64_t tq_begin) {
  __shared__ TileTableLds tls;
  __shared__ int32_t off[kScanMaxE + 1];
  __shared__ int32_t tot_s[kScanMaxE], pre_s[kScanMaxE];
  __shared__ int32_t wsum[kScanWaves];
  const int tid = threadIdx.x;
  const int E = a.num_experts, k = a.topk;
  const int64_t bx = blockIdx.x;
  if (bx >= nroute) {    // the quantization of tokens [tq_begin, tokens), one per wave
    const int64_t t = tq_begin + (bx - nroute) * 4 + threadIdx.x / kWave;
    if (t < a.tokens) quantize_token_wave<BPL>(a, t);
    return;
  }
  grid_zero_fill(a.zero_per_row, a.zero_rows, nroute);
  const int64_t chunk = (bx >= twg && bx < twg + nchunks) ? bx - twg : -1;
  // this chunk's entries [i0, i1); the first kEntryPreload per thread load now
  const int64_t i0 = chunk >= 0 ? chunk * kChunk * k : 0;
  const int64_t i1 = chunk >= 0 ? std::min<int64_t>((chunk + 1) * kChunk, a.tokens) * k : 0;
  int pe[kEntryPreload], pr[kEntryPreload];
  float pp[kEntryPreload];
#pragma unroll
  for (int u = 0; u < kEntryPreload; ++u) {
    const int64_t i = i0 + tid + 256 * u;
    const bool live = i < i1;
    pe[u] = live ? a.topk_idx[i] : -1;
    pp[u] = live ? a.topk_prob[i] : 0.0f;
    pr[u] = live ? (int)a.entry_rank[i] : 0;
  }
  for (int e = tid; e < E; e += 256) { tot_s[e] = 0; pre_s[e] = 0; }
  __syncthreads();
  // thread stretch [j0, j1) of the flattened matrix (a multiple of 4 long,
  // so with 4 | nchunks an int4 never crosses a row), walked with its row e
  // and column c (32-bit: E * nchunks <= kFusedScanInts); a stretch spans
  // at most a few rows, each flushed to LDS once
  const int32_t nc = (int32_t)nchunks, cc = (int32_t)chunk;
  const int32_t n = E * nc;
  const int32_t per = (((n + 255) / 256) + 3) & ~3;
  const int32_t j0 = std::min(tid * per, n), j1 = std::min(j0 + per, n);
  int32_t e = j0 / nc, c = j0 - e * nc, ecur = e;
  int32_t st = 0, sp = 0;
  auto flush = [&]() {
    if (st) atomicAdd(&tot_s[ecur], st);
    if (sp) atomicAdd(&pre_s[ecur], sp);
    st = 0; sp = 0;
  };
  if ((nc & 3) == 0) {
    for (int32_t jb = j0; jb < j1; jb += 64) {     // sixteen 16-byte loads in flight
      int4 q[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int32_t j = jb + 4 * u;
        q[u] = j < j1 ? *reinterpret_cast<const int4*>(hist + j) : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (jb + 4 * u >= j1) break;
        if (e != ecur) { flush(); ecur = e; }
        st += q[u].x + q[u].y + q[u].z + q[u].w;
        sp += (c < cc ? q[u].x : 0) + (c + 1 < cc ? q[u].y : 0) + (c + 2 < cc ? q[u].z : 0) +
              (c + 3 < cc ? q[u].w : 0);
        c += 4;
        if (c == nc) { c = 0; ++e; }
      }
    }
  } else {
    for (int32_t j = j0; j < j1; ++j) {
      if (e != ecur) { flush(); ecur = e; }
      const int32_t v = hist[j];
      st += v;
      sp += c < cc ? v : 0;
      if (++c == nc) { c = 0; ++e; }
    }
  }
  flush();
  __syncthreads();
  int32_t tot[kScanPer];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int e = tid + kScanThreads * i;
    tot[i] = e < E ? tot_s[e] : 0;
  }
  block_expert_offsets(tot, E, a.align, off, wsum);
  if (bx == 0)
    for (int e = tid; e <= E; e += 256) a.offsets[e] = off[e];
  if (bx < twg) {
    // as in route_entries_kernel: a third of them write table 0 (FC1)
    const int64_t w0 = a.num_tables > 1 ? twg / 3 : twg;
    if (bx < w0)
      build_tile_tables(off, E, a.tables[0], a.tables[0], 1, bx * 256 + tid, w0 * 256, tls);
    else
      build_tile_tables(off, E, a.tables[1], a.tables[1], 1, (bx - w0) * 256 + tid,
                        (twg - w0) * 256, tls);
    return;
  }
  if (chunk >= 0) {
    // entry i = i0 + l of the chunk: token chunk * kChunk + l / k
    auto place = [&](int64_t i, int32_t l, int e, float p, int r) {
#ifdef NVFP4_DEBUG_CHECKS
      report_bits(a.error_word, !__builtin_isfinite(p), NVFP4_PRECONDITION_NONFINITE_PROB);
#endif
      int64_t d = -1;
      if (e >= 0 && e < E) {
        d = (int64_t)off[e] + pre_s[e] + r;
        a.row_src[d] = (int32_t)(chunk * kChunk + l / k);
        a.row_prob[d] = p;
      }
      a.dst_row[i] = (int32_t)d;
    };
#pragma unroll
    for (int u = 0; u < kEntryPreload; ++u) {
      const int64_t i = i0 + tid + 256 * u;
      if (i < i1) place(i, tid + 256 * u, pe[u], pp[u], pr[u]);
    }
    for (int32_t l = tid + 256 * kEntryPreload; i0 + l < i1; l += 256) {
      const int64_t i = i0 + l;
      place(i, l, a.topk_idx[i], a.topk_prob[i], (int)a.entry_rank[i]);
    }
    return;
  }
  // the expert whose padding rows this wave writes
  const int64_t ep = (bx - twg - nchunks) * 4 + tid / kWave;
  if (ep >= E) return;
  const int lane = tid & (kWave - 1);
  const int64_t r1 = off[ep + 1];
  for (int64_t r = (int64_t)off[ep] + tot_s[ep] + lane; r < r1; r += kWave) {
    a.row_src[r] = -1;
    a.row_prob[r] = 0.0f;
  }
}

// The routed rows of the permuted layout from the token-major rows of gather
// mode (debug intermediates): row r < *rows_end takes token row_src[r]'s
// codes, scales and outer scale, padding rows (row_src < 0) zeros; each
// output is nullable.  One wave per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* tok_codes,
                                                          const uint8_t* tok_scales,
                                                          const float* tok_gscale,
                                                          const int32_t* row_src,
                                                          const int32_t* rows_end, int64_t cap,
                                                          int64_t H, uint8_t* codes,
                                                          uint8_t* scales, float* gscale) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (r >= cap || r >= (int64_t)*rows_end) return;
  const int64_t t = row_src[r];
  if (codes)
    for (int64_t i = 8 * lane; i < H / 2; i += 8 * kWave) {
      const uint2 v = t >= 0 ? *reinterpret_cast<const uint2*>(tok_codes + t * (H / 2) + i)
                             : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(codes + r * (H / 2) + i) = v;
    }
  if (scales)
    for (int64_t i = lane; i < H / 16; i += kWave)
      scales[r * (H / 16) + i] = t >= 0 ? tok_scales[t * (H / 16) + i] : (uint8_t)0;
  if (gscale && lane == 0) gscale[r] = t >= 0 ? tok_gscale[t] : 0.0f;
}

hipError_t launch_gather_rows(const uint8_t* tok_codes, const uint8_t* tok_scales,
                              const float* tok_gscale, const int32_t* row_src,
                              const int32_t* rows_end, int64_t cap, int64_t hidden,
                              uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t s) {
  if (cap <= 0 || (!codes && !scales && !gscale)) return hipSuccess;
  gather_rows_kernel<<<(unsigned)((cap + 3) / 4), 256, 0, s>>>(
      tok_codes, tok_scales, tok_gscale, row_src, rows_end, cap, hidden, codes, scales, gscale);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& args, hipStream_t s) {
  RouteArgs a = args;
  const int64_t nchunks = route_num_chunks(a.tokens);
  const int E = a.num_experts;
  const size_t mbytes = route_matrix_bytes(a.tokens, E);
  char* ws = static_cast<char*>(a.workspace);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + kErrorSlot);
  int32_t* base = reinterpret_cast<int32_t*>(ws + kErrorSlot + mbytes);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + kErrorSlot + 2 * mbytes);
#ifdef NVFP4_DEBUG_CHECKS
  a.error_word = reinterpret_cast<uint32_t*>(ws);
  clear_word_kernel<<<1, 64, 0, s>>>(a.error_word);
#endif
  const bool small = a.tokens * a.topk <= kSmallEntries;
  const bool gather = a.tok_codes != nullptr && a.x != nullptr;
  // gather mode: the tokens are quantized in the second launch, beside the
  // fused launch's scan and entries (or the three-launch form's scan): a
  // latency-bound chain on a few hundred workgroups, which the quantization
  // runs beside, while the histogram launch stays short (the entries read
  // no outer scale, so nothing waits for the quantization)
  const int bpl_g = gather ? blocks_per_lane(a.hidden) : 1;
  const bool fused = gather && (int64_t)E * nchunks <= kFusedScanInts;
  if (!small) {
    if (nchunks > 0) {
      const unsigned hg = (unsigned)((nchunks + 3) / 4);
      const size_t hl = 4 * E * sizeof(int32_t);
      const int kmax = a.topk <= 8 ? 8 : (a.topk <= 16 ? 16 : 0);
      if (gather) {
        // the ranked histogram
        if (bpl_g == 0) return hipErrorInvalidValue;
        const size_t hl64 = 4 * E * sizeof(unsigned long long);
        switch (kmax) {
          case 8: route_hist_rank_kernel<8><<<hg, 256, hl64, s>>>(a, nchunks, hist); break;
          case 16: route_hist_rank_kernel<16><<<hg, 256, hl64, s>>>(a, nchunks, hist); break;
          default: route_hist_rank_kernel<0><<<hg, 256, hl64, s>>>(a, nchunks, hist); break;
        }
      } else if (kmax == 8) {
        route_hist_kernel<8><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
      } else if (kmax == 16) {
        route_hist_kernel<16><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
      } else {
        route_hist_kernel<0><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
      }
    }
    if (fused) {
      // the scan, the entries' rows, the padding rows and the tile tables
      const int64_t twg = a.num_tables > 0 ? 3 * kTableWorkgroups : 0;
      const int64_t nroute = twg + nchunks + (E + 3) / 4;
      const unsigned grid = (unsigned)(nroute + (a.tokens + 3) / 4);
      switch (bpl_g) {
#define NVFP4_SCANE(B) \
        case B: route_scan_entries_kernel<B><<<grid, 256, 0, s>>>(a, hist, nchunks, twg, nroute, 0); break;
        NVFP4_SCANE(1) NVFP4_SCANE(2) NVFP4_SCANE(4) NVFP4_SCANE(8) NVFP4_SCANE(16)
#undef NVFP4_SCANE
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    const int64_t scan_wgs = (E + kScanExperts - 1) / kScanExperts;
    if (gather) {
      const unsigned grid = (unsigned)(scan_wgs + (a.tokens + 3) / 4);
      switch (bpl_g) {
#define NVFP4_SCANQ(B) \
        case B: route_scan_quant_kernel<B><<<grid, 256, 0, s>>>(a, hist, base, counts, nchunks, scan_wgs, 0); break;
        NVFP4_SCANQ(1) NVFP4_SCANQ(2) NVFP4_SCANQ(4) NVFP4_SCANQ(8) NVFP4_SCANQ(16)
#undef NVFP4_SCANQ
        default: return hipErrorInvalidValue;
      }
    } else {
      route_scan_kernel<<<(unsigned)scan_wgs, kScanThreads, 0, s>>>(
          hist, base, nchunks, E, a.align, counts, a.offsets, a.zero_per_row, a.zero_rows);
    }
    if (gather) {
      // the entries' rows from the chunk bases and ranks, the padding rows and
      // the tile tables
      const int64_t entry_wgs = (a.tokens * a.topk + 255) / 256;
      const int64_t twg = a.num_tables > 0 ? 3 * kTableWorkgroups : 0;
      const unsigned grid = (unsigned)(twg + entry_wgs + (E + 3) / 4);
      route_entries_kernel<<<grid, 256, 0, s>>>(a, base, counts, nchunks, entry_wgs, twg);
      return hipGetLastError();
    }
  }
  const int bpl = a.x ? blocks_per_lane(a.hidden) : 1;
  if (bpl == 0) return hipErrorInvalidValue;
  const int tpw = tokens_per_wave(bpl);
  const int64_t token_waves = (a.tokens + tpw - 1) / tpw;
  const int64_t waves = token_waves + E;
  const int64_t permute_wgs = (waves + 3) / 4;
  const int64_t twg = a.num_tables > 0 ? kTableWorkgroups : 0;
  dim3 grid((unsigned)(twg + permute_wgs)), block(256);
  const int kmax = a.topk <= 8 ? 8 : (a.topk <= 16 ? 16 : 0);
  switch (bpl * 100 + kmax) {
#define NVFP4_SCATTER(B, KM) \
    case B * 100 + KM:                                                                              \
      if (small) route_scatter_kernel<B, KM, true><<<grid, block, 0, s>>>(a, base, counts, token_waves, nchunks, twg); \
      else route_scatter_kernel<B, KM, false><<<grid, block, 0, s>>>(a, base, counts, token_waves, nchunks, twg); \
      break;
    NVFP4_SCATTER(1, 8) NVFP4_SCATTER(2, 8) NVFP4_SCATTER(4, 8) NVFP4_SCATTER(8, 8) NVFP4_SCATTER(16, 8)
    NVFP4_SCATTER(1, 16) NVFP4_SCATTER(2, 16) NVFP4_SCATTER(4, 16) NVFP4_SCATTER(8, 16) NVFP4_SCATTER(16, 16)
    NVFP4_SCATTER(1, 0) NVFP4_SCATTER(2, 0) NVFP4_SCATTER(4, 0) NVFP4_SCATTER(8, 0) NVFP4_SCATTER(16, 0)
#undef NVFP4_SCATTER
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
