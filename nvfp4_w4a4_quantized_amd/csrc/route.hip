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
template <int KMAX>
__global__ __launch_bounds__(256) void route_hist_kernel(const int32_t* idx, int64_t tokens,
                                                          int32_t topk, int32_t E,
                                                          int64_t nchunks, int32_t* hist) {
  extern __shared__ int32_t lds[];   // [4 waves][E]
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  int32_t* h = lds + wave * E;
  for (int e = lane; e < E; e += kWave) h[e] = 0;
  __syncthreads();
  const int64_t chunk = (int64_t)blockIdx.x * 4 + wave;
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

// zero[0, n) = 0 by the whole grid (grid-stride, 16-byte stores where aligned)
__device__ __forceinline__ void grid_zero_fill(float* zero, int64_t n) {
  if (!zero) return;
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = (reinterpret_cast<uintptr_t>(zero) & 15u) == 0 ? n / 4 : 0;
  for (int64_t i = i0; i < n4; i += nt) reinterpret_cast<float4*>(zero)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = 4 * n4 + i0; i < n; i += nt) zero[i] = 0.0f;
}

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(const int32_t* hist, int32_t* base,
                                                                  int64_t nchunks, int32_t E,
                                                                  int32_t align, int32_t* counts,
                                                                  int32_t* offsets, float* zero,
                                                                  int64_t nzero) {
  constexpr int NWAVES = kScanWaves;
  constexpr int PER = kScanPer;
  __shared__ int32_t off[kScanMaxE + 1];
  __shared__ int32_t wsum[NWAVES];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  grid_zero_fill(zero, nzero);
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

// Small batches (SMALL: at most kSmallEntries routing entries) run the
// whole permutation in this one launch: every workgroup histograms all the
// expert ids in LDS, also counting those of the tokens before its own chunk
// (a workgroup's 4*TPW tokens lie in one chunk), derives the offsets with
// the block scan, and takes its chunk bases from LDS.  The redundant
// histograms (a few KiB of ids per workgroup) cost less than the two extra
// dependent launches.  Workgroup 0 publishes offsets[].
constexpr int64_t kSmallEntries = 4096;

// Workgroups appended to the scatter grid that write the GEMMs' tile tables
// (RouteArgs::tables) from the offsets, while the other workgroups permute:
// the tables cost no launch and no time on the routing's critical path.
constexpr int kTableWorkgroups = 16;

template <int BPL, int KMAX, bool SMALL>
__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a, const int32_t* base,
                                                            const int32_t* counts,
                                                            int64_t token_waves, int64_t nchunks,
                                                            int64_t table_wg0) {
  constexpr int TPW = tokens_per_wave(BPL);
  static_assert(kChunk % TPW == 0, "a wave's tokens share one chunk");
  static_assert(kChunk % (4 * TPW) == 0, "a workgroup's tokens share one chunk");
  static_assert(!SMALL || kScanThreads == 256, "the block scan runs on the 256 threads");
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int k = a.topk, E = a.num_experts;
  const int64_t H = a.hidden;
  const bool table_wg = (int64_t)blockIdx.x >= table_wg0;   // uniform per workgroup
  __shared__ TileTableLds tls;
  if constexpr (!SMALL) {
    if (table_wg) {                      // offsets come from the scan launch
      const int64_t wg = (int64_t)blockIdx.x - table_wg0;
      build_tile_tables(a.offsets, E, a.tables[0], a.tables[1], a.num_tables, wg * 256 + threadIdx.x,
                        (int64_t)kTableWorkgroups * 256, tls);
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
  if constexpr (KMAX > 0) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ids[i] = (lane_valid && i < k) ? a.topk_idx[tl * k + i] : -1;
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) prob_l[ti] = (ti < nt && lane < k) ? a.topk_prob[(t0 + ti) * k + lane] : 0.0f;
  }
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
    const int64_t c0 = ((int64_t)blockIdx.x * 4 * TPW) / kChunk * kChunk;   // the chunk's first token
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
    grid_zero_fill(a.zero_per_row, a.zero_rows);
    if (table_wg) {                      // offsets from this workgroup's own histogram
      const int64_t wg = (int64_t)blockIdx.x - table_wg0;
      build_tile_tables(s_off, E, a.tables[0], a.tables[1], a.num_tables, wg * 256 + threadIdx.x,
                        (int64_t)kTableWorkgroups * 256, tls);
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
        if (a.x) a.gscale[r] = 0.0f;
      }
      if (a.x) {
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
    // every lane holds the k expert ids of its own chunk token, so the
    // ballots need no memory traffic; a token's ids come from its lane
#pragma unroll
    for (int ti = 0; ti < TPW; ++ti) {
      dst_l[ti] = -1;
      const int pos = (int)((t0 + ti) % kChunk);
      const uint64_t below_mask = pos == 0 ? 0ull : ((1ull << pos) - 1ull);
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k && ti < nt) {
          const int e = __shfl(ids[j], pos, kWave);
          if (e >= 0 && e < E) {
            bool hit = false;
#pragma unroll
            for (int i = 0; i < KMAX; ++i) hit |= (ids[i] == e);
            const uint64_t mask = __ballot(hit);
            const int64_t d = chunk_base(e, chunk) + __popcll(mask & below_mask);
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
    float s_g = 0.0f;
    if (a.x) {
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const uint32_t mi = bf16_absmax_bits(w[ti][i]);
        m = m > mi ? m : mi;
      }
      const float amax = __uint_as_float(wave_max_u32(m) << 16);
      s_g = outer_scale(amax, a.block_rule);
#pragma unroll
      for (int i = 0; i < BPL; ++i) codes[i] = quantize_block16(w[ti][i], s_g, a.block_rule, &sbytes[i]);
    }
    // the quantized token into row dst (all lanes)
    auto store_row = [&](int64_t dst) {
      if (dst < 0 || !a.x) return;
      uint8_t* cr = a.codes + dst * (H / 2);
      uint8_t* sr = a.scales + dst * (H / 16);
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const int b = lane + kWave * i;
        if (b < nblocks) {
          *reinterpret_cast<uint2*>(cr + (int64_t)b * 8) = codes[i];
          sr[b] = (uint8_t)sbytes[i];
        }
      }
    };
    // the maps of entry j (router weight p), by the lane that holds it
    auto store_meta = [&](int j, int64_t dst, float p) {
      a.dst_row[t * k + j] = (int32_t)dst;
      if (dst < 0) return;
      if (a.row_src) a.row_src[dst] = (int32_t)t;
      a.row_prob[dst] = p;
      if (a.x) a.gscale[dst] = s_g;
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
  if (!small) {
    if (nchunks > 0) {
      const unsigned hg = (unsigned)((nchunks + 3) / 4);
      const size_t hl = 4 * E * sizeof(int32_t);
      if (a.topk <= 8)
        route_hist_kernel<8><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
      else if (a.topk <= 16)
        route_hist_kernel<16><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
      else
        route_hist_kernel<0><<<hg, 256, hl, s>>>(a.topk_idx, a.tokens, a.topk, E, nchunks, hist);
    }
    route_scan_kernel<<<(unsigned)((E + kScanExperts - 1) / kScanExperts), kScanThreads, 0, s>>>(
        hist, base, nchunks, E, a.align, counts, a.offsets, a.zero_per_row, a.zero_rows);
  }
  const int bpl = a.x ? blocks_per_lane(a.hidden) : 1;
  if (bpl == 0) return hipErrorInvalidValue;
  const int tpw = tokens_per_wave(bpl);
  const int64_t token_waves = (a.tokens + tpw - 1) / tpw;
  const int64_t waves = token_waves + E;
  const int64_t table_wg0 = (waves + 3) / 4;
  const int64_t twg = a.num_tables > 0 ? kTableWorkgroups : 0;
  dim3 grid((unsigned)(table_wg0 + twg)), block(256);
  const int kmax = a.topk <= 8 ? 8 : (a.topk <= 16 ? 16 : 0);
  switch (bpl * 100 + kmax) {
#define NVFP4_SCATTER(B, KM) \
    case B * 100 + KM:                                                                              \
      if (small) route_scatter_kernel<B, KM, true><<<grid, block, 0, s>>>(a, base, counts, token_waves, nchunks, table_wg0); \
      else route_scatter_kernel<B, KM, false><<<grid, block, 0, s>>>(a, base, counts, token_waves, nchunks, table_wg0); \
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
