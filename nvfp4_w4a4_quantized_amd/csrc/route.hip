// route.hip -- MoE routing permutation fused with per-token NVFP4
// quantization (miniTE Technical Report §5.2: contiguous expert-major buffers
// with device-side offsets, zero-token experts and padding in the same path;
// §5.3: the row amax is collected while the token is being permuted and the
// quantizer reuses it).
//
// Three launches, no host synchronisation:
//   1. hist:    one wave per chunk of 64 tokens counts its entries per expert
//               (LDS histogram) -> hist[chunk][e].
//   2. scan:    one workgroup turns the chunk histograms into
//               base[chunk][e] = offsets[e] + #entries of e in earlier chunks,
//               counts[e], and offsets[] (exclusive scan of counts rounded up
//               to `align`).
//   3. scatter: one wave per token quantizes the token once (row amax, block
//               scales, codes in registers) and writes it to each of its k
//               destination rows.  The rank of token t inside expert e is
//               base[chunk][e] + popcount of the chunk's ballot mask of
//               tokens choosing e below t: a stable order (ascending token)
//               without any order-dependent atomics.  Extra waves (one per
//               expert) fill the padding rows.
#include "launch.h"
#include "nvfp4_device.h"

namespace nvfp4 {

constexpr int kChunk = 64;          // tokens per chunk = lanes of one wave
constexpr int kScanThreads = 1024;

int64_t route_num_chunks(int64_t tokens) { return (tokens + kChunk - 1) / kChunk; }

// workspace: base[nchunks][E] int32, counts[E] int32 (each 256-byte aligned)
size_t route_workspace_bytes(int64_t tokens, int32_t num_experts) {
  size_t base = (size_t)route_num_chunks(tokens) * (size_t)num_experts * 4u;
  base = (base + 255u) & ~(size_t)255u;
  size_t counts = ((size_t)num_experts * 4u + 255u) & ~(size_t)255u;
  return base + counts;
}

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
      for (int j = 0; j < topk; ++j) {
        int e = idx[t * topk + j];
        if (e >= 0 && e < E) atomicAdd(h + e, 1);
      }
    }
  }
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < E; e += kWave) hist[chunk * E + e] = h[e];
}

// Single workgroup.  Thread (part, e) handles chunks [part*L, (part+1)*L).
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int32_t* hist, int64_t nchunks,
                                                                  int32_t E, int32_t align,
                                                                  int32_t* counts,
                                                                  int32_t* offsets) {
  __shared__ int32_t partial[kScanThreads];
  __shared__ int32_t cnt[1024];
  __shared__ int32_t off[1025];
  __shared__ int32_t wsum[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int parts = kScanThreads / E;            // >= 1 since E <= 1024
  const int e = tid % E, part = tid / E;
  const bool active = part < parts;
  const int64_t L = (nchunks + parts - 1) / parts;
  const int64_t c0 = active ? (int64_t)part * L : 0;
  const int64_t c1 = active ? ((c0 + L < nchunks) ? c0 + L : nchunks) : 0;
  int32_t s = 0;
  for (int64_t c = c0; c < c1; ++c) s += hist[c * E + e];
  partial[tid] = active ? s : 0;
  __syncthreads();
  int32_t before = 0;
  if (active) {
    for (int p = 0; p < part; ++p) before += partial[p * E + e];
    if (part == 0) {
      int32_t total = 0;
      for (int p = 0; p < parts; ++p) total += partial[p * E + e];
      cnt[e] = total;
    }
  }
  __syncthreads();
  // exclusive scan of padded counts over experts (E <= 1024 = block size)
  int32_t v = 0;
  if (tid < E) v = (cnt[tid] + align - 1) / align * align;
  const int lane = tid & (kWave - 1), w = tid / kWave;
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int32_t y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int32_t ws = (lane < kScanThreads / kWave) ? wsum[lane] : 0;
    int32_t wi = ws;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      int32_t y = __shfl_up(wi, o, kWave);
      if (lane >= o) wi += y;
    }
    if (lane < kScanThreads / kWave) wsum[lane] = wi - ws;   // exclusive
  }
  __syncthreads();
  const int32_t excl = incl - v + wsum[w];
  if (tid < E) {
    off[tid] = excl;
    offsets[tid] = excl;
    counts[tid] = cnt[tid];
    if (tid == E - 1) { off[E] = excl + v; offsets[E] = excl + v; }
  }
  __syncthreads();
  if (active) {
    int32_t run = off[e] + before;
    for (int64_t c = c0; c < c1; ++c) {
      int32_t h = hist[c * E + e];
      hist[c * E + e] = run;
      run += h;
    }
  }
}

template <int BPL, int KMAX>
__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a, const int32_t* base,
                                                            const int32_t* counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  const int k = a.topk, E = a.num_experts;
  const int64_t H = a.hidden;
  if (wid >= a.tokens) {
    // padding rows of expert e: [offsets[e] + counts[e], offsets[e+1])
    const int64_t e = wid - a.tokens;
    if (e >= E) return;
    const int64_t r0 = (int64_t)a.offsets[e] + counts[e], r1 = a.offsets[e + 1];
    for (int64_t r = r0; r < r1; ++r) {
      if (lane == 0) {
        a.row_src[r] = -1;
        a.row_prob[r] = 0.0f;
        if (a.zero_per_row) a.zero_per_row[r] = 0.0f;
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
  const int64_t t = wid;
  const int64_t chunk = t / kChunk;
  const int pos = (int)(t % kChunk);
  const int64_t tl = chunk * kChunk + lane;            // token of this lane in the chunk
  const bool lane_valid = tl < a.tokens;

  // quantize the token once
  const int nblocks = (int)(H / 16);
  uint32_t w[BPL][8];
  uint2 codes[BPL];
  uint32_t sbytes[BPL];
  float s_g = 0.0f;
  if (a.x) {
    const uint16_t* xr = a.x + t * H;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const int b = lane + kWave * i;
      if (b < nblocks) {
        const uint16_t* p = xr + (int64_t)b * 16;
        u32x4_t u0 = load_stream16(p);
        u32x4_t u1 = load_stream16(p + 8);
        w[i][0] = u0.x; w[i][1] = u0.y; w[i][2] = u0.z; w[i][3] = u0.w;
        w[i][4] = u1.x; w[i][5] = u1.y; w[i][6] = u1.z; w[i][7] = u1.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) w[i][j] = 0u;
      }
    }
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      const uint32_t mi = bf16_absmax_bits(w[i]);
      m = m > mi ? m : mi;
    }
    const float amax = __uint_as_float(wave_max_u32(m) << 16);
    s_g = amax / 2688.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      codes[i] = quantize_block16(w[i], s_g, &sbytes[i]);
    }
  }

  // Destination row of each of the token's k entries.  With KMAX > 0 every
  // lane first holds the k expert ids of its own chunk token in registers, so
  // the ballots need no memory traffic; the current token's ids come from
  // lane `pos` by a shuffle.
  auto store_row = [&](int j, int64_t dst) {
    if (lane == 0) a.dst_row[t * k + j] = (int32_t)dst;
    if (dst < 0) return;
    if (lane == 0) {
      a.row_src[dst] = (int32_t)t;
      a.row_prob[dst] = a.topk_prob[t * k + j];
      if (a.zero_per_row) a.zero_per_row[dst] = 0.0f;
      if (a.x) a.gscale[dst] = s_g;
    }
    if (a.x) {
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
    }
  };
  const uint64_t below_mask = pos == 0 ? 0ull : ((1ull << pos) - 1ull);
  if constexpr (KMAX > 0) {
    int ids[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) ids[i] = (lane_valid && i < k) ? a.topk_idx[tl * k + i] : -1;
    int64_t dsts[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      dsts[j] = -1;
      if (j < k) {
        const int e = __shfl(ids[j], pos, kWave);
        if (e >= 0 && e < E) {
          bool hit = false;
#pragma unroll
          for (int i = 0; i < KMAX; ++i) hit |= (ids[i] == e);
          const uint64_t mask = __ballot(hit);
          dsts[j] = (int64_t)base[chunk * E + e] + __popcll(mask & below_mask);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) store_row(j, dsts[j]);
  } else {
    for (int j = 0; j < k; ++j) {
      const int e = a.topk_idx[t * k + j];
      int64_t dst = -1;
      if (e >= 0 && e < E) {
        bool hit = false;
        if (lane_valid)
          for (int i = 0; i < k; ++i) hit |= (a.topk_idx[tl * k + i] == e);
        const uint64_t mask = __ballot(hit);
        dst = (int64_t)base[chunk * E + e] + __popcll(mask & below_mask);
      }
      store_row(j, dst);
    }
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int64_t nchunks = route_num_chunks(a.tokens);
  const int E = a.num_experts;
  int32_t* base = static_cast<int32_t*>(a.workspace);
  size_t base_bytes = ((size_t)nchunks * (size_t)E * 4u + 255u) & ~(size_t)255u;
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) + base_bytes);
  if (nchunks > 0) {
    route_hist_kernel<<<(unsigned)((nchunks + 3) / 4), 256, 4 * E * sizeof(int32_t), s>>>(
        a.topk_idx, a.tokens, a.topk, E, nchunks, base);
  }
  route_scan_kernel<<<1, kScanThreads, 0, s>>>(base, nchunks, E, a.align, counts, a.offsets);
  const int64_t waves = a.tokens + E;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  int bpl = a.x ? blocks_per_lane(a.hidden) : 1;
  const int kmax = a.topk <= 8 ? 8 : (a.topk <= 16 ? 16 : 0);
  switch (bpl * 100 + kmax) {
#define NVFP4_SCATTER(B, KM) \
    case B * 100 + KM: route_scatter_kernel<B, KM><<<grid, block, 0, s>>>(a, base, counts); break;
    NVFP4_SCATTER(1, 8) NVFP4_SCATTER(2, 8) NVFP4_SCATTER(4, 8) NVFP4_SCATTER(8, 8) NVFP4_SCATTER(16, 8)
    NVFP4_SCATTER(1, 16) NVFP4_SCATTER(2, 16) NVFP4_SCATTER(4, 16) NVFP4_SCATTER(8, 16) NVFP4_SCATTER(16, 16)
    NVFP4_SCATTER(1, 0) NVFP4_SCATTER(2, 0) NVFP4_SCATTER(4, 0) NVFP4_SCATTER(8, 0) NVFP4_SCATTER(16, 0)
#undef NVFP4_SCATTER
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
