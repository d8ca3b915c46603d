// FP8 dispatch of MoE tokens on one GPU, for gfx950.
//
// "Six Reasons Deepseek Ai Is A Waste Of Time" (the paragraph on the combine
// and dispatch components): activations are quantized to FP8 before the MoE
// up-projections and the dispatch then moves FP8. This is the part of the
// dispatch that stays on a GPU: every token is quantized once (1x128 tiles,
// the activation rule) and its codes and scales are written into the row
// block of each expert the router chose, in the padded per-expert layout of
// the grouped GEMM (rows of expert e from m_offsets[e], blocks rounded up to
// multiples of 128, padding rows zero).
//
// Row order inside an expert's block is slot order, slot = token * k + choice,
// so the layout is deterministic. Five launches:
//   count  per 256-slot block, a histogram of the valid choices (LDS atomics);
//   scan   one workgroup: per-expert totals, padded offsets, and for every
//          (block, expert) the first row that block's slots of that expert take;
//   rank   per block: each wavefront ranks its 64 slots among equal experts
//          (one ballot per distinct expert present), the 4 wavefronts' counts
//          are added in LDS, and row = base + earlier waves + rank;
//   quant  one wavefront per token: read and quantize the token once, store
//          its codes and scales to each of its rows;
//   pad    one workgroup per expert: zero its padding rows.
#include "common.hpp"

namespace fp8q {

constexpr int kDispBlock = 256;      // slots per count/rank block, one per thread
constexpr int kDispWaves = kDispBlock / 64;
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(kDispBlock) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                                    int S, int G,
                                                                    int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < G; e += kDispBlock) h[e] = 0;
  __syncthreads();
  const int slot = blockIdx.x * kDispBlock + threadIdx.x;
  if (slot < S) {
    const int e = ids[slot];
    if (e >= 0 && e < G) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G; e += kDispBlock) hist[(int64_t)blockIdx.x * G + e] = h[e];
}

__global__ __launch_bounds__(kMaxExperts) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int n_blk, int G, int32_t* __restrict__ base,
    int32_t* __restrict__ counts, int32_t* __restrict__ m_offsets) {
  __shared__ int32_t padded[kMaxExperts];
  __shared__ int32_t off[kMaxExperts + 1];
  const int e = threadIdx.x;
  if (e < G) {
    int total = 0;
    for (int b = 0; b < n_blk; ++b) total += hist[(int64_t)b * G + e];
    counts[e] = total;
    padded[e] = (total + kGroup - 1) / kGroup * kGroup;
  }
  __syncthreads();
  if (e == 0) {
    int run = 0;
    for (int i = 0; i < G; ++i) {
      off[i] = run;
      run += padded[i];
    }
    off[G] = run;
  }
  __syncthreads();
  if (e < G) m_offsets[e] = off[e];
  if (e == 0) m_offsets[G] = off[G];
  if (e < G) {
    int run = off[e];
    for (int b = 0; b < n_blk; ++b) {
      const int64_t i = (int64_t)b * G + e;
      const int c = hist[i];
      base[i] = run;
      run += c;
    }
  }
}

__global__ __launch_bounds__(kDispBlock) void dispatch_rank_kernel(const int32_t* __restrict__ ids,
                                                                   int S, int G,
                                                                   const int32_t* __restrict__ base,
                                                                   int32_t* __restrict__ row_of_slot) {
  __shared__ int32_t wave_cnt[kDispWaves * kMaxExperts];  // [wave][expert]
  for (int i = threadIdx.x; i < kDispWaves * G; i += kDispBlock) wave_cnt[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int slot = blockIdx.x * kDispBlock + threadIdx.x;
  const int e = (slot < S) ? ids[slot] : -1;
  const bool valid = e >= 0 && e < G;
  // rank among the earlier lanes of this wavefront that chose the same expert
  int rank = 0;
  uint64_t todo = __ballot(valid);
  while (todo) {  // wave-uniform: one pass per distinct expert in the wavefront
    const int leader = __builtin_ctzll(todo);
    const int el = __builtin_amdgcn_readlane(e, leader);
    const bool mine = valid && e == el;
    const uint64_t m = __ballot(mine);
    if (mine) rank = __popcll(m & ((1ull << lane) - 1));
    if (lane == leader) wave_cnt[w * G + el] = __popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  if (slot < S) {
    int row = -1;
    if (valid) {
      row = base[(int64_t)blockIdx.x * G + e] + rank;
      for (int v = 0; v < w; ++v) row += wave_cnt[v * G + e];
    }
    row_of_slot[slot] = row;
  }
}

// One wavefront per token; a 1x128 tile is 16 chunks of 16 bytes = one DPP
// row of 16 lanes, so 64 lanes quantize 4 tiles per step.
__global__ __launch_bounds__(256) void dispatch_quant_kernel(const uint4* __restrict__ x, int T,
                                                             int K, int k,
                                                             const int32_t* __restrict__ row_of_slot,
                                                             uint2* __restrict__ q,
                                                             float* __restrict__ sa) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  const int n_chunks = K / 8;
  const int G = K / kGroup;
  const uint4* xr = x + (int64_t)t * n_chunks;
  const int32_t* rows = row_of_slot + (int64_t)t * k;
  for (int c0 = 0; c0 < n_chunks; c0 += 64) {
    const int c = c0 + lane;
    const bool have = c < n_chunks;  // whole tiles (DPP rows) are present or absent
    const uint4 v = have ? load_nt(xr + c) : make_uint4(0, 0, 0, 0);
    float m = 0.0f;
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                       fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                       fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
    const float amax = __uint_as_float(row16_max_u32(__float_as_uint(m)));
    const float s = __fdiv_rn(amax, kFp8Max);
    const TileDivisor d = make_divisor(s, amax);
    const uint2 codes = quant8(v, d);
    if (have) {
      for (int j = 0; j < k; ++j) {
        const int row = rows[j];  // same for the whole wavefront
        if (row < 0) continue;   // dropped choice
        q[(int64_t)row * n_chunks + c] = codes;
        if ((lane & 15) == 0) sa[(int64_t)row * G + (c >> 4)] = s;
      }
    }
  }
}

__global__ __launch_bounds__(256) void dispatch_pad_kernel(const int32_t* __restrict__ m_offsets,
                                                           const int32_t* __restrict__ counts,
                                                           int K, uint4* __restrict__ q,
                                                           float* __restrict__ sa) {
  const int e = blockIdx.x;
  const int64_t r0 = (int64_t)m_offsets[e] + counts[e];
  const int64_t n_rows = (int64_t)m_offsets[e + 1] - r0;  // at most 127
  const int n16 = K / 16;
  for (int64_t i = threadIdx.x; i < n_rows * n16; i += 256)
    q[(r0 + i / n16) * n16 + i % n16] = make_uint4(0, 0, 0, 0);
  const int G = K / kGroup;
  for (int64_t i = threadIdx.x; i < n_rows * G; i += 256) sa[(r0 + i / G) * G + i % G] = 0.0f;
}

int64_t dispatch_blocks(int64_t slots) { return (slots + kDispBlock - 1) / kDispBlock; }

int64_t dispatch_workspace_bytes(int64_t slots, int64_t G) {
  return (2 * dispatch_blocks(slots) * G + G) * 4;  // hist, base, counts
}

hipError_t launch_moe_dispatch(const void* x, const int32_t* ids, int64_t T, int64_t K, int64_t k,
                               int64_t G, uint8_t* q, float* sa, int32_t* m_offsets,
                               int32_t* row_of_slot, void* workspace, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t n_blk = dispatch_blocks(S);
  int32_t* hist = (int32_t*)workspace;
  int32_t* base = hist + n_blk * G;
  int32_t* counts = base + n_blk * G;
  if (n_blk > 0)
    hipLaunchKernelGGL(dispatch_count_kernel, dim3((unsigned)n_blk), dim3(kDispBlock), 0, stream,
                       ids, (int)S, (int)G, hist);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kMaxExperts), 0, stream, hist, (int)n_blk,
                     (int)G, base, counts, m_offsets);
  if (n_blk > 0)
    hipLaunchKernelGGL(dispatch_rank_kernel, dim3((unsigned)n_blk), dim3(kDispBlock), 0, stream, ids,
                       (int)S, (int)G, base, row_of_slot);
  if (K > 0) {
    if (T > 0)
      hipLaunchKernelGGL(dispatch_quant_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream,
                         (const uint4*)x, (int)T, (int)K, (int)k, row_of_slot, (uint2*)q, sa);
    hipLaunchKernelGGL(dispatch_pad_kernel, dim3((unsigned)G), dim3(256), 0, stream, m_offsets,
                       counts, (int)K, (uint4*)q, sa);
  }
  return hipGetLastError();
}

}  // namespace fp8q
