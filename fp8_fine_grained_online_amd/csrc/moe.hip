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
// so the layout is deterministic. Three launches:
//   count  per 256-slot block: each wavefront ranks its 64 slots among equal
//          experts (one ballot per distinct expert present), the 4 wavefronts'
//          counts are added in LDS; the block's histogram goes to the
//          workspace and each slot's rank inside the block (earlier waves +
//          rank in its wave, -1 for an invalid choice) to row_of_slot;
//   scan   one workgroup, 1024/G threads per expert: per-expert totals, padded
//          offsets, and for every (block, expert) the first row that block's
//          slots of that expert take;
//   quant  one wavefront per token: its rows are base + in-block rank; read
//          and quantize the token once, store its codes and scales to each of
//          its rows, then overwrite its slots' ranks with their rows; further
//          wavefronts, one per possible padding row (127 per expert), zero the
//          padding rows.
// Ranking in the count pass, rather than in a kernel of its own between the
// scan and the scatter, saves a launch. With the parallel scan below, the
// whole dispatch on MI355X (interleaved, same outputs bit for bit): 8192
// tokens x top-8 of 32 experts, K = 7168: 148.2 -> 133.9 us; 4096 x top-8 of
// 256, K = 7168: 99.1 -> 97.2 us; 16384 x top-6 of 64, K = 2048: 65.0 ->
// 62.4 us.
#include "common.hpp"

namespace fp8q {

constexpr int kDispBlock = 256;      // slots per count/rank block, one per thread
constexpr int kDispWaves = kDispBlock / 64;
constexpr int kMaxExperts = 1024;
constexpr int kHeldSteps = 8;  // quantize/scatter: steps of codes a lane holds (K <= 8192)

__global__ __launch_bounds__(kDispBlock) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                                    int S, int G,
                                                                    int32_t* __restrict__ hist,
                                                                    int32_t* __restrict__ in_block) {
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
    int r = -1;
    if (valid) {
      r = rank;
      for (int v = 0; v < w; ++v) r += wave_cnt[v * G + e];
    }
    in_block[slot] = r;
  }
  for (int x = threadIdx.x; x < G; x += kDispBlock) {
    int c = 0;
#pragma unroll
    for (int v = 0; v < kDispWaves; ++v) c += wave_cnt[v * G + x];
    hist[(int64_t)blockIdx.x * G + x] = c;
  }
}

// One workgroup. Thread (e, p) = (tid % G, tid / G), p < tpe = 1024 / G
// threads per expert, owns the contiguous run of blocks [p * chunk, (p+1) *
// chunk) of expert e's column of the histogram: it sums them (holding up to
// kScanHeld values in registers for the second pass), the partial sums of an
// expert get an inclusive prefix over p in LDS (Hillis-Steele, stride G),
// whose last entry is the expert's total, the padded totals a prefix over
// the experts, and the thread writes the base row of each of its blocks.
// Neighbouring threads take neighbouring experts, so each histogram row is
// read and written coalesced. Every step is parallel: an earlier version
// summed the partials and formed the prefix over p in loops of up to tpe
// dependent LDS reads, and read its run of the histogram twice.
constexpr int kScanHeld = 16;
__global__ __launch_bounds__(kMaxExperts) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int n_blk, int G, int32_t* __restrict__ base,
    int32_t* __restrict__ counts, int32_t* __restrict__ m_offsets) {
  __shared__ int32_t part[kMaxExperts];  // [p * G + e]
  __shared__ int32_t scan[kMaxExperts];
  const int tid = threadIdx.x;
  const int tpe = kMaxExperts / G;
  const int e = tid % G, p = tid / G;
  const bool on = p < tpe;
  const int chunk = (n_blk + tpe - 1) / tpe;
  const int b0 = min(p * chunk, n_blk), b1 = min(b0 + chunk, n_blk);
  const bool held = chunk <= kScanHeld;  // uniform
  int v[kScanHeld];
  int sum = 0;
  if (on) {
    if (held) {
#pragma unroll
      for (int j = 0; j < kScanHeld; ++j) v[j] = (b0 + j < b1) ? hist[(int64_t)(b0 + j) * G + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanHeld; ++j) sum += v[j];
    } else {
#pragma unroll 8
      for (int b = b0; b < b1; ++b) sum += hist[(int64_t)b * G + e];
    }
  }
  part[tid] = sum;  // zero for p >= tpe
  __syncthreads();
  for (int d = 1; d < tpe; d <<= 1) {
    const int add = (on && p >= d) ? part[tid - d * G] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  // expert totals (the last p's inclusive prefix), then an inclusive scan of
  // the padded totals (entries from G on are zero, so steps d < G give every
  // expert's full prefix)
  int padded = 0;
  if (tid < G) {
    const int total = part[(tpe - 1) * G + tid];
    counts[tid] = total;
    padded = (total + kGroup - 1) / kGroup * kGroup;
  }
  scan[tid] = padded;
  __syncthreads();
  for (int d = 1; d < G; d <<= 1) {
    const int add = tid >= d ? scan[tid - d] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  if (tid < G) m_offsets[tid + 1] = scan[tid];
  if (tid == 0) m_offsets[0] = 0;
  if (on) {
    int run = (e > 0 ? scan[e - 1] : 0) + part[tid] - sum;  // expert offset + earlier runs
    if (held) {
#pragma unroll
      for (int j = 0; j < kScanHeld; ++j) {
        if (b0 + j < b1) {
          base[(int64_t)(b0 + j) * G + e] = run;
          run += v[j];
        }
      }
    } else {
      // eight blocks at a time: their loads are issued together
      for (int b = b0; b < b1; b += 8) {
        int c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (b + j < b1) ? hist[(int64_t)(b + j) * G + e] : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (b + j < b1) {
            base[(int64_t)(b + j) * G + e] = run;
            run += c[j];
          }
        }
      }
    }
  }
}

// One wavefront per token. Lane l owns 16 consecutive values (32 bytes in, 16
// bytes of codes out) of each 1024-value step, so a 1x128 tile is 8 lanes
// (half a DPP row) and every destination row gets one 16-byte store per lane
// per step. The scales are gathered across steps, one lane shuffle per step,
// until lane l holds the scale of tile 64 w + l of window w (8 steps); each
// destination row then gets the window's scales in one contiguous store.
//
// A token's row for choice j is base[block][expert] + the slot's rank inside
// its 256-slot block, which the count pass left in row_of_slot; the wavefront
// replaces those ranks by the rows once it has used them (-1 stays -1).
//
// Wavefronts past the T tokens zero the padding rows: wavefront T + 127 e + i
// takes row m_offsets[e] + counts[e] + i when that row is below m_offsets[e+1].
// With K == 0 only the tokens' wavefronts run, for the row map.
__global__ __launch_bounds__(256) void dispatch_quant_kernel(const uint4* __restrict__ x, int T,
                                                             int K, int k,
                                                             const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ row_of_slot,
                                                             const int32_t* __restrict__ m_offsets,
                                                             const int32_t* __restrict__ counts,
                                                             int n_experts, uint2* __restrict__ q,
                                                             float* __restrict__ sa) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_chunks = K / 8;
  const int G = K / kGroup;
  if (t >= T) {
    const int pi = t - T;
    const int e = pi / (kGroup - 1);
    if (e >= n_experts) return;
    const int64_t row = (int64_t)m_offsets[e] + counts[e] + pi % (kGroup - 1);
    if (row >= m_offsets[e + 1]) return;  // at most 127 padding rows per expert
    uint4* qr = (uint4*)q + row * (K / 16);
    for (int c = lane; c < K / 16; c += 64) qr[c] = make_uint4(0, 0, 0, 0);
    for (int c = lane; c < G; c += 64) sa[row * G + c] = 0.0f;
    return;
  }
  const uint4* xr = x + (int64_t)t * n_chunks;
  // row of the token's choice j: the ranks are only read here, and
  // overwritten after their last use
  auto slot_row = [&](int j) {
    const int64_t slot = (int64_t)t * k + j;
    const int r = row_of_slot[slot];
    return r < 0 ? -1 : base[(slot / kDispBlock) * n_experts + ids[slot]] + r;
  };
  // lane j holds the row of choice j < 64, looked up once, all lanes together
  // (a chain of dependent loads per choice and use cost 5% at K = 2048)
  const int lane_row = lane < k ? slot_row(lane) : -1;
  auto row_of = [&](int j) {  // wave-uniform j
    return j < 64 ? __builtin_amdgcn_readlane(lane_row, j) : slot_row(j);
  };
  auto write_rows = [&]() {
    if (lane < k) row_of_slot[(int64_t)t * k + lane] = lane_row;
    int r[4];
    for (int j0 = 64; j0 < k; j0 += 256) {  // all loads of a batch before any store
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * 64 + lane;
        r[u] = j < k ? slot_row(j) : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * 64 + lane;
        if (j < k) row_of_slot[(int64_t)t * k + j] = r[u];
      }
    }
  };
  const int n_steps = (n_chunks + 127) / 128;
  float win = 0.0f;          // this lane's tile of the current window, once gathered
  constexpr int kBatch = 2;  // steps whose loads are in flight together
  // step st: this lane's two chunks st * 128 + 2 lane (+1), loaded into v
  auto load_step = [&](int st, uint4 (&v)[2]) {
    const int c = st * 128 + 2 * lane;
    const bool have = c < n_chunks;  // whole tiles (8 lanes) are present or absent
    v[0] = have ? load_nt(xr + c) : make_uint4(0, 0, 0, 0);
    v[1] = have ? load_nt(xr + c + 1) : make_uint4(0, 0, 0, 0);
  };
  // the step's codes; its tile scale joins the current window of 8 steps, and
  // a finished window's 64 scales go to every destination row at once
  auto quantize_step = [&](int st, const uint4 (&v)[2]) {
    const float m = fmaxf(absmax8(v[0]), absmax8(v[1]));
    const float amax = __uint_as_float(row8_max_u32(__float_as_uint(m)));
    const float s = tile_scale(amax);
    const TileDivisor d = make_divisor(s, amax);
    const uint2 lo = quant8(v[0], d), hi = quant8(v[1], d);
    // at step st, lane l with l / 8 == st % 8 takes the scale of tile
    // 8 st + l % 8, which lanes 8 (l % 8) .. 8 (l % 8) + 7 hold
    const float got = __shfl(s, (lane & 7) * 8);
    if ((lane >> 3) == (st & 7)) win = got;
    if ((st & 7) == 7 || st == n_steps - 1) {
      const int tile = (st & ~7) * 8 + lane;  // window st / 8 covers tiles 64 (st / 8) + 0..63
      if (tile < G) {
        for (int j = 0; j < k; ++j) {
          const int row = row_of(j);
          if (row < 0) continue;
          sa[(int64_t)row * G + tile] = win;
        }
      }
    }
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  };
  auto store_codes = [&](int row, int st, uint4 codes) {
    const int c = st * 128 + 2 * lane;
    if (c < n_chunks) *(uint4*)(q + ((int64_t)row * n_chunks + c)) = codes;
  };

  if (n_steps <= kHeldSteps) {
    // K <= 8192: the token's codes stay in registers (kHeldSteps x 16 bytes
    // per lane) and each destination row is written in one pass, its steps
    // back to back, instead of eight rows taking turns at every step
    // (8192 tokens x top-8 x 7168: 156 -> 150 us)
    uint4 cd[kHeldSteps];
#pragma unroll
    for (int s0 = 0; s0 < kHeldSteps; s0 += kBatch) {
      if (s0 >= n_steps) break;  // wave-uniform
      uint4 v[kBatch][2];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) load_step(s0 + u, v[u]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u < n_steps) cd[s0 + u] = quantize_step(s0 + u, v[u]);
    }
    for (int j = 0; j < k; ++j) {
      const int row = row_of(j);  // same for the whole wavefront
      if (row < 0) continue;       // dropped choice
#pragma unroll
      for (int st = 0; st < kHeldSteps; ++st)
        if (st < n_steps) store_codes(row, st, cd[st]);
    }
    write_rows();
    return;
  }
  for (int s0 = 0; s0 < n_steps; s0 += kBatch) {
    uint4 v[kBatch][2];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) load_step(s0 + u, v[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int st = s0 + u;
      if (st >= n_steps) break;  // wave-uniform
      const uint4 codes = quantize_step(st, v[u]);
      for (int j = 0; j < k; ++j) {
        const int row = row_of(j);
        if (row < 0) continue;
        store_codes(row, st, codes);
      }
    }
  }
  write_rows();
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
                       ids, (int)S, (int)G, hist, row_of_slot);
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kMaxExperts), 0, stream, hist, (int)n_blk,
                     (int)G, base, counts, m_offsets);
  if (T > 0) {
    // the tokens' wavefronts, then (with K > 0) one per possible padding row;
    // with T == 0 every expert is empty and has no padding rows
    const int64_t waves = T + (K > 0 ? (kGroup - 1) * G : 0);
    hipLaunchKernelGGL(dispatch_quant_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream,
                       (const uint4*)x, (int)T, (int)K, (int)k, ids, base, row_of_slot, m_offsets,
                       counts, (int)G, (uint2*)q, sa);
  }
  return hipGetLastError();
}

}  // namespace fp8q
