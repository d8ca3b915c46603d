// Block-scaled FP8 GEMM for gfx950 (CDNA4 MFMA): dense and grouped (MoE).
//
// C = A * B^T with A (M x K) quantized per 1x128 tile and B (N x K) per
// 128x128 block. For each 128-wide K group g the FP8 matrix cores produce the
// FP32 partial P_g of one v_mfma_f32_16x16x128_f8f6f4 (one MFMA spans exactly
// one K group), and the vector ALU promotes it into the FP32 accumulator with
// that group's scales:
//     acc[m, n] += (sa[m, g] * sb[n / 128, g]) * P_g[m, n]
// This is the per-group scaling along K and the promotion of MMA partials to
// FP32 described in "Six Reasons Deepseek Ai Is A Waste Of Time"
// (myomija.com), paragraphs on fine-grained quantization and on promotion,
// with the promotion interval read as one scale group (128).
//
// Tiling. A workgroup computes a BM x BN output tile with WAVES_M x WAVES_N
// waves; each wave owns a WM x WN sub-tile (WM = BM / WAVES_M, WN = BN /
// WAVES_N <= 128, so a wave's columns share one weight block and one sb).
// Per K group the workgroup stages the BM x 128 slab of A, the BN x 128 slab
// of B and the BM A-scales of that group in LDS. The copies go straight from
// global memory to LDS (buffer_load_dwordx4 ... lds: no VGPR round trip), into
// one of two stages, so the loads of group g+1 run under the MFMAs of group g.
//
// LDS layout: rows of 128 bytes; the eight 16-byte chunks of row r are stored
// at chunk positions c ^ (r & 7), so the 16 rows read by one MFMA operand
// load fall in distinct banks. A direct-to-LDS load writes 64 consecutive
// 16-byte slots per wave instruction; each lane therefore fetches the global
// chunk that belongs in its slot.
//
// Operand lanes: for the 16x16x128 MFMA, lane l supplies row l % 16 of the A
// block (and row l % 16 of the B block, i.e. a column of B^T) with 32 bytes
// of K. Which 32 of the 128 K bytes a lane carries only has to agree between A
// and B: lane l takes chunks l/16 and 4 + l/16. Accumulator lanes: lane l
// holds rows 4 (l/16) + r, r = 0..3, of column l % 16.
//
// Ragged edges: the loads go through buffer descriptors sized to the tile's
// valid rows, so rows past the end of A (or B) read as zeros; their results
// are never stored.
//
// Tile order is XCD-aware: the hardware hands workgroup ids to the 8 XCDs
// round-robin, so ids are remapped such that each XCD works on a contiguous
// run of tiles (neighbouring tiles share A rows / B columns in its L2).
#include "common.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  const uint8_t* b;
  const float* sb;
  void* c;
  const int32_t* m_offsets;  // grouped only
  int M;                     // rows of A / C (M_total when grouped)
  int N;
  int K;
  int G;        // experts (grouped); 1 for dense
  int n_tiles;  // number of real tiles (dense) / upper bound (grouped)
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct TileCfg {
  static constexpr int kWM = BM / WAVES_M;
  static constexpr int kWN = BN / WAVES_N;
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kSubM = kWM / 16;
  static constexpr int kSubN = kWN / 16;
  static constexpr int kLdsA = BM * 128;  // bytes per stage
  static constexpr int kLdsB = BN * 128;
  static constexpr int kLdsSa = BM * 4;
  static constexpr int kStage = kLdsA + kLdsB + kLdsSa;
  static constexpr int kLdsBytes = 2 * kStage;
  static constexpr int kLoadsA = BM * 8 / kThreads;  // 16-byte chunks per thread per group
  static constexpr int kLoadsB = BN * 8 / kThreads;
  static_assert(kWN <= 128 && 128 % kWN == 0, "a wave's columns must share one weight block");
  static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "whole wave loads");
  static_assert(BM % 64 == 0 && BM <= kThreads, "A-scales: whole waves, one per thread");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int swz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

// Raw buffer descriptor over `bytes` bytes at `base` (dword 3: the gfx9
// raw-buffer format word); loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct global -> LDS copy: lane l of the wave writes `size` bytes at
// lds + l * size (lds must be wave-uniform).
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int size,
                                         uint32_t voffset, uint32_t soffset) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voffset, soffset, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voffset, soffset, 0, 0);
}

// Workgroup id -> tile index such that each XCD gets a contiguous run.
__device__ __forceinline__ int xcd_tile(int id, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = id % kXcds, local = id / kXcds;
  return x * q + (x < r ? x : r) + local;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool kBf16Out, bool kGrouped>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_blockscaled_kernel(GemmArgs p) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N>;
  constexpr int WM = Cfg::kWM, WN = Cfg::kWN;
  constexpr int SUBM = Cfg::kSubM, SUBN = Cfg::kSubN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[Cfg::kLdsBytes];  // two stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int G = p.K / kGroup;
  const int n_tiles_n = (p.N + BN - 1) / BN;

  // ---- tile -> (rows [m0, m_end), columns n0, expert) ----
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  int m0, m_end, tile_n;
  const uint8_t* bmat = p.b;
  const float* sbmat = p.sb;
  if constexpr (kGrouped) {
    // tiles are numbered expert by expert: ceil(rows_e / BM) row tiles each
    const int tile_m_global = tile / n_tiles_n;
    tile_n = tile % n_tiles_n;
    int e = 0, before = 0, lo = 0, hi = 0;
    for (; e < p.G; ++e) {
      lo = min(max(p.m_offsets[e], 0), p.M);
      hi = min(max(p.m_offsets[e + 1], lo), p.M);
      const int t = (hi - lo + BM - 1) / BM;
      if (tile_m_global < before + t) break;
      before += t;
    }
    if (e == p.G) return;  // beyond the last real tile (grid is an upper bound)
    m0 = lo + (tile_m_global - before) * BM;
    m_end = min(m0 + BM, hi);
    bmat += (int64_t)e * p.N * p.K;
    sbmat += (int64_t)e * (p.N / kGroup) * G;
  } else {
    const int tile_m = tile / n_tiles_n;
    tile_n = tile % n_tiles_n;
    m0 = tile_m * BM;
    m_end = min(m0 + BM, p.M);
  }
  const int n0 = tile_n * BN;
  const int n_last = p.N - 1;

  // ---- global -> LDS copies through buffer descriptors ----
  // One descriptor per operand covers exactly the tile's valid rows, so rows
  // past the end of A (or B) read as zeros. Their outputs are never stored;
  // every output row depends only on its own A row. Slot s = i * kThreads +
  // tid of a stage holds row s / 8, stored chunk s % 8, i.e. the global chunk
  // (s % 8) ^ (row % 8); the per-group advance (g * 128 bytes) is the
  // instruction's scalar offset.
  const int rows_a = m_end - m0;
  const int rows_b = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(p.a + (int64_t)m0 * p.K, (uint32_t)rows_a * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(bmat + (int64_t)n0 * p.K, (uint32_t)rows_b * (uint32_t)p.K);
  const __amdgpu_buffer_rsrc_t rsrc_sa = make_rsrc(p.sa + (int64_t)m0 * G, (uint32_t)rows_a * (uint32_t)G * 4);
  uint32_t offa[Cfg::kLoadsA], offb[Cfg::kLoadsB];
#pragma unroll
  for (int i = 0; i < Cfg::kLoadsA; ++i) {
    const int slot = i * Cfg::kThreads + tid;
    const int row = slot >> 3, lc = (slot & 7) ^ (row & 7);
    offa[i] = (uint32_t)row * (uint32_t)p.K + lc * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kLoadsB; ++i) {
    const int slot = i * Cfg::kThreads + tid;
    const int row = slot >> 3, lc = (slot & 7) ^ (row & 7);
    offb[i] = (uint32_t)row * (uint32_t)p.K + lc * 16;
  }
  const uint32_t offsa = (uint32_t)tid * (uint32_t)G * 4;

  auto issue_loads = [&](int g, uint8_t* __restrict__ stage) {
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i)
      load_lds(rsrc_a, stage + (i * Cfg::kThreads + wave * 64) * 16, 16, offa[i], g * kGroup);
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i)
      load_lds(rsrc_b, stage + Cfg::kLdsA + (i * Cfg::kThreads + wave * 64) * 16, 16, offb[i], g * kGroup);
    if (wave < BM / 64)
      load_lds(rsrc_sa, stage + Cfg::kLdsA + Cfg::kLdsB + wave * 64 * 4, 4, offsa, g * 4);
  };

  v4f acc[SUBM][SUBN];
#pragma unroll
  for (int i = 0; i < SUBM; ++i)
#pragma unroll
    for (int j = 0; j < SUBN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;  // operand row within a 16-row block
  const int lk = lane >> 4;  // which 16-byte chunk pair of the group
  const int nb = min(n0 + wn * WN, n_last) / kGroup;
  const float* gsb = sbmat + (int64_t)nb * G;

  // Operand fragment of the 16-row block starting at `blk` (a row index that
  // is a multiple of 16, so row % 8 == lr % 8): the lane's two chunks sit at
  // fixed per-lane offsets from the block start.
  const int lane_lo = lr * 128 + ((lk ^ (lr & 7)) << 4);
  const int lane_hi = lr * 128 + (((4 + lk) ^ (lr & 7)) << 4);
  auto load_frag = [&](const uint8_t* blk) {
    const uint4 lo = *(const uint4*)(blk + lane_lo);
    const uint4 hi = *(const uint4*)(blk + lane_hi);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // One K group from one LDS stage. sbv: this group's weight scale.
  // The wave's SUBM x SUBN MFMAs run in sequence t = i * SUBN + j; the FMAs
  // promoting MFMA t-1 are issued right after MFMA t, so each promotion waits
  // on a result that is one MFMA old.
  auto compute = [&](const uint8_t* __restrict__ stage, float sbv) {
    const uint8_t* sA = stage;
    const uint8_t* sB = stage + Cfg::kLdsA;
    const float* sSa = (const float*)(stage + Cfg::kLdsA + Cfg::kLdsB) + wm * WM + 4 * lk;
    v8i bf[SUBN];
#pragma unroll
    for (int j = 0; j < SUBN; ++j) bf[j] = load_frag(sB + (wn * WN + j * 16) * 128);
    v8i af;
    float4 sc, sc_prev;
    v4f part_prev;
#pragma unroll
    for (int t = 0; t < SUBM * SUBN; ++t) {
      const int i = t / SUBN, j = t % SUBN;
      if (j == 0) {
        af = load_frag(sA + (wm * WM + i * 16) * 128);
        const float4 sav = *(const float4*)(sSa + i * 16);
        sc = make_float4(sav.x * sbv, sav.y * sbv, sav.z * sbv, sav.w * sbv);
      }
      const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      if (t > 0) {
        v4f& c = acc[(t - 1) / SUBN][(t - 1) % SUBN];
        c[0] = __builtin_fmaf(part_prev[0], sc_prev.x, c[0]);
        c[1] = __builtin_fmaf(part_prev[1], sc_prev.y, c[1]);
        c[2] = __builtin_fmaf(part_prev[2], sc_prev.z, c[2]);
        c[3] = __builtin_fmaf(part_prev[3], sc_prev.w, c[3]);
      }
      part_prev = part;
      sc_prev = sc;
    }
    v4f& c = acc[SUBM - 1][SUBN - 1];
    c[0] = __builtin_fmaf(part_prev[0], sc_prev.x, c[0]);
    c[1] = __builtin_fmaf(part_prev[1], sc_prev.y, c[1]);
    c[2] = __builtin_fmaf(part_prev[2], sc_prev.z, c[2]);
    c[3] = __builtin_fmaf(part_prev[3], sc_prev.w, c[3]);
  };

  // One pipeline step: copy group g_next into `nxt` while computing the group
  // held in `cur`. The restrict-qualified stages tell the compiler (and its
  // wait-count pass) that the LDS reads of `cur` never alias the in-flight
  // copies into `nxt`, so the copies are not waited on until the barrier.
  auto step = [&](const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt, int g_next,
                  float sbv) {
    if (g_next < G) issue_loads(g_next, nxt);
    compute(cur, sbv);
  };

  // ---- main loop: group g computes from stage g % 2 while g+1 streams into the other ----
  float sbv = 0.0f;
  if (G > 0) {
    sbv = gsb[0];
    issue_loads(0, lds);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    uint8_t* cur = lds + (g & 1) * Cfg::kStage;
    uint8_t* nxt = lds + ((g + 1) & 1) * Cfg::kStage;
    const float sbv_next = (g + 1 < G) ? gsb[g + 1] : 0.0f;
    step(cur, nxt, g + 1, sbv);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this thread's copies have landed
    __syncthreads();                     // ... and everyone's; `cur` is free again
    sbv = sbv_next;
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < SUBM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gm = m0 + wm * WM + i * 16 + 4 * lk + r;
      if (gm >= m_end) continue;
#pragma unroll
      for (int j = 0; j < SUBN; ++j) {
        const int gn = n0 + wn * WN + j * 16 + lr;
        if (gn >= p.N) continue;
        const int64_t off = (int64_t)gm * p.N + gn;
        if constexpr (kBf16Out) {
          ((__bf16*)p.c)[off] = (__bf16)acc[i][j][r];
        } else {
          ((float*)p.c)[off] = acc[i][j][r];
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool kGrouped>
static hipError_t launch_cfg(GemmArgs args, bool bf16_out, int m_tiles, hipStream_t stream) {
  using Cfg = TileCfg<BM, BN, WAVES_M, WAVES_N>;
  args.n_tiles = m_tiles * ((args.N + BN - 1) / BN);
  const dim3 grid((unsigned)args.n_tiles);
  const dim3 block(Cfg::kThreads);
  if (bf16_out) {
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, true, kGrouped>), grid,
                       block, 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WAVES_M, WAVES_N, false, kGrouped>), grid,
                       block, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, void* c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream) {
  GemmArgs args{a, sa, b, sb, c, nullptr, (int)M, (int)N, (int)K, 1, 0};
  return launch_cfg<256, 256, 2, 4, false>(args, bf16_out, (int)((M + 255) / 256), stream);
}

hipError_t launch_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b,
                               const float* sb, void* c, bool bf16_out, const int32_t* m_offsets,
                               int64_t G, int64_t M_total, int64_t N, int64_t K,
                               hipStream_t stream) {
  GemmArgs args{a, sa, b, sb, c, m_offsets, (int)M_total, (int)N, (int)K, (int)G, 0};
  // upper bound on sum_e ceil(rows_e / 256) for rows_e multiples of 128
  const int64_t m_tiles = (M_total / 128 + G + 1) / 2;
  return launch_cfg<256, 256, 2, 4, true>(args, bf16_out, (int)m_tiles, stream);
}

}  // namespace fp8q
