// Block-scaled FP8 GEMM for gfx950 (CDNA4 MFMA): dense and grouped (MoE).
//
// C = A * B^T with A (M x K) quantized per 1x128 tile and B (N x K) per
// 128x128 block. For each 128-wide K group g the FP8 matrix cores produce the
// exact-product FP32 partial P_g of one v_mfma_f32_16x16x128_f8f6f4 (one MFMA
// spans exactly one K group), and the vector ALU promotes it into the FP32
// accumulator with that group's scales:
//     acc[m, n] += (sa[m, g] * sb[n / 128, g]) * P_g[m, n]
// This is the per-group scaling along K and the promotion of MMA partials to
// FP32 described in "Six Reasons Deepseek Ai Is A Waste Of Time"
// (myomija.com), paragraphs on fine-grained quantization and on promotion,
// with the promotion interval read as one scale group (128).
//
// Tiling: a workgroup computes a BM x BN tile with (BM/WM) x (BN/WN) waves,
// each wave a WM x WN sub-tile of 16x16 MFMA blocks. K-group slabs of A and B
// (BM x 128 and BN x 128 bytes) and the group's A-scale column are staged in
// LDS, double-buffered, so loads of group g+1 overlap the MFMAs of group g.
// LDS rows are 128 bytes; their eight 16-byte chunks are XOR-swizzled by the
// row index so that the 16 rows read by one MFMA operand load hit distinct
// banks.
//
// Operand lanes: for the 16x16x128 MFMA, lane l supplies row l % 16 of A (of
// B^T's column, i.e. B's row) with 32 bytes of K. Which 32 of the 128 K
// bytes a lane carries only has to agree between A and B (the products are
// summed over the whole group), so lane l takes chunks l/16 and 4 + l/16.
// Accumulator lanes: lane l holds rows 4 (l/16) + r, r = 0..3, of column l % 16.
#include "common.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

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
  int G;  // experts (grouped); 1 for dense
};

template <int BM, int BN, int WM, int WN>
struct TileCfg {
  static constexpr int kWavesM = BM / WM;
  static constexpr int kWavesN = BN / WN;
  static constexpr int kThreads = 64 * kWavesM * kWavesN;
  static constexpr int kSubM = WM / 16;
  static constexpr int kSubN = WN / 16;
  static constexpr int kLdsA = BM * 128;            // bytes per stage
  static constexpr int kLdsB = BN * 128;
  static constexpr int kLdsSa = BM * 4;
  static constexpr int kStage = kLdsA + kLdsB + kLdsSa;
  static constexpr int kChunksA = BM * 8 / kThreads;  // 16-byte chunks per thread
  static constexpr int kChunksB = BN * 8 / kThreads;
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one weight block");
  static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "even chunk split");
  static_assert(BM <= kThreads, "one A-scale per thread");
};

__device__ __forceinline__ int swz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

template <int BM, int BN, int WM, int WN, bool kBf16Out, bool kGrouped>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN)) void gemm_blockscaled_kernel(GemmArgs p) {
  using Cfg = TileCfg<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / Cfg::kWavesN;
  const int wn = wave % Cfg::kWavesN;

  const int n_tiles_n = p.N / BN;
  const int tile_n = blockIdx.x % n_tiles_n;
  const int tile_m = blockIdx.x / n_tiles_n;
  const int m0 = tile_m * BM;
  const int n0 = tile_n * BN;
  const int G = p.K / kGroup;

  const uint8_t* bmat = p.b;
  const float* sbmat = p.sb;
  if constexpr (kGrouped) {
    // expert owning this tile's first row: last e with m_offsets[e] <= m0
    int lo = 0, hi = p.G;  // invariant: answer in [lo, hi)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.m_offsets[mid] <= m0) lo = mid; else hi = mid;
    }
    bmat += (int64_t)lo * p.N * p.K;
    sbmat += (int64_t)lo * (p.N / kGroup) * G;
  }

  // ---- global -> register staging for one K group ----
  uint4 ra[Cfg::kChunksA], rb[Cfg::kChunksB];
  float rsa = 0.0f;
  auto load_group = [&](int g) {
#pragma unroll
    for (int i = 0; i < Cfg::kChunksA; ++i) {
      const int idx = tid + i * Cfg::kThreads;
      const int row = idx >> 3, ch = idx & 7;
      const int gm = m0 + row;
      ra[i] = (gm < p.M) ? *(const uint4*)(p.a + (int64_t)gm * p.K + g * kGroup + ch * 16)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::kChunksB; ++i) {
      const int idx = tid + i * Cfg::kThreads;
      const int row = idx >> 3, ch = idx & 7;
      rb[i] = *(const uint4*)(bmat + (int64_t)(n0 + row) * p.K + g * kGroup + ch * 16);
    }
    if (tid < BM) {
      const int gm = m0 + tid;
      rsa = (gm < p.M) ? p.sa[(int64_t)gm * G + g] : 0.0f;
    }
  };
  auto store_group = [&](int stage) {
    uint8_t* sA = lds + stage * Cfg::kStage;
    uint8_t* sB = sA + Cfg::kLdsA;
    float* sSa = (float*)(sB + Cfg::kLdsB);
#pragma unroll
    for (int i = 0; i < Cfg::kChunksA; ++i) {
      const int idx = tid + i * Cfg::kThreads;
      *(uint4*)(sA + swz(idx >> 3, idx & 7)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::kChunksB; ++i) {
      const int idx = tid + i * Cfg::kThreads;
      *(uint4*)(sB + swz(idx >> 3, idx & 7)) = rb[i];
    }
    if (tid < BM) sSa[tid] = rsa;
  };

  v4f acc[Cfg::kSubM][Cfg::kSubN];
#pragma unroll
  for (int i = 0; i < Cfg::kSubM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kSubN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;   // operand row within a 16-row block
  const int lk = lane >> 4;   // which 16-byte chunk pair of the group
  const int sb_row = (n0 + wn * WN) / kGroup;

  if (G > 0) {
    load_group(0);
    store_group(0);
  }
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int stage = g & 1;
    if (g + 1 < G) load_group(g + 1);

    const uint8_t* sA = lds + stage * Cfg::kStage;
    const uint8_t* sB = sA + Cfg::kLdsA;
    const float* sSa = (const float*)(sB + Cfg::kLdsB);

    // B fragments for the wave's WN columns
    v8i bf[Cfg::kSubN];
#pragma unroll
    for (int j = 0; j < Cfg::kSubN; ++j) {
      const int row = wn * WN + j * 16 + lr;
      const uint4 lo = *(const uint4*)(sB + swz(row, lk));
      const uint4 hi = *(const uint4*)(sB + swz(row, 4 + lk));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const float sbv = sbmat[(int64_t)sb_row * G + g];

#pragma unroll
    for (int i = 0; i < Cfg::kSubM; ++i) {
      const int row = wm * WM + i * 16 + lr;
      const uint4 lo = *(const uint4*)(sA + swz(row, lk));
      const uint4 hi = *(const uint4*)(sA + swz(row, 4 + lk));
      const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float4 sav = *(const float4*)(sSa + wm * WM + i * 16 + 4 * lk);
      const float sc0 = sav.x * sbv, sc1 = sav.y * sbv, sc2 = sav.z * sbv, sc3 = sav.w * sbv;
#pragma unroll
      for (int j = 0; j < Cfg::kSubN; ++j) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[i][j][0] = __builtin_fmaf(part[0], sc0, acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(part[1], sc1, acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(part[2], sc2, acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(part[3], sc3, acc[i][j][3]);
      }
    }

    if (g + 1 < G) store_group(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < Cfg::kSubM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gm = m0 + wm * WM + i * 16 + 4 * lk + r;
      if (gm >= p.M) continue;
#pragma unroll
      for (int j = 0; j < Cfg::kSubN; ++j) {
        const int gn = n0 + wn * WN + j * 16 + lr;
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

template <int BM, int BN, int WM, int WN, bool kGrouped>
static hipError_t launch_cfg(const GemmArgs& args, bool bf16_out, int m_tiles, hipStream_t stream) {
  using Cfg = TileCfg<BM, BN, WM, WN>;
  const dim3 grid((unsigned)(m_tiles * (args.N / BN)));
  const dim3 block(Cfg::kThreads);
  const size_t lds = 2 * Cfg::kStage;
  // the LDS limit above 64 KB is raised once per kernel instantiation
  static const hipError_t attr_bf16 = hipFuncSetAttribute(
      (const void*)gemm_blockscaled_kernel<BM, BN, WM, WN, true, kGrouped>,
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  static const hipError_t attr_f32 = hipFuncSetAttribute(
      (const void*)gemm_blockscaled_kernel<BM, BN, WM, WN, false, kGrouped>,
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (bf16_out) {
    if (attr_bf16 != hipSuccess) return attr_bf16;
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WM, WN, true, kGrouped>), grid, block, lds,
                       stream, args);
  } else {
    if (attr_f32 != hipSuccess) return attr_f32;
    hipLaunchKernelGGL((gemm_blockscaled_kernel<BM, BN, WM, WN, false, kGrouped>), grid, block, lds,
                       stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, void* c, bool bf16_out, int64_t M, int64_t N,
                                   int64_t K, hipStream_t stream) {
  GemmArgs args{a, sa, b, sb, c, nullptr, (int)M, (int)N, (int)K, 1};
  const int m_tiles = (int)((M + 127) / 128);
  return launch_cfg<128, 128, 64, 64, false>(args, bf16_out, m_tiles, stream);
}

hipError_t launch_gemm_grouped(const uint8_t* a, const float* sa, const uint8_t* b,
                               const float* sb, void* c, bool bf16_out, const int32_t* m_offsets,
                               int64_t G, int64_t M_total, int64_t N, int64_t K,
                               hipStream_t stream) {
  GemmArgs args{a, sa, b, sb, c, m_offsets, (int)M_total, (int)N, (int)K, (int)G};
  const int m_tiles = (int)((M_total + 127) / 128);
  return launch_cfg<128, 128, 64, 64, true>(args, bf16_out, m_tiles, stream);
}

}  // namespace fp8q
