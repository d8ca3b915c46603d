// Quantize-on-load block-scaled FP8 GEMM for gfx950: C = Q(A) · B^T, where A
// arrives in bf16 and Q is the 1x128 activation quantization, applied inside
// the GEMM's load stage instead of by a separate pass over A.
//
// The woojincopolymer.co.kr post, paragraph of hardware suggestions: fuse the
// FP8 cast with the global-to-shared transfer, so that activations are
// quantized while they are loaded for the MMA, the BF16 activations are read
// once and no FP8 copy round-trips through HBM.
// The arithmetic is exactly that of fp8q_quant_act_1x128 followed by
// fp8_gemm_blockscaled (same codes, same scales, same per-group promotion).
//
// On gfx950 the direct global -> LDS copy cannot transform data, so the
// quantization goes through VGPRs: per K group each thread loads 4 chunks of
// 8 bf16 values (buffer loads, one group ahead), a 1x128 tile being the 16
// chunks of 16 consecutive lanes (one DPP row) as in the standalone
// quantizer; the tile's amax is reduced with DPP, and the codes (8 bytes per
// chunk) and the scale are written into the LDS stage the MFMAs read next.
// B (FP8) arrives by direct global -> LDS copies as in the other GEMMs.
//
// Tile 128 x 256 with 8 waves of 64 x 64 (the 256 x 256 tile leaves no
// registers for the bf16 staging). Every column tile quantizes its A rows
// again, N / 256 times in all; the workgroups of column tile 0 also store the
// codes and scales (optional outputs), e.g. for the backward pass.
#include "common.hpp"
#include "tiles.hpp"

namespace fp8q {

constexpr int kQaBM = 128;
constexpr int kQaBN = 256;
constexpr int kQaWavesN = 4;                      // 2 x 4 waves
constexpr int kQaWM = 64;
constexpr int kQaWN = 64;
constexpr int kQaSubM = kQaWM / 16;
constexpr int kQaSubN = kQaWN / 16;
constexpr int kQaThreads = 512;
constexpr int kQaLdsA = kQaBM * 128;              // FP8 A slab of one group
constexpr int kQaLdsB = kQaBN * 128;              // FP8 B slab of one group
constexpr int kQaStage = kQaLdsA + kQaLdsB + kQaBM * 4;  // + the A scales
constexpr int kQaChunks = kQaBM * 16 / kQaThreads;       // bf16 chunks of A per thread per group
constexpr int kQaLoadsB = kQaBN * 8 / kQaThreads;        // 16-byte copies of B per thread per group
constexpr int kQaCopyEvery = 2;                           // MFMAs between B copies

struct QaArgs {
  const void* a;  // bf16 bits, M x K
  const uint8_t* b;
  const float* sb;
  void* c;
  uint8_t* qa;    // optional outputs: codes and scales of A (nullptr: not stored)
  float* sa;
  int M, N, K;
};

template <bool kBf16Out>
__global__ __launch_bounds__(kQaThreads) void gemm_qa_kernel(QaArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kQaStage];  // two stages; the epilogue's staging
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kQaWavesN, wn = wave % kQaWavesN;
  const int lr = lane & 15, lk = lane >> 4;
  const int G = p.K / kGroup;
  const int n_tiles_n = (p.N + kQaBN - 1) / kQaBN;
  const int m_tiles = (p.M + kQaBM - 1) / kQaBM;
  int tm, tn;
  band_tile(xcd_tile(blockIdx.x, gridDim.x), m_tiles, n_tiles_n, tm, tn);
  const int m0 = tm * kQaBM, n0 = tn * kQaBN;
  const int rows_a = min(kQaBM, p.M - m0);
  const int rows_b = min(kQaBN, p.N - n0);
  const bool side = p.qa != nullptr && tn == 0;  // this workgroup stores A's codes and scales

  // bf16 A: thread t holds chunk t % 16 (8 values) of rows t / 16 + 32 i of
  // the group, so a DPP row of 16 lanes holds one 1x128 tile; rows past M
  // read as zeros through the descriptor (and are never stored).
  const __amdgpu_buffer_rsrc_t rsrc_a =
      make_rsrc((const uint8_t*)p.a + (int64_t)m0 * p.K * 2, (uint32_t)rows_a * (uint32_t)p.K * 2);
  const int qc = tid & 15;
  const int qrow0 = tid >> 4;
  auto load_a = [&](int g, uint4 (&r)[kQaChunks]) {
#pragma unroll
    for (int i = 0; i < kQaChunks; ++i) {
      const uint32_t off = (uint32_t)(qrow0 + 32 * i) * (uint32_t)p.K * 2 + qc * 16;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, off, g * 256, 0);
      r[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  // quantize the group held in r into `stage` (codes at the swizzled slots of
  // the FP8 slab, scales after the B slab) and, with `store`, to the outputs
  auto quantize_a = [&](int g, const uint4 (&r)[kQaChunks], uint8_t* stage, bool store) {
#pragma unroll
    for (int i = 0; i < kQaChunks; ++i) {
      const int row = qrow0 + 32 * i;
      const float amax = __uint_as_float(row16_max_u32(__float_as_uint(absmax8(r[i]))));
      const float s = tile_scale(amax);
      const TileDivisor d = make_divisor(s, amax);
      const uint2 codes = quant8(r[i], d);
      *(uint2*)(stage + swz(row, qc >> 1) + (qc & 1) * 8) = codes;
      if (qc == 0) ((float*)(stage + kQaLdsA + kQaLdsB))[row] = s;
      if (store && row < rows_a) {
        const int64_t gm = m0 + row;
        *(uint2*)(p.qa + gm * p.K + g * kGroup + qc * 8) = codes;
        if (qc == 0) p.sa[gm * G + g] = s;
      }
    }
  };

  // B: slot q * 512 + tid of a stage holds row (q * 512 + tid) / 8, stored
  // chunk tid % 8, i.e. global chunk (tid % 8) ^ (row % 8)
  const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(p.b + (int64_t)n0 * p.K, (uint32_t)rows_b * (uint32_t)p.K);
  const int brow0 = tid >> 3, blc0 = (tid & 7) ^ (brow0 & 7);
  const uint32_t offb = (uint32_t)brow0 * (uint32_t)p.K + blc0 * 16;
  const uint32_t brow_step = (uint32_t)(kQaThreads / 8) * (uint32_t)p.K;
  auto copy_b = [&](int q, int g, uint8_t* __restrict__ stage) {
    load_lds(rsrc_b, stage + kQaLdsA + (q * kQaThreads + wave * 64) * 16, 16, offb + q * brow_step,
             g * kGroup);
  };

  v4f acc[kQaSubM][kQaSubN];
#pragma unroll
  for (int i = 0; i < kQaSubM; ++i)
#pragma unroll
    for (int j = 0; j < kQaSubN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nb = min(n0 + wn * kQaWN, p.N - 1) / kGroup;  // the wave's weight block column
  const float* gsb = p.sb + (int64_t)nb * G;
  const int lane_lo = lr * 128 + ((lk ^ (lr & 7)) << 4);
  const int lane_hi = lr * 128 + (((4 + lk) ^ (lr & 7)) << 4);
  auto load_frag = [&](const uint8_t* blk) {
    const uint4 lo = *(const uint4*)(blk + lane_lo);
    const uint4 hi = *(const uint4*)(blk + lane_hi);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  // One step: multiply group g from `stage`; meanwhile copy B of g_next into
  // `nxt`, quantize A of g_next (held in ra, loaded one step earlier) into
  // `nxt`, and load A of g_load into rb. The MFMA order and the promotion of
  // MFMA t-1 after MFMA t are those of the large-tile kernel.
  uint4 ra[kQaChunks], rb[kQaChunks];
  auto step = [&](const uint8_t* __restrict__ stage, uint8_t* __restrict__ nxt, int g_next, int g_load,
                  float sbv, bool store) {
    load_a(g_load, rb);
    const float* sSa = (const float*)(stage + kQaLdsA + kQaLdsB) + wm * kQaWM + lr;
    v8i bf[kQaSubN];
#pragma unroll
    for (int j = 0; j < kQaSubN; ++j) bf[j] = load_frag(stage + kQaLdsA + (wn * kQaWN + j * 16) * 128);
    v8i af = load_frag(stage + wm * kQaWM * 128);
    float sav = sSa[0];
    v8i af_next;
    float sav_next, sc, sc_prev;
    v4f part_prev;
#pragma unroll
    for (int t = 0; t < kQaSubM * kQaSubN; ++t) {
      const int i = t / kQaSubN, j = t % kQaSubN;
      if (t % kQaCopyEvery == 0 && t / kQaCopyEvery < kQaLoadsB) copy_b(t / kQaCopyEvery, g_next, nxt);
      if (t == kQaSubN) quantize_a(g_next, ra, nxt, store);
      if (j == 0) {
        sc = sav * sbv;
        if (i + 1 < kQaSubM) {
          af_next = load_frag(stage + (wm * kQaWM + (i + 1) * 16) * 128);
          sav_next = sSa[(i + 1) * 16];
        }
      }
      const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          bf[j], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      if (t > 0) {
        v4f& c = acc[(t - 1) / kQaSubN][(t - 1) % kQaSubN];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = __builtin_fmaf(part_prev[r], sc_prev, c[r]);
      }
      part_prev = part;
      sc_prev = sc;
      if (j == kQaSubN - 1 && i + 1 < kQaSubM) {
        af = af_next;
        sav = sav_next;
      }
    }
    {
      v4f& c = acc[kQaSubM - 1][kQaSubN - 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) c[r] = __builtin_fmaf(part_prev[r], sc_prev, c[r]);
    }
  };

  // prologue: group 0 into stage 0; A of group 1 into registers
  if (G > 0) {
#pragma unroll
    for (int q = 0; q < kQaLoadsB; ++q) copy_b(q, 0, lds);
    load_a(0, ra);
    load_a(min(1, G - 1), rb);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    quantize_a(0, ra, lds, side);
#pragma unroll
    for (int i = 0; i < kQaChunks; ++i) ra[i] = rb[i];
  }
  __syncthreads();
  for (int g = 0; g < G; ++g) {
    uint8_t* cur = lds + (g & 1) * kQaStage;
    uint8_t* nxt = lds + ((g + 1) & 1) * kQaStage;
    // the last group re-copies and re-quantizes itself into the idle stage
    // (never read, and not stored): no branch in the step
    step(cur, nxt, min(g + 1, G - 1), min(g + 2, G - 1), gsb[g], side && g + 1 < G);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this thread's copies and loads have landed
    __syncthreads();                     // ... and everyone's; `cur` is free again
#pragma unroll
    for (int i = 0; i < kQaChunks; ++i) ra[i] = rb[i];
  }

  // ---- epilogue: the wave's 64 x 64 tile staged in LDS, whole row segments stored ----
  const int nw = n0 + wn * kQaWN;  // N % 128 == 0: the wave's 64 columns are all in or all out
  if constexpr (kBf16Out) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    static_assert(8 * kQaWM * 128 <= 2 * kQaStage, "staging fits in the stages");
    uint8_t* tile = lds + wave * (kQaWM * 128);
#pragma unroll
    for (int i = 0; i < kQaSubM; ++i) {
      const int m = i * 16 + lr;
#pragma unroll
      for (int j = 0; j < kQaSubN; ++j) {
        const int byte = j * 32 + lk * 8;
        const bf16x4 v = {(__bf16)acc[i][j][0], (__bf16)acc[i][j][1], (__bf16)acc[i][j][2],
                          (__bf16)acc[i][j][3]};
        *(bf16x4*)(tile + m * 128 + (((byte >> 4) ^ (m & 7)) << 4) + (byte & 15)) = v;
      }
    }
    __syncthreads();
    if (nw < p.N) {
      const int c = lane & 7;
#pragma unroll
      for (int k = 0; k < kQaWM / 8; ++k) {
        const int m = k * 8 + (lane >> 3);
        const int gm = m0 + wm * kQaWM + m;
        const uint4 v = *(const uint4*)(tile + m * 128 + ((c ^ (m & 7)) << 4));
        if (gm < p.M) *(uint4*)((__bf16*)p.c + (int64_t)gm * p.N + nw + c * 8) = v;
      }
    }
  } else {
    static_assert(8 * (kQaWM / 2) * 256 <= 2 * kQaStage, "staging fits in the stages");
    uint8_t* tile = lds + wave * ((kQaWM / 2) * 256);
    const int c = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h) __syncthreads();
#pragma unroll
      for (int i = 0; i < kQaSubM / 2; ++i) {
        const int m = i * 16 + lr;
#pragma unroll
        for (int j = 0; j < kQaSubN; ++j)
          *(v4f*)(tile + m * 256 + (((j * 4 + lk) ^ (m & 15)) << 4)) = acc[h * (kQaSubM / 2) + i][j];
      }
      __syncthreads();
      if (nw < p.N) {
#pragma unroll
        for (int k = 0; k < kQaWM / 8; ++k) {
          const int m = k * 4 + (lane >> 4);
          const int gm = m0 + wm * kQaWM + h * (kQaWM / 2) + m;
          const v4f v = *(const v4f*)(tile + m * 256 + ((c ^ (m & 15)) << 4));
          if (gm < p.M) *(v4f*)((float*)p.c + (int64_t)gm * p.N + nw + c * 4) = v;
        }
      }
    }
  }
}

hipError_t launch_gemm_quant_a(const void* a, const uint8_t* b, const float* sb, void* c,
                               bool bf16_out, int64_t M, int64_t N, int64_t K, uint8_t* qa,
                               float* sa, hipStream_t stream) {
  QaArgs args{a, b, sb, c, qa, sa, (int)M, (int)N, (int)K};
  const int64_t tiles = ((M + kQaBM - 1) / kQaBM) * ((N + kQaBN - 1) / kQaBN);
  const dim3 grid((unsigned)tiles), block(kQaThreads);
  if (bf16_out)
    hipLaunchKernelGGL(gemm_qa_kernel<true>, grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL(gemm_qa_kernel<false>, grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace fp8q
