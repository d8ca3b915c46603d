// Backward-pass re-tiling kernels for gfx950: 128x1 activation tiles and the
// 128x128 weight-block transpose.
//
// The backward pass of a linear layer Y = X W^T needs
//   dX = dY W      : dY in 1x128 tiles (the forward quantizer), W^T in
//                    128x128 blocks -> the weight codes transposed;
//   dW = dY^T X    : both operands reduced over the tokens M, i.e. quantized
//                    in 128x1 tiles (128 tokens of one channel) and laid out
//                    channel-major so that M is the contiguous dimension.
// The conversion of activations from 1x128 to 128x1 tiles for the backward
// pass is in the Figure 7 (a) passage of "Six Reasons Deepseek Ai Is A Waste
// Of Time" (myomija.com); that the forward activations are kept as 1x128 FP8
// tiles is in the memory paragraph of the woojincopolymer.co.kr post.
//
// One kernel template covers four sources, all mapped 128 x 128 tile by tile
// from a row-major R x C input to the row-major C x R output:
//   kBf16      : bf16 activations -> 128x1 quantization (transposed codes)
//   kBf16Dual  : as kBf16, and also the 1x128 quantization of the same tile
//                (its 128 rows are whole 1x128 tiles): both layouts of an
//                output gradient from one read of it
//   kFp8Scaled : stored 1x128 codes + scales -> each element dequantized to
//                binary32 (one rounding of code * scale) -> 128x1 quantization
//   kFp8Copy   : 128x128-block codes copied transposed, block scale moved
//
// Per workgroup (256 threads): the tile is read row by row with 16-byte
// coalesced loads into LDS; thread t then walks column t % 128 over rows
// 64 (t / 128) .. +63 (one 128x1 tile per column, split between two waves
// whose maxima meet in LDS), quantizes its 64 values and writes the 64 codes
// as one contiguous piece of a transposed row in LDS; finally 8 lanes per
// output row store 128-byte runs. The input bytes are read once from HBM and
// the output bytes written once; the kernels are HBM-streaming.
#include "common.hpp"

namespace fp8q {

enum class Retile { kBf16, kBf16Dual, kFp8Scaled, kFp8Copy };

constexpr int kRtThreads = 256;
constexpr int kRtOutStride = 144;  // LDS bytes per transposed row: 128 codes + 16 pad

template <Retile S>
struct RetileCfg {
  static constexpr bool kBf16In = (S == Retile::kBf16 || S == Retile::kBf16Dual);
  static constexpr int kInRowBytes = kBf16In ? 256 : 128;  // one tile row in global memory
  // LDS row stride: bf16 rows padded by 16 bytes so that the row pass's
  // 16-byte reads (two threads per row) fall in distinct banks
  static constexpr int kLdsRow = kBf16In ? 272 : 128;
  static constexpr int kInBytes = 128 * kLdsRow;
  static constexpr int kBufBytes = kInBytes > 128 * kRtOutStride ? kInBytes : 128 * kRtOutStride;
  static constexpr int kLoads = 128 * kInRowBytes / 16 / kRtThreads;  // 16-byte chunks per thread
};

// Decode one E4M3 byte (exact in binary32).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// in:  R x C row-major (bf16 or E4M3 bytes)
// in_s: kFp8Scaled: R x (C/128) scales; kFp8Copy: (R/128) x (C/128) block scales
// out: C x R E4M3 bytes;  out_s: kBf16/kFp8Scaled: C x (R/128); kFp8Copy: (C/128) x (R/128)
// kBf16Dual only: row_q R x C E4M3 bytes and row_s R x (C/128), the 1x128 quantization
template <Retile S>
__global__ __launch_bounds__(kRtThreads) void retile_kernel(const uint8_t* __restrict__ in,
                                                            const float* __restrict__ in_s,
                                                            uint8_t* __restrict__ out,
                                                            float* __restrict__ out_s,
                                                            uint8_t* __restrict__ row_q,
                                                            float* __restrict__ row_s, int R,
                                                            int C) {
  using Cfg = RetileCfg<S>;
  __shared__ __attribute__((aligned(16))) uint8_t buf[Cfg::kBufBytes];
  __shared__ float row_scale[128];
  __shared__ float half_max[128];
  __shared__ float full_max[128];

  const int t = threadIdx.x;
  const int rt = blockIdx.x;  // tile row: input rows 128 rt ..
  const int ct = blockIdx.y;  // tile column: input columns 128 ct ..
  const int Gc = C / kGroup;
  const int Gr = R / kGroup;

  // ---- input tile -> LDS, row-major, 16-byte chunks ----
  {
    constexpr int kChunksPerRow = Cfg::kInRowBytes / 16;
    const int64_t row_bytes = (int64_t)C * (Cfg::kInRowBytes / 128);
    const uint8_t* src = in + (int64_t)rt * 128 * row_bytes + (int64_t)ct * Cfg::kInRowBytes;
    uint4 v[Cfg::kLoads];
#pragma unroll
    for (int i = 0; i < Cfg::kLoads; ++i) {
      const int c = t + i * kRtThreads;
      v[i] = load_nt((const uint4*)(src + (c / kChunksPerRow) * row_bytes + (c % kChunksPerRow) * 16));
    }
    if constexpr (S == Retile::kFp8Scaled) {
      if (t < 128) row_scale[t] = in_s[((int64_t)rt * 128 + t) * Gc + ct];
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoads; ++i) {
      const int c = t + i * kRtThreads;
      *(uint4*)(buf + (c / kChunksPerRow) * Cfg::kLdsRow + (c % kChunksPerRow) * 16) = v[i];
    }
  }
  __syncthreads();

  // ---- kBf16Dual, row pass: each tile row is one 1x128 tile; thread t
  // quantizes half t & 1 (64 values) of row t >> 1, the pair exchanging maxima
  if constexpr (S == Retile::kBf16Dual) {
    const int row = t >> 1, half = t & 1;
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *(const uint4*)(buf + row * Cfg::kLdsRow + half * 128 + j * 16);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v[j].x)), fabsf(bf16_hi(v[j].x))),
                               fmaxf(fabsf(bf16_lo(v[j].y)), fabsf(bf16_hi(v[j].y)))),
                         fmaxf(fmaxf(fabsf(bf16_lo(v[j].z)), fabsf(bf16_hi(v[j].z))),
                               fmaxf(fabsf(bf16_lo(v[j].w)), fabsf(bf16_hi(v[j].w))))));
    // partner lane t ^ 1 (quad_perm [1,0,3,2]); non-negative floats order like their bits
    const uint32_t mb = __float_as_uint(m);
    const float amax = __uint_as_float(
        umax(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0xB1, 0xF, 0xF, false)));
    const float s = tile_scale(amax);
    const TileDivisor d = make_divisor(s, amax);
    uint8_t* dst = row_q + ((int64_t)rt * 128 + row) * C + (int64_t)ct * 128 + half * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 lo = quant8(v[2 * j], d), hi = quant8(v[2 * j + 1], d);
      *(uint4*)(dst + 16 * j) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    if (half == 0) row_s[((int64_t)rt * 128 + row) * Gc + ct] = s;
  }

  // ---- column pass: thread t owns column k, rows 64 h .. 64 h + 63 ----
  const int k = t & 127;
  const int h = t >> 7;
  uint32_t w[16];  // the 64 output codes, little-endian in 16 dwords

  if constexpr (S == Retile::kFp8Copy) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t d = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) d |= (uint32_t)buf[(64 * h + 4 * j + b) * Cfg::kLdsRow + k] << (8 * b);
      w[j] = d;
    }
    __syncthreads();  // every read of the input tile is done before it is overwritten
  } else {
    float v[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int row = 64 * h + i;
      if constexpr (Cfg::kBf16In) {
        v[i] = __uint_as_float((uint32_t)(*(const uint16_t*)(buf + row * Cfg::kLdsRow + 2 * k)) << 16);
      } else {
        v[i] = __fmul_rn(e4m3_to_f32(buf[row * Cfg::kLdsRow + k]), row_scale[row]);
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(v[i]));
    if (h == 1) half_max[k] = m;
    __syncthreads();  // also: every read of the input tile is done
    if (h == 0) full_max[k] = fmaxf(m, half_max[k]);
    __syncthreads();
    const float amax = full_max[k];
    const float s = tile_scale(amax);
    const TileDivisor d = make_divisor(s, amax);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      w[j] = pack4_e4m3(quotient(v[4 * j], d), quotient(v[4 * j + 1], d), quotient(v[4 * j + 2], d),
                        quotient(v[4 * j + 3], d));
    if (h == 0) out_s[((int64_t)ct * 128 + k) * Gr + rt] = s;
  }
  if constexpr (S == Retile::kFp8Copy) {
    if (t == 0) out_s[(int64_t)ct * Gr + rt] = in_s[(int64_t)rt * Gc + ct];
  }

  // ---- codes -> LDS, transposed: output row k, bytes 64 h .. 64 h + 63 ----
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *(uint4*)(buf + k * kRtOutStride + 64 * h + 16 * j) =
        make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  __syncthreads();

  // ---- LDS -> output: 8 lanes per 128-byte output row ----
  uint8_t* dst = out + (int64_t)ct * 128 * R + (int64_t)rt * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + i * kRtThreads;
    const int row = c >> 3, ch = c & 7;
    *(uint4*)(dst + (int64_t)row * R + ch * 16) = *(const uint4*)(buf + row * kRtOutStride + ch * 16);
  }
}

template <Retile S>
static hipError_t launch_retile(const void* in, const float* in_s, uint8_t* out, float* out_s,
                                int64_t R, int64_t C, hipStream_t stream,
                                uint8_t* row_q = nullptr, float* row_s = nullptr) {
  const dim3 grid((unsigned)(R / kGroup), (unsigned)(C / kGroup));
  hipLaunchKernelGGL(retile_kernel<S>, grid, dim3(kRtThreads), 0, stream, (const uint8_t*)in, in_s,
                     out, out_s, row_q, row_s, (int)R, (int)C);
  return hipGetLastError();
}

hipError_t launch_quant_act_dual(const void* x, int64_t M, int64_t K, uint8_t* q, float* sa,
                                 uint8_t* qt, float* st, hipStream_t stream) {
  return launch_retile<Retile::kBf16Dual>(x, nullptr, qt, st, M, K, stream, q, sa);
}

hipError_t launch_quant_act_128x1(const void* x, int64_t M, int64_t K, uint8_t* qt, float* st,
                                  hipStream_t stream) {
  return launch_retile<Retile::kBf16>(x, nullptr, qt, st, M, K, stream);
}

hipError_t launch_requant_1x128_to_128x1(const uint8_t* q, const float* sa, int64_t M, int64_t K,
                                         uint8_t* qt, float* st, hipStream_t stream) {
  return launch_retile<Retile::kFp8Scaled>(q, sa, qt, st, M, K, stream);
}

hipError_t launch_transpose_weight_128x128(const uint8_t* q, const float* sb, int64_t N, int64_t K,
                                           uint8_t* qt, float* sbt, hipStream_t stream) {
  return launch_retile<Retile::kFp8Copy>(q, sb, qt, sbt, N, K, stream);
}

}  // namespace fp8q
