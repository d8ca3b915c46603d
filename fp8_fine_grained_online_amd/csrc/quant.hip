// Online fine-grained FP8 quantization kernels for gfx950.
//
//  * 1x128 activation tiles ("per token per 128 channels") and 128x128 weight
//    blocks ("per 128 input channels per 128 output channels"): the Figure 7 (a)
//    passage of "Six Reasons Deepseek Ai Is A Waste Of Time" (myomija.com).
//  * The scale maps each tile's/block's current maximum |x| to 448, the largest
//    E4M3 value (standard-practice paragraph of the same page; computed online,
//    per the "online quantization" section of the Greek codingmall.com page).
//
// Both kernels are HBM-streaming: 2 bytes read, 1 byte + 4/128 bytes written
// per element. Loads and stores are 16-byte / 8-byte per lane and coalesced.
// The bf16 inputs are read once (non-temporal loads); the codes and scales are
// stored normally so that the GEMM consuming them next finds them in cache,
// unless the codes are larger than that cache (then non-temporally, and the
// activation kernel also has an explicitly non-temporal entry point).
#include "common.hpp"

namespace fp8q {

// ---------------------------------------------------------------------------
// 1x128 activation quantization.
//
// A row-major M x K matrix with K % 128 == 0 is a flat array of 1x128 tiles:
// tile t holds elements [128 t, 128 t + 128), its scale is sa[t]. A tile is
// 16 chunks of 16 bytes (8 bf16), one chunk per lane, so a DPP row of 16 lanes
// owns one tile and reduces its amax with four DPP steps. Each thread handles
// kActUnroll chunks spaced one block-width apart, all loads issued first.
// kNt: codes and scales go out with non-temporal stores, which do not keep
// them in the Infinity Cache (for outputs that are not read next on this GPU).
// ---------------------------------------------------------------------------
constexpr int kActThreads = 256;
constexpr int kActUnroll = 2;

template <bool kNt>
__global__ __launch_bounds__(kActThreads) void quant_act_1x128_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ sa, int64_t n_tiles) {
  const int64_t n_chunks = n_tiles * 16;
  const int64_t base = (int64_t)blockIdx.x * (kActThreads * kActUnroll) + threadIdx.x;
  uint4 v[kActUnroll];
#pragma unroll
  for (int u = 0; u < kActUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kActThreads;
    v[u] = (c < n_chunks) ? load_nt(x + c) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kActUnroll; ++u) {
    const int64_t c = base + (int64_t)u * kActThreads;
    float f[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                  bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    // non-negative floats order like their bit patterns
    const float amax = __uint_as_float(row16_max_u32(__float_as_uint(m)));
    const float s = tile_scale(amax);
    const TileDivisor d = make_divisor(s, amax);
    uint2 out;
    out.x = pack4_e4m3(quotient(f[0], d), quotient(f[1], d), quotient(f[2], d), quotient(f[3], d));
    out.y = pack4_e4m3(quotient(f[4], d), quotient(f[5], d), quotient(f[6], d), quotient(f[7], d));
    if (c < n_chunks) {
      if constexpr (kNt) {
        __builtin_nontemporal_store(out.x, &q[c].x);
        __builtin_nontemporal_store(out.y, &q[c].y);
        if ((threadIdx.x & 15) == 0) __builtin_nontemporal_store(s, &sa[c >> 4]);
      } else {
        q[c] = out;  // ordinary store: a GEMM reading the codes next finds them cached
        if ((threadIdx.x & 15) == 0) sa[c >> 4] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 128x128 weight quantization: one workgroup per block, the whole block
// (32 KB of bf16) held in registers: 256 threads x 8 chunks of 16 bytes.
// Thread t owns chunk column t % 16 of rows t / 16 + 16 i, i = 0..7.
// ---------------------------------------------------------------------------
constexpr int kWThreads = 256;

template <bool kNt>
__global__ __launch_bounds__(kWThreads) void quant_weight_128x128_kernel(
    const uint4* __restrict__ w, uint2* __restrict__ q, float* __restrict__ sb, int64_t K,
    int nblk_k) {
  __shared__ uint32_t wave_max[kWThreads / 64];
  const int bk = blockIdx.x;
  const int64_t bn = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t chunks_per_row = K / 8;
  const int64_t c0 = (bn * kGroup + (t >> 4)) * chunks_per_row + (int64_t)bk * 16 + (t & 15);
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load_nt(w + c0 + (int64_t)i * 16 * chunks_per_row);

  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v[i].x)), fabsf(bf16_hi(v[i].x))),
                       fmaxf(fabsf(bf16_lo(v[i].y)), fabsf(bf16_hi(v[i].y)))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v[i].z)), fabsf(bf16_hi(v[i].z))),
                       fmaxf(fabsf(bf16_lo(v[i].w)), fabsf(bf16_hi(v[i].w)))));
  }
  uint32_t mb = row16_max_u32(__float_as_uint(m));
  mb = umax(umax(__builtin_amdgcn_readlane(mb, 0), __builtin_amdgcn_readlane(mb, 16)),
            umax(__builtin_amdgcn_readlane(mb, 32), __builtin_amdgcn_readlane(mb, 48)));
  if ((t & 63) == 0) wave_max[t >> 6] = mb;
  __syncthreads();
  mb = umax(umax(wave_max[0], wave_max[1]), umax(wave_max[2], wave_max[3]));
  const float amax = __uint_as_float(mb);
  const float s = tile_scale(amax);
  const TileDivisor d = make_divisor(s, amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint2 o = quant8(v[i], d);
    if constexpr (kNt) {
      __builtin_nontemporal_store(o.x, &q[c0 + (int64_t)i * 16 * chunks_per_row].x);
      __builtin_nontemporal_store(o.y, &q[c0 + (int64_t)i * 16 * chunks_per_row].y);
    } else {
      q[c0 + (int64_t)i * 16 * chunks_per_row] = o;
    }
  }
  if (t == 0) sb[bn * nblk_k + bk] = s;
}

// Codes beyond the 256 MB Infinity Cache cannot stay cached for the kernel
// that reads them next, so above that size both quantizers store them
// non-temporally (same bytes; the streaming stores move HBM traffic faster).
constexpr int64_t kCachedCodesMax = (int64_t)256 << 20;

hipError_t launch_quant_act_1x128(const void* x, int64_t M, int64_t K, uint8_t* q, float* sa,
                                  bool nontemporal, hipStream_t stream) {
  const int64_t n_tiles = M * (K / kGroup);
  const int64_t per_block = (int64_t)kActThreads * kActUnroll / 16;  // tiles per block
  const int64_t blocks = (n_tiles + per_block - 1) / per_block;
  if (nontemporal || M * K > kCachedCodesMax)
    hipLaunchKernelGGL(quant_act_1x128_kernel<true>, dim3((unsigned)blocks), dim3(kActThreads), 0,
                       stream, (const uint4*)x, (uint2*)q, sa, n_tiles);
  else
    hipLaunchKernelGGL(quant_act_1x128_kernel<false>, dim3((unsigned)blocks), dim3(kActThreads), 0,
                       stream, (const uint4*)x, (uint2*)q, sa, n_tiles);
  return hipGetLastError();
}

hipError_t launch_quant_weight_128x128(const void* w, int64_t N, int64_t K, uint8_t* q, float* sb,
                                       hipStream_t stream) {
  const int nblk_k = (int)(K / kGroup);
  const int nblk_n = (int)(N / kGroup);
  if (N * K > kCachedCodesMax)
    hipLaunchKernelGGL(quant_weight_128x128_kernel<true>, dim3(nblk_k, nblk_n), dim3(kWThreads), 0, stream,
                       (const uint4*)w, (uint2*)q, sb, K, nblk_k);
  else
    hipLaunchKernelGGL(quant_weight_128x128_kernel<false>, dim3(nblk_k, nblk_n), dim3(kWThreads), 0, stream,
                       (const uint4*)w, (uint2*)q, sb, K, nblk_k);
  return hipGetLastError();
}

}  // namespace fp8q
