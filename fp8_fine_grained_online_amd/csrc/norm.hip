// Layer normalization fused with the 1x128 FP8 cast, for gfx950.
//
// The woojincopolymer.co.kr post (hardware suggestions) wants layer
// normalization and the FP8 cast fused; "Six Reasons Deepseek Ai Is A Waste Of
// Time" keeps normalization in higher precision while the GEMMs run in FP8.
// Here one wavefront normalizes one row held in its registers (four rows per
// workgroup share gamma and beta, staged once in LDS) and quantizes
// the binary32 result per 1x128 tile straight to E4M3 codes and scales: the
// row is read from HBM once and no BF16 copy of the normalized row exists.
//
// Per row x (K bf16 values):
//   RMS:      S = sum x^2,  r = fl32(1 / sqrt(S/K + eps)),  y = fl32(fl32(x r) g)
//   centred:  mu = sum x / K,  var = sum fl64(x - mu)^2 / K,
//             r = fl32(1 / sqrt(var + eps)),
//             y = fl32(fl32(fl32(fl32(x - fl32(mu)) r) g) + b)
// with every float64 step correctly rounded (division, square root) and the
// statistics equal to the correctly rounded exact sums, not a function of the
// summation order: a fast plain float64 pass whose result is certified (see
// certified_inv_std and the exponent-span test of the mean), with an
// error-free double-double pass (TwoSum per term, then a butterfly across the
// wavefront whose every combination is symmetric, so all lanes hold the same
// bits) where the certificate fails. Then y is quantized per 1x128 tile with
// the activation rule (amax, s = fl32(amax/448), codes of fl32(y/s)).
//
// Every rounding above must happen as written: the library is compiled with
// floating-point contraction off, so no product is fused into the addition
// that follows it (e.g. the "+ b" or the sum of d * d).
#include "common.hpp"

namespace fp8q {

constexpr int kNormThreads = 256;  // 4 rows per workgroup, one per wavefront (faster than 8 or 16)

struct DD {
  double hi, lo;
};

// Knuth's TwoSum: s + e == a + b exactly
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = __dadd_rn(a, b);
  const double bb = __dsub_rn(s, a);
  e = __dadd_rn(__dsub_rn(a, __dsub_rn(s, bb)), __dsub_rn(b, bb));
}

__device__ __forceinline__ DD dd_add_term(DD acc, double p) {
  double s, e;
  two_sum(acc.hi, p, s, e);
  return DD{s, __dadd_rn(acc.lo, e)};
}

// (a.hi + a.lo) + (b.hi + b.lo), renormalized; symmetric in a and b
__device__ __forceinline__ DD dd_add(DD a, DD b) {
  double s, e;
  two_sum(a.hi, b.hi, s, e);
  e = __dadd_rn(e, __dadd_rn(a.lo, b.lo));
  const double hi = __dadd_rn(s, e);
  return DD{hi, __dsub_rn(e, __dsub_rn(hi, s))};
}

__device__ __forceinline__ double wave_sum(DD v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    DD o;
    o.hi = __shfl_xor(v.hi, m);
    o.lo = __shfl_xor(v.lo, m);
    v = dd_add(v, o);
  }
  return __dadd_rn(v.hi, v.lo);
}

__device__ __forceinline__ float inv_std(double stat_over_k, float eps) {
  const double t = __dadd_rn(stat_over_k, (double)eps);
  return (float)__ddiv_rn(1.0, __dsqrt_rn(t));
}

// Plain float64 sum over the wavefront; every combination is a symmetric
// addition, so all lanes end with the same bits.
__device__ __forceinline__ double wave_sum_plain(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = __dadd_rn(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m));
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m));
  return v;
}

// The fast statistics are plain float64 sums of nonnegative terms with at
// most 256 + 6 roundings in any chain (a lane's terms, then the butterfly),
// so they are within a relative 263 * 2^-53 < 2^-44 of the exact sum, and the
// exact sum's float64 rounding lies in S_fast * [1 - 2^-43, 1 + 2^-43]. Every
// step from S to r (S/K, + eps, sqrt, 1/x, then to binary32) is correctly
// rounded and monotone in S, so when both ends of that interval give the same
// binary32 r, it is the r of the exact sum; otherwise the caller recomputes
// the sum exactly (double-double). Returns true when r is certified.
__device__ __forceinline__ bool certified_inv_std(double S_fast, int K, float eps, float& r) {
  const double m = __dmul_rn(S_fast, 0x1p-43);
  const float lo = inv_std(__ddiv_rn(__dadd_rn(S_fast, m), (double)K), eps);  // largest sum
  const float hi = inv_std(__ddiv_rn(__dsub_rn(S_fast, m), (double)K), eps);  // smallest sum
  r = lo;
  return lo == hi;
}

// biased exponent field of a nonzero bf16 value, subnormals counted as 1 (they
// are multiples of the same quantum as exponent 1); zeros give `none`
__device__ __forceinline__ uint32_t bf16_exp_or(uint32_t half, uint32_t none) {
  const uint32_t e = (half >> 7) & 0xFFu;
  return (half & 0x7FFFu) ? (e ? e : 1u) : none;
}

// An empty asm that "modifies" the packed row: values unpacked from it before
// cannot be reused after, so each pass re-unpacks (a few bit operations)
// instead of keeping 8 floats or doubles per chunk live across passes.
template <int N>
__device__ __forceinline__ void reunpack_fence(uint4 (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
}

__device__ __forceinline__ void unpack8(uint4 w, float f[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Wavefronts per SIMD the compiler must fit: five for the RMS kernel up to 14
// chunks per lane (K <= 7168), which then keeps four VGPRs in scratch and runs
// 3% faster at 16384 x 7168 (89.7 against 92.7 us); otherwise no constraint
// (the centred kernel would spill 40 VGPRs and ran 134 against 108 us).
template <int kChunks, bool kCentred>
constexpr int kNormWavesPerSimd = (!kCentred && kChunks <= 14) ? 5 : 1;

// kChunks: the most 16-byte chunks (8 values) a lane holds, K <= kChunks * 512
template <int kChunks, bool kCentred>
__global__ __launch_bounds__(kNormThreads) __attribute__((amdgpu_waves_per_eu(kNormWavesPerSimd<kChunks, kCentred>)))
void norm_quant_1x128_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ gamma, const uint4* __restrict__ beta,
    float eps, uint2* __restrict__ q, float* __restrict__ sa, int M, int K) {
  // gamma (and beta) for all rows of the workgroup, staged once in LDS
  extern __shared__ uint4 params[];  // [K/8] gamma, then [K/8] beta when centred
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kNormThreads / 64) + (threadIdx.x >> 6);
  const bool active = row < M;  // whole wavefront
  const int n_chunks = K / 8;
  const uint4* xr = x + (int64_t)row * n_chunks;

  // chunk lane + 64 i of the row; a 1x128 tile is 16 chunks = one DPP row of
  // 16 lanes within one i. The row's loads are issued first.
  uint4 v[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = lane + 64 * i;
    v[i] = (active && c < n_chunks) ? load_nt(xr + c) : make_uint4(0, 0, 0, 0);  // absent: zeros
  }
  for (int c = threadIdx.x; c < n_chunks; c += kNormThreads) {
    params[c] = gamma[c];
    if constexpr (kCentred) params[n_chunks + c] = beta[c];
  }
  __syncthreads();
  if (!active) return;

  // Statistics: a fast float64 pass whose result is certified exact, with an
  // error-free double-double pass only where the certificate fails (rare:
  // r within 2^-43 of a binary32 rounding boundary, or a centred row whose
  // magnitudes span more than 31 binades).
  float r, mu32 = 0.0f;
  if constexpr (kCentred) {
    // The values of the row are multiples of 2^(emin - 134) below 2^(emax - 126);
    // with K <= 2^14 every partial sum then fits in 53 bits when
    // emax - emin <= 31, so the plain float64 sum is exact in any order.
    double s1 = 0.0;
    uint32_t emax = 0, emin = 255;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        emax = max(emax, max(bf16_exp_or(w[h] & 0xFFFFu, 0u), bf16_exp_or(w[h] >> 16, 0u)));
        emin = min(emin, min(bf16_exp_or(w[h] & 0xFFFFu, 255u), bf16_exp_or(w[h] >> 16, 255u)));
        s1 = __dadd_rn(s1, (double)bf16_lo(w[h]));
        s1 = __dadd_rn(s1, (double)bf16_hi(w[h]));
      }
    }
    emax = wave_max_u32(emax);
    emin = wave_min_u32(emin);
    double S1;
    if ((int)emax - (int)emin <= 31) {
      S1 = wave_sum_plain(s1);
    } else {
      reunpack_fence(v);
      DD d1{0.0, 0.0};
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) d1 = dd_add_term(d1, (double)f[e]);
      }
      S1 = wave_sum(d1);
    }
    const double mu = __ddiv_rn(S1, (double)K);
    reunpack_fence(v);
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (lane + 64 * i >= n_chunks) continue;  // absent chunks would add mu^2
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double d = __dsub_rn((double)f[e], mu);
        s2 = __dadd_rn(s2, __dmul_rn(d, d));
      }
    }
    if (!certified_inv_std(wave_sum_plain(s2), K, eps, r)) {
      reunpack_fence(v);
      DD d2{0.0, 0.0};
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        if (lane + 64 * i >= n_chunks) continue;
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = __dsub_rn((double)f[e], mu);
          d2 = dd_add_term(d2, __dmul_rn(d, d));
        }
      }
      r = inv_std(__ddiv_rn(wave_sum(d2), (double)K), eps);
    }
    mu32 = (float)mu;
  } else {
    double s2 = 0.0;  // squares of bf16 values are exact in float64: one rounding per term
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s2 = __fma_rn((double)f[e], (double)f[e], s2);
    }
    if (!certified_inv_std(wave_sum_plain(s2), K, eps, r)) {
      reunpack_fence(v);
      DD d2{0.0, 0.0};
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        float f[8];
        unpack8(v[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) d2 = dd_add_term(d2, __dmul_rn((double)f[e], (double)f[e]));
      }
      r = inv_std(__ddiv_rn(wave_sum(d2), (double)K), eps);
    }
  }

  reunpack_fence(v);
  const int G = K / kGroup;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = lane + 64 * i;
    if (64 * i >= n_chunks) break;  // uniform: no chunk of this i exists
    const bool have = c < n_chunks;  // whole DPP rows (tiles) are present or absent
    float f[8], g[8], b[8];
    unpack8(v[i], f);
    unpack8(have ? params[c] : make_uint4(0, 0, 0, 0), g);
    if constexpr (kCentred) unpack8(have ? params[n_chunks + c] : make_uint4(0, 0, 0, 0), b);
    float y[8];
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (kCentred)
        y[e] = __fadd_rn(__fmul_rn(__fmul_rn(__fsub_rn(f[e], mu32), r), g[e]), b[e]);
      else
        y[e] = __fmul_rn(__fmul_rn(f[e], r), g[e]);
      m = fmaxf(m, fabsf(y[e]));
    }
    const float amax = __uint_as_float(row16_max_u32(__float_as_uint(m)));
    const float s = tile_scale(amax);
    const TileDivisor d = make_divisor(s, amax);
    uint2 out;
    out.x = pack4_e4m3(quotient(y[0], d), quotient(y[1], d), quotient(y[2], d), quotient(y[3], d));
    out.y = pack4_e4m3(quotient(y[4], d), quotient(y[5], d), quotient(y[6], d), quotient(y[7], d));
    if (have) {
      q[(int64_t)row * n_chunks + c] = out;
      if ((lane & 15) == 0) sa[(int64_t)row * G + (c >> 4)] = s;
    }
  }
}

template <int kChunks>
static hipError_t launch_norm_chunks(const void* x, const void* gamma, const void* beta, float eps,
                                     bool centred, int64_t M, int64_t K, uint8_t* q, float* sa,
                                     hipStream_t stream) {
  const int rows = kNormThreads / 64;
  const dim3 grid((unsigned)((M + rows - 1) / rows));
  const size_t lds = (size_t)(centred ? 2 : 1) * (size_t)K * 2;  // gamma (+ beta), bf16
  if (centred)
    hipLaunchKernelGGL((norm_quant_1x128_kernel<kChunks, true>), grid, dim3(kNormThreads), lds,
                       stream, (const uint4*)x, (const uint4*)gamma, (const uint4*)beta, eps,
                       (uint2*)q, sa, (int)M, (int)K);
  else
    hipLaunchKernelGGL((norm_quant_1x128_kernel<kChunks, false>), grid, dim3(kNormThreads), lds,
                       stream, (const uint4*)x, (const uint4*)gamma, (const uint4*)beta, eps,
                       (uint2*)q, sa, (int)M, (int)K);
  return hipGetLastError();
}

constexpr int64_t kNormMaxK = 16384;

hipError_t launch_norm_quant_act_1x128(const void* x, const void* gamma, const void* beta,
                                       float eps, bool centred, int64_t M, int64_t K, uint8_t* q,
                                       float* sa, hipStream_t stream) {
  // chunks per lane; the row array is sized to the next instantiated count,
  // since unused entries still take registers (K = 7168 with 16 chunks per
  // lane instead of 14: centred 142 us instead of 114 at 16384 rows)
  const int64_t per_lane = (K / 8 + 63) / 64;
#define FP8Q_NORM_CHUNKS(n) \
  if (per_lane <= n) return launch_norm_chunks<n>(x, gamma, beta, eps, centred, M, K, q, sa, stream);
  FP8Q_NORM_CHUNKS(2)
  FP8Q_NORM_CHUNKS(4)
  FP8Q_NORM_CHUNKS(6)
  FP8Q_NORM_CHUNKS(8)
  FP8Q_NORM_CHUNKS(10)
  FP8Q_NORM_CHUNKS(12)
  FP8Q_NORM_CHUNKS(14)
  FP8Q_NORM_CHUNKS(16)
  FP8Q_NORM_CHUNKS(20)
  FP8Q_NORM_CHUNKS(24)
  FP8Q_NORM_CHUNKS(28)
#undef FP8Q_NORM_CHUNKS
  return launch_norm_chunks<32>(x, gamma, beta, eps, centred, M, K, q, sa, stream);
}

}  // namespace fp8q
