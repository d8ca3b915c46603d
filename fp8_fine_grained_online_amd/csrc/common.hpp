// Device helpers shared by the gfx950 kernels: bf16 unpacking, the E4M3
// conversion, and cross-lane reductions inside 16-lane DPP rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load: data read once need not stay cached.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kGroup = 128;       // K-group (1x128 tile width, 128x128 block side)
constexpr float kFp8Max = 448.0f; // largest finite OCP E4M3FN value

// bf16 bit pairs packed in a dword -> the two float32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |bf16| bits of both halves; comparing these as unsigned integers orders the
// magnitudes of finite values.
__device__ __forceinline__ uint32_t abs2_bits(uint32_t w) { return w & 0x7FFF7FFFu; }

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over the 16 lanes of each DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the result.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// max over the 8 lanes of each half DPP row (lanes 8r .. 8r+7)
__device__ __forceinline__ uint32_t row8_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

// Tile scale s = fl32(amax / 448), the correctly rounded binary32 quotient.
// For amax >= 2^-116 (every quotient normal) it is one multiply by
// c = RN(1/448) and one FMA correction, q0 = RN(amax c), then
// q = RN(q0 + RN(amax - 448 q0) c): an exhaustive host comparison over every
// binary32 amax found it equal to the correctly rounded quotient wherever
// that quotient is normal, and only there, so smaller amax take the IEEE
// division (a branch no tile of ordinary data takes).
__device__ __forceinline__ float tile_scale(float amax) {
  constexpr float kInv448 = 1.0f / 448.0f;  // RN(1/448)
  if (amax < 0x1p-116f) return __fdiv_rn(amax, kFp8Max);
  const float q0 = amax * kInv448;
  return __builtin_fmaf(__builtin_fmaf(-q0, kFp8Max, amax), kInv448, q0);
}

// RN(1/x) for binary32 x in [2^-85, 2^120): one Newton step from the hardware
// reciprocal estimate, r = RN(r0 + RN(1 - x r0) r0) with r0 = v_rcp_f32(x).
// An exhaustive GPU comparison with the IEEE division over every binary32 in
// that range found no difference (outside it, for subnormal x or a subnormal
// result, there are).
__device__ __forceinline__ float recip_rn(float x) {
  const float r0 = __builtin_amdgcn_rcpf(x);
  return __builtin_fmaf(__builtin_fmaf(-x, r0, 1.0f), r0, r0);
}

// Per-tile quotient x / s, correctly rounded in binary32.
//
// The divide is replaced by a reciprocal and one FMA correction
// (Markstein's scheme): r = RN(1/s') once per tile, then
//   q0 = RN(x' r),  e = RN(x' - s' q0) (exact),  q = RN(q0 + e r).
// With s' and x' scaled by the same power of two p (chosen so that amax * p is
// not tiny), x'/s' = x/s exactly, and the residual e never underflows. An
// exhaustive host comparison against IEEE division over every bf16 amax and
// every bf16 |x| <= amax showed identical quotients wherever the quotient can
// change an E4M3 code (|x/s| > 2^-11); below that every code is a signed
// zero either way. The sign of x is re-attached so that -0 and negative
// underflows keep their sign.
struct TileDivisor {
  float sp;  // s * p
  float r;   // RN(1 / (s * p))
  float p;   // power of two applied to x (1 unless amax < 2^-64)
};

__device__ __forceinline__ TileDivisor make_divisor(float s, float amax) {
  TileDivisor d;
  if (s == 0.0f) {
    // all-zero tile (scale 0): every x is +-0 and passes through unchanged,
    // so the codes are zeros carrying the sign of x
    d.p = 1.0f;
    d.sp = 1.0f;
    d.r = 1.0f;
    return d;
  }
  d.p = (amax < 0x1p-64f) ? 0x1p+64f : 1.0f;
  d.sp = s * d.p;  // exact: power-of-two scaling of a finite value
  // s > 0 here, so s >= 2^-149 and sp >= 2^-85 (tiny tiles are scaled by
  // 2^64); sp <= FLT_MAX / 448 < 2^120: inside recip_rn's verified range
  d.r = recip_rn(d.sp);
  return d;
}

__device__ __forceinline__ float quotient(float x, const TileDivisor& d) {
  float xs = x * d.p;
  float q0 = xs * d.r;
  float e = __builtin_fmaf(-q0, d.sp, xs);
  float q = __builtin_fmaf(e, d.r, q0);
  // copysign(q, x) as one bitfield insert
  return __uint_as_float((__float_as_uint(q) & 0x7FFFFFFFu) | (__float_as_uint(x) & 0x80000000u));
}

// Four quotients -> four E4M3 codes packed little-endian in a dword.
// Saturation at +-448 is explicit (fmed3), then the hardware converts with
// round-to-nearest-even.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
  b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
  c = __builtin_amdgcn_fmed3f(c, -kFp8Max, kFp8Max);
  d = __builtin_amdgcn_fmed3f(d, -kFp8Max, kFp8Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// max |x| over the 8 bf16 values of a 16-byte chunk
__device__ __forceinline__ float absmax8(uint4 v) {
  return fmaxf(fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                     fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))),
               fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                     fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
}

// Quantize the 8 bf16 values in `in` (4 dwords) to 8 codes (2 dwords).
__device__ __forceinline__ uint2 quant8(uint4 in, const TileDivisor& d) {
  uint2 out;
  out.x = pack4_e4m3(quotient(bf16_lo(in.x), d), quotient(bf16_hi(in.x), d),
                     quotient(bf16_lo(in.y), d), quotient(bf16_hi(in.y), d));
  out.y = pack4_e4m3(quotient(bf16_lo(in.z), d), quotient(bf16_hi(in.z), d),
                     quotient(bf16_lo(in.w), d), quotient(bf16_hi(in.w), d));
  return out;
}

}  // namespace fp8q
