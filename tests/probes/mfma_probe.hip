// Test-only probe of gfx950's FP8 matrix core (not part of the library): one
// wavefront computes D = A * B^T + C for a 16 x 16 tile over G K-groups of
// 128, with the same operand layout as the library's GEMM (B first, so lane l
// holds D[l % 16][4 (l / 16) + r], r = 0..3), either
//   mode 0: chaining the MFMAs through their accumulator input
//           (D = mfma(g = G-1, ... mfma(g = 0, C))), or
//   mode 1: one MFMA per group with a zero accumulator, the partials added to
//           C in FP32 by the vector ALU (what the library does).
// It answers whether the FP8 MFMA also loses low bits when it accumulates into
// a nonzero C, the question of the limited accumulation width the pages raise
// for H800 Tensor Cores ("Six Reasons Deepseek Ai Is A Waste Of Time",
// preliminary test and promotion passages).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// a: 16 x K codes, b: 16 x K codes (K = 128 G), c_in and d: 16 x 16 floats
__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint8_t* __restrict__ a,
                                                        const uint8_t* __restrict__ b,
                                                        const float* __restrict__ c_in,
                                                        float* __restrict__ d, int G, int mode) {
  const int lane = threadIdx.x;
  const int lr = lane & 15, lk = lane >> 4;
  const int K = 128 * G;
  v4f acc, sum;
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = c_in[lr * 16 + 4 * lk + r];
  sum = acc;
  for (int g = 0; g < G; ++g) {
    const uint8_t* ar = a + lr * K + g * 128 + lk * 16;
    const uint8_t* br = b + lr * K + g * 128 + lk * 16;
    const uint4 alo = *(const uint4*)ar, ahi = *(const uint4*)(ar + 64);
    const uint4 blo = *(const uint4*)br, bhi = *(const uint4*)(br + 64);
    const v8i af = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                    (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
    const v8i bf = {(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w,
                    (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
    if (mode == 0) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc, 0, 0, 0, 0, 0, 0);
    } else {
      const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          bf, af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] = sum[r] + p[r];
    }
  }
  const v4f out = mode == 0 ? acc : sum;
#pragma unroll
  for (int r = 0; r < 4; ++r) d[lr * 16 + 4 * lk + r] = out[r];
}

extern "C" __attribute__((visibility("default"))) int mfma_probe(const uint8_t* a, const uint8_t* b,
                                                                 const float* c_in, float* d,
                                                                 int G, int mode, void* stream) {
  if (!a || !b || !c_in || !d || G < 1 || (mode != 0 && mode != 1)) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, c_in, d, G,
                     mode);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
