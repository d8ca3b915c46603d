// Test-only probe: is RN(1/x) equal to one Newton step from the hardware
// reciprocal estimate, r1 = fma(fma(-x, r0, 1), r0, r0) with r0 = v_rcp_f32(x),
// for every binary32 x in [lo_bits, hi_bits)? Counts the mismatches against
// the correctly rounded division and records the smallest failing x.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ void rcp_check(uint32_t lo, uint32_t hi, unsigned long long* bad, uint32_t* first) {
  unsigned long long count = 0;
  uint32_t f = 0xFFFFFFFFu;
  for (uint64_t u = (uint64_t)lo + blockIdx.x * 256ull + threadIdx.x; u < hi;
       u += (uint64_t)gridDim.x * 256ull) {
    const float x = __uint_as_float((uint32_t)u);
    const float ref = __fdiv_rn(1.0f, x);
    const float r0 = __builtin_amdgcn_rcpf(x);
    const float r1 = __builtin_fmaf(__builtin_fmaf(-x, r0, 1.0f), r0, r0);
    if (__float_as_uint(r1) != __float_as_uint(ref)) {
      ++count;
      f = min(f, (uint32_t)u);
    }
  }
  if (count) {
    atomicAdd(bad, count);
    atomicMin(first, f);
  }
}

extern "C" __attribute__((visibility("default"))) int rcp_probe_run(uint32_t lo, uint32_t hi, unsigned long long* bad, uint32_t* first,
                             void* stream) {
  hipLaunchKernelGGL(rcp_check, dim3(8192), dim3(256), 0, (hipStream_t)stream, lo, hi, bad, first);
  return (int)hipGetLastError();
}
