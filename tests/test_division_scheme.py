"""The kernels' tile scale s = fl32(amax / 448) is computed as q0 = RN(amax c),
q = RN(q0 + RN(amax - 448 q0) c) with c = RN(1/448) whenever amax >= 2^-116
(the IEEE division otherwise). This checks, exhaustively over every binary32
amax in that range, that the sequence equals the correctly rounded quotient.

The reference is (float)((double)amax / 448): amax / 448 = (amax / 7) 2^-6, and
a quotient by 7 that is not exact has a binary expansion of period 3, so its
53-bit rounding never lands on a binary32 midpoint (no double rounding).
Host arithmetic: C's fmaf (correctly rounded), compiled here with gcc."""

import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
  const float c = (float)(1.0 / 448.0);
  unsigned long long bad = 0, n = 0;
  const uint32_t lo = 0x05800000u;  /* 2^-116 */
  #pragma omp parallel for reduction(+:bad,n) schedule(static, 1 << 16)
  for (long long v = lo; v < 0x7F800000LL; ++v) {
    uint32_t u = (uint32_t)v;
    float a; memcpy(&a, &u, 4);
    const float ref = (float)((double)a / 448.0);
    const float q0 = a * c;
    const float q = fmaf(fmaf(-q0, 448.0f, a), c, q0);
    ++n;
    if (memcmp(&q, &ref, 4) != 0) ++bad;
  }
  printf("%llu %llu\n", n, bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_scale_sequence_equals_the_correctly_rounded_quotient():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "s.c"), os.path.join(d, "s")
        open(src, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", src, "-o", exe, "-lm"],
                       check=True)
        n, bad = map(int, subprocess.run([exe], check=True, capture_output=True,
                                         text=True).stdout.split())
    assert n == 0x7F800000 - 0x05800000  # every binary32 from 2^-116 to the largest finite
    assert bad == 0
