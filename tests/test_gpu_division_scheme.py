"""The kernels' per-tile reciprocal RN(1/sp) is one Newton step from the
hardware estimate, r = RN(r0 + RN(1 - sp r0) r0), r0 = v_rcp_f32(sp). Every sp
a kernel forms lies in [2^-85, 2^120) (a positive scale is at least 2^-149,
tiles with amax < 2^-64 are scaled by 2^64, and s <= FLT_MAX/448). This checks
every binary32 in that range against the correctly rounded division on the
GPU itself (tests/probes/rcp_probe.hip)."""

import ctypes
import os
import struct

import pytest

from conftest import ROOT, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def bits(f):
    return struct.unpack("<I", struct.pack("<f", f))[0]


def test_reciprocal_newton_step_is_correctly_rounded_on_the_whole_range():
    import torch
    path = os.path.join(ROOT, "tests", "probes", "librcp_probe.so")
    if not os.path.exists(path):
        pytest.fail("probe not built (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    L.rcp_probe_run.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    lo, hi = bits(2.0 ** -85), bits(2.0 ** 120)
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    assert L.rcp_probe_run(lo, hi, bad.data_ptr(), first.data_ptr(),
                           torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert bad.item() == 0, hex(first.item() & 0xFFFFFFFF)
    # and the range's edges are where the scheme stops holding
    bad.zero_()
    assert L.rcp_probe_run(bits(2.0 ** 127), bits(2.0 ** 127) + 4096, bad.data_ptr(), first.data_ptr(),
                           torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert bad.item() > 0  # a subnormal result: outside the verified range
