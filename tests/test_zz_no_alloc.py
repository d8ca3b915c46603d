"""The allocation-free GEMM entry point (fp8_gemm_blockscaled_noalloc, C ABI
through the ctypes binding) against fp8_gemm_blockscaled_ws, the entry point
it is a variant of: same kernels, so the outputs must agree bit for bit.
Two calls in a row on the library's one static scratch, the second smaller;
a third shape that does not split; and no device memory allocated by torch
during the calls (outputs passed in)."""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SHAPES = [(64, 7168, 7168), (16, 1024, 2048), (256, 256, 1024)]


def operands(M, N, K, seed):
    import fp8_fine_grained_online_amd as F
    a = S.activations(M, K, S.rng_for(1200 + seed, 0))
    b = S.weights(N, K, S.rng_for(1200 + seed, 1))
    qa, sa = F.fp8q_quant_act_1x128(to_dev_bf16(a))
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(b))
    return qa, sa, qb, sb


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(out):
    import fp8_fine_grained_online_amd as F
    import torch
    L = F.lib()
    assert L.fp8_gemm_blockscaled_ws_bytes(*SHAPES[0]) > 0   # split path, large partials
    assert L.fp8_gemm_blockscaled_ws_bytes(*SHAPES[1]) > 0   # split path, smaller partials
    assert L.fp8_gemm_blockscaled_ws_bytes(*SHAPES[2]) == 0  # one launch, no scratch
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    for i, (M, N, K) in enumerate(SHAPES):
        qa, sa, qb, sb = operands(M, N, K, i)
        want = F.fp8_gemm_blockscaled_ws(qa, sa, qb, sb, out)
        c = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        F.fp8_gemm_blockscaled_noalloc(qa, sa, qb, sb, out, c=c)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(c.view(torch.int16 if out == "bf16" else torch.int32),
                           want.view(torch.int16 if out == "bf16" else torch.int32)), (M, N, K)


def test_noalloc_against_the_oracle_small_case():
    """The split path at 64 x 1024 x 2048 within the GEMM parity rule."""
    import fp8_fine_grained_online_amd as F
    from oracle import quant
    from helpers import check_gemm, from_dev_bf16_bits, reference
    M, N, K = 64, 1024, 2048
    a = S.activations(M, K, S.rng_for(1210, 0))
    b = S.weights(N, K, S.rng_for(1210, 1))
    qa, sa = F.fp8q_quant_act_1x128(to_dev_bf16(a))
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(b))
    c = F.fp8_gemm_blockscaled_noalloc(qa, sa, qb, sb, "bf16")
    oqa, osa = quant.quant_act_1x128(a)
    oqb, osb = quant.quant_weight_128x128(b)
    check_gemm(from_dev_bf16_bits(c), reference(oqa, osa, oqb, osb), "bf16")
