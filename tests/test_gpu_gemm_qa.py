"""GPU parity of the quantize-on-load GEMM (fp8_gemm_blockscaled_bf16a) vs the
oracle: C against the oracle's 1x128 quantization of A, 128x128 quantization
of B and float64 per-group GEMM (within the GEMM tolerance); the optional
codes and scales of A bit-exact; and, on the large-tile path, C bit-identical
to fp8q_quant_act_1x128 + fp8_gemm_blockscaled (same per-element arithmetic
in the same group order)."""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import from_dev_bf16_bits, to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S
from test_gpu_gemm import check, oracle_rows, poisoned

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def fused(a_bits, b_bits, out, rows=None, with_codes=True):
    """GPU: quantize B, then the fused GEMM. Returns (C, qa, sa) on the host."""
    import fp8_fine_grained_online_amd as F
    import torch
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(b_bits))
    M, N = a_bits.shape[0], b_bits.shape[0]
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = poisoned((M, N), dt)
    qa = torch.full(a_bits.shape, 0xAB, dtype=torch.uint8, device="cuda")
    sa = torch.full((M, a_bits.shape[1] // 128), float("nan"), device="cuda")
    if with_codes:
        F.fp8_gemm_blockscaled_bf16a(to_dev_bf16(a_bits), qb, sb, out, c=c, qa=qa, sa=sa)
    else:
        F.fp8_gemm_blockscaled_bf16a(to_dev_bf16(a_bits), qb, sb, out, c=c)
    torch.cuda.synchronize()
    if rows is not None:
        idx = torch.as_tensor(rows, device="cuda")
        c, qa, sa = c[idx], qa[idx], sa[idx]
    got = from_dev_bf16_bits(c) if out == "bf16" else c.cpu().numpy()
    return got, qa.cpu().numpy(), sa.cpu().numpy()


def check_codes(a_bits, qa, sa):
    from oracle import quant
    q_o, s_o = quant.quant_act_1x128(a_bits)
    assert np.array_equal(qa, q_o)
    assert np.array_equal(sa.view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (100, 256, 384), (300, 384, 256),
                                   (129, 128, 1024), (640, 512, 2048), (77, 1024, 7168),
                                   (256, 256, 1024)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_small_and_ragged_shapes(M, N, K, out):
    a = S.activations(M, K, S.rng_for(880 + M, N))
    b = S.weights(N, K, S.rng_for(880 + M, N + 1))
    got, qa, sa = fused(a, b, out)
    check(got, oracle_rows(a, b), out)
    check_codes(a, qa, sa)


def test_without_code_outputs():
    a = S.activations(200, 512, S.rng_for(881, 0))
    b = S.weights(384, 512, S.rng_for(881, 1))
    got, qa, sa = fused(a, b, "f32", with_codes=False)
    check(got, oracle_rows(a, b), "f32")
    assert np.all(qa == 0xAB) and np.all(np.isnan(sa))  # nothing written


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_bit_identical_to_the_unfused_large_tile_path(out):
    """M = 1900 (a ragged last row tile), N = 4224 (a half column tile)."""
    import fp8_fine_grained_online_amd as F
    import torch
    M, N, K = 1900, 4224, 512
    a = S.activations(M, K, S.rng_for(882, 0))
    b = S.weights(N, K, S.rng_for(882, 1))
    got, qa, sa = fused(a, b, out)
    qa2, sa2 = F.fp8q_quant_act_1x128(to_dev_bf16(a))
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(b))
    c = F.fp8_gemm_blockscaled(qa2, sa2, qb, sb, out)
    torch.cuda.synchronize()
    want = from_dev_bf16_bits(c) if out == "bf16" else c.cpu().numpy()
    assert np.array_equal(got.view(np.uint16 if out == "bf16" else np.uint32),
                          want.view(np.uint16 if out == "bf16" else np.uint32))
    assert np.array_equal(qa, qa2.cpu().numpy())
    assert np.array_equal(sa.view(np.uint32), sa2.cpu().numpy().view(np.uint32))


def test_full_size_4096_sampled_rows():
    """The dense 4096^3 workload through the fused path; 24 sampled rows of C
    against the oracle, their codes and scales bit-exact."""
    w = S.WORKLOADS["dense_4096x4096x4096"]
    a, b = S.dense_inputs(w)
    rows = np.unique(np.concatenate([[0, 127, 128, 4095], S.rng_for(883, 0).integers(0, w.M, 20)]))
    got, qa, sa = fused(a, b, "bf16", rows=rows)
    check(got, oracle_rows(a, b, rows), "bf16")
    check_codes(a[rows], qa, sa)


def test_k_zero_writes_zeros_and_m_zero_is_a_no_op():
    import fp8_fine_grained_online_amd as F
    import torch
    L = F.lib()
    c = poisoned((64, 256), torch.float32)
    assert L.fp8_gemm_blockscaled_bf16a(None, None, None, c.data_ptr(), F.FP8Q_OUT_F32, 64, 256, 0,
                                        None, None, None) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0
    c = poisoned((1, 256), torch.float32)
    assert L.fp8_gemm_blockscaled_bf16a(None, None, None, c.data_ptr(), F.FP8Q_OUT_F32, 0, 256, 128,
                                        None, None, None) == 0
    torch.cuda.synchronize()
    assert torch.isnan(c).all()
