"""Host-side shape checks of the Python binding (no GPU, no library call):
a mis-shaped operand is rejected before any device pointer is formed."""

import pytest


def _grouped_args(G=4, N=256, K=512, M=512):
    import torch
    a = torch.zeros((M, K), dtype=torch.uint8)
    sa = torch.zeros((M, K // 128), dtype=torch.float32)
    b = torch.zeros((G, N, K), dtype=torch.uint8)
    sb = torch.zeros((G, N // 128, K // 128), dtype=torch.float32)
    off = torch.zeros(G + 1, dtype=torch.int32)
    return a, sa, b, sb, off


def test_grouped_accepts_matching_shapes():
    from fp8_fine_grained_online_amd import _lib
    a, sa, b, sb, off = _grouped_args()
    assert _lib._grouped_shapes(a, sa, b, sb, off, None) == (4, 256, 512, 512)


@pytest.mark.parametrize("sb_shape", [(3, 2, 4), (4, 1, 4), (4, 2, 3), (4, 2, 5), (5, 2, 4)])
def test_grouped_rejects_mis_shaped_block_scales(sb_shape):
    import torch
    from fp8_fine_grained_online_amd import fp8_gemm_grouped
    a, sa, b, _, off = _grouped_args()
    sb = torch.zeros(sb_shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="sb must have shape"):
        fp8_gemm_grouped(a, sa, b, sb, off)


def test_grouped_rejects_other_mismatches():
    import torch
    from fp8_fine_grained_online_amd import fp8_gemm_grouped
    a, sa, b, sb, off = _grouped_args()
    with pytest.raises(ValueError, match="G\\+1"):
        fp8_gemm_grouped(a, sa, b, sb, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="sa must be"):
        fp8_gemm_grouped(a, sa[:, :3].contiguous(), b, sb, off)
    with pytest.raises(ValueError, match="a must be"):
        fp8_gemm_grouped(a[:, :384].contiguous(), sa, b, sb, off)
    with pytest.raises(ValueError, match="3 dims"):
        fp8_gemm_grouped(a, sa, b, sb[0], off)
