"""GPU parity of the quantization kernels (C ABI through the binding) vs the oracle.

Codes and scales must be bit-exact. Covers the exhaustive (amax significand, x)
table at several amax exponents (including bf16-subnormal amax and tiny tiles
that take the rescaled divide), ragged and edge shapes, all-zero tiles, and
the full-size 16384 x 7168 activation tensor (sampled rows) and weights.
"""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev, to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def gpu_act(bits, nt=False):
    import fp8_fine_grained_online_amd as F
    import torch
    f = F.fp8q_quant_act_1x128_nt if nt else F.fp8q_quant_act_1x128
    q, sa = f(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), sa.cpu().numpy()


def gpu_weight(bits):
    import fp8_fine_grained_online_amd as F
    import torch
    q, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(bits))
    torch.cuda.synchronize()
    return q.cpu().numpy(), sb.cpu().numpy()


def assert_same(got_q, got_s, want_q, want_s):
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), \
        f"{int((got_s.view(np.uint32) != want_s.view(np.uint32)).sum())} scales differ"
    diff = got_q != want_q
    if diff.any():
        i = np.argwhere(diff)[0]
        raise AssertionError(f"{int(diff.sum())} codes differ; first at {tuple(i)}: "
                             f"got {got_q[tuple(i)]:#04x} want {want_q[tuple(i)]:#04x}")


@pytest.mark.parametrize("exp_field", [127, 1, 0, 30, 62, 63, 64, 100, 200, 254])
def test_exhaustive_table(exp_field):
    from oracle import quant
    tiles = S.exhaustive_tiles(exp_field)
    want = quant.quant_act_1x128(tiles)
    assert_same(*gpu_act(tiles), *want)
    assert_same(*gpu_act(tiles, nt=True), *want)  # the non-temporal-store form
    # the same rows through the weight kernel, 128 rows per block
    rows = tiles.shape[0] // 128 * 128
    w = tiles[:rows]
    assert_same(*gpu_weight(w), *quant.quant_weight_128x128(w))


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (257, 1024), (64, 7168), (1000, 256)])
@pytest.mark.parametrize("nt", [False, True])
def test_random_shapes(M, K, nt):
    from oracle import quant
    x = S.activations(M, K, S.rng_for(500 + M, K))
    assert_same(*gpu_act(x, nt), *quant.quant_act_1x128(x))


@pytest.mark.parametrize("N,K", [(128, 128), (384, 256), (256, 7168)])
def test_weight_shapes(N, K):
    from oracle import quant
    w = S.weights(N, K, S.rng_for(600 + N, K))
    assert_same(*gpu_weight(w), *quant.quant_weight_128x128(w))


def test_zero_and_signed_zero_tiles():
    from oracle import quant
    x = S.activations(4, 512, S.rng_for(700, 0))
    x[0, :128] = 0
    x[1, 128:256] = 0x8000
    x[2, 256:384] = np.where(np.arange(128) % 2, 0x8000, 0).astype(np.uint16)
    x[3, 384:] = 1  # a tile of bf16 subnormals
    got = gpu_act(x)
    assert_same(*got, *quant.quant_act_1x128(x))
    assert got[1][0, 0] == 0 and np.all(got[0][1, 128:256] == 0x80)
    w = np.zeros((256, 256), np.uint16)
    w[128:, 128:] = 0x8000
    w[:128, 128:] = S.weights(128, 128, S.rng_for(700, 1))
    assert_same(*gpu_weight(w), *quant.quant_weight_128x128(w))


def test_grouped_weights_3d():
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    w = np.stack([S.weights(256, 384, S.rng_for(710, e)) for e in range(3)])
    q, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(w))
    torch.cuda.synchronize()
    q, sb = q.cpu().numpy(), sb.cpu().numpy()
    for e in range(3):
        assert_same(q[e], sb[e], *quant.quant_weight_128x128(w[e]))


def test_full_size_activation_sampled_rows_and_determinism():
    """16384 x 7168 (the standalone activation-quantization workload)."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    w = S.WORKLOADS["actquant_16384x7168"]
    x, _ = S.dense_inputs(w)
    xd = to_dev_bf16(x)
    q1, s1 = F.fp8q_quant_act_1x128(xd)
    q2, s2 = F.fp8q_quant_act_1x128(xd)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    rows = np.unique(np.concatenate([[0, 1, w.M - 1], S.rng_for(720, 0).integers(0, w.M, 61)]))
    want_q, want_s = quant.quant_act_1x128(x[rows])
    assert_same(q1.cpu().numpy()[rows], s1.cpu().numpy()[rows], want_q, want_s)
    # the non-temporal-store form (the one the standalone workload times): every
    # code and scale equal to the cached form's
    q3, s3 = F.fp8q_quant_act_1x128_nt(xd)
    torch.cuda.synchronize()
    assert torch.equal(q3, q1) and torch.equal(s3.view(torch.int32), s1.view(torch.int32))


def test_full_size_weights_sampled_blocks():
    """7168 x 7168 weights; block rows sampled."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    w = S.weights(7168, 7168, S.rng_for(30, 1))
    q, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(w))
    torch.cuda.synchronize()
    q, sb = q.cpu().numpy(), sb.cpu().numpy()
    for nb in [0, 17, 55]:
        r = slice(nb * 128, (nb + 1) * 128)
        wq, ws = quant.quant_weight_128x128(w[r])
        assert_same(q[r], sb[nb:nb + 1], wq, ws)


def test_codes_beyond_the_cache_bit_exact():
    """Above 256 MiB of codes both quantizers store non-temporally. A 4096-row
    block repeated on the device to 40960 x 7168 activations and to
    32 x 4096 x 7168 weights; sampled rows and blocks bit-exact against the
    oracle on the host block they repeat."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    K = 7168
    x = S.activations(4096, K, S.rng_for(730, 0))
    q, sa = F.fp8q_quant_act_1x128(to_dev_bf16(x).repeat(10, 1))
    torch.cuda.synchronize()
    assert q.shape[0] * K > 256 << 20
    rows = np.array([0, 4095, 4096 + 17, 20000, 40959])
    want_q, want_s = quant.quant_act_1x128(x[rows % 4096])
    idx = torch.as_tensor(rows, device="cuda")
    assert_same(q[idx].cpu().numpy(), sa[idx].cpu().numpy(), want_q, want_s)
    del q, sa
    w = S.weights(4096, K, S.rng_for(730, 1))
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(w).repeat(32, 1))
    torch.cuda.synchronize()
    assert qb.shape[0] * K > 256 << 20
    for nb in [0, 31, 32 + 5, 1023]:
        r = slice(nb * 128, (nb + 1) * 128)
        h = slice((nb % 32) * 128, (nb % 32 + 1) * 128)
        wq, ws = quant.quant_weight_128x128(w[h])
        assert_same(qb[r].cpu().numpy(), sb[nb:nb + 1].cpu().numpy(), wq, ws)
