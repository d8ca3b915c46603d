"""GPU parity of the backward-pass pieces vs the oracle.

* 128x1 quantization (bf16 -> transposed codes): bit-exact, including the
  exhaustive (amax significand, x) table laid out as 128x1 tiles;
* re-tiling of stored 1x128 FP8 activations into 128x1 tiles: bit-exact, on
  quantized activations and on random codes with scales over the whole
  binary32 range (products that are binary32 subnormals included);
* the 128x128 weight transpose: bit-exact for every byte value;
* the row-scaled (Wgrad) GEMM: element by element on small and ragged shapes
  (both kernels), on sampled rows at a full layer size;
* Dgrad and Wgrad composed from the calls above, against the oracle's
  composition of the same steps.
"""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_gemm, from_dev_bf16_bits, reference, to_dev, to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_same(got_q, got_s, want_q, want_s):
    assert got_q.shape == want_q.shape and got_s.shape == want_s.shape
    ds = got_s.view(np.uint32) != np.asarray(want_s, np.float32).view(np.uint32)
    assert not ds.any(), f"{int(ds.sum())} scales differ; first at {tuple(np.argwhere(ds)[0])}"
    dq = got_q != want_q
    if dq.any():
        i = tuple(np.argwhere(dq)[0])
        raise AssertionError(f"{int(dq.sum())} codes differ; first at {i}: "
                             f"got {got_q[i]:#04x} want {want_q[i]:#04x}")


def gpu_128x1(x_bits):
    import fp8_fine_grained_online_amd as F
    qt, st = F.fp8q_quant_act_128x1(to_dev_bf16(x_bits))
    return host(qt), host(st)


def gpu_requant(codes, scales):
    import fp8_fine_grained_online_amd as F
    qt, st = F.fp8q_requant_1x128_to_128x1(to_dev(codes), to_dev(scales))
    return host(qt), host(st)


# ---------------------------------------------------------------- 128x1 quant

@pytest.mark.parametrize("exp_field", [127, 0, 1, 63, 64, 200, 254])
def test_128x1_exhaustive_table(exp_field):
    """Every tile of the exhaustive table becomes one column of X (M = 128)."""
    from oracle import quant
    tiles = S.exhaustive_tiles(exp_field)
    pad = (-tiles.shape[0]) % 128
    tiles = np.concatenate([tiles, np.zeros((pad, 128), np.uint16)])
    x = np.ascontiguousarray(tiles.T)  # 128 x T
    got = gpu_128x1(x)
    assert_same(*got, *quant.quant_act_128x1(x))
    assert_same(*got, *quant.quant_act_1x128(tiles))


@pytest.mark.parametrize("M,K", [(128, 128), (256, 384), (384, 1024), (1024, 7168)])
def test_128x1_random_shapes(M, K):
    from oracle import quant
    x = S.activations(M, K, S.rng_for(940 + M, K))
    assert_same(*gpu_128x1(x), *quant.quant_act_128x1(x))


def test_128x1_zero_and_signed_zero_tiles():
    from oracle import quant
    x = S.activations(256, 256, S.rng_for(941, 0))
    x[:128, 3] = 0            # +0 tile
    x[128:, 5] = 0x8000       # -0 tile
    x[:128, 7] = np.where(np.arange(128) % 2, 0x8000, 0).astype(np.uint16)  # mixed zeros
    qt, st = gpu_128x1(x)
    assert_same(qt, st, *quant.quant_act_128x1(x))
    assert st[3, 0] == 0 and st[5, 1] == 0 and np.all(qt[3, :128] == 0) and np.all(qt[5, 128:] == 0x80)


def test_128x1_full_size_sampled_columns():
    """dY (8192 tokens x 7168 channels): every 128x1 tile of 96 sampled columns."""
    from oracle import quant
    x = S.activations(8192, 7168, S.rng_for(942, 1))
    qt, st = gpu_128x1(x)
    cols = np.sort(S.rng_for(942, 0).choice(x.shape[1], 96, replace=False))
    want_q, want_s = quant.quant_act_1x128(np.ascontiguousarray(x[:, cols].T))
    assert_same(qt[cols], st[cols], want_q, want_s)


@pytest.mark.parametrize("M,K", [(128, 128), (256, 384), (1024, 7168)])
def test_dual_quant_matches_both_tilings(M, K):
    """One read, both outputs: bit-exact against the 1x128 and 128x1 oracles."""
    import fp8_fine_grained_online_amd as F
    from oracle import quant
    x = S.activations(M, K, S.rng_for(948 + M, K))
    x[:128, :128] = 0  # a zero 128x128 corner: zero tiles in both tilings
    q, sa, qt, st = F.fp8q_quant_act_1x128_128x1(to_dev_bf16(x))
    assert_same(host(q), host(sa), *quant.quant_act_1x128(x))
    assert_same(host(qt), host(st), *quant.quant_act_128x1(x))


def test_dual_quant_exhaustive_rows_and_columns():
    """The exhaustive table's tiles as rows (1x128) of one 128-row slab and as
    columns (128x1) of the transposed layout, through the fused kernel."""
    import fp8_fine_grained_online_amd as F
    from oracle import quant
    tiles = S.exhaustive_tiles(127)
    tiles = tiles[: tiles.shape[0] // 128 * 128]
    x = np.ascontiguousarray(tiles.reshape(-1, 128, 128).transpose(1, 0, 2).reshape(128, -1))
    q, sa, qt, st = F.fp8q_quant_act_1x128_128x1(to_dev_bf16(x))
    assert_same(host(q), host(sa), *quant.quant_act_1x128(x))
    assert_same(host(qt), host(st), *quant.quant_act_128x1(x))
    xt = np.ascontiguousarray(tiles.T)  # 128 x T: every tile a column
    q, sa, qt, st = F.fp8q_quant_act_1x128_128x1(to_dev_bf16(xt))
    assert_same(host(qt), host(st), *quant.quant_act_1x128(tiles))
    assert_same(host(q), host(sa), *quant.quant_act_1x128(xt))


# ------------------------------------------------------------------- requant

@pytest.mark.parametrize("M,K", [(128, 128), (256, 384), (512, 2048)])
def test_requant_of_quantized_activations(M, K):
    from oracle import quant
    x = S.activations(M, K, S.rng_for(943 + M, K))
    q, s = quant.quant_act_1x128(x)
    assert_same(*gpu_requant(q, s), *quant.requant_1x128_to_128x1(q, s))


def test_requant_random_codes_all_scale_ranges():
    """Random finite codes; per-tile scales from 2^-149 to just below 2^119
    (products that are binary32 subnormals, normal and large; 448 * scale stays
    finite, as it does for every scale the quantizer produces), and zero scales."""
    from oracle import e4m3, quant
    rng = S.rng_for(944, 0)
    M, K = 1024, 512
    codes = rng.choice(e4m3.finite_codes(), (M, K)).astype(np.uint8)
    exps = rng.integers(-149, 119, (M, K // 128))
    scales = np.ldexp(rng.uniform(1, 2, (M, K // 128)), exps).astype(np.float32)
    scales[::17, 1] = 0
    codes[::17, 128:256] = np.where(rng.random((len(range(0, M, 17)), 128)) < 0.5, 0, 0x80)
    assert_same(*gpu_requant(codes, scales), *quant.requant_1x128_to_128x1(codes, scales))


def test_requant_full_size_sampled():
    """X (8192 tokens x 7168 channels) stored as 1x128 FP8, re-tiled; three whole
    128-channel groups of the output compared (a column group of the input is
    re-tiled independently of the others)."""
    from oracle import quant
    x = S.activations(8192, 7168, S.rng_for(945, 0))
    q, s = quant.quant_act_1x128(x)
    qt, st = gpu_requant(q, s)
    for g in [0, 29, 55]:
        cols = slice(128 * g, 128 * (g + 1))
        want_q, want_s = quant.requant_1x128_to_128x1(np.ascontiguousarray(q[:, cols]),
                                                      np.ascontiguousarray(s[:, g:g + 1]))
        assert_same(qt[cols], st[cols], want_q, want_s)


# ------------------------------------------------------------ weight transpose

@pytest.mark.parametrize("N,K", [(128, 128), (384, 256), (2048, 7168)])
def test_transpose_every_byte(N, K):
    import fp8_fine_grained_online_amd as F
    from oracle import quant
    rng = S.rng_for(946, N)
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)  # every byte value, NaN codes too
    sb = rng.standard_normal((N // 128, K // 128)).astype(np.float32)
    qt, sbt = F.fp8q_transpose_weight_128x128(to_dev(q), to_dev(sb))
    want_q, want_s = quant.transpose_weight_128x128(q, sb)
    assert np.array_equal(host(qt), want_q)
    assert np.array_equal(host(sbt).view(np.uint32), want_s.view(np.uint32))


# ------------------------------------------------------------ row-scaled GEMM

def poisoned(shape, dtype):
    import torch
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def rowscaled_operands(M, N, K, seed):
    """A (M x K) and B (N x K) codes with 1x128 scales, made by the oracle's
    128x1 quantizer from seeded gradient-like (M tokens = K here) tensors."""
    from oracle import quant
    dy = S.activations(K, M, S.rng_for(seed, 0))   # tokens x out-channels
    x = S.activations(K, N, S.rng_for(seed, 1))    # tokens x in-channels
    qa, sa = quant.quant_act_128x1(dy)
    qb, sb = quant.quant_act_128x1(x)
    return qa, sa, qb, sb


def gpu_rowscaled(qa, sa, qb, sb, out, rows=None):
    import fp8_fine_grained_online_amd as F
    import torch
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = poisoned((qa.shape[0], qb.shape[0]), dt)
    F.fp8_gemm_rowscaled(to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb), out, c=c)
    torch.cuda.synchronize()
    if rows is not None:
        c = c[torch.as_tensor(rows, device="cuda")]
    return from_dev_bf16_bits(c) if out == "bf16" else c.cpu().numpy()


def check_rowscaled(got, qa, sa, qb, sb, out):
    return check_gemm(got, reference(qa, sa, qb, sb, row_scales=True), out)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (100, 256, 384), (300, 384, 256),
                                   (1, 128, 1024), (640, 512, 2048)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_rowscaled_small_and_ragged(M, N, K, out):
    qa, sa, qb, sb = rowscaled_operands(M, N, K, 950 + M)
    check_rowscaled(gpu_rowscaled(qa, sa, qb, sb, out), qa, sa, qb, sb, out)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M", [2000, 1900])
def test_rowscaled_big_tile_path_ragged_m(M, out):
    """Enough tiles for the large-tile kernel, M ragged against 256; sampled
    rows including the last tile's. With M = 1900 the last row tile has 108
    rows, so the waves of its upper 128 rows only copy (no MFMAs)."""
    N, K = 4224, 512
    qa, sa, qb, sb = rowscaled_operands(M, N, K, 951)
    rows = np.concatenate([np.arange(0, 16), np.arange(1000, 1008), np.arange(1780, 1800),
                           np.arange(M - 16, M)])
    got = gpu_rowscaled(qa, sa, qb, sb, out, rows)
    check_rowscaled(got, qa[rows], sa[rows], qb, sb, out)


def test_rowscaled_one_hot_indexing():
    """One nonzero code in A at (m0, k0), one in B at (n0, k0): C has a single
    nonzero, dec * dec * sa[m0, g] * sb[n0, g], at (m0, n0)."""
    M, N, K = 256, 512, 512
    rng = np.random.default_rng(7)
    for m0, n0, k0 in [(0, 0, 0), (255, 511, 511), (17, 300, 129), (128, 127, 383)]:
        qa = np.zeros((M, K), np.uint8)
        qb = np.zeros((N, K), np.uint8)
        qa[m0, k0] = 0x40   # 2.0
        qb[n0, k0] = 0xB0   # -0.5
        sa = np.ldexp(1.0, rng.integers(-8, 8, (M, K // 128))).astype(np.float32)
        sb = np.ldexp(1.0, rng.integers(-8, 8, (N, K // 128))).astype(np.float32)
        c = gpu_rowscaled(qa, sa, qb, sb, "f32")
        want = np.zeros((M, N), np.float32)
        want[m0, n0] = 2.0 * -0.5 * sa[m0, k0 // 128] * sb[n0, k0 // 128]
        assert np.array_equal(c, want), (m0, n0, k0)


def test_rowscaled_k_zero_writes_zeros():
    import fp8_fine_grained_online_amd as F
    import torch
    c = poisoned((64, 256), torch.float32)
    L = F.lib()
    st = L.fp8_gemm_rowscaled(None, None, None, None, c.data_ptr(), F.FP8Q_OUT_F32, 64, 256, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert np.all(host(c) == 0)


# ------------------------------------------------------- Dgrad / Wgrad composed

def test_dgrad_composed():
    """dX = dY W: dY 1x128-quantized, W 128x128-quantized then transposed."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import gemm, quant
    M, N, K = 384, 256, 640       # tokens, out-channels, in-channels
    dy = S.activations(M, N, S.rng_for(960, 0))
    w = S.weights(N, K, S.rng_for(960, 1))
    qd, sd = F.fp8q_quant_act_1x128(to_dev_bf16(dy))
    qw, sw = F.fp8q_quant_weight_128x128(to_dev_bf16(w))
    qwt, swt = F.fp8q_transpose_weight_128x128(qw, sw)
    dx = poisoned((M, K), torch.float32)
    F.fp8_gemm_blockscaled(qd, sd, qwt, swt, "f32", c=dx)
    oqd, osd = quant.quant_act_1x128(dy)
    oqwt, oswt = quant.transpose_weight_128x128(*quant.quant_weight_128x128(w))
    check_gemm(host(dx), reference(oqd, osd, oqwt, oswt), "f32")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wgrad_composed(out):
    """dW = dY^T X: dY quantized 128x1 from bf16, X stored as 1x128 FP8 and re-tiled."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    M, N, K = 512, 384, 256       # tokens, out-channels, in-channels
    dy = S.activations(M, N, S.rng_for(961, 0))
    x = S.activations(M, K, S.rng_for(961, 1))
    qdt, sdt = F.fp8q_quant_act_128x1(to_dev_bf16(dy))
    qx, sx = F.fp8q_quant_act_1x128(to_dev_bf16(x))
    qxt, sxt = F.fp8q_requant_1x128_to_128x1(qx, sx)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    dw = poisoned((N, K), dt)
    F.fp8_gemm_rowscaled(qdt, sdt, qxt, sxt, out, c=dw)
    torch.cuda.synchronize()
    got = from_dev_bf16_bits(dw) if out == "bf16" else host(dw)
    oa, osa = quant.quant_act_128x1(dy)
    ob, osb = quant.requant_1x128_to_128x1(*quant.quant_act_1x128(x))
    check_rowscaled(got, oa, osa, ob, osb, out)


def test_wgrad_full_size_sampled():
    """Wgrad of the 8192-token x 7168 -> 2048 projection: dW (7168 x 2048)
    with K = 8192 tokens, in the launch configuration the bench times; 12
    sampled rows compared in full."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import quant
    T, N, K = 8192, 7168, 2048
    dy = S.activations(T, N, S.rng_for(962, 0))
    x = S.activations(T, K, S.rng_for(962, 1))
    _, _, qdt, sdt = F.fp8q_quant_act_1x128_128x1(to_dev_bf16(dy))
    qx, sx = F.fp8q_quant_act_1x128(to_dev_bf16(x))
    qxt, sxt = F.fp8q_requant_1x128_to_128x1(qx, sx)
    dw = poisoned((N, K), torch.float32)
    F.fp8_gemm_rowscaled(qdt, sdt, qxt, sxt, "f32", c=dw)
    rows = np.array([0, 1, 255, 256, 3000, 4097, 5555, 7000, 7166, 7167, 128, 6143])
    got = host(dw)[rows]
    oa, osa = quant.quant_act_1x128(np.ascontiguousarray(dy[:, rows].T))
    ob, osb = quant.requant_1x128_to_128x1(*quant.quant_act_1x128(x))
    check_rowscaled(got, oa, osa, ob, osb, "f32")
