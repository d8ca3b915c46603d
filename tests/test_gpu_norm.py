"""GPU parity of the fused normalization + 1x128 cast vs the oracle: codes and
scales bit-exact, RMS and centred, every register-tiling variant of the
kernel (K from 128 to 16384), edge rows, and sampled rows at full size."""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def bits(v):
    return S.f32_to_bf16_bits(np.asarray(v, np.float32))


def params(K, seed):
    g = bits(1.0 + 0.1 * S.rng_for(seed, 1).standard_normal(K))
    b = bits(0.05 * S.rng_for(seed, 2).standard_normal(K))
    return g, b


def gpu(x, g, b, eps, centred):
    import fp8_fine_grained_online_amd as F
    import torch
    q, sa = F.fp8q_norm_quant_act_1x128(to_dev_bf16(x), to_dev_bf16(g), eps,
                                        to_dev_bf16(b) if centred else None, centred)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sa.cpu().numpy()


def check(x, g, b, eps, centred):
    from oracle import norm
    q, s = gpu(x, g, b, eps, centred)
    wq, ws = norm.norm_quant_act_1x128(x, g, eps, b, centred)
    ds = s.view(np.uint32) != ws.view(np.uint32)
    assert not ds.any(), f"{int(ds.sum())} scales differ; first {tuple(np.argwhere(ds)[0])}"
    dq = q != wq
    assert not dq.any(), f"{int(dq.sum())} codes differ; first {tuple(np.argwhere(dq)[0])}"


# K = 128 .. 16384 covers every instantiated row size (2, 4, 6, 8, 10, 12, 14,
# 16, 20, 24, 28 and 32 chunks per lane), with partially filled wavefronts
# (K = 128, 384, 2944)
@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (64, 1024), (33, 2048), (6, 2944), (5, 3072),
                                 (4, 4096), (3, 5120), (4, 6144), (64, 7168), (9, 8192),
                                 (3, 10240), (2, 12288), (2, 14336), (7, 16384)])
@pytest.mark.parametrize("centred", [False, True])
def test_shapes(M, K, centred):
    x = S.activations(M, K, S.rng_for(980 + M, K))
    g, b = params(K, 981)
    check(x, g, b, 1e-6, centred)


@pytest.mark.parametrize("centred", [False, True])
def test_edge_rows(centred):
    K = 1024
    rng = S.rng_for(982, 0)
    x = S.activations(8, K, rng)
    x[0] = 0                                                   # zero row (eps > 0)
    x[1] = bits(np.full(K, 3.0))                               # constant row
    x[2] = bits(np.ldexp(rng.standard_normal(K), -120))        # tiny values
    x[3] = bits(np.ldexp(rng.standard_normal(K), 100))         # huge values
    x[4, 5] = bits([2.0 ** 60])[0]                             # one dominant entry
    x[5] = bits(np.where(np.arange(K) % 2, 1.0, -1.0))         # zero mean, unit variance
    x[6, :128] = 0                                             # a zero tile in a normal row
    g, b = params(K, 983)
    g[128:256] = 0                                             # gamma zero: zero output tile
    check(x, g, b, 1e-6, centred)
    # eps = 0 away from the zero and constant rows (zero variance divides by zero there)
    check(x[2:], g, b, 0.0, centred)


@pytest.mark.parametrize("centred", [False, True])
def test_full_size_sampled_rows(centred):
    """8192 x 7168 activations; 48 sampled rows compared (rows are independent)."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import norm
    M, K = 8192, 7168
    x = S.activations(M, K, S.rng_for(984, 0))
    g, b = params(K, 985)
    q, sa = F.fp8q_norm_quant_act_1x128(to_dev_bf16(x), to_dev_bf16(g), 1e-6,
                                        to_dev_bf16(b) if centred else None, centred)
    torch.cuda.synchronize()
    rows = np.sort(S.rng_for(984, 1).choice(M, 48, replace=False))
    wq, ws = norm.norm_quant_act_1x128(x[rows], g, 1e-6, b, centred)
    assert np.array_equal(sa.cpu().numpy()[rows].view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(q.cpu().numpy()[rows], wq)


def eps_defeating_certificate(ms, seed=0, n=1 << 22):
    """A binary32 eps for which r = 1/sqrt(ms + eps) (float64 steps) lies within
    2^-45 r of a binary32 rounding midpoint, so that the kernel's fast,
    certified statistics cannot decide r and its exact (double-double) path
    must run. Found by a seeded search on the CPU."""
    rng = np.random.default_rng(seed)
    eps = rng.uniform(2.0 ** -20, 1.0, n).astype(np.float32)
    r = 1.0 / np.sqrt(np.float64(ms) + eps.astype(np.float64))
    r32 = r.astype(np.float32)
    up = np.nextafter(r32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r32, np.float32(0)).astype(np.float64)
    r32 = r32.astype(np.float64)
    mid = np.where(r >= r32, (r32 + up) / 2, (r32 + dn) / 2)
    d = np.abs(r - mid) / r
    i = int(np.argmin(d))
    assert d[i] < 2.0 ** -45
    return float(eps[i])


@pytest.mark.parametrize("a", [1.0, 3.0, 0.5])
@pytest.mark.parametrize("centred", [False, True])
def test_rows_whose_inverse_std_sits_on_a_rounding_boundary(a, centred):
    """Rows with mean square a^2 (constant rows; for the centred form rows of
    +-a, mean 0, variance a^2) and an eps that puts r within 2^-45 of a binary32
    midpoint: the fast path's certificate fails and the exact path decides."""
    K = 1024
    eps = eps_defeating_certificate(a * a)
    x = np.tile(bits(np.where(np.arange(K) % 2, a, -a) if centred else np.full(K, a)), (8, 1))
    x[1::2] = S.activations(4, K, S.rng_for(986, int(a * 4)))  # ordinary rows beside them
    g, b = params(K, 987)
    check(x, g, b, eps, centred)


def test_centred_rows_spanning_many_binades():
    """Magnitudes spanning more than 31 binades: the plain float64 mean is not
    exact, so the kernel sums the row in double-double."""
    K = 2048
    rng = S.rng_for(988, 0)
    x = S.activations(6, K, rng)
    x[0, 3] = bits([2.0 ** 40])[0]
    x[1, 10] = bits([-(2.0 ** 50)])[0]
    x[2, :] = bits(np.ldexp(rng.standard_normal(K), rng.integers(-60, 60, K)))
    g, b = params(K, 989)
    check(x, g, b, 1e-6, True)
    check(x, g, b, 1e-6, False)
