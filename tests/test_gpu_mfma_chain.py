"""Does gfx950's FP8 MFMA lose low bits when it accumulates into a nonzero C,
i.e. across chained MFMAs (the limited accumulation the pages report for H800
Tensor Cores)? Measured with the test-only probe tests/probes/mfma_probe.hip,
which runs D = A * B^T + C on one 16 x 16 tile either by chaining the MFMAs
through their accumulator (mode 0) or, like the library, with a zero
accumulator per group and FP32 additions on the vector ALU (mode 1).

Findings pinned here:
* C is added at FP32 precision: with one exact product the result is the
  correctly rounded (nearest-even) C + product, ties and both signs included;
* C takes no part in the block alignment that truncates the products inside
  an instruction (models where C raises a block's exponent miss by orders of
  magnitude);
* chained and FP32-promoted accumulation agree to FP32 rounding over 1 to 16
  groups. Across MFMAs the matrix core accumulates like FP32; the precision
  loss is the truncation inside one instruction (test_gpu_mfma_model.py).
"""

import ctypes
import os

import numpy as np
import pytest

from conftest import ROOT, gpu_available
from helpers import e4m3_exponent, mfma_group_model, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

PROBE = os.path.join(ROOT, "tests", "probes", "libmfma_probe.so")


def probe():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBE)
    L.mfma_probe.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return L


def run(a, b, c, mode):
    import torch
    G = a.shape[1] // 128
    A, B, C = to_dev(a), to_dev(b), to_dev(c.astype(np.float32))
    D = torch.full((16, 16), float("nan"), device="cuda")
    assert probe().mfma_probe(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), G, mode,
                              None) == 0
    torch.cuda.synchronize()
    return D.cpu().numpy().astype(np.float64)


def enc(v):
    import torch
    return torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# (C, [(k, a, b), ...]) for output (0, 0); every product is exact in binary32
CASES = {
    "0.75 ulp above 512 rounds up": (512.0, [(0, 1.5 * 2 ** -6, 2 ** -9)]),
    "0.75 ulp below -512 rounds down": (-512.0, [(0, -1.5 * 2 ** -6, 2 ** -9)]),
    "tie onto an even significand": (512.0, [(0, 2 ** -6, 2 ** -9)]),
    "tie from an odd significand": (512.0 + 2 ** -14, [(0, 2 ** -6, 2 ** -9)]),
    "16 half-ulp products in 16 blocks add up first": (64.0, [(8 * i, 2 ** -9, 2 ** -9) for i in range(16)]),
    "0.75 ulp at 2^24": (2.0 ** 24, [(0, 1.5, 1.0)]),
    "tie at 2^24": (2.0 ** 24, [(0, 1.0, 1.0)]),
    "tie at 2^24 + 2": (2.0 ** 24 + 2, [(0, 1.0, 1.0)]),
    "tiny C below half an ulp of the product": (2.0 ** -30, [(0, 1.0, 1.0)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_accumulator_is_added_with_fp32_round_to_nearest_even(name):
    c00, prods = CASES[name]
    a = np.zeros((16, 128), np.uint8)
    b = np.zeros((16, 128), np.uint8)
    exact = c00
    for k, av, bv in prods:
        a[0, k], b[0, k] = enc([av])[0], enc([bv])[0]
        exact += av * bv
    c = np.zeros((16, 16))
    c[0, 0] = c00
    want = np.float32(exact)  # one rounding of the exact sum (numpy rounds to nearest even)
    assert run(a, b, c, 0)[0, 0] == want
    assert run(a, b, c, 1)[0, 0] == want


def random_operands(G, seed, active_blocks=16):
    rng = np.random.default_rng(seed)
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    a = np.zeros((16, 128 * G), np.uint8)
    b = np.zeros((16, 128 * G), np.uint8)
    for g in range(G):
        cols = slice(128 * g, 128 * g + 8 * active_blocks)
        a[:, cols] = rng.choice(fin, (16, 8 * active_blocks))
        b[:, cols] = rng.choice(fin, (16, 8 * active_blocks))
    e = rng.integers(-12, 32, (16, 16))
    c = np.ldexp(rng.uniform(1, 2, (16, 16)), e) * rng.choice([-1, 1], (16, 16))
    c[::5] = 0
    return a, b, np.float32(c).astype(np.float64)


@pytest.mark.parametrize("active_blocks", [1, 3, 16])
def test_accumulator_takes_no_part_in_block_alignment(active_blocks):
    """One group: D = C + (exactly summed truncated products) to FP32 rounding;
    letting C raise the first block's alignment exponent would be far off."""
    a, b, c = random_operands(1, 7 + active_blocks, active_blocks)
    d = run(a, b, c, 0)
    kept, S = mfma_group_model(a, b)
    scale = 2.0 ** -24 * (S + np.abs(c))
    assert np.all(np.abs(d - (kept + c)) <= 8 * scale)
    # the alternative: C's exponent joins block 0's alignment exponent
    from oracle import e4m3
    ec = np.where(c == 0, -1000, np.frexp(np.abs(c))[1] - 1)
    p = e4m3.decode(a)[:, None, :8] * e4m3.decode(b)[None, :, :8]
    E0 = np.max(e4m3_exponent(a)[:, None, :8] + e4m3_exponent(b)[None, :, :8], axis=2)
    q_alt = np.ldexp(1.0, np.maximum(np.maximum(E0, ec), -500) - 13)
    q_hw = np.ldexp(1.0, np.maximum(E0, -500) - 13)
    alt = kept - (np.trunc(p / q_hw[..., None]) * q_hw[..., None]).sum(2) \
        + (np.trunc(p / q_alt[..., None]) * q_alt[..., None]).sum(2) + c
    assert np.max(np.abs(d - alt) / scale) > 100


@pytest.mark.parametrize("G", [1, 4, 16])
def test_chained_equals_fp32_promotion(G):
    """Chaining G groups through the accumulator matches adding each group's
    MFMA result in FP32, to FP32 rounding of the running sum."""
    a, b, c = random_operands(G, 20 + G)
    d_chain = run(a, b, c, 0)
    d_prom = run(a, b, c, 1)
    S = np.abs(c).copy()
    for g in range(G):
        S += mfma_group_model(a[:, 128 * g:128 * (g + 1)], b[:, 128 * g:128 * (g + 1)])[1]
    assert np.all(np.abs(d_chain - d_prom) <= 4 * G * 2.0 ** -24 * S)
