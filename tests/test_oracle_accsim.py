"""The K = 4096 accumulation-precision demonstration, pinned to the pages' figure.

The pages report a maximum relative error of nearly 2% from limited Tensor-Core
accumulation at K = 4096 and none of the setup. The oracle's chunked 14-bit
accumulator model, run on the 4096^3 workload's distributions, must land within
a factor of four of that figure, while per-group FP32 promotion stays at least
1000 times smaller on the same outputs. The accumulator model itself is pinned
separately: with enough bits it is exact, and with truncation it errs toward zero.
"""

import json
import os

import numpy as np
import pytest

from fp8_fine_grained_online_amd import synthetic as S
from oracle import accsim, quant


@pytest.fixture(scope="module")
def sample():
    K = 4096
    a = S.activations(64, K, S.rng_for(1, 0))
    b = S.weights(128, K, S.rng_for(1, 1))
    qa, sa = quant.quant_act_1x128(a)
    qb, sb = quant.quant_weight_128x128(b)
    sb_rows = np.repeat(sb, 128, axis=0)[:64]
    return qa, sa, qb[:64], sb_rows


def test_limited_accumulation_reproduces_pages_figure(sample, golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "pages_facts.json")))["limited_accumulation"]
    qa, sa, qb, sb_rows = sample
    assert qa.shape[1] == facts["K"]
    lim, pg, _ = accsim.demonstration(qa, sa, qb, sb_rows, mant_bits=14, chunk=32, mode="rne")
    target = facts["max_relative_error"]
    assert target / 4 <= lim <= target * 4, lim
    assert pg * 1000 <= lim, (pg, lim)
    assert pg < 1e-4


def test_limited_sum_exact_with_wide_accumulator():
    rng = np.random.default_rng(0)
    # integers below 2^20: exact with 40 bits even after alignment
    t = rng.integers(-2 ** 20, 2 ** 20, (50, 300)).astype(np.float64)
    assert np.array_equal(accsim.limited_sum(t, mant_bits=40, chunk=32), t.sum(axis=1))


def test_limited_sum_truncation_biases_toward_zero():
    t = np.full((1, 4096), 1.0 + 2.0 ** -10)
    exact = t.sum()
    rz = accsim.limited_sum(t, mant_bits=8, chunk=1, mode="rz")[0]
    rne = accsim.limited_sum(t, mant_bits=8, chunk=1, mode="rne")[0]
    assert rz < exact
    assert abs(rne - exact) <= abs(rz - exact)


def test_limited_sum_swamping_closed_form():
    """A running sum of 2^14 and unit terms with 14 bits: the units vanish."""
    t = np.zeros((1, 65))
    t[0, 0] = 2.0 ** 14
    t[0, 1:] = 0.5
    # per-add alignment (chunk 1): 14 bits at 2^14 leave a quantum of 2, so 0.5 is lost
    assert accsim.limited_sum(t, mant_bits=14, chunk=1, mode="rz")[0] == 2.0 ** 14
    assert accsim.limited_sum(t, mant_bits=30, chunk=1)[0] == 2.0 ** 14 + 32
