"""Pins for the oracle's MoE dispatch (oracle/moe.py).

Independent references: a hand-worked tiny example, numpy's stable argsort as a
second formulation of the row assignment, invariants of the layout (ranges,
order, padding, bijection) and the dense 1x128 quantizer for the row contents.
"""

import numpy as np
import pytest

from fp8_fine_grained_online_amd import synthetic as S
from oracle import moe, quant


def test_hand_worked_example():
    """T = 4 tokens, k = 2, G = 3. Expert 0 gets (t0,j0) (t2,j1) (t3,j0); expert 1
    gets nothing; expert 2 gets (t0,j1) (t1,j0) (t1,j1) (t2,j0); (t3,j1) = 5 is dropped."""
    x = S.activations(4, 256, S.rng_for(995, 0))
    ids = np.array([[0, 2], [2, 2], [2, 0], [0, 5]])
    a, sa, off, row, counts = moe.dispatch_1x128(x, ids, 3)
    assert counts.tolist() == [3, 0, 4]
    assert off.tolist() == [0, 128, 128, 256]
    assert row.tolist() == [[0, 128], [129, 130], [131, 1], [2, -1]]
    q, s = quant.quant_act_1x128(x)
    for (t, j), r in np.ndenumerate(row):
        if r >= 0:
            assert np.array_equal(a[r], q[t]) and np.array_equal(sa[r], s[t])
    pad = np.ones(256, bool)
    pad[[0, 1, 2, 128, 129, 130, 131]] = False
    assert not a[pad].any() and not sa[pad].any()


def routing(T, k, G, seed):
    """Distinct experts per token, uniform (the router's top-k choices)."""
    rng = S.rng_for(seed, 0)
    return np.argsort(rng.random((T, G)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,k,G", [(64, 8, 32), (300, 2, 7), (129, 1, 1), (50, 6, 256)])
def test_rows_equal_stable_argsort_formulation(T, k, G):
    x = S.activations(T, 128, S.rng_for(996, T))
    ids = routing(T, k, G, 997 + T)
    a, sa, off, row, counts = moe.dispatch_1x128(x, ids, G)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # slots grouped by expert, slot order kept
    rank = np.empty_like(order)
    starts = np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=G))])
    for e in range(G):
        sel = order[starts[e]:starts[e + 1]]
        rank[sel] = np.arange(sel.size)
    want = off[flat].astype(np.int64) + rank
    assert np.array_equal(row.reshape(-1), want)


@pytest.mark.parametrize("T,k,G", [(512, 8, 32), (77, 3, 5)])
def test_layout_invariants(T, k, G):
    x = S.activations(T, 256, S.rng_for(998, T))
    ids = routing(T, k, G, 999 + T)
    ids[::13, 0] = -1                                   # some dropped choices
    a, sa, off, row, counts = moe.dispatch_1x128(x, ids, G)
    assert off[0] == 0 and np.all(np.diff(off) % 128 == 0) and np.all(np.diff(off) >= counts)
    assert np.all(np.diff(off) - counts < 128)
    assert a.shape[0] == off[-1] <= moe.max_rows(T, k, G)
    valid = (ids >= 0) & (ids < G)
    assert np.array_equal(row >= 0, valid)
    rows = row[valid]
    assert np.unique(rows).size == rows.size            # one slot per row
    e_of = np.searchsorted(off, rows, side="right") - 1
    assert np.array_equal(e_of, ids[valid])              # each row inside its expert's block
    tok = np.nonzero(valid)[0]
    for e in range(G):
        sel = ids[valid] == e
        r = rows[sel]
        assert np.array_equal(np.sort(r), np.arange(off[e], off[e] + counts[e]))
        assert np.all(np.diff(tok[sel][np.argsort(r)]) >= 0)  # token order within the expert
    q, s = quant.quant_act_1x128(x)
    assert np.array_equal(a[rows], q[tok]) and np.array_equal(sa[rows], s[tok])
    used = np.zeros(a.shape[0], bool)
    used[rows] = True
    assert not a[~used].any() and not sa[~used].any()
