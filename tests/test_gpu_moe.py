"""GPU parity of the FP8 MoE dispatch vs the oracle: offsets, the slot -> row map,
codes and scales bit-exact; rows past m_offsets[G] untouched; dispatch feeding
the grouped GEMM without a host synchronization."""

import numpy as np
import pytest

from conftest import gpu_available
from helpers import check_gemm, from_dev_bf16_bits, grouped_reference, to_dev, to_dev_bf16
from fp8_fine_grained_online_amd import synthetic as S

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

POISON = 0xAB


def routing(T, k, G, seed, drop_every=0):
    """Distinct experts per token, uniform; optionally some invalid choices."""
    rng = S.rng_for(seed, 0)
    ids = np.argsort(rng.random((T, G)), axis=1)[:, :k].astype(np.int32)
    if drop_every:
        ids[::drop_every, 0] = -1
        ids[1::drop_every, k - 1] = G + 3
    return ids


def poisoned_outputs(T, k, G, K):
    """Dispatch outputs pre-filled with a marker, so unwritten rows can be seen."""
    import fp8_fine_grained_online_amd as F
    import torch
    cap = F.lib().fp8q_moe_dispatch_max_rows(T, k, G)
    q = torch.full((cap, K), POISON, dtype=torch.uint8, device="cuda")
    sa = torch.full((cap, K // 128), float("nan"), dtype=torch.float32, device="cuda")
    return q, sa


def check_against_oracle(x, ids, G):
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import moe
    q, sa = poisoned_outputs(x.shape[0], ids.shape[1], G, x.shape[1])
    q, sa, off, rows = F.fp8q_moe_dispatch_1x128(to_dev_bf16(x), to_dev(ids), G, q=q, sa=sa)
    torch.cuda.synchronize()
    a_o, sa_o, off_o, rows_o, _ = moe.dispatch_1x128(x, ids, G)
    assert np.array_equal(off.cpu().numpy(), off_o)
    assert np.array_equal(rows.cpu().numpy(), rows_o)
    M = int(off_o[-1])
    qh, sah = q.cpu().numpy(), sa.cpu().numpy()
    assert np.array_equal(qh[:M], a_o)
    assert np.array_equal(sah[:M].view(np.uint32), sa_o.view(np.uint32))
    assert np.all(qh[M:] == POISON) and np.all(np.isnan(sah[M:]))  # not written


# K up to 8192 keeps a token's codes in registers and writes each destination
# row in one pass (8192: 8 steps, the limit); larger K stores step by step
# Rows 10-12 give the offsets scan several 256-slot blocks per thread
# with ragged runs (305 and 625 blocks over 64 threads per expert) and, at
# G = 600, ten experts per lane in the prefix over the experts' totals. The
# last two give a token more choices than a wavefront has lanes: 70 (the
# choices past 64 looked up one by one, their rows written in one batch of
# 4 x 64 lanes) and 300 (two batches; a token's slots span two 256-slot
# blocks).
@pytest.mark.parametrize("T,k,G,K", [(64, 8, 32, 256), (300, 2, 7, 384), (129, 1, 1, 128),
                                     (50, 6, 256, 128), (1000, 8, 32, 1024), (257, 3, 1024, 128),
                                     (40, 4, 16, 8192), (33, 3, 8, 9216), (20, 2, 4, 16384),
                                     (26000, 3, 3, 128), (40000, 4, 6, 128), (3000, 8, 600, 128),
                                     (9, 70, 128, 256), (6, 300, 1024, 128)])
def test_small(T, k, G, K):
    x = S.activations(T, K, S.rng_for(1000 + T, K))
    check_against_oracle(x, routing(T, k, G, 1001 + T, drop_every=7), G)


def test_repeated_expert_choices_and_zero_tokens():
    """A token may list an expert twice (two rows); a zero token gives zero tiles."""
    x = S.activations(40, 256, S.rng_for(1002, 0))
    x[3] = 0
    ids = np.tile(np.array([[1, 1, 0]], np.int32), (40, 1))
    check_against_oracle(x, ids, 2)


def test_row_map_without_codes():
    """K == 0: only the offsets and the slot -> row map are produced."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import moe
    T, k, G = 1000, 8, 32
    ids = routing(T, k, G, 1005, drop_every=5)
    x = torch.empty((T, 0), dtype=torch.bfloat16, device="cuda")
    _, _, off, rows = F.fp8q_moe_dispatch_1x128(x, to_dev(ids), G)
    torch.cuda.synchronize()
    # the oracle's row assignment on zero tokens of one tile (rows do not depend on K)
    _, _, off_o, rows_o, _ = moe.dispatch_1x128(np.zeros((T, 128), np.uint16), ids, G)
    assert np.array_equal(off.cpu().numpy(), off_o)
    assert np.array_equal(rows.cpu().numpy(), rows_o)


def test_no_tokens_writes_zero_offsets():
    import fp8_fine_grained_online_amd as F
    import torch
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    off = torch.full((9,), -7, dtype=torch.int32, device="cuda")
    F.fp8q_moe_dispatch_1x128(x, ids, 8, m_offsets=off)
    torch.cuda.synchronize()
    assert np.all(off.cpu().numpy() == 0)


def test_full_size_8192_tokens_top8_of_32():
    """The grouped workload's token layout: 8192 tokens x top-8 of 32 experts =
    65536 rows, K = 7168. Offsets and the row map compared in full, codes and
    scales on sampled rows of every expert."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import moe, quant
    T, k, G, K = 8192, 8, 32, 7168
    x = S.activations(T, K, S.rng_for(1003, 0))
    ids = routing(T, k, G, 1004)
    q, sa, off, rows = F.fp8q_moe_dispatch_1x128(to_dev_bf16(x), to_dev(ids), G)
    torch.cuda.synchronize()
    # the oracle's row assignment, on a 128-column slice (rows do not depend on K)
    _, _, off_o, rows_o, counts = moe.dispatch_1x128(np.ascontiguousarray(x[:, :128]), ids, G)
    assert np.array_equal(off.cpu().numpy(), off_o)
    assert np.array_equal(rows.cpu().numpy(), rows_o)
    tok = np.repeat(np.arange(T), k).reshape(T, k)
    rng = S.rng_for(1003, 1)
    pick = rng.choice(T * k, 256, replace=False)
    r = rows_o.reshape(-1)[pick]
    t = tok.reshape(-1)[pick]
    q_o, s_o = quant.quant_act_1x128(x[t])
    qh = q.cpu().numpy()
    sah = sa.cpu().numpy()
    assert np.array_equal(qh[r], q_o) and np.array_equal(sah[r].view(np.uint32), s_o.view(np.uint32))
    for e in range(G):  # padding rows zero
        pad = slice(int(off_o[e] + counts[e]), int(off_o[e + 1]))
        assert not qh[pad].any() and not sah[pad].any()


def test_dispatch_feeds_grouped_gemm_without_host_sync():
    """Dispatch, then the grouped GEMM with M_total = the dispatch capacity: rows
    past m_offsets[G] of C stay untouched; the rest matches the oracle's
    dispatch + grouped GEMM."""
    import fp8_fine_grained_online_amd as F
    import torch
    from oracle import bf16, gemm, moe, quant
    T, k, G, K, N = 256, 4, 8, 512, 256
    x = S.activations(T, K, S.rng_for(1005, 0))
    ids = routing(T, k, G, 1006)
    w = np.stack([S.weights(N, K, S.rng_for(1005, 1 + e)) for e in range(G)])
    q, sa, off, rows = F.fp8q_moe_dispatch_1x128(to_dev_bf16(x), to_dev(ids), G)
    qb, sb = F.fp8q_quant_weight_128x128(to_dev_bf16(w))
    cap = q.shape[0]
    c = torch.full((cap, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    F.fp8_gemm_grouped(q, sa, qb, sb, off, "bf16", c=c, M_total=cap)
    torch.cuda.synchronize()
    a_o, sa_o, off_o, _, _ = moe.dispatch_1x128(x, ids, G)
    qw, sw = zip(*[quant.quant_weight_128x128(w[e]) for e in range(G)])
    qw, sw = np.stack(qw), np.stack(sw)
    M = int(off_o[-1])
    got = from_dev_bf16_bits(c)
    check_gemm(got[:M], grouped_reference(a_o[:M], sa_o[:M], qw, sw, off_o), "bf16")
    assert np.all(np.isnan(c[M:].float().cpu().numpy()))
