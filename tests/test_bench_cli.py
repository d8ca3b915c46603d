"""bench.py's contract on the CPU: it refuses more than one GPU with a message,
rejects unknown workloads, and its CPU-baseline legs (the oracle on a bounded
sample) produce the fields the JSON line carries."""

import os
import subprocess
import sys

import numpy as np

from conftest import ROOT

sys.path.insert(0, ROOT)


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_unknown_workload_is_rejected():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode == 2 and "unknown" in r.stderr


def check_baseline(d):
    assert d["kind"] == "oracle" and d["unit"] == "TFLOP/s"
    assert d["value"] > 0 and d["cores"] >= 1 and d["sample"]


def test_cpu_baseline_legs_on_tiny_inputs():
    import bench
    from fp8_fine_grained_online_amd import synthetic as S
    a = S.activations(256, 256, S.rng_for(990, 0))
    b = S.weights(128, 256, S.rng_for(990, 1))
    check_baseline(bench.cpu_baseline("tiny", a, b, 128))
    dy = S.activations(256, 128, S.rng_for(990, 2))
    check_baseline(bench.cpu_baseline_backward("tiny", a, b, dy, 64))
    d = bench.cpu_baseline_weights("tiny", b, 256 * 3.0, 128)
    assert d["unit"] == "GB/s" and d["kind"] == "oracle" and d["value"] > 0
    g, _ = S.norm_params(256, S.rng_for(990, 3))
    for gamma in (None, g):
        d = bench.cpu_baseline_stream("tiny", a, 256 * 3.03, 64, gamma)
        assert d["unit"] == "GB/s" and d["kind"] == "oracle" and d["value"] > 0


def test_dispatch_inputs_and_baseline():
    import bench
    from fp8_fine_grained_online_amd import synthetic as S
    w = S.Workload(33, "small", 64, 0, 256, G=8, topk=3)
    x, ids, b = S.dispatch_inputs(w)
    assert x.shape == (64, 256) and ids.shape == (64, 3) and b is None
    assert all(len(set(r)) == 3 for r in ids.tolist()) and ids.min() >= 0 and ids.max() < 8
    d = bench.cpu_baseline_dispatch("small", x, ids, 8, 32)
    assert d["unit"] == "GB/s" and d["kind"] == "oracle" and d["value"] > 0


def test_backward_workload_inputs_have_the_layer_shapes():
    from fp8_fine_grained_online_amd import synthetic as S
    w = S.WORKLOADS["bwd_proj_8192x7168x2048"]
    assert w.backward and (w.M, w.N, w.K) == (8192, 7168, 2048)
    small = S.Workload(w.wid, "small", 256, 128, 384, backward=True)
    x, wt, dy = S.backward_inputs(small)
    assert x.shape == (256, 384) and wt.shape == (128, 384) and dy.shape == (256, 128)
    assert x.dtype == wt.dtype == dy.dtype == np.uint16


def test_counter_records_are_keyed_by_source(tmp_path):
    """Recorded MFMA counters are reported only for the kernel source they were
    taken on: a record whose source hash differs from the current source gives
    null, as does a workload with no record."""
    import json
    import bench
    src = ("gemm.hip", "tiles.hpp", "common.hpp")
    path = str(tmp_path / "mfma_counters.json")
    json.dump({"w_cur": {"source_hash": bench.source_hash(*src), "mfma_busy": 0.5,
                         "mfma_flop_per_launch": 1.0},
               "w_old": {"source_hash": "0" * 16, "mfma_busy": 0.5}}, open(path, "w"))
    assert bench.measured_mfma("w_cur", src, path) == {"mfma_busy": 0.5, "mfma_flop_per_launch": 1.0}
    assert bench.measured_mfma("w_old", src, path) is None
    assert bench.measured_mfma("no_such_workload", src, path) is None


def test_accumulation_demo_leg():
    """The limited-accumulation leg on a 64 x 64 corner, with the oracle's own
    FP32-rounded GEMM standing in for the GPU's output: the 14-bit model lands
    near the pages' ~2%, and an FP32 result stays orders of magnitude below it."""
    import bench
    from fp8_fine_grained_online_amd import synthetic as S
    from oracle import gemm, quant
    a = S.activations(64, 4096, S.rng_for(991, 0))
    b = S.weights(128, 4096, S.rng_for(991, 1))

    def corner(n):
        qa, sa = quant.quant_act_1x128(a[:n])
        qb, sb = quant.quant_weight_128x128(b)
        return gemm.gemm_blockscaled(qa, sa, qb, sb, "f32")[:n, :n]

    d = bench.accumulation_demo(a, b, corner, n=64)
    assert d["sample"] == "C[0:64, 0:64], K = 4096"
    assert 0.005 <= d["limited_14bit_chunk32"] <= 0.08
    assert d["gpu_kernel_fp32_out"] * 1000 <= d["limited_14bit_chunk32"]
    assert d["per_group_fp32_model"] * 1000 <= d["limited_14bit_chunk32"]
