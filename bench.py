#!/usr/bin/env python3
"""Throughput of the fine-grained FP8 hot path on one MI355X.

One step = the whole path over one batch of synthetic inputs already resident
in HBM: online 1x128 activation quantization, 128x128 weight quantization and
the block-scaled FP8 GEMM (grouped for the MoE workload). `value` is the GEMM's
algorithmic FLOPs per step (2*M*N*K; real tokens for MoE) divided by the step
time, i.e. quantization time is charged to the step. Two timed passes of K
steps each: the first, with HIP events only at its ends, gives the step time
and `value`; the second records an event pair around every kernel on the
launch stream and gives the per-kernel durations (the markers themselves cost
a few microseconds per kernel, so they are kept out of the first pass).

Prints one JSON line. Options: --steps K --warmup W --workload NAME --gpus 1.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOPS & % of FP8 MFMA peak (4096^3, grouped MoE)"
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_fine_grained_online_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel_src):
    """HBM bytes per launch from committed counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(*kernel_src):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(workload, a_bits, b_bits, rows):
    """The oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np
    from oracle import gemm, quant
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    qa, sa = quant.quant_act_1x128(a_bits[:rows])
    qb, sb = quant.quant_weight_128x128(b_bits)
    c64 = gemm.gemm_blockscaled_f64(qa, sa, qb, sb)
    gemm.round_bf16(c64)
    dt = time.perf_counter() - t0
    N, K = b_bits.shape
    return {
        "value": 2.0 * rows * N * K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{workload}: oracle quantization of the first {rows} rows of A and all of B "
                   f"({N}x{K}), float64 per-group GEMM of those rows, bf16 rounding; {dt:.2f} s"),
    }


def copy_calibration(steps, warmup):
    """A plain 512 MiB device-to-device copy: bytes moved are known exactly."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        dst.copy_(src)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 5),
                      "copy_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense_4096x4096x4096")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of 512 MiB (HBM ceiling and the "
                         "reference launch for calibrating FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(args.steps, args.warmup)
        return

    import fp8_fine_grained_online_amd as F
    from fp8_fine_grained_online_amd import synthetic as S

    if args.workload not in S.WORKLOADS or args.workload == "actquant_16384x7168":
        print(f"unknown GEMM workload {args.workload}; choose from "
              f"{[k for k in S.WORKLOADS if not k.startswith('actquant')]}", file=sys.stderr)
        sys.exit(2)
    w = S.WORKLOADS[args.workload]
    L = F.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    grouped = w.G > 0
    if grouped:
        a_bits, b_bits, counts, off = S.grouped_inputs(w, args.seed)
        M, N, K = a_bits.shape[0], w.N, w.K
        off_d = torch.from_numpy(off).to(dev)
        flops = 2.0 * w.tokens * N * K
        flops_padded = 2.0 * M * N * K
        b_rows = w.G * N
    else:
        a_bits, b_bits = S.dense_inputs(w, args.seed)
        M, N, K = w.M, w.N, w.K
        flops = flops_padded = 2.0 * M * N * K
        b_rows = N
    A = up_bf16(a_bits)
    B = up_bf16(b_bits)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    qb = torch.empty((b_rows, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((b_rows // 128, K // 128), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        s = L.fp8q_quant_act_1x128(A.data_ptr(), M, K, qa.data_ptr(), sa.data_ptr(), sp)
        if ev:
            ev[1].record(stream)
        s |= L.fp8q_quant_weight_128x128(B.data_ptr(), b_rows, K, qb.data_ptr(), sb.data_ptr(), sp)
        if ev:
            ev[2].record(stream)
        if grouped:
            s |= L.fp8_gemm_grouped(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                    C.data_ptr(), F.FP8Q_OUT_BF16, off_d.data_ptr(), w.G, M, N, K, sp)
        else:
            s |= L.fp8_gemm_blockscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                        C.data_ptr(), F.FP8Q_OUT_BF16, M, N, K, sp)
        if ev:
            ev[3].record(stream)
        if s:
            raise RuntimeError(f"launch failed with status {s}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # pass 1: the step time, events only at the ends
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_begin.elapsed_time(t_end) / args.steps

    # pass 2: per-kernel durations from event pairs on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    q_act = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    q_w = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    g_ms = np.mean([e[2].elapsed_time(e[3]) for e in evs])

    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    act_bytes = M * K * (2 + 1) + M * (K // 128) * 4
    w_bytes = b_rows * K * (2 + 1) + (b_rows // 128) * (K // 128) * 4
    kernel_src = ("gemm.hip", "common.hpp")
    traffic = measured_traffic(args.workload, kernel_src)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "M": M, "N": N, "K": K, "G": w.G or None,
            "tokens": w.tokens or None, "out": "bf16",
            "step": "quant_act_1x128 + quant_weight_128x128 + " +
                    ("fp8_gemm_grouped" if grouped else "fp8_gemm_blockscaled"),
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "fp8_gemm_grouped" if grouped else "fp8_gemm_blockscaled",
            "achieved": round(gemm_tflops, 2),
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "kernels_ms": {
            "quant_act_1x128": round(q_act, 5),
            "quant_weight_128x128": round(q_w, 5),
            "gemm": round(g_ms, 5),
        },
        "quant_act_GBps": round(act_bytes / (q_act * 1e-3) / 1e9, 1),
        "quant_weight_GBps": round(w_bytes / (q_w * 1e-3) / 1e9, 1),
        "gemm_tflops_padded": round(flops_padded / (g_ms * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        if grouped:
            e = 0
            r0 = int(off[e])
            out["cpu_baseline"] = cpu_baseline(args.workload + f" expert {e}", a_bits[r0:r0 + 128],
                                               b_bits[e], 128)
        else:
            out["cpu_baseline"] = cpu_baseline(args.workload, a_bits, b_bits, min(M, 1024))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
