#!/usr/bin/env python3
"""Throughput of the fine-grained FP8 hot path on one MI355X.

One step = the whole path over one batch of synthetic inputs already resident
in HBM: online 1x128 activation quantization, 128x128 weight quantization and
the block-scaled FP8 GEMM (grouped for the MoE workload). `value` is the GEMM's
algorithmic FLOPs per step (2*M*N*K; real tokens for MoE) divided by the step
time, i.e. quantization time is charged to the step. A backward workload
(bwd_*) times the layer's Dgrad and Wgrad instead: quantization of dY in 1x128
and 128x1 tiles (one fused kernel), the weight transpose, re-tiling of the
stored FP8 X, and the two GEMMs (value = 4*M*N*K per step). Two timed passes of K steps each: the
first, with HIP events only at its ends, gives the step time and `value`; the
second records an event pair around every kernel on the launch stream and
gives the per-kernel durations (the markers themselves cost a few
microseconds per kernel, so they are kept out of the first pass).

Stream workloads (actquant_*, normquant_*) time one HBM-bound kernel and report
GB/s of algorithmic traffic against the 8 TB/s HBM peak.

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
DEFAULT_WORKLOAD = "dense_4096x4096x4096"
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MALL_BYTES = 256 << 20     # MI355X Infinity Cache
# sources whose hash keys the recorded counters of each streaming kernel
STREAM_SOURCES = {"quant_act_1x128": ("quant.hip", "common.hpp"),
                  "quant_act_1x128_nt": ("quant.hip", "common.hpp"),
                  "quant_weight_128x128": ("quant.hip", "common.hpp"),
                  "norm_quant_act_1x128": ("norm.hip", "common.hpp"),
                  "moe_dispatch_1x128": ("moe.hip", "common.hpp")}


def source_hash(*names):
    """Hash of the kernel sources with comments and whitespace removed, so that
    recorded counters stay valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_fine_grained_online_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
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


def measured_mfma(workload, kernel_src, path=None):
    """MFMA-unit counters of the roofline kernel from committed rocprofv3 --pmc
    runs (profiles/mfma_counters.json), if the kernel's source is unchanged:
    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES over the cycles the chip's SIMDs could
    have kept the matrix units busy during the kernel, and the FP8 MFMA FLOP
    the counters saw per launch."""
    path = path or os.path.join(ROOT, "profiles", "mfma_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(*kernel_src):
        return None
    return {k: rec[k] for k in ("mfma_busy", "mfma_flop_per_launch") if k in rec}


def oracle_threads():
    """Threads the oracle's BLAS calls use."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(workload, a_bits, b_bits, rows):
    """The oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np
    from oracle import gemm, quant
    threads = oracle_threads()
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


def cpu_baseline_grouped(workload, a_bits, b_bits, off, counts, budget_s=10.0):
    """The oracle, untuned, on the real rows of experts 0, 1, ... until about
    `budget_s` seconds of CPU work (at least one expert)."""
    from oracle import gemm, quant
    threads = oracle_threads()
    N, K = b_bits.shape[1:]
    t0 = time.perf_counter()
    e, rows = 0, 0
    while e < len(counts) and (e == 0 or time.perf_counter() - t0 < budget_s):
        r0, n = int(off[e]), int(counts[e])
        qa, sa = quant.quant_act_1x128(a_bits[r0:r0 + n])
        qb, sb = quant.quant_weight_128x128(b_bits[e])
        gemm.round_bf16(gemm.gemm_blockscaled_f64(qa, sa, qb, sb))
        e, rows = e + 1, rows + n
    dt = time.perf_counter() - t0
    return {
        "value": 2.0 * rows * N * K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{workload}: oracle quantization of the real rows of experts 0..{e - 1} "
                   f"({rows} rows) and of their weights ({N}x{K} each), float64 per-group GEMM, "
                   f"bf16 rounding; {dt:.2f} s"),
    }


def copy_rate(steps, warmup):
    """A plain 512 MiB device-to-device copy (bytes moved known exactly; the
    source is twice the Infinity Cache, so it streams from HBM). Returns
    (bytes each way, ms per copy)."""
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
    return n, t0.elapsed_time(t1) / steps


def copy_calibration(steps, warmup):
    n, ms = copy_rate(steps, warmup)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 5),
                      "copy_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def plan_forward(w, args, F, S, L, dev, sp, up_bf16):
    """Quantize A and B, then the (grouped) block-scaled GEMM."""
    import numpy as np
    import torch
    grouped = w.G > 0
    if grouped:
        a_bits, b_bits, counts, off = S.grouped_inputs(w, args.seed)
        M, N, K = a_bits.shape[0], w.N, w.K
        off_d = torch.from_numpy(off).to(dev)
        flops = 2.0 * w.tokens * N * K
        b_rows = w.G * N
    else:
        a_bits, b_bits = S.dense_inputs(w, args.seed)
        M, N, K = w.M, w.N, w.K
        flops = 2.0 * M * N * K
        b_rows = N
    A = up_bf16(a_bits)
    B = up_bf16(b_bits)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    qb = torch.empty((b_rows, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((b_rows // 128, K // 128), dtype=torch.float32, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    gemm_name = "fp8_gemm_grouped" if grouped else "fp8_gemm_blockscaled"
    # small-M shapes take the split-K entry point; its workspace is allocated
    # here, before anything is timed
    ws_bytes = 0 if grouped or w.quant_on_load else L.fp8_gemm_blockscaled_ws_bytes(M, N, K)
    if w.quant_on_load:
        # A is quantized inside the GEMM (its codes and scales are stored too,
        # as the activation quantizer would store them for the backward pass)
        gemm_name = "fp8_gemm_blockscaled_bf16a"
        gemm = lambda: L.fp8_gemm_blockscaled_bf16a(A.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                                    C.data_ptr(), F.FP8Q_OUT_BF16, M, N, K,
                                                    qa.data_ptr(), sa.data_ptr(), sp)
    elif ws_bytes:
        gemm_name = "fp8_gemm_blockscaled_ws"
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        gemm = lambda: L.fp8_gemm_blockscaled_ws(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(),
                                                 sb.data_ptr(), C.data_ptr(), F.FP8Q_OUT_BF16, M,
                                                 N, K, ws.data_ptr(), ws_bytes, sp)
    elif grouped:
        gemm = lambda: L.fp8_gemm_grouped(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                          C.data_ptr(), F.FP8Q_OUT_BF16, off_d.data_ptr(), w.G, M,
                                          N, K, sp)
    else:
        gemm = lambda: L.fp8_gemm_blockscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(),
                                              sb.data_ptr(), C.data_ptr(), F.FP8Q_OUT_BF16, M, N,
                                              K, sp)
    launches = [
        ("quant_act_1x128",
         lambda: L.fp8q_quant_act_1x128(A.data_ptr(), M, K, qa.data_ptr(), sa.data_ptr(), sp)),
        ("quant_weight_128x128",
         lambda: L.fp8q_quant_weight_128x128(B.data_ptr(), b_rows, K, qb.data_ptr(), sb.data_ptr(),
                                             sp)),
        (gemm_name, gemm),
    ]
    if w.quant_on_load:
        launches = launches[1:]

    def cpu():
        if grouped:
            return cpu_baseline_grouped(args.workload, a_bits, b_bits, off, counts)
        return cpu_baseline(args.workload, a_bits, b_bits, M)  # the whole workload

    def gemm_f32_corner(n):
        """C[:n, :n] of this GEMM with FP32 output, from the operands the timed
        steps quantized on the device."""
        c32 = torch.empty((M, N), dtype=torch.float32, device=dev)
        st = L.fp8_gemm_blockscaled(qa.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                    c32.data_ptr(), F.FP8Q_OUT_F32, M, N, K, sp)
        torch.cuda.synchronize()
        if st:
            raise RuntimeError(f"fp8_gemm_blockscaled failed with status {st}")
        return c32[:n, :n].cpu().numpy()

    # algorithmic bytes of the GEMM: operands, scales and output, each once
    gemm_bytes = (M * K + b_rows * K + M * (K // 128) * 4 + (b_rows // 128) * (K // 128) * 4
                  + 2 * M * N)
    if w.quant_on_load:
        gemm_bytes += 2 * M * K  # A read in bf16 (2 B, not 1) and its codes written
    return {
        "launches": launches,
        "flops": {gemm_name: flops},
        "flops_step": flops,
        "gemm_bytes": {gemm_name: gemm_bytes},
        "bytes": {n: b for n, b in (("quant_act_1x128", M * K * 3 + M * (K // 128) * 4),
                                    ("quant_weight_128x128",
                                     b_rows * K * 3 + (b_rows // 128) * (K // 128) * 4))
                  if n in [name for name, _ in launches]},
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "G": w.G or None,
                   "tokens": w.tokens or None, "out": "bf16",
                   "step": " + ".join(name for name, _ in launches)},
        "extra": {"gemm_tflops_padded": (gemm_name, 2.0 * M * N * K)},
        "cpu": cpu,
        # the limited-accumulation demonstration belongs to the K = 4096 GEMM
        "accum": (lambda: accumulation_demo(a_bits, b_bits, gemm_f32_corner))
                 if gemm_name == "fp8_gemm_blockscaled" and M >= 256 and N >= 256 and K == 4096
                 else None,
    }


def grouped_moe_line(args, F, S, L, dev, sp, up_bf16, steps, warmup):
    """The grouped half of the headline metric: the 32-expert MoE GEMM
    (65536 tokens, N = 4096, K = 7168, bf16 out) timed on its own after its
    operands are quantized once. TFLOP/s over the real tokens (the algorithmic
    count) and over the padded rows; fraction of the FP8 MFMA peak."""
    import torch
    name = "moe_g32_65536x4096x7168"
    w = S.WORKLOADS[name]
    sub = argparse.Namespace(**dict(vars(args), workload=name))
    plan = plan_forward(w, sub, F, S, L, dev, sp, up_bf16)
    launches = dict(plan["launches"])
    for n in ("quant_act_1x128", "quant_weight_128x128"):
        if launches[n]():
            raise RuntimeError(f"{n} failed")
    gemm = launches["fp8_gemm_grouped"]
    for _ in range(warmup):
        gemm()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    st = 0
    for _ in range(steps):
        st |= gemm()
    t1.record(stream)
    torch.cuda.synchronize()
    if st:
        raise RuntimeError(f"fp8_gemm_grouped failed with status {st}")
    ms = t0.elapsed_time(t1) / steps
    real = plan["flops"]["fp8_gemm_grouped"] / (ms * 1e-3) / 1e12
    padded = plan["extra"]["gemm_tflops_padded"][1] / (ms * 1e-3) / 1e12
    src = ("gemm.hip", "tiles.hpp", "common.hpp")
    out = {"workload": name, "kernel": "fp8_gemm_grouped", "kernel_ms": round(ms, 5),
           "steps": steps, "tokens": w.tokens, "rows_padded": plan["config"]["M"],
           "tflops": round(real, 2), "frac": round(real / FP8_PEAK_TFLOPS, 4),
           "tflops_padded": round(padded, 2), "peak": FP8_PEAK_TFLOPS,
           "traffic": measured_traffic(name, src)}
    counters = measured_mfma(name, src)
    if counters:
        out.update(counters)
    del plan, launches, gemm
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def accumulation_demo(a_bits, b_bits, gpu_corner, n=256):
    """The pages' limited-accumulation experiment (an FP8 GEMM with K = 4096
    whose Tensor-Core accumulation loses nearly 2%), on C[:n, :n] of this
    workload: the oracle's chunked 14-bit accumulator model and its per-group
    FP32 promotion model, beside the GPU kernel's own FP32 output, each as the
    largest relative error against the exact sum over outputs with
    |C| >= 0.1 RMS(C). Quantizing only the sampled rows of A and of B is exact:
    1x128 tiles and 128x128 blocks do not reach across rows or blocks."""
    import numpy as np
    from oracle import accsim, quant
    t0 = time.perf_counter()
    qa, sa = quant.quant_act_1x128(a_bits[:n])
    qb, sb = quant.quant_weight_128x128(b_bits[:-(-n // 128) * 128])  # whole weight blocks
    sb_rows = np.repeat(sb, 128, axis=0)[:n]
    lim, pg, ref = accsim.demonstration(qa, sa, qb[:n], sb_rows, mant_bits=14, chunk=32, mode="rne")
    gpu = accsim.max_rel_error(gpu_corner(n), ref)
    return {"sample": f"C[0:{n}, 0:{n}], K = {qa.shape[1]}",
            "metric": "max |C - C_exact| / |C_exact| over |C_exact| >= 0.1 RMS",
            "limited_14bit_chunk32": round(lim, 5), "per_group_fp32_model": float(f"{pg:.3g}"),
            "gpu_kernel_fp32_out": float(f"{gpu:.3g}"), "seconds": round(time.perf_counter() - t0, 1)}


def plan_backward(w, args, F, S, L, dev, sp, up_bf16):
    """Dgrad and Wgrad of Y = X W^T (X: M x K, W: N x K, dY: M x N), from the
    forward's stored FP8 X (1x128) and W (128x128) and the bf16 dY."""
    import torch
    M, N, K = w.M, w.N, w.K
    x_bits, w_bits, dy_bits = S.backward_inputs(w, args.seed)
    X, W, DY = up_bf16(x_bits), up_bf16(w_bits), up_bf16(dy_bits)
    u8, f32 = torch.uint8, torch.float32
    e = lambda *shape, dt=u8: torch.empty(shape, dtype=dt, device=dev)
    # stored by the forward pass (not part of the timed step)
    qx, sx = e(M, K), e(M, K // 128, dt=f32)
    qw, sw = e(N, K), e(N // 128, K // 128, dt=f32)
    for st in (L.fp8q_quant_act_1x128(X.data_ptr(), M, K, qx.data_ptr(), sx.data_ptr(), sp),
               L.fp8q_quant_weight_128x128(W.data_ptr(), N, K, qw.data_ptr(), sw.data_ptr(), sp)):
        if st:
            raise RuntimeError(f"forward quantization failed with status {st}")
    qdy, sdy = e(M, N), e(M, N // 128, dt=f32)          # Dgrad A: dY, 1x128
    qdyt, sdyt = e(N, M), e(N, M // 128, dt=f32)        # Wgrad A: dY^T, 128x1
    qwt, swt = e(K, N), e(K // 128, N // 128, dt=f32)   # Dgrad B: W^T
    qxt, sxt = e(K, M), e(K, M // 128, dt=f32)          # Wgrad B: X^T, 128x1
    dX = e(M, K, dt=torch.bfloat16)
    dW = e(N, K, dt=f32)
    launches = [
        ("quant_act_1x128_128x1",  # dY in both tilings from one read
         lambda: L.fp8q_quant_act_1x128_128x1(DY.data_ptr(), M, N, qdy.data_ptr(), sdy.data_ptr(),
                                              qdyt.data_ptr(), sdyt.data_ptr(), sp)),
        ("transpose_weight_128x128",
         lambda: L.fp8q_transpose_weight_128x128(qw.data_ptr(), sw.data_ptr(), N, K, qwt.data_ptr(),
                                                 swt.data_ptr(), sp)),
        ("requant_1x128_to_128x1",
         lambda: L.fp8q_requant_1x128_to_128x1(qx.data_ptr(), sx.data_ptr(), M, K, qxt.data_ptr(),
                                               sxt.data_ptr(), sp)),
        ("fp8_gemm_blockscaled",   # Dgrad: dX = dY W, reduction over N
         lambda: L.fp8_gemm_blockscaled(qdy.data_ptr(), sdy.data_ptr(), qwt.data_ptr(),
                                        swt.data_ptr(), dX.data_ptr(), F.FP8Q_OUT_BF16, M, K, N, sp)),
        ("fp8_gemm_rowscaled",     # Wgrad: dW = dY^T X, reduction over the M tokens
         lambda: L.fp8_gemm_rowscaled(qdyt.data_ptr(), sdyt.data_ptr(), qxt.data_ptr(),
                                      sxt.data_ptr(), dW.data_ptr(), F.FP8Q_OUT_F32, N, K, M, sp)),
    ]
    f = 2.0 * M * N * K
    return {
        "launches": launches,
        "flops": {"fp8_gemm_blockscaled": f, "fp8_gemm_rowscaled": f},
        "flops_step": 2 * f,
        "bytes": {"quant_act_1x128_128x1": M * N * 4 + 2 * M * (N // 128) * 4,
                  "transpose_weight_128x128": N * K * 2 + 2 * (N // 128) * (K // 128) * 4,
                  "requant_1x128_to_128x1": M * K * 2 + 2 * M * (K // 128) * 4},
        "config": {"workload": args.workload, "M": M, "N": N, "K": K, "G": None, "tokens": M,
                   "out": {"dX": "bf16", "dW": "f32"},
                   "step": "quant_act_1x128_128x1(dY) + Dgrad (transpose_weight_128x128(W) + "
                           "fp8_gemm_blockscaled) + Wgrad (requant_1x128_to_128x1(X) + "
                           "fp8_gemm_rowscaled)"},
        "extra": {},
        "cpu": lambda: cpu_baseline_backward(args.workload, x_bits, w_bits, dy_bits, 256),
    }


def plan_stream(w, args, F, S, L, dev, sp, up_bf16):
    """HBM-streaming workloads: standalone 1x128 quantization, or RMS
    normalization fused with it; value in GB/s of algorithmic traffic."""
    import torch
    from fp8_fine_grained_online_amd.synthetic import T_B
    M, K = w.M, w.K
    if w.name.startswith("wquant"):
        # weights (N(0, 0.02)), 128x128 blocks: M x K codes, (M/128) x (K/128) scales
        x_bits = S.weights(M, K, S.rng_for(w.wid, T_B, args.seed))
        X = up_bf16(x_bits)
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sb = torch.empty((M // 128, K // 128), dtype=torch.float32, device=dev)
        nbytes = M * K * 3 + (M // 128) * (K // 128) * 4
        name = "quant_weight_128x128"
        fn = lambda: L.fp8q_quant_weight_128x128(X.data_ptr(), M, K, q.data_ptr(), sb.data_ptr(), sp)
        cpu = lambda: cpu_baseline_weights(args.workload, x_bits, nbytes / M, 32768)  # 8 experts
        return {
            "launches": [(name, fn)], "flops": {}, "bytes": {name: nbytes}, "stream": name,
            "config": {"workload": args.workload, "M": M, "K": K, "step": name,
                       "bytes_per_step": nbytes},
            "extra": {}, "cpu": cpu,
        }
    x_bits, _ = S.dense_inputs(w, args.seed)
    X = up_bf16(x_bits)
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    nbytes = M * K * 3 + M * (K // 128) * 4
    if w.name.startswith("normquant"):
        g_bits, _ = S.norm_params(K, S.rng_for(w.wid, T_B, args.seed))
        g = up_bf16(g_bits)
        name = "norm_quant_act_1x128"
        fn = lambda: L.fp8q_norm_quant_act_1x128(X.data_ptr(), g.data_ptr(), None, 1e-6, 0, M, K,
                                                 q.data_ptr(), sa.data_ptr(), sp)
        nbytes += 2 * K
        cpu = lambda: cpu_baseline_stream(args.workload, x_bits, nbytes / M, M, g_bits)
    else:
        # standalone quantization: nothing reads the codes next on this GPU, so
        # the non-temporal-store form (same codes, not kept in the cache)
        name = "quant_act_1x128_nt"
        fn = lambda: L.fp8q_quant_act_1x128_nt(X.data_ptr(), M, K, q.data_ptr(), sa.data_ptr(), sp)
        cpu = lambda: cpu_baseline_stream(args.workload, x_bits, nbytes / M, M, None)
    return {
        "launches": [(name, fn)],
        "flops": {},
        "bytes": {name: nbytes},
        "stream": name,
        "config": {"workload": args.workload, "M": M, "K": K,
                   "step": name + (" (RMS, eps 1e-6)" if name.startswith("norm") else ""),
                   "bytes_per_step": nbytes},
        "extra": {},
        "cpu": cpu,
    }


def plan_dispatch(w, args, F, S, L, dev, sp, up_bf16):
    """MoE FP8 dispatch (quantize + permute), optionally followed by the
    expert weights' quantization and the grouped up-projection GEMM fed the
    dispatch output with no host synchronization."""
    import torch
    T, K, G, k = w.M, w.K, w.G, w.topk
    x_bits, ids, b_bits = S.dispatch_inputs(w, args.seed)
    X = up_bf16(x_bits)
    ids_d = torch.from_numpy(ids).to(dev)
    cap = L.fp8q_moe_dispatch_max_rows(T, k, G)
    ws_bytes = L.fp8q_moe_dispatch_workspace_bytes(T, k, G)
    q = torch.empty((cap, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((cap, K // 128), dtype=torch.float32, device=dev)
    off = torch.empty((G + 1,), dtype=torch.int32, device=dev)
    rows = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    launches = [("moe_dispatch_1x128",
                 lambda: L.fp8q_moe_dispatch_1x128(X.data_ptr(), ids_d.data_ptr(), T, K, k, G,
                                                   q.data_ptr(), sa.data_ptr(), cap, off.data_ptr(),
                                                   rows.data_ptr(), ws.data_ptr(), ws_bytes, sp))]
    # real rows only: read x once, write every chosen row's codes and scales, the row map
    nbytes = T * K * 2 + T * k * (K + (K // 128) * 4) + T * k * 4 * 2
    config = {"workload": args.workload, "tokens": T, "K": K, "G": G, "topk": k,
              "step": "moe_dispatch_1x128"}
    if not w.N:
        return {"launches": launches, "flops": {}, "bytes": {"moe_dispatch_1x128": nbytes},
                "stream": "moe_dispatch_1x128", "config": config, "extra": {},
                "cpu": lambda: cpu_baseline_dispatch(args.workload, x_bits, ids, G, T)}
    N = w.N
    B = up_bf16(b_bits)
    qb = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((G * N // 128, K // 128), dtype=torch.float32, device=dev)
    C = torch.empty((cap, N), dtype=torch.bfloat16, device=dev)
    launches += [
        ("quant_weight_128x128",
         lambda: L.fp8q_quant_weight_128x128(B.data_ptr(), G * N, K, qb.data_ptr(), sb.data_ptr(), sp)),
        ("fp8_gemm_grouped",
         lambda: L.fp8_gemm_grouped(q.data_ptr(), sa.data_ptr(), qb.data_ptr(), sb.data_ptr(),
                                    C.data_ptr(), F.FP8Q_OUT_BF16, off.data_ptr(), G, cap, N, K, sp)),
    ]
    flops = 2.0 * T * k * N * K
    config.update({"N": N, "out": "bf16",
                   "step": "moe_dispatch_1x128 + quant_weight_128x128 + fp8_gemm_grouped "
                           "(M_total = dispatch capacity, no host sync)"})
    return {"launches": launches, "flops": {"fp8_gemm_grouped": flops}, "flops_step": flops,
            "bytes": {"moe_dispatch_1x128": nbytes,
                      "quant_weight_128x128": G * N * K * 3 + (G * N // 128) * (K // 128) * 4},
            "config": config, "extra": {},
            "cpu": lambda: cpu_baseline(args.workload + " expert 0", x_bits[:2048], b_bits[0], 2048)}


def cpu_baseline_dispatch(workload, x_bits, ids, G, tokens):
    """The oracle, untuned, dispatching the first `tokens` tokens."""
    from oracle import moe
    threads = oracle_threads()
    t0 = time.perf_counter()
    moe.dispatch_1x128(x_bits[:tokens], ids[:tokens], G)
    dt = time.perf_counter() - t0
    T, K = x_bits.shape
    k = ids.shape[1]
    nbytes = tokens * K * 2 + tokens * k * (K + (K // 128) * 4) + tokens * k * 8
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{workload}: oracle dispatch of the first {tokens} tokens; {dt:.2f} s"}


def cpu_baseline_stream(workload, x_bits, bytes_per_row, rows, gamma_bits):
    """The oracle, untuned, on the first `rows` rows."""
    from oracle import norm, quant
    threads = oracle_threads()
    t0 = time.perf_counter()
    if gamma_bits is None:
        quant.quant_act_1x128(x_bits[:rows])
        what = "1x128 quantization"
    else:
        norm.norm_quant_act_1x128(x_bits[:rows], gamma_bits, 1e-6)
        what = "RMS normalization + 1x128 quantization"
    dt = time.perf_counter() - t0
    return {
        "value": bytes_per_row * rows / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{workload}: oracle {what} of the first {rows} rows; {dt:.2f} s",
    }


def cpu_baseline_weights(workload, w_bits, bytes_per_row, rows):
    """The oracle, untuned, on the first `rows` rows (whole 128x128 blocks)."""
    from oracle import quant
    threads = oracle_threads()
    t0 = time.perf_counter()
    quant.quant_weight_128x128(w_bits[:rows])
    dt = time.perf_counter() - t0
    return {
        "value": bytes_per_row * rows / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{workload}: oracle 128x128 quantization of the first {rows} rows; {dt:.2f} s",
    }


def cpu_baseline_backward(workload, x_bits, w_bits, dy_bits, rows):
    """The oracle, untuned: `rows` rows of dX and `rows` rows of dW."""
    import numpy as np
    from oracle import gemm, quant
    threads = oracle_threads()
    M, K = x_bits.shape
    N = w_bits.shape[0]
    t0 = time.perf_counter()
    qd, sd = quant.quant_act_1x128(dy_bits[:rows])
    qwt, swt = quant.transpose_weight_128x128(*quant.quant_weight_128x128(w_bits))
    gemm.round_bf16(gemm.gemm_blockscaled_f64(qd, sd, qwt, swt))
    qdt, sdt = quant.quant_act_1x128(np.ascontiguousarray(dy_bits[:, :rows].T))
    qxt, sxt = quant.requant_1x128_to_128x1(*quant.quant_act_1x128(x_bits))
    gemm.round_f32(gemm.gemm_rowscaled_f64(qdt, sdt, qxt, sxt))
    dt = time.perf_counter() - t0
    return {
        "value": (2.0 * rows * K * N + 2.0 * rows * K * M) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{workload}: oracle Dgrad of the first {rows} token rows (1x128 quantization of "
                   f"dY, weight quantization and transpose, float64 per-group GEMM, bf16) and "
                   f"Wgrad of the first {rows} output channels (128x1 quantization of dY, "
                   f"re-tiling of all of X, float64 row-scaled GEMM, float32); {dt:.2f} s"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the clock takes a few hundred microseconds of load to settle: the default
    # warms up long enough for the short steps too
    ap.add_argument("--warmup", type=int, default=200)
    # untimed steps for this many seconds before the W warm-up steps: the
    # shader clock needs tens of milliseconds of load to ramp, and a handful
    # of warm-up steps (e.g. --warmup 5) leaves the timed steps on a cold
    # clock (4096^3 GEMM measured 88 us cold against 61-66 us settled)
    ap.add_argument("--settle", type=float, default=0.3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-grouped", action="store_true",
                    help="skip the grouped MoE GEMM line that the default workload also reports")
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

    if args.workload not in S.WORKLOADS:
        print(f"unknown workload {args.workload}; choose from {list(S.WORKLOADS)}",
              file=sys.stderr)
        sys.exit(2)
    w = S.WORKLOADS[args.workload]
    L = F.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if w.topk:
        kind = plan_dispatch
    elif w.backward:
        kind = plan_backward
    else:
        kind = plan_stream if w.N == 0 else plan_forward
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    plan = kind(w, args, F, S, L, dev, sp, up_bf16)
    resident = torch.cuda.memory_allocated(dev) - mem0
    names = [n for n, _ in plan["launches"]]
    # HBM-bound workloads cycle through copies of their buffers whose total
    # exceeds three times the 256 MB Infinity Cache, so that each step reads
    # its inputs from HBM rather than from the cache the previous step filled
    ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    hbm_bound = "stream" in plan or any(
        plan["flops"][n] / b < ridge for n, b in plan.get("gemm_bytes", {}).items())
    n_copies = 1
    if hbm_bound and resident > 0:
        n_copies = int(min(8, max(1, -(-3 * MALL_BYTES // resident))))
    copies = [plan["launches"]] + [kind(w, args, F, S, L, dev, sp, up_bf16)["launches"]
                                   for _ in range(n_copies - 1)]
    step_no = [0]

    def step(ev=None):
        s = 0
        launches = copies[step_no[0] % n_copies]
        step_no[0] += 1
        for i, (_, fn) in enumerate(launches):
            if ev:
                ev[i].record(stream)
            s |= fn()
        if ev:
            ev[len(launches)].record(stream)
        if s:
            raise RuntimeError(f"launch failed with status {s}")

    settle_end = time.perf_counter() + max(0.0, args.settle)
    settle_steps = 0
    while time.perf_counter() < settle_end:
        for _ in range(8):
            step()
        settle_steps += 8
        torch.cuda.synchronize()
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per_launch = {n: np.array([e[i].elapsed_time(e[i + 1]) for e in evs]) for i, n in enumerate(names)}
    kms = {n: float(v.mean()) for n, v in per_launch.items()}
    kpct = {n: [round(float(x), 5) for x in np.percentile(v, [10, 50, 90])]
            for n, v in per_launch.items()}
    if len(names) == 1:
        # one launch per step: the step timing (events only at the ends of the
        # timed pass) is that kernel's duration without per-launch marker cost
        kms = {names[0]: ms_step}

    if "stream" in plan:
        # HBM-bound workload: GB/s of algorithmic traffic against the HBM peak
        name = plan["stream"]
        gbps = plan["bytes"][name] / (kms[name] * 1e-3) / 1e9
        metric = f"{name} HBM GB/s & % of HBM peak"
        value, unit = plan["bytes"][name] / (ms_step * 1e-3) / 1e9, "GB/s"
        roofline = {"bound": "hbm", "kernel": name, "achieved": round(gbps, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(args.workload, STREAM_SOURCES[name])}
    else:
        # the roofline kernel: the slowest contraction of the step; its roof is
        # the MFMA peak unless its arithmetic intensity (FLOP per algorithmic
        # byte) is below the ridge point, as for small-M shapes
        gemm_name = max(plan["flops"], key=lambda n: kms[n])
        gemm_tflops = plan["flops"][gemm_name] / (kms[gemm_name] * 1e-3) / 1e12
        metric = METRIC
        value, unit = plan["flops_step"] / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        gemm_src = ("gemm_qa.hip" if gemm_name == "fp8_gemm_blockscaled_bf16a" else "gemm.hip",
                    "tiles.hpp", "common.hpp")
        traffic = measured_traffic(args.workload, gemm_src)
        gbytes = plan.get("gemm_bytes", {}).get(gemm_name)
        ridge = FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if gbytes and plan["flops"][gemm_name] / gbytes < ridge:
            gbps = gbytes / (kms[gemm_name] * 1e-3) / 1e9
            roofline = {"bound": "hbm", "kernel": gemm_name, "achieved": round(gbps, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                        "traffic": traffic, "tflops": round(gemm_tflops, 2)}
        else:
            roofline = {"bound": "mfma", "kernel": gemm_name, "achieved": round(gemm_tflops, 2),
                        "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic}
            counters = measured_mfma(args.workload, gemm_src)
            if counters:
                roofline.update(counters)

    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": dict(plan["config"], buffer_copies=n_copies,
                       buffer_MB_per_copy=round(resident / 1e6, 1),
                       settle_s=args.settle, settle_steps=settle_steps),
        "roofline": roofline,
        "kernels_ms": {n: round(v, 5) for n, v in kms.items()},
        "kernels_ms_p10_p50_p90": kpct,
        "kernels_GBps": {n: round(b / (kms[n] * 1e-3) / 1e9, 1) for n, b in plan["bytes"].items()},
        "kernels_TFLOPs": {n: round(f / (kms[n] * 1e-3) / 1e12, 2) for n, f in plan["flops"].items()},
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": None,
    }
    for key, (n, f) in plan["extra"].items():
        out[key] = round(f / (kms[n] * 1e-3) / 1e12, 2)
    if roofline["bound"] == "hbm":
        # practical ceiling: a plain device-to-device copy on this GPU
        n_copy, ms_copy = copy_rate(20, 5)
        copy_gbps = 2 * n_copy / (ms_copy * 1e-3) / 1e9
        roofline["copy_GBps"] = round(copy_gbps, 1)
        roofline["frac_of_copy"] = round(roofline["achieved"] / copy_gbps, 4)
    cpu_fn, accum_fn = plan["cpu"], plan.get("accum")
    if args.workload == DEFAULT_WORKLOAD and not args.no_grouped:
        # the metric names both the 4096^3 GEMM and the grouped MoE GEMM
        del copies, plan
        out["grouped_moe"] = grouped_moe_line(args, F, S, L, dev, sp, up_bf16,
                                              steps=max(5, min(args.steps, 50)),
                                              warmup=20)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_fn()
        if accum_fn:
            out["accumulation_demo"] = accum_fn()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
