"""Seeded synthetic inputs: the only code shared by the GPU path's tests and the oracle.

Holds none of the method's arithmetic: it draws bf16 activations and weights,
and MoE expert offsets, with the shapes and value distributions of the
workloads below. Everything is a pure function of (seed, workload, tensor id).

Distributions (the pages give no data; these follow the workloads' own
definitions): activations are N(0, 1) with exactly round(0.001 * numel)
distinct entries, drawn without replacement, multiplied by 100 (outliers, the
case the pages' fine-grained scaling is meant for); weights are N(0, 0.02).
Values are drawn in float32 and rounded to bf16 (nearest, ties to even).
Output gradients dY of the backward workloads are drawn like activations;
normalization scales are 1 + N(0, 0.1) and shifts N(0, 0.05).
MoE token counts per expert are multinomial(total, uniform), each padded up to a
multiple of 128 with all-zero rows.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 100.0
WEIGHT_STD = 0.02


def rng_for(workload: int, tensor: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, workload, tensor])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def activations(M: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """M x K bf16 bits: N(0,1), 0.1% of entries (exact count) times 100."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n_out = int(round(OUTLIER_FRACTION * M * K))
    if n_out:
        idx = rng.choice(M * K, size=n_out, replace=False)
        x.reshape(-1)[idx] *= np.float32(OUTLIER_FACTOR)
    return f32_to_bf16_bits(x)


def weights(N: int, K: int, rng: np.random.Generator) -> np.ndarray:
    """N x K bf16 bits: N(0, 0.02)."""
    x = rng.standard_normal((N, K), dtype=np.float32) * np.float32(WEIGHT_STD)
    return f32_to_bf16_bits(x)


def moe_offsets(total_tokens: int, G: int, rng: np.random.Generator):
    """(real counts, padded offsets int32[G+1]) for multinomial(total, 1/G) counts."""
    counts = rng.multinomial(total_tokens, [1.0 / G] * G).astype(np.int64)
    padded = (counts + 127) // 128 * 128
    off = np.zeros(G + 1, dtype=np.int64)
    off[1:] = np.cumsum(padded)
    return counts, off.astype(np.int32)


def moe_activations(counts, offsets, K: int, rng: np.random.Generator) -> np.ndarray:
    """Padded M_total x K bf16 bits; expert e's real tokens first, padding rows +0."""
    counts = np.asarray(counts)
    offsets = np.asarray(offsets, dtype=np.int64)
    real = activations(int(counts.sum()), K, rng)
    out = np.zeros((int(offsets[-1]), K), dtype=np.uint16)
    src = 0
    for e, c in enumerate(counts):
        out[offsets[e]:offsets[e] + c] = real[src:src + c]
        src += c
    return out


@dataclass
class Workload:
    """One of the synthetic workloads; ids match the list below."""
    wid: int
    name: str
    M: int
    N: int
    K: int
    out: List[str] = field(default_factory=lambda: ["bf16"])
    G: int = 0  # experts (grouped); 0 = dense
    tokens: int = 0  # grouped: real tokens before padding
    backward: bool = False  # Dgrad + Wgrad of the layer Y[M x N] = X[M x K] W[N x K]^T
    topk: int = 0  # MoE dispatch: router choices per token (M = tokens)
    quant_on_load: bool = False  # A quantized inside the GEMM (fp8_gemm_blockscaled_bf16a)


WORKLOADS = {
    "dense_256x256x1024": Workload(0, "dense_256x256x1024", 256, 256, 1024, ["f32", "bf16"]),
    "dense_4096x4096x4096": Workload(1, "dense_4096x4096x4096", 4096, 4096, 4096),
    # the same inputs (same id) through the quantize-on-load GEMM
    "qol_4096x4096x4096": Workload(1, "qol_4096x4096x4096", 4096, 4096, 4096, quant_on_load=True),
    "proj_8192x7168x2048": Workload(20, "proj_8192x7168x2048", 8192, 7168, 2048),
    "proj_8192x2048x7168": Workload(21, "proj_8192x2048x7168", 8192, 2048, 7168),
    "bwd_proj_8192x7168x2048": Workload(22, "bwd_proj_8192x7168x2048", 8192, 7168, 2048,
                                        backward=True),
    "skinny_64x7168x7168": Workload(30, "skinny_64x7168x7168", 64, 7168, 7168),
    "actquant_16384x7168": Workload(31, "actquant_16384x7168", 16384, 0, 7168),
    "normquant_16384x7168": Workload(32, "normquant_16384x7168", 16384, 0, 7168),
    # standalone 128x128 weight quantization: 32 experts' 4096 x 7168 weights as
    # one 131072 x 7168 tensor
    "wquant_32x4096x7168": Workload(35, "wquant_32x4096x7168", 32 * 4096, 0, 7168),
    "dispatch_8192x7168_top8_g32": Workload(33, "dispatch_8192x7168_top8_g32", 8192, 0, 7168,
                                            G=32, topk=8),
    "moe_up_8192x4096x7168_top8_g32": Workload(34, "moe_up_8192x4096x7168_top8_g32", 8192, 4096,
                                               7168, G=32, topk=8),
    "moe_g32_65536x4096x7168": Workload(4, "moe_g32_65536x4096x7168", 0, 4096, 7168,
                                        G=32, tokens=65536),
}

# tensor ids inside a workload's seed stream
T_A, T_B, T_OFFSETS, T_DY = 0, 1, 2, 3


def dense_inputs(w: Workload, seed: int = 0, M: Optional[int] = None):
    """(A bits M x K, B bits N x K) for a dense workload."""
    M = w.M if M is None else M
    a = activations(M, w.K, rng_for(w.wid, T_A, seed))
    b = weights(w.N, w.K, rng_for(w.wid, T_B, seed)) if w.N else None
    return a, b


def norm_params(K: int, rng: np.random.Generator):
    """(gamma, beta) bf16 bits of a normalization layer: 1 + N(0, 0.1), N(0, 0.05)."""
    g = f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(K, dtype=np.float32))
    b = f32_to_bf16_bits(0.05 * rng.standard_normal(K, dtype=np.float32))
    return g, b


def routing(T: int, k: int, G: int, rng: np.random.Generator) -> np.ndarray:
    """Router choices T x k (int32): k distinct experts per token, uniform."""
    return np.argsort(rng.random((T, G)), axis=1)[:, :k].astype(np.int32)


def dispatch_inputs(w: Workload, seed: int = 0):
    """(x bits T x K, topk_ids T x k, expert weights G x N x K or None)."""
    x = activations(w.M, w.K, rng_for(w.wid, T_A, seed))
    ids = routing(w.M, w.topk, w.G, rng_for(w.wid, T_OFFSETS, seed))
    b = None
    if w.N:
        rb = rng_for(w.wid, T_B, seed)
        b = np.stack([weights(w.N, w.K, rb) for _ in range(w.G)])
    return x, ids, b


def backward_inputs(w: Workload, seed: int = 0):
    """(X bits M x K, W bits N x K, dY bits M x N) for a backward workload."""
    x, wt = dense_inputs(w, seed)
    dy = activations(w.M, w.N, rng_for(w.wid, T_DY, seed))
    return x, wt, dy


def grouped_inputs(w: Workload, seed: int = 0):
    """(A bits M_total x K, B bits G x N x K, counts, offsets int32[G+1])."""
    counts, off = moe_offsets(w.tokens, w.G, rng_for(w.wid, T_OFFSETS, seed))
    a = moe_activations(counts, off, w.K, rng_for(w.wid, T_A, seed))
    rb = rng_for(w.wid, T_B, seed)
    b = np.stack([weights(w.N, w.K, rb) for _ in range(w.G)])
    return a, b, counts, off


def exhaustive_tiles(amax_exp_field: int, depth: int = 21) -> np.ndarray:
    """bf16 bits, T x 128: every (amax significand, x) pair at one amax exponent.

    Each row is one 1x128 tile: element 0 is the tile's amax (positive, bf16
    exponent field ``amax_exp_field``, significand 0..127), the other 127 are
    bf16 values x with |x| <= amax, both signs, covering every bf16 pattern whose
    exponent field lies within ``depth`` binades below amax's (smaller x round
    to zero codes). Rows of one significand are consecutive. Exponent field 0
    makes amax a bf16 subnormal (x then spans the subnormals below it).
    """
    rows = []
    lo_field = max(amax_exp_field - depth, 0)
    for sig in range(128):
        amax_bits = (amax_exp_field << 7) | sig
        if amax_bits == 0:
            continue
        mags = np.arange(lo_field << 7, amax_bits + 1, dtype=np.uint32)
        xs = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-xs.size) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)])
        body = xs.reshape(-1, 127)
        head = np.full((body.shape[0], 1), amax_bits, np.uint16)
        rows.append(np.concatenate([head, body], axis=1))
    return np.concatenate(rows, axis=0)
