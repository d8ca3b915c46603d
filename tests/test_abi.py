"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any HIP call.

Every call here either fails validation (a status other than FP8Q_OK, returned
before the first HIP call) or is a zero-size no-op that returns FP8Q_OK before
the first HIP call. No call carries arguments that pass validation, so none
can reach a kernel launch on the fake addresses it passes, on any machine. As
a second guard the module still skips itself where a GPU is visible (torch
sees one, or the kernel driver's device node exists); the GPU suites exercise
every entry point with real buffers."""

import ctypes
import os
import re

import pytest

from conftest import ROOT, gpu_available

pytestmark = pytest.mark.skipif(gpu_available() or os.path.exists("/dev/kfd"),
                                reason="fake device addresses: runs only without a GPU")

HEADER = os.path.join(ROOT, "include", "fp8q.h")


def _lib():
    from fp8_fine_grained_online_amd import _lib as L
    if not os.path.exists(L.lib_path()):
        pytest.fail("libfp8q.so not built (run __graft_entry__.build())")
    return L.lib()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"FP8Q_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


ENTRY_POINTS = ["fp8q_quant_act_1x128", "fp8q_quant_act_1x128_nt", "fp8q_quant_weight_128x128", "fp8_gemm_blockscaled",
                "fp8_gemm_grouped", "fp8q_quant_act_128x1", "fp8q_requant_1x128_to_128x1",
                "fp8q_transpose_weight_128x128", "fp8_gemm_rowscaled", "fp8q_quant_act_1x128_128x1",
                "fp8q_norm_quant_act_1x128", "fp8q_moe_dispatch_1x128", "fp8_gemm_blockscaled_ws",
                "fp8_gemm_blockscaled_bf16a", "fp8_gemm_blockscaled_noalloc"]


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ENTRY_POINTS + ["fp8q_version", "fp8q_status_string"]:
        assert name in syms


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert L.fp8q_version() == 202
    for s in range(9):
        assert L.fp8q_status_string(s) != b"unknown status"
    assert L.fp8q_status_string(99) == b"unknown status"


# fake, suitably aligned addresses (never dereferenced: no GPU here)
P = 0x100000
A, SA, B, SB, C, OFF, X, Q = (P * i for i in range(1, 9))


@pytest.mark.parametrize("name", ["fp8q_quant_act_1x128", "fp8q_quant_act_1x128_nt"])
def test_quant_act_validation(name):
    L = _lib()
    f = getattr(L, name)
    assert f(X, 4, 100, Q, SA, None) == 2  # K % 128
    assert f(X, -1, 128, Q, SA, None) == 2
    assert f(X, 4, -128, Q, SA, None) == 2
    assert f(None, 4, 128, Q, SA, None) == 1
    assert f(X, 4, 128, None, SA, None) == 1
    assert f(X, 4, 128, Q, None, None) == 1
    assert f(X + 2, 4, 128, Q, SA, None) == 3
    assert f(X, 4, 128, Q + 8, SA, None) == 3
    assert f(X, 4, 128, Q, SA + 2, None) == 3
    assert f(X, 1 << 31, 128, Q, SA, None) == 7
    # zero sizes: success without touching anything (NULL pointers allowed)
    assert f(None, 0, 128, None, None, None) == 0
    assert f(None, 5, 0, None, None, None) == 0


def test_quant_weight_validation():
    L = _lib()
    f = L.fp8q_quant_weight_128x128
    assert f(X, 100, 128, Q, SB, None) == 2
    assert f(X, 128, 100, Q, SB, None) == 2
    assert f(X, -128, 128, Q, SB, None) == 2
    assert f(None, 128, 128, Q, SB, None) == 1
    assert f(X, 128, 128, Q, None, None) == 1
    assert f(X + 4, 128, 128, Q, SB, None) == 3
    assert f(X, 128, 128, Q, SB + 1, None) == 3
    assert f(X, 128 * 65536, 128, Q, SB, None) == 7
    assert f(None, 0, 128, None, None, None) == 0


def test_gemm_validation():
    L = _lib()
    f = L.fp8_gemm_blockscaled
    assert f(A, SA, B, SB, C, 1, 64, 100, 128, None) == 2  # N % 128
    assert f(A, SA, B, SB, C, 1, 64, 128, 100, None) == 2  # K % 128
    assert f(A, SA, B, SB, C, 1, -1, 128, 128, None) == 2
    assert f(A, SA, B, SB, C, 2, 64, 128, 128, None) == 4  # dtype
    assert f(A, SA, B, SB, C, -1, 64, 128, 128, None) == 4
    for i in range(5):
        args = [A, SA, B, SB, C]
        args[i] = None
        assert f(*args, 1, 64, 128, 128, None) == 1, i
    assert f(A + 8, SA, B, SB, C, 1, 64, 128, 128, None) == 3
    assert f(A, SA, B + 1, SB, C, 1, 64, 128, 128, None) == 3
    assert f(A, SA, B, SB, C + 4, 0, 64, 128, 128, None) == 3
    assert f(A, SA + 2, B, SB, C, 0, 64, 128, 128, None) == 3
    assert f(A, SA, B, SB + 2, C, 0, 64, 128, 128, None) == 3
    assert f(A, SA, B, SB, C, 0, 1 << 31, 128, 128, None) == 7
    assert f(A, SA, B, SB, C, 0, 64, 128, (1 << 23) + 128, None) == 7  # K limit
    assert f(A + 8, SA, B, SB, C, 0, 64, 128, 1 << 23, None) == 3  # the largest K gets past the size checks
    assert f(None, None, None, None, None, 0, 0, 128, 128, None) == 0
    assert f(None, None, None, None, None, 0, 64, 0, 128, None) == 0


def test_grouped_validation():
    L = _lib()
    f = L.fp8_gemm_grouped
    assert f(A, SA, B, SB, C, 1, OFF, 0, 256, 128, 128, None) == 2  # G < 1
    assert f(A, SA, B, SB, C, 1, OFF, 2, 200, 128, 128, None) == 2  # M_total % 128
    assert f(A, SA, B, SB, C, 1, OFF, 2, 256, 100, 128, None) == 2
    assert f(A, SA, B, SB, C, 1, OFF, 2, 256, 128, 100, None) == 2
    assert f(A, SA, B, SB, C, 3, OFF, 2, 256, 128, 128, None) == 4
    assert f(A, SA, B, SB, C, 1, None, 2, 256, 128, 128, None) == 1
    assert f(A, SA, B, SB, C, 1, OFF + 2, 2, 256, 128, 128, None) == 3
    assert f(None, SA, B, SB, C, 1, OFF, 2, 256, 128, 128, None) == 1
    assert f(None, None, None, None, None, 1, None, 2, 0, 128, 128, None) == 0


@pytest.mark.parametrize("name", ["fp8q_quant_act_128x1", "fp8q_requant_1x128_to_128x1",
                                  "fp8q_transpose_weight_128x128"])
def test_retile_validation(name):
    L = _lib()
    with_scales = name != "fp8q_quant_act_128x1"

    def f(inp, ins, R, C_, out, outs):
        fn = getattr(L, name)
        return fn(inp, ins, R, C_, out, outs, None) if with_scales else fn(inp, R, C_, out, outs, None)

    assert f(X, SA, 100, 128, Q, SB) == 2  # rows % 128
    assert f(X, SA, 128, 100, Q, SB) == 2  # cols % 128
    assert f(X, SA, -128, 128, Q, SB) == 2
    assert f(None, SA, 128, 128, Q, SB) == 1
    assert f(X, SA, 128, 128, None, SB) == 1
    assert f(X, SA, 128, 128, Q, None) == 1
    if with_scales:
        assert f(X, None, 128, 128, Q, SB) == 1
        assert f(X, SA + 2, 128, 128, Q, SB) == 3
    assert f(X + 8, SA, 128, 128, Q, SB) == 3
    assert f(X, SA, 128, 128, Q + 4, SB) == 3
    assert f(X, SA, 128, 128, Q, SB + 1) == 3
    assert f(X, SA, 1 << 31, 128, Q, SB) == 7
    assert f(X, SA, 128, 128 * 65536, Q, SB) == 7
    assert f(None, None, 0, 128, None, None) == 0
    assert f(None, None, 128, 0, None, None) == 0


def test_dual_quant_validation():
    L = _lib()
    f = L.fp8q_quant_act_1x128_128x1
    assert f(X, 100, 128, Q, SA, B, SB, None) == 2
    assert f(X, 128, 100, Q, SA, B, SB, None) == 2
    for i in range(5):
        args = [X, Q, SA, B, SB]
        args[i] = None
        assert f(args[0], 128, 128, *args[1:], None) == 1, i
    assert f(X, 128, 128, Q + 8, SA, B, SB, None) == 3
    assert f(X, 128, 128, Q, SA + 2, B, SB, None) == 3
    assert f(X, 128, 128, Q, SA, B + 8, SB, None) == 3
    assert f(None, 0, 128, None, None, None, None, None) == 0


def test_norm_quant_validation():
    L = _lib()
    f = L.fp8q_norm_quant_act_1x128
    G_, BETA = B, SB  # fake gamma / beta addresses (16-byte aligned)
    assert f(X, G_, BETA, 1e-6, 0, 4, 100, Q, SA, None) == 2           # K % 128
    assert f(X, G_, BETA, 1e-6, 0, -1, 128, Q, SA, None) == 2
    assert f(X, G_, BETA, 1e-6, 2, 4, 128, Q, SA, None) == 2           # centred flag
    assert f(X, G_, BETA, -1.0, 0, 4, 128, Q, SA, None) == 2           # eps < 0
    assert f(X, G_, BETA, float("nan"), 0, 4, 128, Q, SA, None) == 2
    assert f(X, G_, BETA, float("inf"), 0, 4, 128, Q, SA, None) == 2
    assert f(X, G_, BETA, 1e-6, 0, 4, 16384 + 128, Q, SA, None) == 7  # row must fit a wavefront
    assert f(None, G_, BETA, 1e-6, 0, 4, 128, Q, SA, None) == 1
    assert f(X, None, BETA, 1e-6, 0, 4, 128, Q, SA, None) == 1
    assert f(X, G_, None, 1e-6, 1, 4, 128, Q, SA, None) == 1          # centred needs beta
    assert f(X, G_, BETA, 1e-6, 0, 4, 128, None, SA, None) == 1
    assert f(X, G_, BETA, 1e-6, 0, 4, 128, Q, None, None) == 1
    assert f(X, G_ + 4, BETA, 1e-6, 0, 4, 128, Q, SA, None) == 3
    assert f(X, G_, BETA + 4, 1e-6, 1, 4, 128, Q, SA, None) == 3
    assert f(X + 2, G_, BETA, 1e-6, 0, 4, 128, Q, SA, None) == 3
    assert f(X, G_, BETA, 1e-6, 0, 4, 128, Q, SA + 1, None) == 3
    assert f(None, None, None, 1e-6, 0, 0, 128, None, None, None) == 0


def test_dispatch_sizes_and_validation():
    import ctypes
    L = _lib()
    assert L.fp8q_moe_dispatch_max_rows(8192, 8, 32) == (8192 * 8 + 127 * 32 + 127) // 128 * 128
    assert L.fp8q_moe_dispatch_max_rows(1, 1, 1) == 128
    assert L.fp8q_moe_dispatch_max_rows(10, 0, 32) == -1
    assert L.fp8q_moe_dispatch_max_rows(10, 2, 1025) == -1
    ws = L.fp8q_moe_dispatch_workspace_bytes(8192, 8, 32)
    assert ws == (2 * (8192 * 8 // 256) * 32 + 32) * 4
    assert L.fp8q_moe_dispatch_workspace_bytes(-1, 8, 32) == -1
    f = L.fp8q_moe_dispatch_1x128
    OFFS, ROWS, WS = OFF, A, C
    cap = L.fp8q_moe_dispatch_max_rows(64, 2, 4)
    wsb = L.fp8q_moe_dispatch_workspace_bytes(64, 2, 4)
    ok = [X, SB, 64, 256, 2, 4, Q, SA, cap, OFFS, ROWS, WS, wsb, None]

    def call(**kw):
        args = list(ok)
        names = ["x", "ids", "T", "K", "topk", "G", "q", "sa", "cap", "off", "rows", "ws", "wsb", "s"]
        for k_, v in kw.items():
            args[names.index(k_)] = v
        return f(*args)

    assert call(K=100) == 2 and call(topk=0) == 2 and call(G=0) == 2 and call(T=-1) == 2
    assert call(G=1025) == 7
    assert call(cap=cap - 1) == 2                      # outputs too small for the padding
    assert call(wsb=wsb - 4) == 2                      # workspace too small
    for name in ["x", "ids", "q", "sa", "off", "rows", "ws"]:
        assert call(**{name: None}) == 1, name
    assert call(x=X + 8) == 3 and call(q=Q + 4) == 3 and call(ids=SB + 2) == 3
    assert call(sa=SA + 2) == 3 and call(off=OFFS + 2) == 3 and call(ws=WS + 2) == 3
    # T = 0 needs no token pointers: with a misaligned m_offsets it reaches the
    # alignment check (valid T = 0 calls still write m_offsets; with real
    # buffers: test_gpu_moe.py::test_no_tokens_writes_zero_offsets)
    assert call(T=0, x=None, ids=None, rows=None, cap=L.fp8q_moe_dispatch_max_rows(0, 2, 4),
                wsb=L.fp8q_moe_dispatch_workspace_bytes(0, 2, 4), off=OFFS + 2) == 3


def test_gemm_ws_validation():
    L = _lib()
    need = L.fp8_gemm_blockscaled_ws_bytes(64, 7168, 7168)
    assert need > 0 and need % (64 * 7168 * 4) == 0
    assert L.fp8_gemm_blockscaled_ws_bytes(4096, 4096, 4096) == 0  # large M: no split
    assert L.fp8_gemm_blockscaled_ws_bytes(64, 100, 128) == -1
    f = L.fp8_gemm_blockscaled_ws
    W = P * 9
    assert f(A, SA, B, SB, C, 1, 64, 7168, 7168, None, need, None) == 1
    assert f(A, SA, B, SB, C, 1, 64, 7168, 7168, W, need - 16, None) == 2
    assert f(A, SA, B, SB, C, 1, 64, 7168, 7168, W + 4, need, None) == 3
    assert f(A, SA, B, SB, C, 1, 64, 100, 7168, W, need, None) == 2
    assert f(None, None, None, None, None, 0, 0, 128, 128, None, 0, None) == 0


def test_noalloc_gemm_validation():
    """Rejected before any HIP call, like fp8_gemm_blockscaled's checks."""
    L = _lib()
    f = L.fp8_gemm_blockscaled_noalloc
    assert f(A, SA, B, SB, C, 1, 64, 100, 7168, None) == 2   # N % 128
    assert f(A, SA, B, SB, C, 1, 64, 7168, 100, None) == 2   # K % 128
    assert f(A, SA, B, SB, C, 3, 64, 7168, 7168, None) == 4  # out dtype
    for i in range(5):
        args = [A, SA, B, SB, C]
        args[i] = None
        assert f(*args, 1, 64, 7168, 7168, None) == 1, i
    assert f(A + 8, SA, B, SB, C, 1, 64, 7168, 7168, None) == 3
    assert f(A, SA, B, SB, C, 1, 64, 7168, (1 << 23) + 128, None) == 7
    assert f(None, None, None, None, None, 1, 0, 7168, 7168, None) == 0  # M = 0: no-op


def test_noalloc_partials_never_exceed_the_static_scratch():
    """The split-K partials of every shape fit the library's 8 MiB: S splits
    of at most 256 / tiles, 64 x 128 tiles, 4 bytes per output per split."""
    L = _lib()
    worst = 0
    for M in [1, 16, 63, 64, 65, 96, 127, 128, 129, 192, 255, 256, 300, 511, 512]:
        for N in [128, 256, 1024, 2048, 4096, 7168, 8192, 16384, 32768]:
            for K in [2048, 4096, 7168, 16384]:
                worst = max(worst, L.fp8_gemm_blockscaled_ws_bytes(M, N, K))
    assert 0 < worst <= 8 << 20


def test_quant_on_load_gemm_validation():
    L = _lib()
    f = L.fp8_gemm_blockscaled_bf16a
    assert f(X, B, SB, C, 1, 64, 100, 128, None, None, None) == 2   # N % 128
    assert f(X, B, SB, C, 1, 64, 128, 100, None, None, None) == 2   # K % 128
    assert f(X, B, SB, C, 7, 64, 128, 128, None, None, None) == 4   # out dtype
    assert f(X, B, SB, None, 1, 64, 128, 128, None, None, None) == 1
    assert f(None, B, SB, C, 1, 64, 128, 128, None, None, None) == 1
    assert f(X, B, SB, C, 1, 64, 128, 128, Q, None, None) == 1      # codes without scales
    assert f(X + 8, B, SB, C, 1, 64, 128, 128, None, None, None) == 3
    assert f(X, B, SB, C, 1, 64, 128, 128, Q + 8, SA, None) == 3
    assert f(X, B, SB, C, 1, 64, 128, (1 << 23) + 128, None, None, None) == 7
    assert f(None, None, None, None, 1, 0, 128, 128, None, None, None) == 0
    # K == 0 reads no operand: without A, B and sb it reaches the check of C
    # (valid K = 0 calls zero-fill C; with a real C:
    # test_gpu_gemm_qa.py::test_k_zero_writes_zeros_and_m_zero_is_a_no_op)
    assert f(None, None, None, C + 8, 1, 64, 128, 0, None, None, None) == 3


def test_rowscaled_gemm_validation():
    L = _lib()
    f = L.fp8_gemm_rowscaled
    assert f(A, SA, B, SB, C, 0, 64, 100, 128, None) == 2
    assert f(A, SA, B, SB, C, 0, 64, 128, 100, None) == 2
    assert f(A, SA, B, SB, C, 5, 64, 128, 128, None) == 4
    for i in range(5):
        args = [A, SA, B, SB, C]
        args[i] = None
        assert f(*args, 0, 64, 128, 128, None) == 1, i
    assert f(A, SA, B, SB + 2, C, 0, 64, 128, 128, None) == 3
    assert f(A, SA, B, SB, C, 0, 64, 128, (1 << 23) + 128, None) == 7
    assert f(None, None, None, None, None, 0, 0, 128, 128, None) == 0


def test_binding_names_match_c_abi():
    import fp8_fine_grained_online_amd as pkg
    for name in ENTRY_POINTS:
        assert callable(getattr(pkg, name))


def test_oracle_and_hip_path_share_no_code():
    """Neither side imports the other; only the synthetic-input module is shared."""
    pkg_dir = os.path.join(ROOT, "fp8_fine_grained_online_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), fn
                assert "oracle/" not in text, fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", fn)).read()
            assert "fp8_fine_grained_online_amd" not in text, fn


def test_device_code_is_built_without_contraction_or_packed_fp32():
    """The kernels' roundings must happen as written (parity is bit-exact for
    codes), and packed FP32 VALU forms stay disabled."""
    from fp8_fine_grained_online_amd import build
    assert "-ffp-contract=off" in build.FLAGS
    i = build.FLAGS.index("-packed-fp32-ops")
    assert build.FLAGS[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
