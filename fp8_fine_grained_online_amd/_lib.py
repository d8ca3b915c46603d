"""ctypes binding of libfp8q.so: argument marshalling only."""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG_DIR, "libfp8q.so")

FP8Q_OUT_F32 = 0
FP8Q_OUT_BF16 = 1

STATUS = {
    0: "FP8Q_OK", 1: "FP8Q_ERR_NULL", 2: "FP8Q_ERR_SHAPE", 3: "FP8Q_ERR_ALIGN",
    4: "FP8Q_ERR_DTYPE", 5: "FP8Q_ERR_LAUNCH", 6: "FP8Q_ERR_NO_DEVICE", 7: "FP8Q_ERR_TOO_LARGE",
    8: "FP8Q_ERR_SCRATCH",
}

_lib = None


class Fp8qError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with `python -m fp8_fine_grained_online_amd.build`"
                " (there is no fallback path)")
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.fp8q_version.restype = i32
        L.fp8q_version.argtypes = []
        L.fp8q_status_string.restype = ctypes.c_char_p
        L.fp8q_status_string.argtypes = [i32]
        L.fp8q_quant_act_1x128.restype = i32
        L.fp8q_quant_act_1x128.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fp8q_quant_act_1x128_nt.restype = i32
        L.fp8q_quant_act_1x128_nt.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fp8q_quant_weight_128x128.restype = i32
        L.fp8q_quant_weight_128x128.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fp8_gemm_blockscaled.restype = i32
        L.fp8_gemm_blockscaled.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
        L.fp8_gemm_blockscaled_bf16a.restype = i32
        L.fp8_gemm_blockscaled_bf16a.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, vp, vp, vp]
        L.fp8_gemm_blockscaled_ws.restype = i32
        L.fp8_gemm_blockscaled_ws.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, i64, vp]
        L.fp8_gemm_blockscaled_noalloc.restype = i32
        L.fp8_gemm_blockscaled_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
        L.fp8_gemm_blockscaled_ws_bytes.restype = i64
        L.fp8_gemm_blockscaled_ws_bytes.argtypes = [i64, i64, i64]
        L.fp8_gemm_grouped.restype = i32
        L.fp8_gemm_grouped.argtypes = [vp, vp, vp, vp, vp, i32, vp, i64, i64, i64, i64, vp]
        L.fp8q_quant_act_128x1.restype = i32
        L.fp8q_quant_act_128x1.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fp8q_moe_dispatch_1x128.restype = i32
        L.fp8q_moe_dispatch_1x128.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, i64, vp, vp, vp,
                                              i64, vp]
        L.fp8q_moe_dispatch_workspace_bytes.restype = i64
        L.fp8q_moe_dispatch_workspace_bytes.argtypes = [i64, i64, i64]
        L.fp8q_moe_dispatch_max_rows.restype = i64
        L.fp8q_moe_dispatch_max_rows.argtypes = [i64, i64, i64]
        L.fp8q_norm_quant_act_1x128.restype = i32
        L.fp8q_norm_quant_act_1x128.argtypes = [vp, vp, vp, ctypes.c_float, i32, i64, i64, vp, vp, vp]
        L.fp8q_quant_act_1x128_128x1.restype = i32
        L.fp8q_quant_act_1x128_128x1.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
        L.fp8q_requant_1x128_to_128x1.restype = i32
        L.fp8q_requant_1x128_to_128x1.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.fp8q_transpose_weight_128x128.restype = i32
        L.fp8q_transpose_weight_128x128.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.fp8_gemm_rowscaled.restype = i32
        L.fp8_gemm_rowscaled.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
        _lib = L
    return _lib


def fp8q_version() -> int:
    return lib().fp8q_version()


def _check(fn, status):
    if status != 0:
        raise Fp8qError(fn, status, lib().fp8q_status_string(status).decode())


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out(t, name, shape, dtype, device):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def fp8q_quant_act_1x128(x, q=None, sa=None, stream=None):
    """x: bf16 M x K device tensor -> (q uint8 M x K, sa float32 M x K/128)."""
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x.device)
    sa = _out(sa, "sa", (M, K // 128 if K % 128 == 0 else 0), torch.float32, x.device)
    _check("fp8q_quant_act_1x128",
           lib().fp8q_quant_act_1x128(px, M, K, q.data_ptr(), sa.data_ptr(), _stream(stream)))
    return q, sa


def fp8q_quant_act_1x128_nt(x, q=None, sa=None, stream=None):
    """fp8q_quant_act_1x128 with non-temporal stores (same results; for codes
    that are not read next on this GPU)."""
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x.device)
    sa = _out(sa, "sa", (M, K // 128 if K % 128 == 0 else 0), torch.float32, x.device)
    _check("fp8q_quant_act_1x128_nt",
           lib().fp8q_quant_act_1x128_nt(px, M, K, q.data_ptr(), sa.data_ptr(), _stream(stream)))
    return q, sa


def fp8q_quant_weight_128x128(w, q=None, sb=None, stream=None):
    """w: bf16 N x K (or G x N x K) device tensor -> (q uint8 like w, sb float32 .../128 x K/128)."""
    torch = _torch()
    if w.dim() == 3:
        G, N, K = w.shape
        q = _out(q, "q", (G, N, K), torch.uint8, w.device)
        sb = _out(sb, "sb", (G, N // 128, K // 128), torch.float32, w.device)
        _dev(w, "w", torch.bfloat16, 3)
        rows = G * N
    else:
        _dev(w, "w", torch.bfloat16, 2)
        N, K = w.shape
        q = _out(q, "q", (N, K), torch.uint8, w.device)
        sb = _out(sb, "sb", (N // 128, K // 128), torch.float32, w.device)
        rows = N
    if w.dim() == 3 and N % 128:
        raise ValueError("per-expert N must be a multiple of 128")
    _check("fp8q_quant_weight_128x128",
           lib().fp8q_quant_weight_128x128(w.data_ptr(), rows, K, q.data_ptr(), sb.data_ptr(),
                                           _stream(stream)))
    return q, sb


def _out_dtype(out_dtype):
    torch = _torch()
    if out_dtype in (torch.bfloat16, "bf16", FP8Q_OUT_BF16):
        return FP8Q_OUT_BF16, torch.bfloat16
    if out_dtype in (torch.float32, "f32", FP8Q_OUT_F32):
        return FP8Q_OUT_F32, torch.float32
    raise ValueError(f"unsupported out_dtype {out_dtype}")


def fp8_gemm_blockscaled(a, sa, b, sb, out_dtype="bf16", c=None, stream=None):
    """C = A * B^T with per-1x128 (sa) and per-128x128 (sb) scales. Returns c (M x N)."""
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    pa = _dev(a, "a", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    pb = _dev(b, "b", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if K % 128 == 0 and N % 128 == 0:
        if tuple(sa.shape) != (M, K // 128) or tuple(sb.shape) != (N // 128, K // 128):
            raise ValueError("scale shapes must be (M, K/128) and (N/128, K/128)")
    c = _out(c, "c", (M, N), tdt, a.device)
    _check("fp8_gemm_blockscaled",
           lib().fp8_gemm_blockscaled(pa, psa, pb, psb, c.data_ptr(), code, M, N, K,
                                      _stream(stream)))
    return c


def fp8_gemm_blockscaled_bf16a(a, b, sb, out_dtype="bf16", c=None, qa=None, sa=None,
                               with_codes=False, stream=None):
    """Quantize-on-load GEMM: a is bf16 M x K, quantized to 1x128 tiles inside
    the GEMM. Returns c, or (c, qa, sa) with with_codes (A's codes and scales,
    as fp8q_quant_act_1x128 gives them)."""
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    pa = _dev(a, "a", torch.bfloat16, 2)
    pb = _dev(b, "b", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if K % 128 == 0 and N % 128 == 0 and tuple(sb.shape) != (N // 128, K // 128):
        raise ValueError("sb must have shape (N/128, K/128)")
    c = _out(c, "c", (M, N), tdt, a.device)
    pq = ps = None
    if with_codes or qa is not None or sa is not None:
        qa = _out(qa, "qa", (M, K), torch.uint8, a.device)
        sa = _out(sa, "sa", (M, K // 128), torch.float32, a.device)
        pq, ps = qa.data_ptr(), sa.data_ptr()
    _check("fp8_gemm_blockscaled_bf16a",
           lib().fp8_gemm_blockscaled_bf16a(pa, pb, psb, c.data_ptr(), code, M, N, K, pq, ps,
                                            _stream(stream)))
    return (c, qa, sa) if pq is not None else c


def fp8_gemm_blockscaled_ws(a, sa, b, sb, out_dtype="bf16", c=None, workspace=None, stream=None):
    """fp8_gemm_blockscaled with a workspace (split-K for small-M shapes).
    The workspace (uint8 device tensor) is allocated when not given."""
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    pa = _dev(a, "a", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    pb = _dev(b, "b", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if K % 128 == 0 and N % 128 == 0:
        if tuple(sa.shape) != (M, K // 128) or tuple(sb.shape) != (N // 128, K // 128):
            raise ValueError("scale shapes must be (M, K/128) and (N/128, K/128)")
    c = _out(c, "c", (M, N), tdt, a.device)
    need = lib().fp8_gemm_blockscaled_ws_bytes(M, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
    pw = workspace.data_ptr() if workspace is not None else None
    nw = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("fp8_gemm_blockscaled_ws",
           lib().fp8_gemm_blockscaled_ws(pa, psa, pb, psb, c.data_ptr(), code, M, N, K, pw, nw,
                                         _stream(stream)))
    return c


def _grouped_shapes(a, sa, b, sb, m_offsets, M_total):
    """Shape checks of the grouped GEMM's operands (before any device access):
    the kernel indexes expert e's block scales at sb + e * (N/128) * (K/128), so
    sb must be exactly G x N/128 x K/128 for the b it goes with."""
    if b.dim() != 3 or a.dim() != 2 or sa.dim() != 2 or sb.dim() != 3 or m_offsets.dim() != 1:
        raise ValueError("a, sa: 2 dims; b, sb: 3 dims; m_offsets: 1 dim")
    G, N, K = b.shape
    if m_offsets.shape[0] != G + 1:
        raise ValueError("m_offsets must have G+1 entries")
    M = a.shape[0] if M_total is None else int(M_total)
    if a.shape[1] != K or a.shape[0] < M:
        raise ValueError("a must be at least M_total x K")
    if K % 128 == 0 and N % 128 == 0:
        if sa.shape[0] < M or sa.shape[1] != K // 128:
            raise ValueError("sa must be at least M_total x K/128")
        if tuple(sb.shape) != (G, N // 128, K // 128):
            raise ValueError(f"sb must have shape {(G, N // 128, K // 128)}, got {tuple(sb.shape)}")
    return G, N, K, M


def fp8_gemm_blockscaled_noalloc(a, sa, b, sb, out_dtype="bf16", c=None, stream=None):
    """fp8_gemm_blockscaled_ws with the split-K partials in the library's
    static per-GPU scratch (no workspace; pass c to allocate nothing at all)."""
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    pa = _dev(a, "a", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    pb = _dev(b, "b", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if K % 128 == 0 and N % 128 == 0:
        if tuple(sa.shape) != (M, K // 128) or tuple(sb.shape) != (N // 128, K // 128):
            raise ValueError("scale shapes must be (M, K/128) and (N/128, K/128)")
    c = _out(c, "c", (M, N), tdt, a.device)
    _check("fp8_gemm_blockscaled_noalloc",
           lib().fp8_gemm_blockscaled_noalloc(pa, psa, pb, psb, c.data_ptr(), code, M, N, K,
                                              _stream(stream)))
    return c


def fp8_gemm_grouped(a, sa, b, sb, m_offsets, out_dtype="bf16", c=None, M_total=None, stream=None):
    """Grouped GEMM. b: G x N x K codes, sb: G x N/128 x K/128, m_offsets: int32[G+1] device.

    M_total defaults to a.shape[0] (the host-side row count; m_offsets is never
    read on the host).
    """
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    G, N, K, M = _grouped_shapes(a, sa, b, sb, m_offsets, M_total)
    pa = _dev(a, "a", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    pb = _dev(b, "b", torch.uint8, 3)
    psb = _dev(sb, "sb", torch.float32, 3)
    poff = _dev(m_offsets, "m_offsets", torch.int32, 1)
    c = _out(c, "c", (M, N), tdt, a.device)
    _check("fp8_gemm_grouped",
           lib().fp8_gemm_grouped(pa, psa, pb, psb, c.data_ptr(), code, poff, G, M, N, K,
                                  _stream(stream)))
    return c


def _div128(n):
    return n // 128 if n % 128 == 0 else 0


def fp8q_quant_act_128x1(x, qt=None, st=None, stream=None):
    """x: bf16 M x K device tensor -> (qt uint8 K x M, st float32 K x M/128): 128x1 tiles, transposed."""
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    qt = _out(qt, "qt", (K, M), torch.uint8, x.device)
    st = _out(st, "st", (K, _div128(M)), torch.float32, x.device)
    _check("fp8q_quant_act_128x1",
           lib().fp8q_quant_act_128x1(px, M, K, qt.data_ptr(), st.data_ptr(), _stream(stream)))
    return qt, st


def fp8q_moe_dispatch_1x128(x, topk_ids, G, q=None, sa=None, m_offsets=None, row_of_slot=None,
                            workspace=None, stream=None):
    """FP8 dispatch: x bf16 T x K, topk_ids int32 T x topk (device) ->
    (q uint8 M_cap x K, sa float32 M_cap x K/128, m_offsets int32[G+1], row_of_slot int32 T x topk).

    M_cap = fp8q_moe_dispatch_max_rows(T, topk, G); only rows below m_offsets[G]
    are written. Pass q.shape[0] as M_total to fp8_gemm_grouped (no host sync).
    """
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    pid = _dev(topk_ids, "topk_ids", torch.int32, 2)
    T, K = x.shape
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must have one row per token")
    topk = topk_ids.shape[1]
    L = lib()
    M_cap = L.fp8q_moe_dispatch_max_rows(T, topk, G)
    ws_bytes = L.fp8q_moe_dispatch_workspace_bytes(T, topk, G)
    if M_cap < 0 or ws_bytes < 0:
        raise ValueError("invalid dispatch sizes")
    q = _out(q, "q", (M_cap, K), torch.uint8, x.device)
    sa = _out(sa, "sa", (M_cap, _div128(K)), torch.float32, x.device)
    m_offsets = _out(m_offsets, "m_offsets", (G + 1,), torch.int32, x.device)
    row_of_slot = _out(row_of_slot, "row_of_slot", (T, topk), torch.int32, x.device)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=x.device)
    _check("fp8q_moe_dispatch_1x128",
           L.fp8q_moe_dispatch_1x128(px, pid, T, K, topk, G, q.data_ptr(), sa.data_ptr(), M_cap,
                                     m_offsets.data_ptr(), row_of_slot.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return q, sa, m_offsets, row_of_slot


def fp8q_norm_quant_act_1x128(x, gamma, eps, beta=None, centred=False, q=None, sa=None,
                              stream=None):
    """Normalize rows of x (bf16 M x K; RMS, or centred with beta) and quantize the
    binary32 result per 1x128 tile -> (q uint8 M x K, sa float32 M x K/128)."""
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    pg = _dev(gamma, "gamma", torch.bfloat16, 1)
    pb = _dev(beta, "beta", torch.bfloat16, 1) if beta is not None else None
    M, K = x.shape
    if gamma.shape[0] != K or (beta is not None and beta.shape[0] != K):
        raise ValueError("gamma and beta must have K entries")
    q = _out(q, "q", (M, K), torch.uint8, x.device)
    sa = _out(sa, "sa", (M, _div128(K)), torch.float32, x.device)
    _check("fp8q_norm_quant_act_1x128",
           lib().fp8q_norm_quant_act_1x128(px, pg, pb, float(eps), int(bool(centred)), M, K,
                                           q.data_ptr(), sa.data_ptr(), _stream(stream)))
    return q, sa


def fp8q_quant_act_1x128_128x1(x, q=None, sa=None, qt=None, st=None, stream=None):
    """x: bf16 M x K -> (q M x K, sa M x K/128, qt K x M, st K x M/128): both tilings, one read."""
    torch = _torch()
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = _out(q, "q", (M, K), torch.uint8, x.device)
    sa = _out(sa, "sa", (M, _div128(K)), torch.float32, x.device)
    qt = _out(qt, "qt", (K, M), torch.uint8, x.device)
    st = _out(st, "st", (K, _div128(M)), torch.float32, x.device)
    _check("fp8q_quant_act_1x128_128x1",
           lib().fp8q_quant_act_1x128_128x1(px, M, K, q.data_ptr(), sa.data_ptr(), qt.data_ptr(),
                                            st.data_ptr(), _stream(stream)))
    return q, sa, qt, st


def fp8q_requant_1x128_to_128x1(q, sa, qt=None, st=None, stream=None):
    """Stored 1x128 codes q (M x K) and sa (M x K/128) -> (qt K x M, st K x M/128)."""
    torch = _torch()
    pq = _dev(q, "q", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    M, K = q.shape
    if tuple(sa.shape) != (M, _div128(K)):
        raise ValueError("sa must have shape (M, K/128)")
    qt = _out(qt, "qt", (K, M), torch.uint8, q.device)
    st = _out(st, "st", (K, _div128(M)), torch.float32, q.device)
    _check("fp8q_requant_1x128_to_128x1",
           lib().fp8q_requant_1x128_to_128x1(pq, psa, M, K, qt.data_ptr(), st.data_ptr(),
                                             _stream(stream)))
    return qt, st


def fp8q_transpose_weight_128x128(q, sb, qt=None, sbt=None, stream=None):
    """Weight codes q (N x K) and block scales sb (N/128 x K/128) -> (qt K x N, sbt K/128 x N/128)."""
    torch = _torch()
    pq = _dev(q, "q", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    N, K = q.shape
    if tuple(sb.shape) != (_div128(N), _div128(K)):
        raise ValueError("sb must have shape (N/128, K/128)")
    qt = _out(qt, "qt", (K, N), torch.uint8, q.device)
    sbt = _out(sbt, "sbt", (_div128(K), _div128(N)), torch.float32, q.device)
    _check("fp8q_transpose_weight_128x128",
           lib().fp8q_transpose_weight_128x128(pq, psb, N, K, qt.data_ptr(), sbt.data_ptr(),
                                               _stream(stream)))
    return qt, sbt


def fp8_gemm_rowscaled(a, sa, b, sb, out_dtype="f32", c=None, stream=None):
    """C = A * B^T with 1x128 scales on both operands: sa (M x K/128), sb (N x K/128)."""
    torch = _torch()
    code, tdt = _out_dtype(out_dtype)
    pa = _dev(a, "a", torch.uint8, 2)
    psa = _dev(sa, "sa", torch.float32, 2)
    pb = _dev(b, "b", torch.uint8, 2)
    psb = _dev(sb, "sb", torch.float32, 2)
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b must share K")
    if K % 128 == 0:
        if tuple(sa.shape) != (M, K // 128) or tuple(sb.shape) != (N, K // 128):
            raise ValueError("scale shapes must be (M, K/128) and (N, K/128)")
    c = _out(c, "c", (M, N), tdt, a.device)
    _check("fp8_gemm_rowscaled",
           lib().fp8_gemm_rowscaled(pa, psa, pb, psb, c.data_ptr(), code, M, N, K, _stream(stream)))
    return c
