"""MI355X (gfx950) MoE FP8 training hot path: fused FP8 quantization and scaled grouped GEMM.

Thin ctypes binding over the C ABI in ``include/fp8_quant_grouped.h`` (library
``libfp8qg.so`` next to this file, built by ``_build.build()``).  Each Python function has the
name of the C entry point it calls and only marshals arguments: it takes torch tensors for
device memory, allocates outputs with torch on the input's device, passes raw pointers and the
current HIP stream, and raises on a non-zero status.  Every step of the computation runs in
the HIP kernels; there is no fallback.  If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8qg.so")

E4M3FNUZ = 0  # AMD e4m3fnuz: largest value 240
E4M3FN = 1    # OCP e4m3fn: largest value 448
FMAX = {E4M3FNUZ: 240.0, E4M3FN: 448.0}
GEMM_FWD_MGROUPED = 0
GEMM_WGRAD_KGROUPED = 1
OUT_BF16 = 0
OUT_FP32 = 1

_lib = None

# name -> (restype, argtypes)
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_I = ctypes.c_int
SIGNATURES = {
    "fp8q_abi_version": (_I, []),
    "fp8q_status_string": (ctypes.c_char_p, [_I]),
    "fp8_abi_version": (_I, []),
    "fp8_status_string": (ctypes.c_char_p, [_I]),
    "fp8_grouped_gemm_workspace_size": (_SZ, [_I, _I64, _I64, _I64, _I32]),
    "fp8_quant_rowwise": (_I, [_P, _I64, _I64, _I64, _I, _P, _I64, _P, _P]),
    "fp8_quant_rowwise_gather": (_I, [_P, _I64, _I64, _I64, _P, _I64, _I, _P, _I64, _P, _P]),
    "fp8_quant_colwise_grouped_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "fp8_quant_colwise_grouped": (_I, [_P, _I64, _I64, _I64, _P, _I32, _I, _P, _I64, _P, _P, _SZ,
                                       _P]),
    "fp8_quant_dual_grouped_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "fp8_quant_dual_grouped": (_I, [_P, _I64, _I64, _I64, _P, _I32, _I, _P, _I64, _P, _P, _I64, _P,
                                    _P, _SZ, _P]),
    "fp8_quant_colwise_grouped_noalloc": (_I, [_P, _I64, _I64, _I64, _P, _I32, _I, _P, _I64, _P,
                                               _P]),
    "fp8_quant_weights_dual_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "fp8_quant_weights_dual": (_I, [_P, _I64, _I64, _I64, _I64, _I, _P, _I64, _P, _P, _I64, _P, _P,
                                    _SZ, _P]),
    "fp8_grouped_gemm": (_I, [_I, _I, _P, _I64, _P, _P, _I64, _I64, _P, _P, _I32, _I64, _I64,
                              _I64, _P, _I64, _I, _P, _SZ, _P]),
    "fp8_mx_quant_rowwise": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_mx_quant_colwise": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P]),
    "fp8_mx_grouped_gemm": (_I, [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _I64, _I64, _P, _I32,
                                 _I64, _I64, _I64, _P, _I64, _I, _P, _SZ, _P]),
    "fp8_mx_grouped_gemm_wgrad": (_I, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _P, _I32, _I64,
                                       _I64, _I64, _P, _I64, _I, _P, _SZ, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "fp8_quantization_grouped_amd._build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(name: str, status: int) -> None:
    if status != 0:
        msg = lib().fp8q_status_string(status).decode()
        raise RuntimeError(f"{name} failed: status {status} ({msg})")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, what: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")


def fp8_quant_rowwise(x: torch.Tensor, fmt: int, q: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None):
    """x: bf16 [rows, cols] (row stride may exceed cols).  Returns (q uint8 [rows, cols],
    scales float32 [rows])."""
    _dev(x, "x")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=x.device)
    st = lib().fp8_quant_rowwise(_ptr(x), rows, cols, x.stride(0), fmt, _ptr(q), q.stride(0),
                                 _ptr(scales), _stream(x))
    _check("fp8_quant_rowwise", st)
    return q, scales


def fp8_quant_rowwise_gather(x: torch.Tensor, row_index: torch.Tensor, fmt: int,
                             q: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    """Rowwise quantization of the rows x[row_index[r]] (indices clamped into range).
    x: bf16 [src_rows, cols]; row_index: int32 [rows] on the device.  Returns (q uint8
    [rows, cols], scales float32 [rows])."""
    _dev(x, "x")
    _dev(row_index, "row_index")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert row_index.dtype == torch.int32 and row_index.dim() == 1 and row_index.is_contiguous()
    src_rows, cols = x.shape
    rows = row_index.numel()
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows,), dtype=torch.float32, device=x.device)
    st = lib().fp8_quant_rowwise_gather(_ptr(x), src_rows, cols, x.stride(0), _ptr(row_index),
                                        rows, fmt, _ptr(q), q.stride(0), _ptr(scales), _stream(x))
    _check("fp8_quant_rowwise_gather", st)
    return q, scales


def fp8_quant_colwise_grouped_workspace_size(rows: int, cols: int, groups: int) -> int:
    return int(lib().fp8_quant_colwise_grouped_workspace_size(rows, cols, groups))


def fp8_quant_colwise_grouped(x: torch.Tensor, offsets: torch.Tensor, fmt: int,
                              q_t: torch.Tensor | None = None,
                              scales: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None):
    """x: bf16 [rows, cols]; offsets: int32 device [groups] (cumulative group ends).
    Returns (q_t uint8 [cols, rows] column-major copy, scales float32 [groups, cols])."""
    _dev(x, "x")
    _dev(offsets, "offsets")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert offsets.dtype == torch.int32 and offsets.is_contiguous()
    rows, cols = x.shape
    groups = offsets.numel()
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((groups, cols), dtype=torch.float32, device=x.device)
    need = fp8_quant_colwise_grouped_workspace_size(rows, cols, groups)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    st = lib().fp8_quant_colwise_grouped(_ptr(x), rows, cols, x.stride(0), _ptr(offsets), groups,
                                         fmt, _ptr(q_t), q_t.stride(0), _ptr(scales),
                                         _ptr(workspace), workspace.numel(), _stream(x))
    _check("fp8_quant_colwise_grouped", st)
    return q_t, scales


def fp8_quant_dual_grouped_workspace_size(rows: int, cols: int, groups: int) -> int:
    return int(lib().fp8_quant_dual_grouped_workspace_size(rows, cols, groups))


def fp8_quant_dual_grouped(x: torch.Tensor, offsets: torch.Tensor, fmt: int,
                           q: torch.Tensor | None = None, s_rows: torch.Tensor | None = None,
                           q_t: torch.Tensor | None = None, s_cols: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None):
    """Both layouts of x [rows, cols] at once: returns ((q uint8 [rows, cols], s_rows float32
    [rows]) as fp8_quant_rowwise would, (q_t uint8 [cols, rows], s_cols float32 [groups, cols])
    as fp8_quant_colwise_grouped with these token offsets would)."""
    _dev(x, "x")
    _dev(offsets, "offsets")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert offsets.dtype == torch.int32 and offsets.is_contiguous()
    rows, cols = x.shape
    groups = offsets.numel()
    e = lambda *s, dt=torch.uint8: torch.empty(s, dtype=dt, device=x.device)
    q = e(rows, cols) if q is None else q
    s_rows = e(rows, dt=torch.float32) if s_rows is None else s_rows
    q_t = e(cols, rows) if q_t is None else q_t
    s_cols = e(groups, cols, dt=torch.float32) if s_cols is None else s_cols
    need = fp8_quant_dual_grouped_workspace_size(rows, cols, groups)
    if workspace is None:
        workspace = e(max(need, 256))
    st = lib().fp8_quant_dual_grouped(_ptr(x), rows, cols, x.stride(0), _ptr(offsets), groups, fmt,
                                      _ptr(q), q.stride(0), _ptr(s_rows), _ptr(q_t), q_t.stride(0),
                                      _ptr(s_cols), _ptr(workspace), workspace.numel(), _stream(x))
    _check("fp8_quant_dual_grouped", st)
    return (q, s_rows), (q_t, s_cols)


def fp8_quant_colwise_grouped_noalloc(x: torch.Tensor, offsets: torch.Tensor, fmt: int,
                                      q_t: torch.Tensor | None = None,
                                      scales: torch.Tensor | None = None):
    """fp8_quant_colwise_grouped through the entry point that allocates nothing (its maxima
    live in the library's static per-GPU array; sizes beyond it raise).  The C call allocates
    nothing; pass q_t and scales to allocate nothing here either."""
    _dev(x, "x")
    _dev(offsets, "offsets")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert offsets.dtype == torch.int32 and offsets.is_contiguous()
    rows, cols = x.shape
    groups = offsets.numel()
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((groups, cols), dtype=torch.float32, device=x.device)
    st = lib().fp8_quant_colwise_grouped_noalloc(_ptr(x), rows, cols, x.stride(0), _ptr(offsets),
                                                 groups, fmt, _ptr(q_t), q_t.stride(0),
                                                 _ptr(scales), _stream(x))
    _check("fp8_quant_colwise_grouped_noalloc", st)
    return q_t, scales


def fp8_quant_weights_dual_workspace_size(experts: int, K: int, N: int) -> int:
    return int(lib().fp8_quant_weights_dual_workspace_size(experts, K, N))


def fp8_quant_weights_dual(w: torch.Tensor, experts: int, fmt: int,
                           q_rows: torch.Tensor | None = None,
                           s_rows: torch.Tensor | None = None,
                           q_t: torch.Tensor | None = None, s_cols: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None):
    """Expert weights w: bf16 [experts*K, N] in both layouts at once.  Returns
    (q_rows uint8 [experts*K, N], s_rows float32 [experts*K]) as fp8_quant_rowwise would and
    (q_t uint8 [N, experts*K], s_cols float32 [experts, N]) as fp8_quant_colwise_grouped with
    offsets K, 2K, .. would."""
    _dev(w, "w")
    assert w.dtype == torch.bfloat16 and w.dim() == 2 and w.stride(1) == 1
    rows, N = w.shape
    assert experts > 0 and rows % experts == 0
    K = rows // experts
    if q_rows is None:
        q_rows = torch.empty((rows, N), dtype=torch.uint8, device=w.device)
    if s_rows is None:
        s_rows = torch.empty((rows,), dtype=torch.float32, device=w.device)
    if q_t is None:
        q_t = torch.empty((N, rows), dtype=torch.uint8, device=w.device)
    if s_cols is None:
        s_cols = torch.empty((experts, N), dtype=torch.float32, device=w.device)
    need = fp8_quant_weights_dual_workspace_size(experts, K, N)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=w.device)
    st = lib().fp8_quant_weights_dual(_ptr(w), experts, K, N, w.stride(0), fmt, _ptr(q_rows),
                                      q_rows.stride(0), _ptr(s_rows), _ptr(q_t), q_t.stride(0),
                                      _ptr(s_cols), _ptr(workspace), workspace.numel(),
                                      _stream(w))
    _check("fp8_quant_weights_dual", st)
    return (q_rows, s_rows), (q_t, s_cols)


def fp8_grouped_gemm_workspace_size(mode: int, M: int, N: int, K: int, groups: int) -> int:
    return int(lib().fp8_grouped_gemm_workspace_size(mode, M, N, K, groups))


_OUT = {torch.bfloat16: OUT_BF16, torch.float32: OUT_FP32}


def _gemm_out(c, shape, out_dtype, dev):
    if c is None:
        c = torch.empty(shape, dtype=out_dtype, device=dev)
    if c.dtype not in _OUT:
        raise ValueError("the GEMM output must be bfloat16 or float32")
    if c.dim() != len(shape) or tuple(c.shape) != tuple(shape) or c.stride(-1) != 1:
        raise ValueError(f"the GEMM output must be {tuple(shape)} with unit column stride")
    if len(shape) == 3 and c.stride(0) != shape[1] * c.stride(1):
        raise ValueError("a weight-gradient output's group stride must be K * ldc")
    return c


def _gemm_ws(workspace, mode, M, N, K, groups, dev):
    need = fp8_grouped_gemm_workspace_size(mode, M, N, K, groups)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    return workspace


def gemm_offsets_status(workspace: torch.Tensor):
    """The offsets check a grouped GEMM wrote into its workspace: (status, first bad group);
    (0, -1) for valid offsets.  Synchronises with the device to read it."""
    w = workspace[:8].view(torch.int32).cpu()
    return int(w[0]), int(w[1])


def fp8_grouped_gemm(mode: int, fmt: int, a: torch.Tensor, a_scales: torch.Tensor,
                     b: torch.Tensor, b_scales: torch.Tensor, offsets: torch.Tensor, M: int,
                     N: int, K: int, ldb: int | None = None, b_group_stride: int = 0,
                     c: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                     workspace: torch.Tensor | None = None):
    """Scaled FP8 grouped GEMM (see the C header for the two modes).
    Forward: a [M, lda], b holds every group's [N, K] rows at ldb / b_group_stride; returns
    [M, N].  Weight gradient: a [K, lda >= M], b [N, ldb >= M]; returns [G, K, N].  The output
    is bfloat16 or float32 (out_dtype, or the dtype of a given c)."""
    _dev(a, "a")
    groups = offsets.numel()
    if ldb is None:
        ldb = b.stride(0)
    shape = (M, N) if mode == GEMM_FWD_MGROUPED else (groups, K, N)
    c = _gemm_out(c, shape, out_dtype, a.device)
    ws = _gemm_ws(workspace, mode, M, N, K, groups, a.device)
    st = lib().fp8_grouped_gemm(mode, fmt, _ptr(a), a.stride(0), _ptr(a_scales), _ptr(b), ldb,
                                b_group_stride, _ptr(b_scales), _ptr(offsets), groups, M, N, K,
                                _ptr(c), c.stride(-2), _OUT[c.dtype], _ptr(ws), ws.numel(),
                                _stream(a))
    _check("fp8_grouped_gemm", st)
    return c


def fp8_mx_quant_rowwise(x: torch.Tensor, q: torch.Tensor | None = None,
                         e8m0: torch.Tensor | None = None):
    """Returns (q uint8 [rows, cols] OCP e4m3fn, e8m0 uint8 [rows, cols/32])."""
    _dev(x, "x")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    st = lib().fp8_mx_quant_rowwise(_ptr(x), rows, cols, x.stride(0), _ptr(q), q.stride(0),
                                    _ptr(e8m0), e8m0.stride(0), _stream(x))
    _check("fp8_mx_quant_rowwise", st)
    return q, e8m0


def fp8_mx_quant_colwise(x: torch.Tensor, q_t: torch.Tensor | None = None,
                         e8m0: torch.Tensor | None = None):
    """Blocks of 32 rows per column, transposed output.  Returns (q_t uint8 [cols, rows],
    e8m0 uint8 [cols, rows/32])."""
    _dev(x, "x")
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    rows, cols = x.shape
    if q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    if e8m0 is None:
        e8m0 = torch.empty((cols, rows // 32), dtype=torch.uint8, device=x.device)
    st = lib().fp8_mx_quant_colwise(_ptr(x), rows, cols, x.stride(0), _ptr(q_t), q_t.stride(0),
                                    _ptr(e8m0), e8m0.stride(0), _stream(x))
    _check("fp8_mx_quant_colwise", st)
    return q_t, e8m0


def fp8_mx_grouped_gemm(a: torch.Tensor, a_e8m0: torch.Tensor, b: torch.Tensor,
                        b_e8m0: torch.Tensor, offsets: torch.Tensor, M: int, N: int, K: int,
                        ldb: int, b_group_stride: int, ld_sb: int, sb_group_stride: int,
                        c: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                        workspace: torch.Tensor | None = None):
    """MX grouped GEMM forward; returns [M, N] (bfloat16 or float32)."""
    _dev(a, "a")
    groups = offsets.numel()
    c = _gemm_out(c, (M, N), out_dtype, a.device)
    ws = _gemm_ws(workspace, GEMM_FWD_MGROUPED, M, N, K, groups, a.device)
    st = lib().fp8_mx_grouped_gemm(_ptr(a), a.stride(0), _ptr(a_e8m0), a_e8m0.stride(0), _ptr(b),
                                   ldb, b_group_stride, _ptr(b_e8m0), ld_sb, sb_group_stride,
                                   _ptr(offsets), groups, M, N, K, _ptr(c), c.stride(0),
                                   _OUT[c.dtype], _ptr(ws), ws.numel(), _stream(a))
    _check("fp8_mx_grouped_gemm", st)
    return c


def fp8_mx_grouped_gemm_wgrad(a: torch.Tensor, a_e8m0: torch.Tensor, b: torch.Tensor,
                              b_e8m0: torch.Tensor, offsets: torch.Tensor, M: int, N: int,
                              K: int, c: torch.Tensor | None = None, out_dtype=torch.bfloat16,
                              workspace: torch.Tensor | None = None):
    """MX weight gradient: a = XqT [K, lda >= M], b = dYqT [N, ldb >= M] with E8M0 per 32
    tokens (fp8_mx_quant_colwise outputs).  Returns [G, K, N] (bfloat16 or float32)."""
    _dev(a, "a")
    groups = offsets.numel()
    c = _gemm_out(c, (groups, K, N), out_dtype, a.device)
    ws = _gemm_ws(workspace, GEMM_WGRAD_KGROUPED, M, N, K, groups, a.device)
    st = lib().fp8_mx_grouped_gemm_wgrad(_ptr(a), a.stride(0), _ptr(a_e8m0), a_e8m0.stride(0),
                                         _ptr(b), b.stride(0), _ptr(b_e8m0), b_e8m0.stride(0),
                                         _ptr(offsets), groups, M, N, K, _ptr(c), c.stride(-2),
                                         _OUT[c.dtype], _ptr(ws), ws.numel(), _stream(a))
    _check("fp8_mx_grouped_gemm_wgrad", st)
    return c
