"""CPU oracle for the MoE FP8 quantize + grouped GEMM hot path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``, never by the GPU library or its Python binding.  The
arithmetic lives in ``fp8_oracle.c`` (plain C, fp32 quantization chain, exact fp64 GEMM sums);
this module builds it with gcc and marshals numpy arrays through ctypes, and adds whole-matrix
GEMMs (below) that use a float64 library matmul as their summation step.

Every function here has a pin in ``tests/test_oracle_pins.py`` except where its docstring says
otherwise.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FNUZ = 0  # e4m3fnuz, max 240
FN = 1    # OCP e4m3fn, max 448

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int32
    I = ctypes.c_int
    lib.or_fmax.restype = ctypes.c_float
    lib.or_fmax.argtypes = [I]
    lib.or_decode.restype = ctypes.c_double
    lib.or_decode.argtypes = [I, ctypes.c_uint]
    lib.or_encode.restype = ctypes.c_uint
    lib.or_encode.argtypes = [I, ctypes.c_float]
    lib.or_encode_array.restype = None
    lib.or_encode_array.argtypes = [I, P, I64, P]
    lib.or_scale.restype = ctypes.c_float
    lib.or_scale.argtypes = [I, ctypes.c_float]
    lib.or_f64_to_bf16.restype = ctypes.c_uint16
    lib.or_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.or_quant_rowwise.restype = None
    lib.or_quant_rowwise.argtypes = [P, I64, I64, I64, I, P, I64, P]
    lib.or_quant_colwise_grouped.restype = None
    lib.or_quant_colwise_grouped.argtypes = [P, I64, I64, I64, P, I32, I, P, I64, P]
    lib.or_gemm_fwd_rows.restype = None
    lib.or_gemm_fwd_rows.argtypes = [I, P, I64, P, P, I64, I64, P, P, I32, I64, I64, P, I64, P]
    lib.or_gemm_wgrad_rows.restype = None
    lib.or_gemm_wgrad_rows.argtypes = [I, P, I64, P, P, I64, P, P, I32, I64, I64, P, P, I64, P]
    lib.or_mx_quant_rowwise.restype = None
    lib.or_mx_quant_rowwise.argtypes = [P, I64, I64, I64, P, I64, P, I64]
    lib.or_mx_quant_colwise.restype = None
    lib.or_mx_quant_colwise.argtypes = [P, I64, I64, I64, P, I64, P, I64]
    lib.or_mx_gemm_fwd_rows.restype = None
    lib.or_mx_gemm_fwd_rows.argtypes = [P, I64, P, I64, P, I64, I64, P, I64, I64, P, I32, I64,
                                        I64, P, I64, P]
    lib.or_mx_gemm_wgrad_rows.restype = None
    lib.or_mx_gemm_wgrad_rows.argtypes = [P, I64, P, I64, P, I64, P, I64, P, I32, I64, P, P, I64,
                                          P]
    lib.or_num_threads.restype = ctypes.c_int
    lib.or_num_threads.argtypes = []
    lib.or_set_num_threads.restype = None
    lib.or_set_num_threads.argtypes = [I]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().or_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls."""
    _load().or_set_num_threads(int(n))


def fmax(fmt: int) -> float:
    return float(_load().or_fmax(fmt))


def decode(fmt: int, b: int) -> float:
    return float(_load().or_decode(fmt, int(b)))


def encode(fmt: int, y: float) -> int:
    """Encode one fp32 value with |y| <= FMAX (nearest, ties to the even code)."""
    return int(_load().or_encode(fmt, float(np.float32(y))))


def encode_array(fmt: int, y: np.ndarray) -> np.ndarray:
    y = _c(y, np.float32)
    out = np.zeros(y.shape, np.uint8)
    _load().or_encode_array(fmt, _p(y), y.size, _p(out))
    return out


def scale(fmt: int, amax: float) -> np.float32:
    return np.float32(_load().or_scale(fmt, float(np.float32(amax))))


def f64_to_bf16(v: float) -> int:
    return int(_load().or_f64_to_bf16(float(v)))


def f64_to_bf16_array(v: np.ndarray) -> np.ndarray:
    f = _load().or_f64_to_bf16
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([f(float(x)) for x in flat], dtype=np.uint16).reshape(np.shape(v))


def quant_rowwise(x_bf16: np.ndarray, fmt: int):
    """x_bf16: uint16 [rows, cols] bf16 bits.  Returns (q uint8 [rows, cols], s float32 [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.uint8)
    s = np.zeros(rows, np.float32)
    _load().or_quant_rowwise(_p(x), rows, cols, cols, fmt, _p(q), cols, _p(s))
    return q, s


def quant_colwise_grouped(x_bf16: np.ndarray, offsets: np.ndarray, fmt: int):
    """Returns (q_t uint8 [cols, rows], s float32 [groups, cols])."""
    x = _c(x_bf16, np.uint16)
    off = _c(offsets, np.int32)
    rows, cols = x.shape
    g = off.shape[0]
    qt = np.zeros((cols, rows), np.uint8)
    s = np.zeros((g, cols), np.float32)
    _load().or_quant_colwise_grouped(_p(x), rows, cols, cols, _p(off), g, fmt, _p(qt), rows, _p(s))
    return qt, s


def gemm_fwd_rows(fmt, a, sa, b, ldb, b_gs, sb, offsets, N, K, rows):
    """Forward grouped GEMM for the listed rows; returns float64 [len(rows), N] (exact sums
    scaled by 1/(sa*sb), before output rounding).  a: uint8 [M, lda]; b: flat uint8 buffer
    addressed as b[g*b_gs + n*ldb + k]."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.float32)
    sb = _c(sb, np.float32)
    off = _c(offsets, np.int32)
    idx = _c(rows, np.int64)
    out = np.zeros((idx.shape[0], N), np.float64)
    _load().or_gemm_fwd_rows(fmt, _p(a), a.shape[1], _p(sa), _p(b), ldb, b_gs, _p(sb), _p(off),
                             off.shape[0], N, K, _p(idx), idx.shape[0], _p(out))
    return out


def gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, offsets, N, K, g_idx, k_idx):
    """Weight-gradient rows dW[g, k, :] for the listed (g, k) pairs; float64 [len, N].
    xt: uint8 [K, ldx]; dyt: uint8 [N, ldd]; sx: [G, K]; sdy: [G, N]."""
    xt = _c(xt, np.uint8)
    dyt = _c(dyt, np.uint8)
    sx = _c(sx, np.float32)
    sdy = _c(sdy, np.float32)
    off = _c(offsets, np.int32)
    gi = _c(g_idx, np.int32)
    ki = _c(k_idx, np.int64)
    out = np.zeros((gi.shape[0], N), np.float64)
    _load().or_gemm_wgrad_rows(fmt, _p(xt), xt.shape[1], _p(sx), _p(dyt), dyt.shape[1], _p(sdy),
                               _p(off), off.shape[0], N, K, _p(gi), _p(ki), gi.shape[0], _p(out))
    return out


def mx_quant_rowwise(x_bf16: np.ndarray):
    """Returns (q uint8 [rows, cols], e8 uint8 [rows, cols/32])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.uint8)
    e8 = np.zeros((rows, cols // 32), np.uint8)
    _load().or_mx_quant_rowwise(_p(x), rows, cols, cols, _p(q), cols, _p(e8), cols // 32)
    return q, e8


def mx_quant_colwise(x_bf16: np.ndarray):
    """Blocks of 32 rows per column, transposed output.  Returns (q_t uint8 [cols, rows],
    e8 uint8 [cols, rows/32])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    qt = np.zeros((cols, rows), np.uint8)
    e8 = np.zeros((cols, rows // 32), np.uint8)
    _load().or_mx_quant_colwise(_p(x), rows, cols, cols, _p(qt), rows, _p(e8), rows // 32)
    return qt, e8


def mx_gemm_fwd_rows(a, ae8, b, ldb, b_gs, be8, ld_sb, bs_gs, offsets, N, K, rows):
    """MX grouped GEMM rows; float64 [len(rows), N].  a: uint8 [M, lda]; ae8: [M, ld_sa];
    b addressed b[g*b_gs + n*ldb + k]; be8 addressed be8[g*bs_gs + n*ld_sb + kb]."""
    a = _c(a, np.uint8)
    ae8 = _c(ae8, np.uint8)
    b = _c(b, np.uint8)
    be8 = _c(be8, np.uint8)
    off = _c(offsets, np.int32)
    idx = _c(rows, np.int64)
    out = np.zeros((idx.shape[0], N), np.float64)
    _load().or_mx_gemm_fwd_rows(_p(a), a.shape[1], _p(ae8), ae8.shape[1], _p(b), ldb, b_gs,
                                _p(be8), ld_sb, bs_gs, _p(off), off.shape[0], N, K, _p(idx),
                                idx.shape[0], _p(out))
    return out


def mx_gemm_wgrad_rows(xt, xe8, dyt, de8, offsets, N, g_idx, k_idx):
    """MX weight-gradient rows dW[g, k, :] for the listed (g, k); float64 [len, N].  xt: uint8
    [K, ldx] with xe8 [K, ld_sx] (E8M0 per 32 absolute tokens); dyt: [N, ldd] with de8 [N, ld_sd].
    Each group sums its own tokens; a 32-token block shared by two groups keeps its scale."""
    xt = _c(xt, np.uint8)
    xe8 = _c(xe8, np.uint8)
    dyt = _c(dyt, np.uint8)
    de8 = _c(de8, np.uint8)
    off = _c(offsets, np.int32)
    gi = _c(g_idx, np.int32)
    ki = _c(k_idx, np.int64)
    out = np.zeros((gi.shape[0], N), np.float64)
    _load().or_mx_gemm_wgrad_rows(_p(xt), xt.shape[1], _p(xe8), xe8.shape[1], _p(dyt),
                                  dyt.shape[1], _p(de8), de8.shape[1], _p(off), off.shape[0], N,
                                  _p(gi), _p(ki), gi.shape[0], _p(out))
    return out

# ----------------------------------------------------------------------------- whole-matrix GEMMs
# The same definitions as gemm_fwd_rows / gemm_wgrad_rows, for every output at once, with a
# library matmul as the summation step (numpy float64, multithreaded BLAS) so that full-size
# outputs take seconds.  Exactness: every decoded FP8 value times 2^9 (e4m3fn) or 2^10
# (e4m3fnuz) is an integer below 2^18 in magnitude, so every product of two such integers is
# an integer below 2^36 and every partial sum of up to 2^17 of them an integer below 2^53:
# float64 adds them without rounding, in whatever order the matmul takes.  The sums are thus
# the exact ones the C oracle forms, and the results equal its output bit for bit.

_INT_SCALE = {FNUZ: 10, FN: 9}  # log2 of the factor that makes every decoded value an integer


def decode_table(fmt: int) -> np.ndarray:
    """float64 [256]: the C oracle's decode of every byte (NaN for the NaN codes)."""
    return np.array([decode(fmt, b) for b in range(256)], np.float64)


def _int_operand(fmt: int, q: np.ndarray) -> np.ndarray:
    lut = decode_table(fmt) * 2.0 ** _INT_SCALE[fmt]
    return lut[np.asarray(q, np.uint8)]


def gemm_fwd_full(fmt, a, sa, b, ldb, b_gs, sb, offsets, N, K):
    """Every row of the forward grouped GEMM: float64 [M, N], the exact sum of
    dec(a[m,k]) dec(b[g*b_gs + n*ldb + k]) over k, divided by sa[m]*sb[g,n] in float64 (the value
    gemm_fwd_rows returns).  a: uint8 [M, >= K]; b: flat uint8 buffer; rows of no group give 0."""
    a = np.asarray(a, np.uint8)
    M = a.shape[0]
    bflat = np.ascontiguousarray(b, np.uint8).reshape(-1)
    off = np.asarray(offsets, np.int64)
    sa = np.asarray(sa, np.float32).astype(np.float64)
    sb = np.asarray(sb, np.float32).astype(np.float64).reshape(off.size, N)
    out = np.zeros((M, N), np.float64)
    unit = 2.0 ** (-2 * _INT_SCALE[fmt])
    lo = 0
    for g, hi in enumerate(off):
        hi = int(hi)
        if hi > lo:
            idx = g * b_gs + np.arange(N)[:, None] * ldb + np.arange(K)[None, :]
            bg = _int_operand(fmt, bflat[idx])                 # [N, K]
            ag = _int_operand(fmt, a[lo:hi, :K])               # [rows, K]
            acc = (ag @ bg.T) * unit                            # exact sums
            out[lo:hi] = acc / (sa[lo:hi, None] * sb[g][None, :])
        lo = max(lo, hi)
    return out


def gemm_wgrad_group(fmt, xt, sx, dyt, sdy, offsets, g):
    """dW_g of the K-grouped weight gradient: float64 [K, N], the exact sum over the group's
    tokens m of dec(xt[k,m]) dec(dyt[n,m]), divided by sx[g,k]*sdy[g,n] in float64 (the value
    gemm_wgrad_rows returns).  xt: uint8 [K, >= M]; dyt: uint8 [N, >= M]."""
    off = np.asarray(offsets, np.int64)
    lo = 0 if g == 0 else int(off[g - 1])
    hi = int(off[g])
    K, N = xt.shape[0], dyt.shape[0]
    if hi <= lo:
        return np.zeros((K, N), np.float64)
    unit = 2.0 ** (-2 * _INT_SCALE[fmt])
    acc = (_int_operand(fmt, xt[:, lo:hi]) @ _int_operand(fmt, dyt[:, lo:hi]).T) * unit
    sxg = np.asarray(sx, np.float32).astype(np.float64).reshape(off.size, K)[g]
    sdg = np.asarray(sdy, np.float32).astype(np.float64).reshape(off.size, N)[g]
    return acc / (sxg[:, None] * sdg[None, :])


def _mx_operand(q: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """float64 values dec(q) * 2^(e8 - 127), one E8M0 byte per 32 consecutive elements of a row
    (exact: a 4-bit significand times a power of two)."""
    lut = decode_table(FN)
    v = lut[np.asarray(q, np.uint8)]
    sc = np.exp2(np.repeat(np.asarray(e8, np.float64), 32, axis=1)[:, :v.shape[1]] - 127.0)
    return v * sc


def mx_gemm_fwd_full(a, ae8, b, ldb, b_gs, be8, ld_sb, bs_gs, offsets, N, K):
    """Every row of the MX grouped GEMM forward: float64 [M, N] of
    sum_kb 2^(ea+eb) sum_{k in kb} dec(a) dec(b) -- the products exact, their sum rounded in
    float64 (relative error below K * 2^-53, far inside any GEMM tolerance)."""
    a = np.asarray(a, np.uint8)
    M = a.shape[0]
    off = np.asarray(offsets, np.int64)
    bflat = np.ascontiguousarray(b, np.uint8).reshape(-1)
    beflat = np.ascontiguousarray(be8, np.uint8).reshape(-1)
    nb = K // 32
    out = np.zeros((M, N), np.float64)
    lo = 0
    for g, hi in enumerate(off):
        hi = int(hi)
        if hi > lo:
            qb = bflat[g * b_gs + np.arange(N)[:, None] * ldb + np.arange(K)[None, :]]
            eb = beflat[g * bs_gs + np.arange(N)[:, None] * ld_sb + np.arange(nb)[None, :]]
            out[lo:hi] = _mx_operand(a[lo:hi, :K], np.asarray(ae8)[lo:hi, :nb]) @ \
                _mx_operand(qb, eb).T
        lo = max(lo, hi)
    return out


def mx_gemm_wgrad_group(xt, xe8, dyt, de8, offsets, g):
    """dW_g of the MX weight gradient: float64 [K, N] of the sum over the group's tokens of
    dec(xt[k,m]) 2^(xe8[k,m/32]-127) dec(dyt[n,m]) 2^(de8[n,m/32]-127), summed in float64."""
    off = np.asarray(offsets, np.int64)
    lo = 0 if g == 0 else int(off[g - 1])
    hi = int(off[g])
    K, N = xt.shape[0], dyt.shape[0]
    if hi <= lo:
        return np.zeros((K, N), np.float64)
    b0, b1 = lo // 32, -(-hi // 32)
    xa = _mx_operand(xt[:, b0 * 32:b1 * 32], np.asarray(xe8)[:, b0:b1])
    da = _mx_operand(dyt[:, b0 * 32:b1 * 32], np.asarray(de8)[:, b0:b1])
    return xa[:, lo - b0 * 32:hi - b0 * 32] @ da[:, lo - b0 * 32:hi - b0 * 32].T
