"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the same seeded
inputs.  Quantized bytes and scales must match bit for bit; GEMM outputs must lie within
1e-3 + 1e-2*|exact| of the oracle's exactly accumulated result (the oracle value is the exact
sum scaled by 1/(sa*sb), before output rounding), except for rare cancelling elements that the
matrix cores' measured accumulation (tests/mfma_model.py, verified in test_gpu_mfma_model.py)
moves past it, each of which must then match that model; their count is reported.

Sizes are small enough for the oracle to finish in seconds while spanning several tiles of
every kernel (256x64 quant tiles, 128x128 GEMM tiles, 128-byte contraction steps) with ragged
tails, empty groups and groups that start or end on tile boundaries.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import mfma_model as mm
from tests import pinlib

pytestmark = pytest.mark.gpu

FNUZ, FN = 0, 1
FMTS = [FNUZ, FN]


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_grouped_amd as m
    m.lib()  # raises if the HIP library is missing
    return m


DEV = "cuda:0"


def dev_bf16(bits, ld=None):
    return workloads.to_torch_bf16(bits, DEV, ld)


def dev_i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device=DEV)




# ----------------------------------------------------------------------------- codec / scale

@pytest.mark.parametrize("fmt", FMTS)
def test_scale_exhaustive_over_bf16_amax(fq, fmt):
    """Every positive finite bf16 value as a row absmax: the GPU's IEEE division must give the
    oracle's fp32 scale bit for bit."""
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    x = np.zeros((bits.size, 8), np.uint16)
    x[:, 3] = bits
    x[1::2, 3] |= np.uint16(0x8000)  # the sign must not matter
    q, s = fq.fp8_quant_rowwise(dev_bf16(x), fmt)
    oq, os_ = oracle.quant_rowwise(x, fmt)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4040, 0x3F33, 0x3A83, 0x4348, 0x7149, 0x0F00])
def test_rowwise_every_bf16_value(fq, fmt, amax_bits):
    """A row holding every finite bf16 value with |x| <= amax (plus the amax itself): the
    hardware conversion path must reproduce the oracle's encoding of every product."""
    allb = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(allb)
    amax = float(workloads.bf16_bits_to_f32(np.array([amax_bits], np.uint16))[0])
    vals = allb[np.isfinite(f) & (np.abs(f) <= amax)]
    row = np.concatenate([vals, np.array([amax_bits], np.uint16)])
    pad = (-row.size) % 8
    row = np.concatenate([row, np.zeros(pad, np.uint16)])
    # split the values over many rows of the same amax so several kernels shapes are used
    nrow = 16
    per = -(-row.size // nrow)
    per += (-per) % 8
    x = np.zeros((nrow, per), np.uint16)
    flat = x.reshape(-1)
    flat[:row.size] = row
    x[:, -1] = amax_bits  # every row has the same absmax
    q, s = fq.fp8_quant_rowwise(dev_bf16(x), fmt)
    oq, os_ = oracle.quant_rowwise(x, fmt)
    assert np.array_equal(s.cpu().numpy(), os_)
    gq = q.cpu().numpy()
    bad = np.argwhere(gq != oq)
    assert bad.size == 0, [(int(x[r, c]), hex(gq[r, c]), hex(oq[r, c])) for r, c in bad[:8]]


# ----------------------------------------------------------------------------- rowwise

ROW_SHAPES = [(1, 8), (5, 24), (33, 256), (100, 520), (64, 1000), (17, 4096), (9, 8200),
              (3, 20000), (2, 40000), (7, 13)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_rowwise_parity(fq, fmt, shape):
    rows, cols = shape
    x = workloads.make_matrix(100 + rows, rows, cols, 1.0, 0.01)
    x[0, :] = 0  # an all-zero row
    q, s = fq.fp8_quant_rowwise(dev_bf16(x), fmt)
    oq, os_ = oracle.quant_rowwise(x, fmt)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)
    if fmt == FNUZ:
        assert not np.any(q.cpu().numpy() == 0x80)


@pytest.mark.parametrize("fmt", FMTS)
def test_rowwise_padded_leading_dims(fq, fmt):
    rows, cols = 37, 384
    x = workloads.make_matrix(7, rows, cols, 3.0, 0.02)
    xd = dev_bf16(x, ld=cols + 64)
    qbuf = torch.full((rows, cols + 32), 0xAB, dtype=torch.uint8, device=DEV)
    q, s = fq.fp8_quant_rowwise(xd, fmt, q=qbuf[:, :cols])
    oq, os_ = oracle.quant_rowwise(x, fmt)
    qb = qbuf.cpu().numpy()
    assert np.array_equal(qb[:, :cols], oq) and np.array_equal(s.cpu().numpy(), os_)
    assert np.all(qb[:, cols:] == 0xAB)  # nothing written past the row


GATHER_CASES = [
    # tokens, cols, topk, ld_x pad
    (256, 256, 4, 0),      # the C1 width, 1024 routed rows
    (300, 6144, 2, 64),    # wider rows (two waves per row), padded source stride
    (50, 100, 3, 0),       # columns not a multiple of 8: element-wise path
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", GATHER_CASES)
def test_rowwise_gather_parity(fq, fmt, case):
    """Routed token rows quantized in expert order: bytes and scales equal the oracle's rowwise
    quantization of x[index] (numpy gather), repeated source rows included."""
    tokens, cols, topk, pad = case
    x = workloads.make_matrix(900 + tokens, tokens, cols, 1.0, 0.01)
    _, idx = workloads.routed_rows_topk(np.random.Generator(np.random.PCG64(tokens)), tokens,
                                        8, topk)
    q, sc = fq.fp8_quant_rowwise_gather(dev_bf16(x, ld=cols + pad), dev_i32(idx), fmt)
    oq, os_ = oracle.quant_rowwise(x[idx], fmt)
    assert np.array_equal(sc.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_rowwise_gather_index_clamped(fq):
    """Out-of-range indices read the nearest end row (never out of bounds)."""
    x = workloads.make_matrix(77, 20, 64, 2.0)
    idx = np.array([5, -3, 19, 20, 1000, 0, -2147483648, 2147483647], np.int32)
    q, sc = fq.fp8_quant_rowwise_gather(dev_bf16(x), dev_i32(idx), FN)
    oq, os_ = oracle.quant_rowwise(x[np.clip(idx, 0, 19)], FN)
    assert np.array_equal(sc.cpu().numpy(), os_) and np.array_equal(q.cpu().numpy(), oq)


# ----------------------------------------------------------------------------- colwise

COL_CASES = [
    # rows, cols, offsets
    (300, 72, [300]),
    (513, 130, [0, 37, 37, 256, 256, 257, 512, 513]),
    (700, 64, [100, 100, 356, 612, 700, 700]),
    (1024, 200, [444, 509, 893, 1024]),
    (96, 40, [10, 20, 30, 40, 50, 60, 70, 80, 90, 91, 92, 96]),
    (1, 8, [1]),
    (259, 21, [3, 259]),          # columns not a multiple of 8 -> element-wise path
    # more groups than the kernels stage in LDS: offsets are read from global memory
    (4300, 24, sorted(np.random.Generator(np.random.PCG64(11)).integers(0, 4301, 2099).tolist())
     + [4300]),
    # long groups (many row blocks per group and strip), alone and next to short ones
    (40000, 24, [40000]),
    (40000, 40, [100, 700, 39000, 40000]),
    # one block per (group, 16-column strip): a group longer than the 8192 rows a block holds
    # (walked twice by its block), one exactly at the limit from an unaligned start, empty and
    # 1-row groups
    (12000, 1024, [5, 5, 17, 33, 40, 41, 60, 80, 100, 130, 200, 300, 301, 302, 310, 320, 9321,
                   12000]),
    (9000, 1024, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 8200, 9000]),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", COL_CASES)
def test_colwise_grouped_parity(fq, fmt, case):
    rows, cols, off = case
    x = workloads.make_matrix(200 + rows + cols, rows, cols, 1.0, 0.01)
    off = np.asarray(off, np.int32)
    qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x), dev_i32(off), fmt)
    oqt, os_ = oracle.quant_colwise_grouped(x, off, fmt)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(qt.cpu().numpy(), oqt)


@functools.lru_cache(maxsize=2)
def _long_group_case(fmt):
    x = workloads.make_matrix(77, 20000, 8192, 1.0, 0.01)
    off = np.array([4999, 4999, 13001, 20000], np.int32)
    return (x, off) + tuple(oracle.quant_colwise_grouped(x, off, fmt))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("pad", [0, 5])
def test_colwise_long_groups(fq, fmt, pad):
    """Groups averaging >= 4096 rows over >= 512 (group, 64-column strip) pairs: one block per
    pair walks its strip twice.  Unaligned group edges, an empty group, and an output stride
    that is not a multiple of 16 (pad 5) for the byte-wise store path."""
    rows, cols = 20000, 8192
    x, off, oqt, os_ = _long_group_case(fmt)
    buf = torch.full((cols, rows + pad), 0xCD, dtype=torch.uint8, device=DEV)
    qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x), dev_i32(off), fmt, q_t=buf[:, :rows])
    b = buf.cpu().numpy()
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(b[:, :rows], oqt)
    assert np.all(b[:, rows:] == 0xCD)


@pytest.mark.parametrize("fmt", FMTS)
def test_colwise_unaligned_output_stride(fq, fmt):
    rows, cols = 300, 64
    x = workloads.make_matrix(5, rows, cols)
    off = np.array([120, 300], np.int32)
    buf = torch.full((cols, rows + 5), 0xCD, dtype=torch.uint8, device=DEV)
    qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x, ld=cols + 8), dev_i32(off), fmt,
                                         q_t=buf[:, :rows])
    oqt, os_ = oracle.quant_colwise_grouped(x, off, fmt)
    b = buf.cpu().numpy()
    assert np.array_equal(b[:, :rows], oqt) and np.array_equal(s.cpu().numpy(), os_)
    assert np.all(b[:, rows:] == 0xCD)


@pytest.mark.parametrize("fmt", FMTS)
def test_colwise_zero_rows_writes_empty_scales(fq, fmt):
    x = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    off = dev_i32([0, 0, 0])
    qt, s = fq.fp8_quant_colwise_grouped(x, off, fmt)
    want = np.float32(pinlib.FMAX[fmt]) / np.float32(1e-12)
    assert np.all(s.cpu().numpy() == want)


def test_colwise_deterministic_across_calls(fq):
    """Relaxed atomics combine maxima in any order; max is exact, so repeated calls (with the
    workspace reused and not cleared by the caller) give identical bytes."""
    x = workloads.make_matrix(9, 1500, 136, 1.0, 0.01)
    off = dev_i32([200, 700, 701, 1500])
    ws = torch.empty(fq.fp8_quant_colwise_grouped_workspace_size(1500, 136, 4) + 256,
                     dtype=torch.uint8, device=DEV)
    ref = None
    for _ in range(5):
        qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x), off, FN, workspace=ws)
        cur = (qt.cpu().numpy(), s.cpu().numpy())
        if ref is None:
            ref = cur
        assert np.array_equal(cur[0], ref[0]) and np.array_equal(cur[1], ref[1])


# ----------------------------------------------------------------------------- weights, both layouts

WDUAL_CASES = [
    # experts, K, N, pad (extra elements in the rows of w, q_rows and q_t)
    (4, 256, 512, 0),
    (4, 200, 512, 8),    # K not a multiple of the 128-row blocks; padded strides (ld_qt 808)
    (3, 64, 2048, 0),    # the widest N
    (2, 130, 8, 16),     # one 8-column chunk per row
    (1, 1, 16, 0),
    (16, 4096, 2048, 16),  # long expert groups, padded strides
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", WDUAL_CASES)
def test_weights_dual_parity(fq, fmt, case):
    """fp8_quant_weights_dual: the rowwise layout (scales along N) and the colwise layout
    (scales along K per expert) in one call, each equal to the oracle bit for bit."""
    E, K, N, pad = case
    w = workloads.make_matrix(300 + E + K + N, E * K, N, 0.02, 0.01)
    q_rows = torch.full((E * K, N + pad), 0xCD, dtype=torch.uint8, device=DEV)
    q_t = torch.full((N, E * K + pad), 0xCD, dtype=torch.uint8, device=DEV)
    (_, sr), (_, sc) = fq.fp8_quant_weights_dual(dev_bf16(w, ld=N + pad), E, fmt,
                                                 q_rows=q_rows[:, :N], q_t=q_t[:, :E * K])
    oq, os_ = oracle.quant_rowwise(w, fmt)
    oqt, osc = oracle.quant_colwise_grouped(w, (np.arange(1, E + 1) * K).astype(np.int32), fmt)
    qr_h, qt_h = q_rows.cpu().numpy(), q_t.cpu().numpy()
    assert np.array_equal(sr.cpu().numpy(), os_) and np.array_equal(qr_h[:, :N], oq)
    assert np.array_equal(sc.cpu().numpy(), osc) and np.array_equal(qt_h[:, :E * K], oqt)
    assert np.all(qr_h[:, N:] == 0xCD) and np.all(qt_h[:, E * K:] == 0xCD)


def test_weights_dual_rejects_wide_rows(fq):
    w = torch.zeros((64, 2056), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="status 2"):
        fq.fp8_quant_weights_dual(w, 1, FN)


# ----------------------------------------------------------------------------- grouped GEMM

def _fwd_operands(fmt, M, K, N, E, seed):
    x = workloads.make_matrix(seed, M, K, 1.0, 0.01)
    w = workloads.make_matrix(seed + 1, E * K, N, 0.02)
    qa, sa = oracle.quant_rowwise(x, fmt)
    qbt, sb = oracle.quant_colwise_grouped(w, (np.arange(1, E + 1) * K).astype(np.int32), fmt)
    return qa, sa, qbt, sb


GEMM_FWD_CASES = [
    # M, K, N, offsets
    (1024, 256, 512, [444, 509, 893, 1024]),
    (300, 144, 200, [0, 1, 129, 129, 300]),
    (64, 128, 16, [64]),
    (515, 512, 130, [128, 128, 256, 300, 515]),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", GEMM_FWD_CASES)
def test_gemm_fwd_parity(fq, fmt, case):
    M, K, N, off = case
    off = np.asarray(off, np.int32)
    E = off.size
    qa, sa, qbt, sb = _fwd_operands(fmt, M, K, N, E, 300 + M)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qbt).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(off), M, N, K,
                            ldb=E * K, b_group_stride=K)
    got = c.float().cpu().numpy()
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, np.arange(M))
    mm.check_gemm(got, ref, f"fwd {case} fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qbt, E * K, K, sb, off, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_fwd_expert_major_weights(fq, fmt):
    """Weights stored [E, N, K] (b_group_stride = N*K, ldb = K), quantized rowwise along K."""
    M, K, N, E = 400, 256, 96, 3
    off = np.array([150, 150, 400], np.int32)
    x = workloads.make_matrix(41, M, K, 1.0, 0.01)
    w = workloads.make_matrix(42, E * N, K, 0.02)  # [E*N, K]
    qa, sa = oracle.quant_rowwise(x, fmt)
    qb, sbf = oracle.quant_rowwise(w, fmt)        # per (e, n) scale over K
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qb).to(DEV),
                            torch.from_numpy(sbf).to(DEV), dev_i32(off), M, N, K, ldb=K,
                            b_group_stride=N * K)
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qb, K, N * K, sbf, off, N, K, np.arange(M))
    mm.check_gemm(c.float().cpu().numpy(), ref, f"fwd expert-major fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qb, K, N * K, sbf, off, N, K))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_fwd_rows_isolated_from_other_groups(fq, fmt):
    """A group's outputs depend on its own rows only: the rows of the next group in its partial
    row tiles hold NaN codes (e4m3fn 0x7F, e4m3fnuz 0x80), and groups 0 (5 rows, inside one
    tile with 251 rows of group 1) and 2 must still match the oracle."""
    M, K, N, E = 600, 256, 128, 3
    off = np.array([5, 300, 600], np.int32)
    qa, sa, qbt, sb = _fwd_operands(fmt, M, K, N, E, 77)
    qa = qa.copy()
    qa[5:300] = 0x7F if fmt == FN else 0x80
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qbt).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(off), M, N, K,
                            ldb=E * K, b_group_stride=K)
    got = c.float().cpu().numpy()
    rows = np.concatenate([np.arange(0, 5), np.arange(300, 600)])
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, rows)
    assert np.all(np.isfinite(got[rows]))
    mm.check_gemm(got[rows], ref, f"fwd rows isolated fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, rows=rows))


DGRAD_CASES = [
    # M (tokens), K (hidden, the output columns), N (intermediate, the contraction), offsets
    (1024, 256, 512, [485, 524, 774, 1024]),    # the C1 shapes and offsets
    (600, 200, 144, [0, 250, 250, 600]),         # empty groups, ragged tiles (N: multiple of 16)
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", DGRAD_CASES)
def test_gemm_dgrad_parity(fq, fmt, case):
    """Data gradient dX_g = dY_g W_g^T: dY [M, N] and the weights [E*K, N] quantized rowwise along
    N (the contraction), then the forward mode with expert g's [K, N] weight rows as B
    (ldb = N, group stride K*N).  Every output element against the oracle."""
    M, K, N, off = case
    off = np.asarray(off, np.int32)
    E = off.size
    dy = workloads.make_matrix(700 + M, M, N)
    w = workloads.make_matrix(701 + M, E * K, N, 0.02)
    qa, sa = oracle.quant_rowwise(dy, fmt)
    qb, sb = oracle.quant_rowwise(w, fmt)        # per (e, k) scale over N
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qb).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(off), M, K, N, ldb=N,
                            b_group_stride=K * N)
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qb, N, K * N, sb, off, K, N, np.arange(M))
    mm.check_gemm(c.float().cpu().numpy(), ref, f"dgrad {case} fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qb, N, K * N, sb, off, K, N))


GEMM_WGRAD_CASES = [
    # M (tokens), K, N, offsets
    (1000, 160, 96, [100, 100, 357, 358, 1000]),
    (300, 128, 128, [300]),
    (777, 200, 72, [16, 32, 300, 301, 700, 777, 777]),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", GEMM_WGRAD_CASES)
def test_gemm_wgrad_parity(fq, fmt, case):
    M, K, N, off = case
    off = np.asarray(off, np.int32)
    G = off.size
    x = workloads.make_matrix(500 + M, M, K)
    dy = workloads.make_matrix(600 + M, M, N)
    xt, sx = oracle.quant_colwise_grouped(x, off, fmt)    # [K, M], [G, K]
    dyt, sdy = oracle.quant_colwise_grouped(dy, off, fmt)  # [N, M], [G, N]
    # the weight-gradient operands need 16-byte aligned rows: pad the token dimension
    ldp = -(-M // 16) * 16

    def padded(a):
        t = torch.zeros((a.shape[0], ldp), dtype=torch.uint8, device=DEV)
        t[:, :M] = torch.from_numpy(a).to(DEV)
        return t

    c = fq.fp8_grouped_gemm(fq.GEMM_WGRAD_KGROUPED, fmt, padded(xt),
                            torch.from_numpy(sx).to(DEV), padded(dyt),
                            torch.from_numpy(sdy).to(DEV), dev_i32(off), M, N, K, ldb=ldp)
    got = c.float().cpu().numpy()
    gi = np.repeat(np.arange(G, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), G)
    ref = oracle.gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, off, N, K, gi, ki).reshape(G, K, N)
    mm.check_gemm(got, ref, f"wgrad {case} fmt {fmt}",
                  mm.explain_wgrad(fmt, xt, sx, dyt, sdy, off, N, K))
    start = 0
    for g, end in enumerate(off):
        if end == start:
            assert np.all(got[g] == 0)
        start = end


# ----------------------------------------------------------------------------- MXFP8

@pytest.mark.parametrize("shape", [(3, 32), (40, 1024), (17, 7168), (5, 2080)])
def test_mx_rowwise_parity(fq, shape):
    rows, cols = shape
    x = workloads.make_matrix(700 + cols, rows, cols, 1.0, 0.02)
    x[0, :32] = 0
    q, e8 = fq.fp8_mx_quant_rowwise(dev_bf16(x))
    oq, oe = oracle.mx_quant_rowwise(x)
    assert np.array_equal(e8.cpu().numpy(), oe)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_mx_rowwise_every_exponent(fq):
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    n = bits.size - bits.size % 4
    x = np.zeros((n // 4, 4 * 32), np.uint16)
    x.reshape(-1, 32)[:, 7] = bits[:n]
    x.reshape(-1, 32)[:, 9] = bits[:n] ^ np.uint16(0x8000)
    q, e8 = fq.fp8_mx_quant_rowwise(dev_bf16(x))
    oq, oe = oracle.mx_quant_rowwise(x)
    assert np.array_equal(e8.cpu().numpy(), oe) and np.array_equal(q.cpu().numpy(), oq)


@pytest.mark.parametrize("shape", [(32, 8), (256, 64), (544, 136), (96, 40)])
def test_mx_colwise_parity(fq, shape):
    rows, cols = shape
    x = workloads.make_matrix(800 + rows, rows, cols, 0.02, 0.01)
    qt, e8 = fq.fp8_mx_quant_colwise(dev_bf16(x))
    oqt, oe = oracle.mx_quant_colwise(x)
    assert np.array_equal(e8.cpu().numpy(), oe)
    assert np.array_equal(qt.cpu().numpy(), oqt)


# (M, K, N, offsets, outlier fraction of x): 1% of x scaled by 50, as in the tiny
# configuration, at every contraction length (at long K, rare cancelling outputs of such data
# are moved past the strict bar by the matrix cores' accumulation; check_gemm holds each of them
# to the measured model).
@pytest.mark.parametrize("case", [(300, 256, 96, [100, 100, 300], 0.01),
                                  (515, 512, 130, [128, 256, 300, 515], 0.01),
                                  (64, 160, 64, [64], 0.01),
                                  (700, 2048, 384, [0, 333, 700], 0.01),
                                  (700, 2048, 384, [0, 333, 700], 0.0)])
def test_mx_gemm_parity(fq, case):
    M, K, N, off, outliers = case
    off = np.asarray(off, np.int32)
    E = off.size
    x = workloads.make_matrix(900 + M, M, K, 1.0, outliers)
    w = workloads.make_matrix(901 + M, E * K, N, 0.02)
    qa, ea = oracle.mx_quant_rowwise(x)
    qbt, eb = oracle.mx_quant_colwise(w)  # [N, E*K], [N, E*K/32]
    c = fq.fp8_mx_grouped_gemm(torch.from_numpy(qa).to(DEV), torch.from_numpy(ea).to(DEV),
                               torch.from_numpy(qbt).to(DEV), torch.from_numpy(eb).to(DEV),
                               dev_i32(off), M, N, K, ldb=E * K, b_group_stride=K,
                               ld_sb=E * K // 32, sb_group_stride=K // 32)
    ref = oracle.mx_gemm_fwd_rows(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K,
                                  np.arange(M))
    mm.check_gemm(c.float().cpu().numpy(), ref, f"mx {case}",
                  mm.explain_mx_fwd(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K))


def test_mx_gemm_padded_scale_rows(fq):
    """16-byte aligned scale rows (padding bytes hold garbage) and 9 contraction steps, so the
    4-step scale chunks end mid-chunk; B scales in an expert-major [E, N, ld] layout."""
    M, K, N = 600, 1152, 200
    off = np.array([250, 250, 600], np.int32)
    E, nb, ld = off.size, K // 32, 48
    x = workloads.make_matrix(911, M, K, 1.0, 0.0)
    w = workloads.make_matrix(912, E * K, N, 0.02)
    qa, ea = oracle.mx_quant_rowwise(x)
    qbt, eb = oracle.mx_quant_colwise(w)
    ea_p = np.full((M, ld), 0xAB, np.uint8)
    ea_p[:, :nb] = ea
    eb_p = np.full((E, N, ld), 0xCD, np.uint8)
    for e in range(E):
        eb_p[e, :, :nb] = eb[:, e * nb:(e + 1) * nb]
    c = fq.fp8_mx_grouped_gemm(torch.from_numpy(qa).to(DEV), torch.from_numpy(ea_p).to(DEV),
                               torch.from_numpy(qbt).to(DEV), torch.from_numpy(eb_p).to(DEV),
                               dev_i32(off), M, N, K, ldb=E * K, b_group_stride=K, ld_sb=ld,
                               sb_group_stride=N * ld)
    ref = oracle.mx_gemm_fwd_rows(qa, ea_p, qbt, E * K, K, eb_p.reshape(-1), ld, N * ld, off, N,
                                  K, np.arange(M))
    mm.check_gemm(c.float().cpu().numpy(), ref, "mx padded scale rows",
                  mm.explain_mx_fwd(qa, ea_p, qbt, E * K, K, eb_p.reshape(-1), ld, N * ld, off,
                                    N, K))


# (M tokens, K, N, offsets): groups that start and end inside 32-token scale blocks, empty
# groups, ragged K and N tiles, one long group.
# (M tokens, K, N, offsets, strict): the strict cases hold every element to the 1e-3 + 1e-2|exact|
# bar with no matrix-core exception (short groups: no output cancels far below its terms).
MX_WGRAD_CASES = [
    (256, 160, 96, [40, 40, 150, 256], True),
    (512, 256, 128, [512], False),
    (1024, 300, 72, [0, 17, 300, 301, 640, 1000, 1024], False),
    (2048, 128, 256, [700, 2048], False),
    (192, 128, 64, [30, 30, 96, 97, 192], True),
]


@pytest.mark.parametrize("case", MX_WGRAD_CASES)
def test_mx_gemm_wgrad_parity(fq, case):
    """MX weight gradient from the transposed MX quantizations of X and dY (32-token blocks
    counted from token 0): every dW element against the oracle."""
    M, K, N, off, strict = case
    off = np.asarray(off, np.int32)
    G = off.size
    x = workloads.make_matrix(950 + M, M, K, 1.0, 0.0)
    dy = workloads.make_matrix(951 + M, M, N)
    xt, xe = oracle.mx_quant_colwise(x)      # [K, M], [K, M/32]
    dyt, de = oracle.mx_quant_colwise(dy)    # [N, M], [N, M/32]
    c = fq.fp8_mx_grouped_gemm_wgrad(torch.from_numpy(xt).to(DEV), torch.from_numpy(xe).to(DEV),
                                     torch.from_numpy(dyt).to(DEV), torch.from_numpy(de).to(DEV),
                                     dev_i32(off), M, N, K)
    gi = np.repeat(np.arange(G, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), G)
    ref = oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, off, N, gi, ki)
    mm.check_gemm(c.float().cpu().numpy().reshape(G * K, N), ref, f"mx wgrad {case}",
                  mm.explain_mx_wgrad(xt, xe, dyt, de, off, N, K), strict=strict)


# ----------------------------------------------------------------------------- argument errors

def test_invalid_arguments_return_status(fq):
    L = fq.lib()
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((4, 8), dtype=torch.uint8, device=DEV)
    s = torch.zeros((4,), dtype=torch.float32, device=DEV)
    p = lambda t: t.data_ptr()
    assert L.fp8_quant_rowwise(p(x), 4, 8, 4, 1, p(q), 8, p(s), None) == 1   # ld_x < cols
    assert L.fp8_quant_rowwise(p(x), 4, 8, 8, 7, p(q), 8, p(s), None) == 1   # bad format
    assert L.fp8_quant_rowwise(None, 4, 8, 8, 1, p(q), 8, p(s), None) == 1   # null input
    off = dev_i32([4])
    assert L.fp8_quant_colwise_grouped(p(x), 4, 8, 8, p(off), 1, 1, p(q), 4, p(s), p(q), 4,
                                       None) == 3  # workspace too small
    ws = torch.zeros((256,), dtype=torch.uint8, device=DEV)
    assert L.fp8_grouped_gemm(0, 1, p(q), 8, p(s), p(q), 8, 0, p(s), p(off), 1, 4, 4, 8, p(x),
                              4, 0, p(ws), 256, None) == 2  # K not a multiple of 16


# ----------------------------------------------------------------------------- GEMM contract

def _wgrad_case(fmt, M, K, N, off, seed):
    x = workloads.make_matrix(seed, M, K)
    dy = workloads.make_matrix(seed + 1, M, N)
    xt, sx = oracle.quant_colwise_grouped(x, off, fmt)
    dyt, sdy = oracle.quant_colwise_grouped(dy, off, fmt)
    return xt, sx, dyt, sdy


def test_gemm_wgrad_ignores_padding_and_other_groups_codes(fq):
    """Weight gradient in e4m3fn with M % 16 != 0: the token padding of both operands holds NaN
    codes (0x7F, 0xFF), as torch.empty memory may, and in a second call group 0's gradient bytes
    are NaN codes too.  Every group's dW must still match the oracle (second call: group 1,
    whose first contraction chunk holds group 0's last tokens)."""
    M, K, N = 777, 200, 72
    off = np.array([300, 777], np.int32)
    xt, sx, dyt, sdy = _wgrad_case(FN, M, K, N, off, 1500)
    ldp = -(-M // 16) * 16
    a = np.full((K, ldp), 0xFF, np.uint8)
    a[:, :M] = xt
    b = np.full((N, ldp), 0x7F, np.uint8)
    b[:, :M] = dyt
    gi = np.repeat(np.arange(2, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), 2)
    ref = oracle.gemm_wgrad_rows(FN, xt, sx, dyt, sdy, off, N, K, gi, ki).reshape(2, K, N)
    run = lambda bb: fq.fp8_grouped_gemm(
        fq.GEMM_WGRAD_KGROUPED, FN, torch.from_numpy(a).to(DEV), torch.from_numpy(sx).to(DEV),
        torch.from_numpy(bb).to(DEV), torch.from_numpy(sdy).to(DEV), dev_i32(off), M, N, K,
        ldb=ldp).float().cpu().numpy()
    got = run(b)
    assert np.all(np.isfinite(got))
    mm.check_gemm(got, ref, "wgrad, NaN codes in the padding",
                  mm.explain_wgrad(FN, xt, sx, dyt, sdy, off, N, K))
    b2 = b.copy()
    b2[:, :300] = 0x7F
    got2 = run(b2)
    assert np.all(np.isfinite(got2[1]))
    mm.check_gemm(got2[1], ref[1], "wgrad, NaN codes in the previous group",
                  mm.explain_wgrad(FN, xt, sx, dyt, sdy, off, N, K,
                                   pairs=[(1, k) for k in range(K)]))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_fp32_output(fq, fmt):
    """out_dtype fp32: forward and weight gradient write fp32 that matches the oracle, and the
    bf16 output is exactly that fp32 value rounded to nearest even."""
    M, K, N, E = 515, 512, 130, 5
    off = np.array([128, 128, 256, 300, 515], np.int32)
    qa, sa, qbt, sb = _fwd_operands(fmt, M, K, N, E, 815)
    args = (fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV),
            torch.from_numpy(qbt).to(DEV), torch.from_numpy(sb).to(DEV), dev_i32(off), M, N, K)
    c32 = fq.fp8_grouped_gemm(*args, ldb=E * K, b_group_stride=K, out_dtype=torch.float32)
    c16 = fq.fp8_grouped_gemm(*args, ldb=E * K, b_group_stride=K)
    assert c32.dtype == torch.float32 and c16.dtype == torch.bfloat16
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, np.arange(M))
    mm.check_gemm(c32.cpu().numpy(), ref, f"fwd fp32 out fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qbt, E * K, K, sb, off, N, K))
    assert torch.equal(c32.to(torch.bfloat16), c16)
    Mw, Kw, Nw = 1000, 160, 96
    offw = np.array([100, 100, 357, 358, 1000], np.int32)
    xt, sx, dyt, sdy = _wgrad_case(fmt, Mw, Kw, Nw, offw, 1600)
    ldp = -(-Mw // 16) * 16
    pad = lambda v: np.pad(v, ((0, 0), (0, ldp - Mw)))
    wargs = (fq.GEMM_WGRAD_KGROUPED, fmt, torch.from_numpy(pad(xt)).to(DEV),
             torch.from_numpy(sx).to(DEV), torch.from_numpy(pad(dyt)).to(DEV),
             torch.from_numpy(sdy).to(DEV), dev_i32(offw), Mw, Nw, Kw)
    w32 = fq.fp8_grouped_gemm(*wargs, ldb=ldp, out_dtype=torch.float32)
    w16 = fq.fp8_grouped_gemm(*wargs, ldb=ldp)
    G = offw.size
    gi = np.repeat(np.arange(G, dtype=np.int32), Kw)
    ki = np.tile(np.arange(Kw, dtype=np.int64), G)
    refw = oracle.gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, offw, Nw, Kw, gi, ki).reshape(G, Kw, Nw)
    mm.check_gemm(w32.cpu().numpy(), refw, f"wgrad fp32 out fmt {fmt}",
                  mm.explain_wgrad(fmt, xt, sx, dyt, sdy, offw, Nw, Kw))
    assert torch.equal(w32.to(torch.bfloat16), w16)


def test_gemm_offsets_check_in_workspace(fq):
    """The GEMM reports its offsets check in the workspace: valid offsets give (0, -1); a
    decreasing end or a last end other than M names the first offending group.  With such
    offsets the kernel only uses clamped rows, so the call itself stays in range."""
    M, K, N, E = 300, 128, 64, 3
    qa, sa, qbt, sb = _fwd_operands(FN, M, K, N, E, 915)
    ws = torch.full((fq.fp8_grouped_gemm_workspace_size(0, M, N, K, E),), 0xAB,
                    dtype=torch.uint8, device=DEV)

    def status(offs):
        fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, FN, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qbt).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(offs), M, N, K, ldb=E * K,
                            b_group_stride=K, workspace=ws)
        return fq.gemm_offsets_status(ws)

    assert status([100, 200, 300]) == (0, -1)
    assert status([0, 0, 300]) == (0, -1)
    assert status([100, 50, 300]) == (1, 1)
    assert status([100, 200, 250]) == (1, 2)
    assert status([-5, 200, 300]) == (1, 0)
    assert status([100, 400, 300]) == (1, 1)


def test_gemm_fwd_stale_lds_rows_never_reach_stored_rows(fq):
    """More tiles than blocks: every block of the last XCD's range first runs a full row tile of
    group 0, whose rows are all NaN codes (e4m3fn 0x7F), then a partial tile of a small group
    whose DMA skips the rows past the group's end (those LDS rows keep group 0's NaN bytes).
    The small groups' rows must be finite and match the oracle."""
    K, N = 128, 256
    small = [5, 17, 40, 1, 200, 33, 64, 129, 255, 7, 90, 3, 16, 250, 77, 100, 2, 60, 31, 180]
    sizes = [256 * 300] + small
    off = np.cumsum(sizes).astype(np.int32)
    M, E = int(off[-1]), len(sizes)
    qa, sa, qbt, sb = _fwd_operands(FN, M, K, N, E, 1015)
    qa = qa.copy()
    qa[:sizes[0]] = 0x7F
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, FN, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qbt).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(off), M, N, K, ldb=E * K,
                            b_group_stride=K)
    rows = np.arange(sizes[0], M)
    got = c[sizes[0]:].float().cpu().numpy()
    ref = oracle.gemm_fwd_rows(FN, qa, sa, qbt, E * K, K, sb, off, N, K, rows)
    assert np.all(np.isfinite(got))
    mm.check_gemm(got, ref, "fwd after NaN tiles",
                  mm.explain_fwd(FN, qa, sa, qbt, E * K, K, sb, off, N, K, rows=rows))


# ----------------------------------------------------------------------------- both layouts

DUAL_CASES = [
    # rows, cols, offsets, ld pad of x, ld pad of q
    (1024, 256, [485, 524, 774, 1024], 0, 0),           # the C1 activation shapes
    (513, 130, [0, 37, 37, 256, 256, 257, 512, 513], 8, 0),  # ragged tiles, empty groups
    (700, 72, [100, 100, 356, 612, 700, 700], 0, 5),    # byte-wise rowwise stores (ld_q % 8)
    (259, 21, [3, 259], 0, 0),                          # columns not a multiple of 8
    (4300, 24, sorted(np.random.Generator(np.random.PCG64(12)).integers(0, 4301, 2099).tolist())
     + [4300], 0, 0),                                    # groups beyond the LDS offsets copy
    (3000, 7168, [150, 900, 901, 2999, 3000], 0, 0),     # the DeepSeek-V3 hidden width
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("case", DUAL_CASES)
def test_dual_layout_parity(fq, fmt, case):
    """fp8_quant_dual_grouped: the rowwise bytes and scales equal the oracle's rowwise
    quantization and the transposed ones its colwise grouped quantization, bit for bit, with
    nothing written past either output's rows."""
    rows, cols, off, padx, padq = case
    x = workloads.make_matrix(1300 + rows + cols, rows, cols, 1.0, 0.01)
    off = np.asarray(off, np.int32)
    qbuf = torch.full((rows, cols + padq), 0xCD, dtype=torch.uint8, device=DEV)
    (q, sr), (qt, sc) = fq.fp8_quant_dual_grouped(dev_bf16(x, ld=cols + padx if padx else None),
                                                  dev_i32(off), fmt, q=qbuf[:, :cols])
    oq, os_ = oracle.quant_rowwise(x, fmt)
    oqt, osc = oracle.quant_colwise_grouped(x, off, fmt)
    qb = qbuf.cpu().numpy()
    assert np.array_equal(sr.cpu().numpy(), os_)
    assert np.array_equal(qb[:, :cols], oq)
    assert np.all(qb[:, cols:] == 0xCD)
    assert np.array_equal(sc.cpu().numpy(), osc)
    assert np.array_equal(qt.cpu().numpy(), oqt)
