"""GPU parity at the configurations' full sizes, through the C ABI, in the launch
configuration the benchmark times (same entry points, shapes, layouts and strides).

Quantizers: every byte and scale is compared with the oracle (bit-exact), for every
configuration.  GEMMs: every output element is compared with the oracle's exact result under
the 1e-3 + 1e-2*|exact| bar, rare cancelling elements being held to the measured matrix-core
model instead (tests/mfma_model.py; their count is reported).  The operands fed to the GEMMs
are the oracle's quantized bytes, so no input or expected value comes from the GPU path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import mfma_model as mm

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda:0"
FNUZ, FN = 0, 1


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_grouped_amd as m
    m.lib()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module")
def dsv3_fwd():
    return workloads.make_forward("dsv3_mx")   # X [16384, 7168], W [32*7168, 2048], offsets


@pytest.fixture(scope="module")
def dsv3_bwd():
    return workloads.make_wgrad("dsv3_bwd")    # X [16384, 7168], dY [16384, 2048], offsets


# ----------------------------------------------------------------------------- quantizers

@pytest.mark.parametrize("fmt", [FN, FNUZ])
def test_rowwise_full_dsv3_activations(fq, dsv3_fwd, fmt):
    x = dsv3_fwd["x"]
    q, s = fq.fp8_quant_rowwise(workloads.to_torch_bf16(x, DEV), fmt)
    oq, os_ = oracle.quant_rowwise(x, fmt)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_rowwise_gather_full_dsv3(fq, dsv3_fwd):
    """2048 tokens x top-8 routed to 32 experts (Zipf): the 16384 expert-ordered rows of hidden
    7168 quantized straight from the token activations."""
    x = dsv3_fwd["x"][:2048]
    _, idx = workloads.routed_rows_topk(np.random.Generator(np.random.PCG64(6)), 2048, 32, 8)
    q, s = fq.fp8_quant_rowwise_gather(workloads.to_torch_bf16(x, DEV), dev(idx), FN)
    oq, os_ = oracle.quant_rowwise(x[idx], FN)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_colwise_full_dsv3_weights(fq, dsv3_fwd):
    d = dsv3_fwd
    E, K = d["E"], d["K"]
    off_w = (np.arange(1, E + 1) * K).astype(np.int32)
    qt, s = fq.fp8_quant_colwise_grouped(workloads.to_torch_bf16(d["w"], DEV), dev(off_w), FN)
    oqt, os_ = oracle.quant_colwise_grouped(d["w"], off_w, FN)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(qt.cpu().numpy(), oqt)


def test_weights_dual_full_dsv3(fq, dsv3_fwd):
    """Both weight layouts of the 32 x 7168 x 2048 experts in one call; three experts (first,
    middle, last) compared with the oracle in full, rows and columns."""
    d = dsv3_fwd
    E, K, N, w = d["E"], d["K"], d["N"], d["w"]
    (qr, sr), (qt, sc) = fq.fp8_quant_weights_dual(workloads.to_torch_bf16(w, DEV), E, FN)
    qr, sr, qt, sc = (t.cpu().numpy() for t in (qr, sr, qt, sc))
    for e in (0, 13, E - 1):
        we = w[e * K:(e + 1) * K]
        oq, os_ = oracle.quant_rowwise(we, FN)
        assert np.array_equal(sr[e * K:(e + 1) * K], os_)
        assert np.array_equal(qr[e * K:(e + 1) * K], oq)
        oqt, osc = oracle.quant_colwise_grouped(we, np.array([K], np.int32), FN)
        assert np.array_equal(sc[e], osc[0])
        assert np.array_equal(qt[:, e * K:(e + 1) * K], oqt)


@pytest.mark.parametrize("which", ["x", "dy"])
def test_colwise_full_dsv3_wgrad_operands(fq, dsv3_bwd, which):
    d = dsv3_bwd
    a = d[which]
    M = d["M"]
    ldm = -(-M // 16) * 16
    buf = torch.empty((a.shape[1], ldm), dtype=torch.uint8, device=DEV)
    qt, s = fq.fp8_quant_colwise_grouped(workloads.to_torch_bf16(a, DEV), dev(d["offsets"]), FN,
                                         q_t=buf[:, :M])
    oqt, os_ = oracle.quant_colwise_grouped(a, d["offsets"], FN)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(buf[:, :M].cpu().numpy(), oqt)


@pytest.mark.parametrize("which", ["x", "dy"])
def test_dual_full_dsv3(fq, dsv3_bwd, which):
    """Both layouts of the dsv3 activations X [16384, 7168] and gradients dY [16384, 2048] in one
    call (the padded transposed buffers the weight gradient reads), every byte and scale."""
    d = dsv3_bwd
    a = d[which]
    M = d["M"]
    ldm = -(-M // 16) * 16
    buf = torch.empty((a.shape[1], ldm), dtype=torch.uint8, device=DEV)
    (q, sr), (qt, sc) = fq.fp8_quant_dual_grouped(workloads.to_torch_bf16(a, DEV),
                                                  dev(d["offsets"]), FN, q_t=buf[:, :M])
    oq, os_ = oracle.quant_rowwise(a, FN)
    assert np.array_equal(sr.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)
    del q, oq
    oqt, osc = oracle.quant_colwise_grouped(a, d["offsets"], FN)
    assert np.array_equal(sc.cpu().numpy(), osc)
    assert np.array_equal(buf[:, :M].cpu().numpy(), oqt)


def test_mx_quant_full_dsv3(fq, dsv3_fwd):
    d = dsv3_fwd
    q, e = fq.fp8_mx_quant_rowwise(workloads.to_torch_bf16(d["x"], DEV))
    oq, oe = oracle.mx_quant_rowwise(d["x"])
    assert np.array_equal(e.cpu().numpy(), oe) and np.array_equal(q.cpu().numpy(), oq)
    del q, e, oq, oe
    qt, et = fq.fp8_mx_quant_colwise(workloads.to_torch_bf16(d["w"], DEV))
    oqt, oet = oracle.mx_quant_colwise(d["w"])
    assert np.array_equal(et.cpu().numpy(), oet) and np.array_equal(qt.cpu().numpy(), oqt)


@pytest.mark.parametrize("name", ["tiny", "dense", "moe16b"])
def test_quant_full_config(fq, name):
    """The other configurations' quantizers at full size, every byte and scale: rowwise X and the
    per-expert colwise W (dense: one 4096-row group over 14336 columns; moe16b: 64 experts of
    2048 rows; both through the two-pass colwise kernels), in the configuration's encoding."""
    d = workloads.make_forward(name)
    fmt, E, K = d["fmt"], d["E"], d["K"]
    q, s = fq.fp8_quant_rowwise(workloads.to_torch_bf16(d["x"], DEV), fmt)
    oq, os_ = oracle.quant_rowwise(d["x"], fmt)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)
    del q, s, oq, os_
    off_w = (np.arange(1, E + 1) * K).astype(np.int32)
    qt, sw = fq.fp8_quant_colwise_grouped(workloads.to_torch_bf16(d["w"], DEV), dev(off_w), fmt)
    oqt, osw = oracle.quant_colwise_grouped(d["w"], off_w, fmt)
    assert np.array_equal(sw.cpu().numpy(), osw)
    assert np.array_equal(qt.cpu().numpy(), oqt)


# ----------------------------------------------------------------------------- GEMMs
# Every output element is compared: the oracle's whole-matrix GEMMs (a float64 library matmul
# over integer-scaled FP8 values, exact sums) take seconds at these sizes.

def _fwd_full(fq, d, fmt, what):
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, sa = oracle.quant_rowwise(d["x"], fmt)
    qbt, sb = oracle.quant_colwise_grouped(d["w"], (np.arange(1, E + 1) * K).astype(np.int32),
                                           fmt)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, dev(qa), dev(sa), dev(qbt), dev(sb),
                            dev(off), M, N, K, ldb=E * K, b_group_stride=K)
    got = c.float().cpu().numpy()
    del c
    ref = oracle.gemm_fwd_full(fmt, qa, sa, qbt, E * K, K, sb, off, N, K)
    mm.check_gemm(got, ref, what, mm.explain_fwd(fmt, qa, sa, qbt, E * K, K, sb, off, N, K))


@pytest.mark.parametrize("fmt", [FN, FNUZ])
def test_gemm_fwd_full_dsv3(fq, dsv3_fwd, fmt):
    """DeepSeek-V3 expert slice forward, 16384 x 2048 x 7168 over 32 Zipf groups: every row."""
    _fwd_full(fq, dsv3_fwd, fmt, f"dsv3 forward fmt {fmt}")


@pytest.mark.parametrize("name", ["tiny", "dense", "moe16b"])
def test_gemm_fwd_full_config(fq, name):
    """The other forward configurations, every row: tiny (e4m3fnuz, 1% outliers x50), the dense
    Llama3-8B FFN GEMM (8192 x 14336 x 4096) and DeepSeek-MoE-16B experts (49152 routed rows,
    64 groups, 1408 x 2048)."""
    d = workloads.make_forward(name)
    _fwd_full(fq, d, d["fmt"], f"{name} forward fmt {d['fmt']}")


def _padded(a, ldm):
    t = torch.zeros((a.shape[0], ldm), dtype=torch.uint8, device=DEV)
    t[:, :a.shape[1]] = dev(a)
    return t


@pytest.mark.parametrize("fmt", [FN, FNUZ])
def test_gemm_wgrad_full_dsv3(fq, dsv3_bwd, fmt):
    """Weight gradient dW_g = X_g^T dY_g of the 32 Zipf groups (7168 x 2048 each): every element
    of every group, in both encodings."""
    d = dsv3_bwd
    M, K, N, G, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    xt, sx = oracle.quant_colwise_grouped(d["x"], off, fmt)     # [K, M], [G, K]
    dyt, sdy = oracle.quant_colwise_grouped(d["dy"], off, fmt)  # [N, M], [G, N]
    ldm = -(-M // 16) * 16
    c = fq.fp8_grouped_gemm(fq.GEMM_WGRAD_KGROUPED, fmt, _padded(xt, ldm), dev(sx),
                            _padded(dyt, ldm), dev(sdy), dev(off), M, N, K, ldb=ldm)
    for g in range(G):
        got = c[g].float().cpu().numpy()
        ref = oracle.gemm_wgrad_group(fmt, xt, sx, dyt, sdy, off, g)
        mm.check_gemm(got, ref, f"dsv3 weight gradient fmt {fmt} group {g}",
                      mm.explain_wgrad(fmt, xt, sx, dyt, sdy, off, N, K,
                                       pairs=[(g, k) for k in range(K)]))


def test_gemm_dgrad_full_dsv3(fq, dsv3_fwd, dsv3_bwd):
    """dX = dY W^T per group at the dsv3 sizes (the bench's data-gradient launch): dY [16384,
    2048] and W [32*7168, 2048] quantized rowwise along N, output [16384, 7168], every row."""
    d = dsv3_bwd
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, sa = oracle.quant_rowwise(d["dy"], FN)
    qb, sb = oracle.quant_rowwise(dsv3_fwd["w"], FN)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, FN, dev(qa), dev(sa), dev(qb), dev(sb),
                            dev(off), M, K, N, ldb=N, b_group_stride=K * N)
    got = c.float().cpu().numpy()
    del c
    ref = oracle.gemm_fwd_full(FN, qa, sa, qb, N, K * N, sb, off, K, N)
    mm.check_gemm(got, ref, "dsv3 data gradient",
                  mm.explain_fwd(FN, qa, sa, qb, N, K * N, sb, off, K, N))


def test_mx_gemm_wgrad_full_dsv3(fq, dsv3_bwd):
    """MX backward at the dsv3 sizes: X [16384, 7168] and dY [16384, 2048] MX-quantized along
    tokens, dW [32, 7168, 2048]: every element."""
    d = dsv3_bwd
    M, K, N, G, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    xt, xe = oracle.mx_quant_colwise(d["x"])
    dyt, de = oracle.mx_quant_colwise(d["dy"])
    c = fq.fp8_mx_grouped_gemm_wgrad(dev(xt), dev(xe), dev(dyt), dev(de), dev(off), M, N, K)
    for g in range(G):
        got = c[g].float().cpu().numpy()
        ref = oracle.mx_gemm_wgrad_group(xt, xe, dyt, de, off, g)
        mm.check_gemm(got, ref, f"dsv3 MX weight gradient group {g}",
                      mm.explain_mx_wgrad(xt, xe, dyt, de, off, N, K,
                                          pairs=[(g, k) for k in range(K)]))


def test_mx_gemm_full_dsv3(fq, dsv3_fwd):
    """MXFP8 forward of the dsv3 slice: every row."""
    d = dsv3_fwd
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, ea = oracle.mx_quant_rowwise(d["x"])
    qbt, eb = oracle.mx_quant_colwise(d["w"])
    c = fq.fp8_mx_grouped_gemm(dev(qa), dev(ea), dev(qbt), dev(eb), dev(off), M, N, K,
                               ldb=E * K, b_group_stride=K, ld_sb=E * K // 32,
                               sb_group_stride=K // 32)
    got = c.float().cpu().numpy()
    del c
    ref = oracle.mx_gemm_fwd_full(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K)
    mm.check_gemm(got, ref, "dsv3 MXFP8 forward",
                  mm.explain_mx_fwd(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K))
