"""GPU parity at the configurations' full sizes, through the C ABI, in the launch
configuration the benchmark times (same entry points, shapes, layouts and strides).

Quantizers: every byte and scale is compared with the oracle (bit-exact).  GEMMs: the oracle
computes sampled output rows one by one -- every group's first and last row plus seeded random
rows (forward), or sampled (group, k) rows of dW (weight gradient) -- and each sampled element
must lie within 1e-3 + 1e-2*|exact|.  The operands fed to the GEMMs are the oracle's quantized
bytes, so no input or expected value comes from the GPU path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.mfma_bound import (check_tol_hw, mx_wgrad_block_truncation_bound,
                               wgrad_block_truncation_bound)

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


def check_tol(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    excess = np.abs(got - ref) - (1e-3 + 1e-2 * np.abs(ref))
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (f"{what}: |err| {abs(got.flat[i] - ref.flat[i]):.4g} at flat "
                                 f"{i} (gpu {got.flat[i]:.6g}, oracle {ref.flat[i]:.6g})")


def sample_rows(offsets, M, n_random, seed):
    """Every non-empty group's first and last row plus n_random seeded rows."""
    off = np.asarray(offsets, np.int64)
    starts = np.concatenate([[0], off[:-1]])
    ne = off > starts
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([starts[ne], off[ne] - 1, rng.integers(0, M, n_random)]))


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


def test_mx_quant_full_dsv3(fq, dsv3_fwd):
    d = dsv3_fwd
    q, e = fq.fp8_mx_quant_rowwise(workloads.to_torch_bf16(d["x"], DEV))
    oq, oe = oracle.mx_quant_rowwise(d["x"])
    assert np.array_equal(e.cpu().numpy(), oe) and np.array_equal(q.cpu().numpy(), oq)
    del q, e, oq, oe
    qt, et = fq.fp8_mx_quant_colwise(workloads.to_torch_bf16(d["w"], DEV))
    oqt, oet = oracle.mx_quant_colwise(d["w"])
    assert np.array_equal(et.cpu().numpy(), oet) and np.array_equal(qt.cpu().numpy(), oqt)


# ----------------------------------------------------------------------------- GEMMs

def _fwd_case(fq, d, fmt, n_random, what):
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, sa = oracle.quant_rowwise(d["x"], fmt)
    qbt, sb = oracle.quant_colwise_grouped(d["w"], (np.arange(1, E + 1) * K).astype(np.int32),
                                           fmt)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, dev(qa), dev(sa), dev(qbt), dev(sb),
                            dev(off), M, N, K, ldb=E * K, b_group_stride=K)
    rows = sample_rows(off, M, n_random, 17)
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, rows)
    check_tol(got, ref, what)


@pytest.mark.parametrize("fmt", [FN, FNUZ])
def test_gemm_fwd_full_dsv3(fq, dsv3_fwd, fmt):
    _fwd_case(fq, dsv3_fwd, fmt, 96, f"dsv3 forward fmt {fmt}")


@pytest.mark.parametrize("name", ["dense", "moe16b"])
def test_gemm_fwd_full_config(fq, name):
    d = workloads.make_forward(name, FN)
    _fwd_case(fq, d, FN, 48, name)


def test_gemm_wgrad_full_dsv3(fq, dsv3_bwd):
    d = dsv3_bwd
    M, K, N, G, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    xt, sx = oracle.quant_colwise_grouped(d["x"], off, FN)     # [K, M], [G, K]
    dyt, sdy = oracle.quant_colwise_grouped(d["dy"], off, FN)  # [N, M], [G, N]
    ldm = -(-M // 16) * 16

    def padded(a):
        t = torch.zeros((a.shape[0], ldm), dtype=torch.uint8, device=DEV)
        t[:, :M] = dev(a)
        return t

    c = fq.fp8_grouped_gemm(fq.GEMM_WGRAD_KGROUPED, FN, padded(xt), dev(sx), padded(dyt),
                            dev(sdy), dev(off), M, N, K, ldb=ldm)
    rng = np.random.default_rng(23)
    gi = np.repeat(np.arange(G, dtype=np.int32), 4)
    ki = np.stack([np.zeros(G, np.int64), np.full(G, K - 1, np.int64),
                   rng.integers(0, K, G), rng.integers(0, K, G)], axis=1).reshape(-1)
    got = c[torch.from_numpy(gi.astype(np.int64)).to(DEV),
            torch.from_numpy(ki).to(DEV)].float().cpu().numpy()
    ref = oracle.gemm_wgrad_rows(FN, xt, sx, dyt, sdy, off, N, K, gi, ki)
    # outputs here reach |dW| ~ 100, so a cancelling element can sit below the 1e-3 absolute
    # bar by less than the matrix cores' block truncation; see wgrad_block_truncation_bound
    hw = wgrad_block_truncation_bound(FN, xt, sx, dyt, sdy, off, gi, ki)
    check_tol_hw(got, ref, hw, "dsv3 weight gradient")


def test_gemm_dgrad_full_dsv3(fq, dsv3_fwd, dsv3_bwd):
    """dX = dY W^T per group at the dsv3 sizes (the bench's data-gradient launch): dY [16384,
    2048] and W [32*7168, 2048] quantized rowwise along N, output [16384, 7168]."""
    d = dsv3_bwd
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, sa = oracle.quant_rowwise(d["dy"], FN)
    qb, sb = oracle.quant_rowwise(dsv3_fwd["w"], FN)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, FN, dev(qa), dev(sa), dev(qb), dev(sb),
                            dev(off), M, K, N, ldb=N, b_group_stride=K * N)
    rows = sample_rows(off, M, 64, 29)
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = oracle.gemm_fwd_rows(FN, qa, sa, qb, N, K * N, sb, off, K, N, rows)
    check_tol(got, ref, "dsv3 data gradient")


def test_mx_gemm_wgrad_full_dsv3(fq, dsv3_bwd):
    """MX backward at the dsv3 sizes: X [16384, 7168] and dY [16384, 2048] MX-quantized along
    tokens, dW [32, 7168, 2048]; four sampled (group, k) rows per group."""
    d = dsv3_bwd
    M, K, N, G, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    xt, xe = oracle.mx_quant_colwise(d["x"])
    dyt, de = oracle.mx_quant_colwise(d["dy"])
    c = fq.fp8_mx_grouped_gemm_wgrad(dev(xt), dev(xe), dev(dyt), dev(de), dev(off), M, N, K)
    rng = np.random.default_rng(31)
    gi = np.repeat(np.arange(G, dtype=np.int32), 4)
    ki = np.stack([np.zeros(G, np.int64), np.full(G, K - 1, np.int64),
                   rng.integers(0, K, G), rng.integers(0, K, G)], axis=1).reshape(-1)
    got = c[torch.from_numpy(gi.astype(np.int64)).to(DEV),
            torch.from_numpy(ki).to(DEV)].float().cpu().numpy()
    ref = oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, off, N, gi, ki)
    hw = mx_wgrad_block_truncation_bound(xt, xe, dyt, de, off, gi, ki)
    check_tol_hw(got, ref, hw, "dsv3 MX weight gradient")


def test_mx_gemm_full_dsv3(fq, dsv3_fwd):
    d = dsv3_fwd
    M, K, N, E, off = d["M"], d["K"], d["N"], d["E"], d["offsets"]
    qa, ea = oracle.mx_quant_rowwise(d["x"])
    qbt, eb = oracle.mx_quant_colwise(d["w"])
    c = fq.fp8_mx_grouped_gemm(dev(qa), dev(ea), dev(qbt), dev(eb), dev(off), M, N, K,
                               ldb=E * K, b_group_stride=K, ld_sb=E * K // 32,
                               sb_group_stride=K // 32)
    rows = sample_rows(off, M, 96, 19)
    got = c[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = oracle.mx_gemm_fwd_rows(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K,
                                  rows)
    check_tol(got, ref, "dsv3 MXFP8 forward")
