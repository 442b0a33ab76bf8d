"""Seeded sweep: random shapes and group layouts for the quantizers and both GEMM modes against the
oracle, beyond the hand-picked parity cases.

Each case draws its sizes from numpy PCG64(seed): row counts that are not multiples of any tile,
column counts around the 64-column strips, group layouts mixing empty groups, one-row groups and
groups longer than a band of 8 forward row tiles (2048 rows), in both encodings.  One colwise case
is large enough (65536 x 4096) for the maxima pass to walk 4 row tiles per block, the path that
the other inputs never take.  Quantized bytes and scales must match bit for bit; GEMM outputs as in
test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import mfma_model as mm

pytestmark = pytest.mark.gpu

FNUZ, FN = 0, 1
DEV = "cuda:0"


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_quantization_grouped_amd as m
    m.lib()  # raises if the HIP library is missing
    return m


def dev_bf16(bits):
    return workloads.to_torch_bf16(bits, DEV)


def dev_i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device=DEV)


def random_offsets(rng, rows, groups, big=0):
    """Cumulative group ends: `big` groups take most rows, the rest split the remainder at random
    (empty groups and one-row groups included)."""
    sizes = np.zeros(groups, np.int64)
    rest = rows
    if big:
        idx = rng.choice(groups, size=big, replace=False)
        for i in idx:
            take = int(rng.integers(rest // (2 * big), rest // big + 1)) if rest else 0
            sizes[i] = take
            rest -= take
    cuts = np.sort(rng.integers(0, rest + 1, size=groups - 1))
    parts = np.diff(np.concatenate([[0], cuts, [rest]]))
    sizes += parts
    zero = rng.random(groups) < 0.15  # some empty groups: move their rows to the next group
    for i in (np.nonzero(zero)[0] if groups > 1 else []):
        j = (i + 1) % groups
        sizes[j] += sizes[i]
        sizes[i] = 0
    assert sizes.sum() == rows
    return np.cumsum(sizes).astype(np.int32)


# ----------------------------------------------------------------------------- quantizers

@pytest.mark.parametrize("seed", range(6))
def test_sweep_colwise_grouped(fq, seed):
    rng = np.random.Generator(np.random.PCG64(9100 + seed))
    rows = int(rng.integers(1, 5000))
    cols = int(rng.choice([8, 64, 72, 200, 1024, 2056]))
    groups = int(rng.integers(1, 40))
    off = random_offsets(rng, rows, groups, big=int(rng.integers(0, 3)))
    fmt = int(rng.integers(0, 2))
    x = workloads.make_matrix(9200 + seed, rows, cols, 1.0, 0.01)
    qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x), dev_i32(off), fmt)
    oqt, os_ = oracle.quant_colwise_grouped(x, off, fmt)
    assert np.array_equal(s.cpu().numpy(), os_), (rows, cols, groups, fmt)
    assert np.array_equal(qt.cpu().numpy(), oqt), (rows, cols, groups, fmt)


def test_sweep_colwise_four_tiles_per_block(fq):
    """65536 x 4096 with 16 groups: enough (row tile, strip) pairs for the maxima pass to walk 4
    row tiles per block."""
    rng = np.random.Generator(np.random.PCG64(9300))
    rows, cols, groups = 65536, 4096, 16
    off = random_offsets(rng, rows, groups, big=2)
    x = workloads.make_matrix(9301, rows, cols)
    qt, s = fq.fp8_quant_colwise_grouped(dev_bf16(x), dev_i32(off), FN)
    oqt, os_ = oracle.quant_colwise_grouped(x, off, FN)
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(qt.cpu().numpy(), oqt)


@pytest.mark.parametrize("seed", range(3))
def test_sweep_dual(fq, seed):
    rng = np.random.Generator(np.random.PCG64(9400 + seed))
    rows = int(rng.integers(1, 3000))
    cols = int(rng.choice([8, 64, 136, 520, 2048]))
    groups = int(rng.integers(1, 24))
    off = random_offsets(rng, rows, groups, big=int(rng.integers(0, 2)))
    fmt = int(rng.integers(0, 2))
    x = workloads.make_matrix(9500 + seed, rows, cols, 1.0, 0.01)
    (q, sr), (qt, sc) = fq.fp8_quant_dual_grouped(dev_bf16(x), dev_i32(off), fmt)
    oq, os_ = oracle.quant_rowwise(x, fmt)
    oqt, osc = oracle.quant_colwise_grouped(x, off, fmt)
    assert np.array_equal(sr.cpu().numpy(), os_) and np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sc.cpu().numpy(), osc) and np.array_equal(qt.cpu().numpy(), oqt)


@pytest.mark.parametrize("seed", range(3))
def test_sweep_mx_colwise(fq, seed):
    """Row counts that are multiples of 32 but not of the 256-row tile, columns around the
    64-column strips: the E8M0 bytes of partial tiles and strips."""
    rng = np.random.Generator(np.random.PCG64(9600 + seed))
    rows = 32 * int(rng.integers(1, 100))
    cols = int(rng.choice([8, 40, 64, 200, 1000]))
    x = workloads.make_matrix(9700 + seed, rows, cols, 1.0, 0.01)
    qt, e8 = fq.fp8_mx_quant_colwise(dev_bf16(x))
    oqt, oe = oracle.mx_quant_colwise(x)
    assert np.array_equal(e8.cpu().numpy(), oe), (rows, cols)
    assert np.array_equal(qt.cpu().numpy(), oqt), (rows, cols)


# ----------------------------------------------------------------------------- grouped GEMMs

FWD_SWEEP = [
    # seed, M, K, N, groups, big groups (one big group takes at least half the rows: in the
    # first two cases it is longer than a band of 8 row tiles)
    (0, 4200, 128, 600, 5, 1),
    (1, 5000, 144, 300, 3, 1),
    (2, 1700, 256, 520, 12, 0),
    (3, 333, 400, 70, 9, 0),
]


@pytest.mark.parametrize("case", FWD_SWEEP)
def test_sweep_gemm_fwd(fq, case):
    seed, M, K, N, E, big = case
    rng = np.random.Generator(np.random.PCG64(9800 + seed))
    off = random_offsets(rng, M, E, big=big)
    if M >= 4200:
        assert np.diff(np.concatenate([[0], off])).max() > 2048  # crosses a band
    fmt = int(rng.integers(0, 2))
    x = workloads.make_matrix(9900 + seed, M, K, 1.0, 0.01)
    w = workloads.make_matrix(9950 + seed, E * K, N, 0.02)
    qa, sa = oracle.quant_rowwise(x, fmt)
    qbt, sb = oracle.quant_colwise_grouped(w, (np.arange(1, E + 1) * K).astype(np.int32), fmt)
    c = fq.fp8_grouped_gemm(fq.GEMM_FWD_MGROUPED, fmt, torch.from_numpy(qa).to(DEV),
                            torch.from_numpy(sa).to(DEV), torch.from_numpy(qbt).to(DEV),
                            torch.from_numpy(sb).to(DEV), dev_i32(off), M, N, K,
                            ldb=E * K, b_group_stride=K)
    ref = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, np.arange(M))
    mm.check_gemm(c.float().cpu().numpy(), ref, f"sweep fwd {case} fmt {fmt}",
                  mm.explain_fwd(fmt, qa, sa, qbt, E * K, K, sb, off, N, K))


WGRAD_SWEEP = [
    # seed, M (tokens), K, N, groups
    (0, 1500, 272, 96, 7),
    (1, 640, 64, 330, 4),
    (2, 2100, 128, 128, 15),
]


@pytest.mark.parametrize("case", WGRAD_SWEEP)
def test_sweep_gemm_wgrad(fq, case):
    seed, M, K, N, G = case
    rng = np.random.Generator(np.random.PCG64(10000 + seed))
    off = random_offsets(rng, M, G, big=1)
    fmt = int(rng.integers(0, 2))
    x = workloads.make_matrix(10100 + seed, M, K)
    dy = workloads.make_matrix(10150 + seed, M, N)
    xt, sx = oracle.quant_colwise_grouped(x, off, fmt)
    dyt, sdy = oracle.quant_colwise_grouped(dy, off, fmt)
    ldp = -(-M // 16) * 16

    def padded(a):
        t = torch.zeros((a.shape[0], ldp), dtype=torch.uint8, device=DEV)
        t[:, :M] = torch.from_numpy(a).to(DEV)
        return t

    c = fq.fp8_grouped_gemm(fq.GEMM_WGRAD_KGROUPED, fmt, padded(xt),
                            torch.from_numpy(sx).to(DEV), padded(dyt),
                            torch.from_numpy(sdy).to(DEV), dev_i32(off), M, N, K, ldb=ldp)
    gi = np.repeat(np.arange(G, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), G)
    ref = oracle.gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, off, N, K, gi, ki).reshape(G, K, N)
    mm.check_gemm(c.float().cpu().numpy(), ref, f"sweep wgrad {case} fmt {fmt}",
                  mm.explain_wgrad(fmt, xt, sx, dyt, sdy, off, N, K))
