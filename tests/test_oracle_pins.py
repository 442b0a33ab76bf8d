"""Pins of the CPU oracle to facts fixed outside the oracle itself (CPU only).

Each test checks an oracle function against one of: a value the pages state (golden file), a
library routine (torch's float8 dtypes, numpy matmul), brute-force search, exact rational or
integer arithmetic, or a metamorphic property that a dropped term, wrong sign, wrong index or
transposed operand would break.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import pinlib

FNUZ, FN = 0, 1
FMT = [FNUZ, FN]
EPS = np.float32(1e-12)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "codec_spot_values.txt")


# ----------------------------------------------------------------------------- codec

def test_codec_golden_spot_values():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt_s, byte_s, val_s = line.split()[:3]
        fmt = FNUZ if fmt_s == "fnuz" else FN
        got = oracle.decode(fmt, int(byte_s, 16))
        if val_s == "nan":
            assert math.isnan(got), line
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), line
        n += 1
    assert n >= 10


@pytest.mark.parametrize("fmt", FMT)
def test_decode_matches_library(fmt):
    tab = pinlib.torch_decode_table(fmt)
    for b in range(256):
        got = oracle.decode(fmt, b)
        if math.isnan(tab[b]):
            assert math.isnan(got), hex(b)
        else:
            assert got == tab[b], hex(b)


def test_decode_cross_format_half():
    # a fnuz code's value is half the fn value of the same byte, except the three special codes
    for b in range(256):
        if b in (0x80, 0x7F, 0xFF):
            continue
        assert oracle.decode(FNUZ, b) == oracle.decode(FN, b) / 2, hex(b)


@pytest.mark.parametrize("fmt", FMT)
def test_format_range_and_special_codes(fmt):
    vals = np.array([oracle.decode(fmt, b) for b in range(256)])
    fin = vals[np.isfinite(vals)]
    assert np.abs(fin).max() == pinlib.FMAX[fmt]
    if fmt == FNUZ:
        # a single NaN code (0x80) and a single zero: 255 finite codes, 255 distinct values
        assert np.isnan(vals).sum() == 1 and math.isnan(vals[0x80])
        assert len(np.unique(fin)) == 255
        assert not any(v == 0 and math.copysign(1, v) < 0 for v in fin)
    else:
        assert np.isnan(vals).sum() == 2 and math.isnan(vals[0x7F]) and math.isnan(vals[0xFF])
        assert len(np.unique(fin)) == 253  # +0 and -0 compare equal


@pytest.mark.parametrize("fmt", FMT)
def test_encode_brute_force(fmt):
    y = pinlib.encode_probe_values(fmt, n_random=300_000)
    got = oracle.encode_array(fmt, y)
    want = pinlib.brute_encode(fmt, y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]
    lib = pinlib.torch_encode(fmt, y)
    bad = np.nonzero(got != lib)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(lib[i])) for i in bad[:8]]


@pytest.mark.parametrize("fmt", FMT)
def test_encode_monotone_and_zero_sign(fmt):
    y = np.sort(pinlib.encode_probe_values(fmt, n_random=50_000))
    q = oracle.encode_array(fmt, y)
    dec = np.array([oracle.decode(fmt, b) for b in range(256)])
    v = dec[q]
    assert np.all(np.diff(v) >= 0)
    if fmt == FNUZ:
        assert not np.any(q == 0x80)
        assert oracle.encode(FNUZ, -0.0) == 0 and oracle.encode(FNUZ, -1e-6) == 0
    else:
        assert oracle.encode(FN, -0.0) == 0x80 and oracle.encode(FN, -1e-6) == 0x80


# ----------------------------------------------------------------------------- scale

def _is_correctly_rounded_f32(s: np.float32, exact: Fraction) -> bool:
    s = np.float32(s)
    lo = np.nextafter(s, np.float32(0))
    hi = np.nextafter(s, np.float32(np.inf))
    fs = Fraction(float(s))
    d = abs(fs - exact)
    if d > abs(Fraction(float(lo)) - exact) or d > abs(Fraction(float(hi)) - exact):
        return False
    if d == abs(Fraction(float(hi)) - exact) or d == abs(Fraction(float(lo)) - exact):
        return int(np.float32(s).view(np.uint32)) % 2 == 0  # tie: even significand
    return True


@pytest.mark.parametrize("fmt", FMT)
def test_scale_exhaustive_over_bf16_amax(fmt):
    # every positive finite bf16 value as a row absmax: s is FMAX / max(amax, 1e-12f) rounded
    # once to fp32 (checked in exact rational arithmetic)
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    amax = (bits << 16).view(np.float32)
    eps = Fraction(float(EPS))
    fm = Fraction(int(pinlib.FMAX[fmt]))
    for a in amax[::1]:
        s = oracle.scale(fmt, float(a))
        d = max(Fraction(float(a)), eps)
        assert _is_correctly_rounded_f32(s, fm / d), (float(a), float(s))


# ----------------------------------------------------------------------------- rowwise

def _rows(seed, rows, cols, outliers=0.01):
    return workloads.make_matrix(seed, rows, cols, 1.0, outliers, 50.0)


@pytest.mark.parametrize("fmt", FMT)
def test_rowwise_saturation_and_scale(fmt):
    x = _rows(1, 64, 300)
    q, s = oracle.quant_rowwise(x, fmt)
    xf = workloads.bf16_bits_to_f32(x)
    dec = pinlib.torch_decode_table(fmt)[q]
    amax = np.abs(xf).max(axis=1)
    maxcode = 0x7F if fmt == FNUZ else 0x7E
    for r in range(x.shape[0]):
        assert s[r] == oracle.scale(fmt, amax[r])
        assert np.abs(dec[r]).max() == pinlib.FMAX[fmt]
        i = int(np.argmax(np.abs(xf[r])))
        assert q[r, i] & 0x7F == maxcode
    assert np.all(np.abs(dec) <= pinlib.FMAX[fmt])


@pytest.mark.parametrize("fmt", FMT)
def test_rowwise_roundtrip_bound(fmt):
    x = _rows(2, 32, 512)
    q, s = oracle.quant_rowwise(x, fmt)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    dec = pinlib.torch_decode_table(fmt)[q]
    y = np.abs(xf * s[:, None].astype(np.float64))
    sub_step = 2.0 ** pinlib.QUANTUM_LOG2[fmt]
    minnorm = sub_step * 8
    e = np.floor(np.log2(np.maximum(y, minnorm)))
    ulp = np.where(y < minnorm, sub_step, np.exp2(e - 3))
    bound = (0.5 * ulp + y * 2.0 ** -24) / s[:, None]
    err = np.abs(dec / s[:, None] - xf)
    assert np.all(err <= bound * (1 + 1e-12))


@pytest.mark.parametrize("fmt", FMT)
def test_rowwise_matches_library_cast(fmt):
    # brute force over every finite bf16 value in a row whose absmax is fixed at 3.0
    allb = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = workloads.bf16_bits_to_f32(allb)
    keep = np.isfinite(f) & (np.abs(f) <= 3.0)
    vals = allb[keep]
    row = np.concatenate([vals, np.array([0x4040], np.uint16)])  # 0x4040 = 3.0
    q, s = oracle.quant_rowwise(row[None, :], fmt)
    assert s[0] == oracle.scale(fmt, 3.0)
    y = workloads.bf16_bits_to_f32(row) * s[0]
    y = np.clip(y, -pinlib.FMAX[fmt], pinlib.FMAX[fmt]).astype(np.float32)
    assert np.array_equal(q[0], pinlib.torch_encode(fmt, y))


@pytest.mark.parametrize("fmt", FMT)
def test_rowwise_metamorphic(fmt):
    x = _rows(3, 16, 256, outliers=0.0)
    q, s = oracle.quant_rowwise(x, fmt)
    xf = workloads.bf16_bits_to_f32(x)
    # scaling by 2^k (exact in bf16 here) leaves bytes unchanged and divides s by 2^k exactly
    for k in (-5, 3):
        xs = workloads.f32_to_bf16_bits(xf * np.float32(2.0 ** k))
        q2, s2 = oracle.quant_rowwise(xs, fmt)
        assert np.array_equal(q, q2)
        assert np.array_equal(s2, (s / np.float32(2.0 ** k)).astype(np.float32))
    # negation flips the sign bit (fnuz zero stays 0x00)
    qn, sn = oracle.quant_rowwise(x ^ np.uint16(0x8000), fmt)
    assert np.array_equal(s, sn)
    flip = q ^ np.uint8(0x80)
    if fmt == FNUZ:
        flip = np.where(q == 0, np.uint8(0), flip)
    assert np.array_equal(qn, flip)
    # permuting columns permutes bytes
    perm = np.random.default_rng(0).permutation(x.shape[1])
    qp, sp = oracle.quant_rowwise(x[:, perm], fmt)
    assert np.array_equal(qp, q[:, perm]) and np.array_equal(sp, s)


@pytest.mark.parametrize("fmt", FMT)
def test_rowwise_zero_row(fmt):
    x = np.zeros((2, 40), np.uint16)
    x[1, ::2] = 0x8000  # negative zeros
    q, s = oracle.quant_rowwise(x, fmt)
    assert np.all(s == np.float32(pinlib.FMAX[fmt]) / EPS)
    if fmt == FNUZ:
        assert np.all(q == 0)
    else:
        assert np.all(q[0] == 0) and np.all(q[1, ::2] == 0x80) and np.all(q[1, 1::2] == 0)


def test_wrong_format_max_clips():
    # the format-correctness point: scaling against 448 but casting into the 240-max format
    # clips every element above 240 (many per row); scaling against 240 saturates only the
    # absmax neighbourhood
    x = _rows(4, 8, 1024, outliers=0.0)
    xf = workloads.bf16_bits_to_f32(x)
    amax = np.abs(xf).max(axis=1, keepdims=True)
    wrong = np.abs(xf * (np.float32(448.0) / amax)) > 240.0
    q, s = oracle.quant_rowwise(x, FNUZ)
    sat = (q & 0x7F) == 0x7F
    assert wrong.sum() > 10 * sat.sum()


# ----------------------------------------------------------------------------- colwise grouped

@pytest.mark.parametrize("fmt", FMT)
def test_colwise_single_group_is_rowwise_of_transpose(fmt):
    x = _rows(5, 200, 72)
    qt, s = oracle.quant_colwise_grouped(x, np.array([200], np.int32), fmt)
    q2, s2 = oracle.quant_rowwise(np.ascontiguousarray(x.T), fmt)
    assert np.array_equal(qt, q2) and np.array_equal(s[0], s2)


@pytest.mark.parametrize("fmt", FMT)
def test_colwise_group_split_and_empty_groups(fmt):
    x = _rows(6, 300, 40)
    off = np.array([0, 37, 37, 180, 181, 300, 300], np.int32)
    qt, s = oracle.quant_colwise_grouped(x, off, fmt)
    start = 0
    for g, end in enumerate(off):
        if end == start:
            assert np.all(s[g] == np.float32(pinlib.FMAX[fmt]) / EPS)
        else:
            qg, sg = oracle.quant_colwise_grouped(x[start:end], np.array([end - start], np.int32), fmt)
            assert np.array_equal(qt[:, start:end], qg) and np.array_equal(s[g], sg[0])
        start = end


@pytest.mark.parametrize("fmt", FMT)
def test_colwise_row_permutation_within_group(fmt):
    x = _rows(7, 120, 24)
    off = np.array([50, 120], np.int32)
    qt, s = oracle.quant_colwise_grouped(x, off, fmt)
    perm = np.concatenate([np.random.default_rng(1).permutation(50), 50 + np.arange(70)])
    qp, sp = oracle.quant_colwise_grouped(x[perm], off, fmt)
    assert np.array_equal(sp, s) and np.array_equal(qp, qt[:, perm])


@pytest.mark.parametrize("fmt", FMT)
def test_colwise_uniform_groups_match_rowwise_on_expert_layout(fmt):
    E, K, N = 3, 64, 48
    w = workloads.make_matrix(8, E * K, N, 0.02)
    off = (np.arange(1, E + 1) * K).astype(np.int32)
    qt, s = oracle.quant_colwise_grouped(w, off, fmt)
    for e in range(E):
        we_t = np.ascontiguousarray(w[e * K:(e + 1) * K].T)  # [N, K]
        q2, s2 = oracle.quant_rowwise(we_t, fmt)
        assert np.array_equal(qt[:, e * K:(e + 1) * K], q2) and np.array_equal(s[e], s2)


# ----------------------------------------------------------------------------- grouped GEMM

def _quantized_operands(fmt, M, K, N, E, seed, offsets):
    x = workloads.make_matrix(seed, M, K, 1.0, 0.01)
    w = workloads.make_matrix(seed + 100, E * K, N, 0.02)
    qa, sa = oracle.quant_rowwise(x, fmt)
    qbt, sb = oracle.quant_colwise_grouped(w, (np.arange(1, E + 1) * K).astype(np.int32), fmt)
    return qa, sa, qbt, sb  # qbt: [N, E*K]


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_fwd_exact_integer_sums(fmt):
    M, K, N, E = 90, 160, 24, 3
    off = np.array([30, 30, 90], np.int32)
    qa, sa, qbt, sb = _quantized_operands(fmt, M, K, N, E, 11, off)
    out = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, np.arange(M))
    ia = pinlib.int_repr(fmt, qa)
    ib = pinlib.int_repr(fmt, qbt)
    start = 0
    for g, end in enumerate(off):
        if end == start:
            continue
        exact = ia[start:end] @ ib[:, g * K:(g + 1) * K].T  # int64, exact
        acc = out[start:end] * (sa[start:end, None].astype(np.float64) * sb[g][None, :].astype(np.float64))
        want = np.ldexp(exact.astype(np.float64), 2 * pinlib.QUANTUM_LOG2[fmt])
        assert np.allclose(acc, want, rtol=4e-16, atol=0)
        start = end


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_fwd_constant_closed_form(fmt):
    # x == cx, w == cw with FMAX/cx and FMAX/cw powers of two: every quantized value is FMAX and
    # C = K * cx * cw exactly
    M, K, N = 8, 96, 16
    fm = pinlib.FMAX[fmt]
    cx, cw = fm / 256, fm / 1024
    x = workloads.f32_to_bf16_bits(np.full((M, K), cx, np.float32))
    w = workloads.f32_to_bf16_bits(np.full((K, N), cw, np.float32))
    assert np.all(workloads.bf16_bits_to_f32(x) == np.float32(cx))
    qa, sa = oracle.quant_rowwise(x, fmt)
    qbt, sb = oracle.quant_colwise_grouped(w, np.array([K], np.int32), fmt)
    out = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, K, 0, sb, np.array([M], np.int32), N, K, np.arange(M))
    assert np.all(out == K * np.float64(np.float32(cx)) * np.float64(np.float32(cw)))


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_fwd_g1_equals_library_matmul(fmt):
    M, K, N = 40, 256, 32
    qa, sa, qbt, sb = _quantized_operands(fmt, M, K, N, 1, 12, None)
    out = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, K, 0, sb, np.array([M], np.int32), N, K, np.arange(M))
    tab = pinlib.torch_decode_table(fmt)
    ref = (tab[qa] @ tab[qbt].T) / (sa[:, None].astype(np.float64) * sb[0][None, :].astype(np.float64))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_wgrad_exact_integer_sums_and_empty_group(fmt):
    M, K, N = 150, 48, 40
    off = np.array([20, 20, 149, 150], np.int32)
    x = workloads.make_matrix(21, M, K)
    dy = workloads.make_matrix(22, M, N)
    xt, sx = oracle.quant_colwise_grouped(x, off, fmt)    # [K, M], [G, K]
    dyt, sdy = oracle.quant_colwise_grouped(dy, off, fmt)  # [N, M], [G, N]
    G = off.size
    gi = np.repeat(np.arange(G, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), G)
    out = oracle.gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, off, N, K, gi, ki).reshape(G, K, N)
    ix = pinlib.int_repr(fmt, xt)
    idy = pinlib.int_repr(fmt, dyt)
    start = 0
    for g, end in enumerate(off):
        if end == start:
            assert np.all(out[g] == 0)
        else:
            exact = ix[:, start:end] @ idy[:, start:end].T
            acc = out[g] * (sx[g][:, None].astype(np.float64) * sdy[g][None, :].astype(np.float64))
            want = np.ldexp(exact.astype(np.float64), 2 * pinlib.QUANTUM_LOG2[fmt])
            assert np.allclose(acc, want, rtol=4e-16, atol=0)
        start = end


def test_bf16_output_rounding_is_nearest_even():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000),
                           [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]])
    for v in vals:
        b = oracle.f64_to_bf16(v)
        got = float(workloads.bf16_bits_to_f32(np.array([b], np.uint16))[0])
        # neighbours of the result in bf16
        up = float(workloads.bf16_bits_to_f32(np.array([b + 1], np.uint16))[0])
        dn = float(workloads.bf16_bits_to_f32(np.array([b - 1 if b & 0x7FFF else b], np.uint16))[0])
        d = abs(Fraction(got) - Fraction(v))
        assert d <= abs(Fraction(up) - Fraction(v)) and d <= abs(Fraction(dn) - Fraction(v))
        if d == abs(Fraction(up) - Fraction(v)) and up != got:
            assert b % 2 == 0
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80      # tie -> even (1.0)
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even (1 + 2^-6)


# ----------------------------------------------------------------------------- MXFP8

def test_mx_exponent_exhaustive_over_bf16_block_max():
    # block = [a, 0, ..., 0] for every positive finite bf16 a: the E8M0 byte equals
    # max(biased_exponent(a) - 8, 0) read off the bf16 bit fields
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    x = np.zeros((bits.size, 32), np.uint16)
    x[:, 5] = bits
    q, e8 = oracle.mx_quant_rowwise(x)
    want = np.maximum((bits.astype(np.int64) >> 7) - 8, 0)
    assert np.array_equal(e8[:, 0].astype(np.int64), want)
    # the block max decodes into [256, 448] whenever the scale is not clamped at 2^-127
    dec = pinlib.torch_decode_table(FN)[q[:, 5]] * np.exp2(e8[:, 0].astype(np.float64) - 127)
    ok = e8[:, 0] > 0
    qmax = pinlib.torch_decode_table(FN)[q[ok, 5]]
    assert np.all((qmax >= 256) & (qmax <= 448))
    xf = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    rel = np.abs(dec[ok] - xf[ok]) / xf[ok]
    # the floor rule puts the block max in [256, 512) before the cast: up to 448 it is an
    # ordinary rounding (relative error <= 2^-4); above, it saturates (error < 64/512)
    scaled = xf[ok] * np.exp2(127.0 - e8[ok, 0])
    assert rel[scaled <= 448].max() <= 2.0 ** -4
    assert rel.max() < 1.0 / 8


def test_mx_saturation_and_power_of_two_roundtrip():
    # a block with max 1.984375 (e = -8): elements in (448, 512)*2^-8 saturate to 448 * 2^-8
    row = np.zeros((1, 32), np.float32)
    row[0, :4] = [1.984375, 1.78125, -1.9375, 1.0]
    q, e8 = oracle.mx_quant_rowwise(workloads.f32_to_bf16_bits(row))
    assert e8[0, 0] == 127 - 8
    assert q[0, 0] == 0x7E and q[0, 2] == 0xFE  # 508 and -496 saturate to +-448
    assert q[0, 1] == 0x7E                       # 456 also rounds/saturates to 448
    # powers of two within the block's range are exact
    p2 = np.zeros((1, 32), np.float32)
    p2[0, :] = [2.0 ** (-k) for k in range(32)]
    q2, e2 = oracle.mx_quant_rowwise(workloads.f32_to_bf16_bits(p2))
    dec = pinlib.torch_decode_table(FN)[q2[0]] * 2.0 ** (int(e2[0, 0]) - 127)
    lim = 2.0 ** (int(e2[0, 0]) - 127 - 9)  # smallest fn subnormal at this scale
    exact = p2[0] >= lim
    assert np.array_equal(dec[exact], p2[0][exact].astype(np.float64))


def test_mx_colwise_is_rowwise_of_transpose():
    x = workloads.make_matrix(31, 96, 40, 1.0, 0.02)
    qt, et = oracle.mx_quant_colwise(x)
    q2, e2 = oracle.mx_quant_rowwise(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q2) and np.array_equal(et, e2)


def test_mx_gemm_exact_block_sums():
    M, K, N, E = 48, 128, 20, 2
    off = np.array([17, 48], np.int32)
    x = workloads.make_matrix(41, M, K, 1.0, 0.01)
    w = workloads.make_matrix(42, E * K, N, 0.02)
    qa, ea = oracle.mx_quant_rowwise(x)
    qbt, eb = oracle.mx_quant_colwise(w)  # [N, E*K], [N, E*K/32]
    out = oracle.mx_gemm_fwd_rows(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K,
                                  np.arange(M))
    ia = pinlib.int_repr(FN, qa)
    ib = pinlib.int_repr(FN, qbt)
    start = 0
    for g, end in enumerate(off):
        for m in range(start, end):
            for n in range(N):
                tot = Fraction(0)
                for kb in range(K // 32):
                    s = int(np.dot(ia[m, kb * 32:(kb + 1) * 32], ib[n, g * K + kb * 32:g * K + (kb + 1) * 32]))
                    e = int(ea[m, kb]) - 127 + int(eb[n, g * K // 32 + kb]) - 127 - 18
                    tot += Fraction(s) * (Fraction(2) ** e)
                assert abs(Fraction(out[m - 0, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 300)
        start = end


def _mx_wgrad_operands(M, K, N, seed):
    """XqT, dYqT and their E8M0 bytes from the MX colwise oracle (blocks of 32 tokens)."""
    x = workloads.make_matrix(seed, M, K, 1.0, 0.01)
    dy = workloads.make_matrix(seed + 1, M, N)
    xt, xe = oracle.mx_quant_colwise(x)      # [K, M], [K, M/32]
    dyt, de = oracle.mx_quant_colwise(dy)    # [N, M], [N, M/32]
    return xt, xe, dyt, de


def test_mx_wgrad_unit_scales_equal_plain_wgrad():
    """With every E8M0 byte 127 (2^0) the MX weight gradient is the plain FP8 one with unit
    scales (a separately pinned oracle function)."""
    M, K, N = 96, 40, 24
    off = np.array([10, 10, 61, 96], np.int32)
    xt, _, dyt, _ = _mx_wgrad_operands(M, K, N, 61)
    ones_x = np.full((K, M // 32), 127, np.uint8)
    ones_d = np.full((N, M // 32), 127, np.uint8)
    gi = np.repeat(np.arange(4, dtype=np.int32), K)
    ki = np.tile(np.arange(K, dtype=np.int64), 4)
    got = oracle.mx_gemm_wgrad_rows(xt, ones_x, dyt, ones_d, off, N, gi, ki)
    ref = oracle.gemm_wgrad_rows(FN, xt, np.ones((4, K), np.float32), dyt,
                                 np.ones((4, N), np.float32), off, N, K, gi, ki)
    assert np.array_equal(got, ref)
    assert np.all(got[gi == 1] == 0.0)  # the empty group


def test_mx_wgrad_single_group_is_mx_forward_over_tokens():
    """One group holding every token: dW[k, n] is the MX forward GEMM of the rows of XqT against
    the rows of dYqT, contracting over tokens (the separately pinned MX forward oracle)."""
    M, K, N = 128, 24, 20
    xt, xe, dyt, de = _mx_wgrad_operands(M, K, N, 63)
    got = oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, np.array([M], np.int32), N,
                                    np.zeros(K, np.int32), np.arange(K, dtype=np.int64))
    ref = oracle.mx_gemm_fwd_rows(xt, xe, dyt, M, 0, de, M // 32, 0, np.array([K], np.int32), N,
                                  M, np.arange(K))
    assert np.array_equal(got, ref)


def test_mx_wgrad_split_inside_a_block_is_additive():
    """Splitting a group inside a 32-token block: both parts keep that block's (absolute) scale,
    so their gradients add up to the merged group's (a group-relative block index would not)."""
    M, K, N = 128, 16, 12
    xt, xe, dyt, de = _mx_wgrad_operands(M, K, N, 67)
    ks = np.arange(K, dtype=np.int64)
    merged = oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, np.array([20, 110, 128], np.int32), N,
                                       np.full(K, 1, np.int32), ks)
    split = np.array([20, 45, 77, 110, 128], np.int32)
    parts = [oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, split, N, np.full(K, g, np.int32), ks)
             for g in (1, 2, 3)]
    assert np.allclose(parts[0] + parts[1] + parts[2], merged, rtol=1e-12, atol=0)
    assert not np.array_equal(parts[0], merged)


# ----------------------------------------------------------------------------- whole-matrix GEMMs

@pytest.mark.parametrize("fmt", FMT)
def test_gemm_fwd_full_exact_integer_sums(fmt):
    """gemm_fwd_full (library matmul as the summation step): every row equals the exact int64
    sum (torch's decode tables) scaled by the float64 scale product, and the row-by-row C
    oracle bit for bit; an empty group and rows of no group give zeros."""
    M, K, N, E = 120, 176, 40, 4
    off = np.array([33, 33, 100, 120], np.int32)
    qa, sa, qbt, sb = _quantized_operands(fmt, M, K, N, E, 31, off)
    full = oracle.gemm_fwd_full(fmt, qa, sa, qbt, E * K, K, sb, off, N, K)
    rows = oracle.gemm_fwd_rows(fmt, qa, sa, qbt, E * K, K, sb, off, N, K, np.arange(M))
    assert np.array_equal(full, rows)
    ia = pinlib.int_repr(fmt, qa)
    ib = pinlib.int_repr(fmt, qbt)
    start = 0
    for g, end in enumerate(off):
        if end > start:
            exact = ia[start:end] @ ib[:, g * K:(g + 1) * K].T
            want = np.ldexp(exact.astype(np.float64), 2 * pinlib.QUANTUM_LOG2[fmt]) / (
                sa[start:end, None].astype(np.float64) * sb[g][None, :].astype(np.float64))
            assert np.array_equal(full[start:end], want)
        start = end


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_fwd_full_extreme_magnitudes_stay_exact(fmt):
    """Every operand byte at the format's largest magnitude with alternating signs over a long
    contraction (K = 16384): the partial sums reach K * FMAX^2 in the integer-scaled domain and
    must still be exact (the integer closed form), which a float32 or low-precision sum fails."""
    M, K, N = 4, 16384, 3
    top = 0x7F if fmt == FNUZ else 0x7E
    qa = np.full((M, K), top, np.uint8)
    qa[:, 1::2] |= 0x80
    qa[1] = top                      # row 1: all positive, sum K * FMAX^2
    qb = np.full((N, K), top, np.uint8)
    qb[2, :K // 2] = 0x01            # the smallest subnormal in half the terms
    ones = np.ones(M, np.float32)
    full = oracle.gemm_fwd_full(fmt, qa, ones, qb, K, 0, np.ones(N, np.float32),
                                np.array([M], np.int32), N, K)
    ia = pinlib.int_repr(fmt, qa)
    ib = pinlib.int_repr(fmt, qb)
    want = np.ldexp((ia @ ib.T).astype(np.float64), 2 * pinlib.QUANTUM_LOG2[fmt])
    assert np.array_equal(full, want)
    assert full[1, 0] == K * pinlib.FMAX[fmt] ** 2


@pytest.mark.parametrize("fmt", FMT)
def test_gemm_wgrad_group_matches_rows_and_integer_sums(fmt):
    M, K, N = 300, 40, 24
    off = np.array([0, 77, 77, 250, 300], np.int32)
    x = workloads.make_matrix(71, M, K)
    dy = workloads.make_matrix(72, M, N)
    xt, sx = oracle.quant_colwise_grouped(x, off, fmt)
    dyt, sdy = oracle.quant_colwise_grouped(dy, off, fmt)
    ix = pinlib.int_repr(fmt, xt)
    idy = pinlib.int_repr(fmt, dyt)
    start = 0
    for g, end in enumerate(off):
        got = oracle.gemm_wgrad_group(fmt, xt, sx, dyt, sdy, off, g)
        rows = oracle.gemm_wgrad_rows(fmt, xt, sx, dyt, sdy, off, N, K,
                                      np.full(K, g, np.int32), np.arange(K, dtype=np.int64))
        assert np.array_equal(got, rows)
        exact = ix[:, start:end] @ idy[:, start:end].T
        want = np.ldexp(exact.astype(np.float64), 2 * pinlib.QUANTUM_LOG2[fmt]) / (
            sx[g][:, None].astype(np.float64) * sdy[g][None, :].astype(np.float64))
        assert np.array_equal(got, want)
        if end == start:
            assert np.all(got == 0)
        start = end


def test_mx_gemm_fwd_full_matches_exact_block_sums():
    """MX forward for every row: within 2^-50 relative of the exact rational block sums (the
    C oracle's per-row function, separately pinned by them, as the comparison)."""
    M, K, N, E = 64, 256, 24, 3
    off = np.array([20, 20, 64], np.int32)
    x = workloads.make_matrix(81, M, K, 1.0, 0.01)
    w = workloads.make_matrix(82, E * K, N, 0.02)
    qa, ea = oracle.mx_quant_rowwise(x)
    qbt, eb = oracle.mx_quant_colwise(w)
    full = oracle.mx_gemm_fwd_full(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K)
    rows = oracle.mx_gemm_fwd_rows(qa, ea, qbt, E * K, K, eb, E * K // 32, K // 32, off, N, K,
                                   np.arange(M))
    assert np.allclose(full, rows, rtol=2.0 ** -45, atol=0)
    ia = pinlib.int_repr(FN, qa)
    ib = pinlib.int_repr(FN, qbt)
    for m, n in [(0, 0), (19, 23), (20, 5), (63, 11)]:
        g = 0 if m < 20 else 2
        tot = Fraction(0)
        for kb in range(K // 32):
            s = int(np.dot(ia[m, kb * 32:(kb + 1) * 32], ib[n, g * K + kb * 32:g * K + (kb + 1) * 32]))
            e = int(ea[m, kb]) - 127 + int(eb[n, g * K // 32 + kb]) - 127 - 18
            tot += Fraction(s) * (Fraction(2) ** e)
        assert abs(Fraction(full[m, n]) - tot) <= abs(tot) * Fraction(1, 2 ** 45)


def test_mx_wgrad_group_matches_rows():
    """MX weight gradient per group (blocks straddling group edges keep their scale) equals the
    separately pinned per-row oracle to float64 rounding, empty groups give zeros."""
    M, K, N = 224, 24, 20
    off = np.array([0, 45, 45, 130, 224], np.int32)
    xt, xe, dyt, de = _mx_wgrad_operands(M, K, N, 91)
    for g in range(off.size):
        got = oracle.mx_gemm_wgrad_group(xt, xe, dyt, de, off, g)
        rows = oracle.mx_gemm_wgrad_rows(xt, xe, dyt, de, off, N, np.full(K, g, np.int32),
                                         np.arange(K, dtype=np.int64))
        assert np.allclose(got, rows, rtol=2.0 ** -45, atol=0)
        if g in (0, 2):
            assert np.all(got == 0)
