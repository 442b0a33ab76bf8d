"""Independent references used to pin the CPU oracle (test-only helpers).

Nothing here calls the oracle or the GPU library.  Decoding uses torch's float8 dtypes (a
library routine); encoding is checked by brute-force nearest search over those decoded tables;
GEMM sums are checked with exact integer arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

FNUZ = 0
FN = 1
FMAX = {FNUZ: 240.0, FN: 448.0}
# every finite value of the format is an integer multiple of its smallest subnormal
QUANTUM_LOG2 = {FNUZ: -10, FN: -9}
_TORCH_DT = {FNUZ: torch.float8_e4m3fnuz, FN: torch.float8_e4m3fn}


def torch_decode_table(fmt: int) -> np.ndarray:
    """float64[256]: the value of every byte according to torch's float8 dtype."""
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(_TORCH_DT[fmt]).to(torch.float64).numpy()


def torch_encode(fmt: int, y: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8 cast (round to nearest even); inputs must be within range."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(_TORCH_DT[fmt]).view(torch.uint8).numpy()


def brute_encode(fmt: int, y: np.ndarray) -> np.ndarray:
    """Nearest representable value by exhaustive distance to every positive finite code; a tie
    goes to the even code.  Sign handled as the format requires (fnuz has a single zero)."""
    tab = torch_decode_table(fmt)
    pos_codes = np.array([c for c in range(128) if np.isfinite(tab[c])], np.int64)
    vals = tab[pos_codes]
    y = np.asarray(y, dtype=np.float32).ravel()
    out = np.empty(y.size, np.uint8)
    a = np.abs(y.astype(np.float64))
    for i in range(0, y.size, 1 << 15):
        d = np.abs(a[i:i + (1 << 15), None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among the minimal-distance codes prefer the even one
        even_pref = cand & ((pos_codes[None, :] & 1) == 0)
        pick = np.where(even_pref.any(axis=1), even_pref.argmax(axis=1), cand.argmax(axis=1))
        code = pos_codes[pick]
        neg = np.signbit(y[i:i + (1 << 15)])
        if fmt == FNUZ:
            code = np.where((code != 0) & neg, code | 0x80, code)
        else:
            code = np.where(neg, code | 0x80, code)
        out[i:i + (1 << 15)] = code.astype(np.uint8)
    return out


def int_repr(fmt: int, q: np.ndarray) -> np.ndarray:
    """Each byte's value as an exact int64 multiple of the format's smallest subnormal."""
    tab = torch_decode_table(fmt)
    ints = np.zeros(256, np.int64)
    fin = np.isfinite(tab)
    ints[fin] = np.rint(np.ldexp(tab[fin], -QUANTUM_LOG2[fmt])).astype(np.int64)
    assert np.all(np.ldexp(ints[fin].astype(np.float64), QUANTUM_LOG2[fmt]) == tab[fin])
    return ints[np.asarray(q, dtype=np.uint8)]


def fp32_neighbors(v: np.ndarray, k: int = 2) -> np.ndarray:
    """v and its fp32 neighbours up to k ulps on each side."""
    v = np.asarray(v, dtype=np.float32)
    out = [v]
    up = v.copy()
    dn = v.copy()
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return np.concatenate(out)


def encode_probe_values(fmt: int, n_random: int = 400_000, seed: int = 0) -> np.ndarray:
    """fp32 values in [-FMAX, FMAX] that exercise every rounding decision: each representable
    value and each midpoint between neighbours (with fp32 neighbours), tiny and subnormal fp32
    values, and uniform random bit patterns."""
    tab = torch_decode_table(fmt)
    pos = np.sort(np.unique(tab[:128][np.isfinite(tab[:128])]))
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [2.0 ** -11, 2.0 ** -12, 1e-30, 1e-40, 1.4e-45]])
    vals = fp32_neighbors(base.astype(np.float32), 2)
    rng = np.random.default_rng(seed)
    fm_bits = np.float32(FMAX[fmt]).view(np.uint32)
    rb = rng.integers(0, int(fm_bits) + 1, size=n_random, dtype=np.uint64).astype(np.uint32)
    vals = np.concatenate([vals, rb.view(np.float32)])
    vals = vals[np.abs(vals) <= FMAX[fmt]]
    return np.concatenate([vals, -vals]).astype(np.float32)
