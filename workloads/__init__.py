"""Seeded synthetic inputs for the MoE FP8 hot path.

This module only draws random numbers and arranges them into the shapes of the workloads; it
holds none of the quantization or GEMM arithmetic.  Both the CPU oracle (in tests) and the GPU
library are fed from here, so they always see the same bytes.

Shapes follow the models the pages measure on (Llama3-8B FFN, DeepSeek-MoE-16B experts,
DeepSeek-V3 expert slice); no dataset is involved.  Recipe: numpy PCG64(seed), fp32 draws,
rounded to bf16 with round-to-nearest-even on the fp32 bit pattern.

Configs:
  tiny      4 experts, K=256, N=512, 1024 tokens N(0,1) with 1% of elements x50, group ends
            from 3 sorted uniform integer cuts of [0, 1024]; e4m3fnuz.
  dense     M=8192, K=4096, N=14336, G=1; X ~ N(0,1), W ~ N(0, 0.02).
  moe16b    64 experts, K=2048, N=1408, 8192 tokens x top-6 distinct experts picked by
            Gumbel-top-k over Zipf(1.1) weights on a seeded permutation of the experts.
  dsv3_bwd  32 experts, hidden 7168, intermediate 2048, 16384 routed rows, group sizes
            multinomial(16384) over Zipf(1.1) expert probabilities; X, dY ~ N(0,1).
  dsv3_mx   forward of dsv3_bwd in MXFP8: W[32, 7168, 2048] ~ N(0, 0.02), same offsets.
"""
from __future__ import annotations

import numpy as np

FNUZ = 0
FN = 1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    chunk = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for i in range(0, flat_u.size, chunk):
        v = flat_u[i:i + chunk].astype(np.uint64)
        v = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        flat_o[i:i + chunk] = v.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws, generated in chunks to bound host memory."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, np.uint16)
    chunk = 1 << 24
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        v = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[i:i + m] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def zipf_probs(rng: np.random.Generator, n: int, s: float = 1.1) -> np.ndarray:
    """p_i proportional to rank^-s, ranks assigned by a seeded permutation."""
    ranks = rng.permutation(n) + 1
    w = ranks.astype(np.float64) ** (-s)
    return w / w.sum()


def offsets_from_sizes(sizes) -> np.ndarray:
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


def random_offsets(rng: np.random.Generator, rows: int, groups: int, allow_empty=True) -> np.ndarray:
    """Group END offsets from sorted uniform integer cuts of [0, rows]."""
    if groups == 1:
        return np.array([rows], np.int32)
    cuts = np.sort(rng.integers(0, rows + 1, size=groups - 1))
    if not allow_empty:
        cuts = np.unique(cuts)
    return np.concatenate([cuts, [rows]]).astype(np.int32)


def routed_offsets_topk(rng: np.random.Generator, tokens: int, experts: int, topk: int,
                        s: float = 1.1) -> np.ndarray:
    """Each token picks topk distinct experts by Gumbel-top-k over log Zipf weights."""
    logp = np.log(zipf_probs(rng, experts, s))
    counts = np.zeros(experts, np.int64)
    chunk = 4096
    for i in range(0, tokens, chunk):
        m = min(chunk, tokens - i)
        g = rng.gumbel(size=(m, experts))
        top = np.argpartition(-(logp[None, :] + g), topk - 1, axis=1)[:, :topk]
        counts += np.bincount(top.ravel(), minlength=experts)
    return offsets_from_sizes(counts)


def routed_rows_topk(rng: np.random.Generator, tokens: int, experts: int, topk: int,
                     s: float = 1.1):
    """Token dispatch in expert order: each token picks topk distinct experts (Gumbel-top-k over
    log Zipf weights); rows are sorted by expert, tokens ascending inside an expert.  Returns
    (offsets int32 [experts], index int32 [tokens*topk]: the source token of each row)."""
    logp = np.log(zipf_probs(rng, experts, s))
    g = rng.gumbel(size=(tokens, experts))
    top = np.argpartition(-(logp[None, :] + g), topk - 1, axis=1)[:, :topk]   # [tokens, topk]
    expert = top.ravel()
    token = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=experts)
    return offsets_from_sizes(counts), token[order].astype(np.int32)


def multinomial_offsets(rng: np.random.Generator, rows: int, experts: int, s: float = 1.1) -> np.ndarray:
    p = zipf_probs(rng, experts, s)
    return offsets_from_sizes(rng.multinomial(rows, p))


# ----------------------------------------------------------------------------- configs

CONFIGS = {
    "tiny": dict(seed=1, M=1024, K=256, N=512, E=4, fmt=FNUZ),
    "dense": dict(seed=2, M=8192, K=4096, N=14336, E=1, fmt=FN),
    "moe16b": dict(seed=3, tokens=8192, topk=6, M=49152, K=2048, N=1408, E=64, fmt=FN),
    "dsv3_bwd": dict(seed=4, M=16384, K=7168, N=2048, E=32, fmt=FN),
    "dsv3_mx": dict(seed=5, M=16384, K=7168, N=2048, E=32, fmt=FN),
}


def make_forward(name: str, fmt: int | None = None):
    """Forward inputs: dict with x [M,K] bf16 bits, w [E*K, N] bf16 bits (the [E,K,N] weights
    viewed as one 2-D matrix), offsets [E] int32, and the sizes."""
    cfg = dict(CONFIGS[name])
    if fmt is not None:
        cfg["fmt"] = fmt
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    M, K, N, E = cfg["M"], cfg["K"], cfg["N"], cfg["E"]
    if name == "tiny":
        x = rng.standard_normal((M, K), dtype=np.float32)
        mask = rng.random((M, K)) < 0.01
        x[mask] *= np.float32(50.0)
        x = f32_to_bf16_bits(x)
        w = normal_bf16(rng, (E * K, N), 0.02)
        offsets = random_offsets(rng, M, E)
    elif name == "dense":
        x = normal_bf16(rng, (M, K))
        w = normal_bf16(rng, (E * K, N), 0.02)
        offsets = np.array([M], np.int32)
    elif name == "moe16b":
        offsets = routed_offsets_topk(rng, cfg["tokens"], E, cfg["topk"])
        assert int(offsets[-1]) == M
        x = normal_bf16(rng, (M, K))
        w = normal_bf16(rng, (E * K, N), 0.02)
    elif name in ("dsv3_bwd", "dsv3_mx"):
        # both share the dsv3_bwd routing so the MX forward sees the backward's groups
        r4 = np.random.Generator(np.random.PCG64(CONFIGS["dsv3_bwd"]["seed"]))
        offsets = multinomial_offsets(r4, M, E)
        x = normal_bf16(rng, (M, K))
        w = normal_bf16(rng, (E * K, N), 0.02)
    else:
        raise KeyError(name)
    return dict(name=name, x=x, w=w, offsets=offsets, M=M, K=K, N=N, E=E, fmt=cfg["fmt"])


def make_wgrad(name: str = "dsv3_bwd", fmt: int | None = None):
    """Backward (weight-gradient) inputs: x [M,K], dy [M,N] bf16 bits and offsets [E]."""
    cfg = dict(CONFIGS[name])
    if fmt is not None:
        cfg["fmt"] = fmt
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    M, K, N, E = cfg["M"], cfg["K"], cfg["N"], cfg["E"]
    offsets = multinomial_offsets(rng, M, E)
    x = normal_bf16(rng, (M, K))
    dy = normal_bf16(rng, (M, N))
    return dict(name=name, x=x, dy=dy, offsets=offsets, M=M, K=K, N=N, E=E, fmt=cfg["fmt"])


def make_matrix(seed: int, rows: int, cols: int, std: float = 1.0, outlier_frac: float = 0.0,
                outlier_mul: float = 50.0) -> np.ndarray:
    """A small bf16 test matrix, optionally with a fraction of outliers."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if outlier_frac > 0:
        mask = rng.random((rows, cols)) < outlier_frac
        x[mask] *= np.float32(outlier_mul)
    return f32_to_bf16_bits(x)


def to_torch_bf16(bits: np.ndarray, device, ld: int | None = None):
    """Copy bf16 bit patterns to a device bf16 tensor (optionally with a padded row stride)."""
    import torch
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    if ld is None or bits.ndim != 2 or ld == bits.shape[1]:
        return t.to(device)
    out = torch.zeros((bits.shape[0], ld), dtype=torch.bfloat16, device=device)
    out[:, :bits.shape[1]] = t.to(device)
    return out[:, :bits.shape[1]]
