"""Seeded synthetic inputs shaped like the LLM linear and MoE layers the pages talk about.

This module only draws random numbers and rounds them to bf16; it holds none of the
quantization or GEMM arithmetic, so both the oracle side and the GPU side of a test can take
their inputs from it.  Every tensor is returned as a numpy uint16 array of bf16 bit patterns
(row-major), so the oracle and the library see identical bytes.

Draws use numpy's PCG64 `default_rng(seed)` in float64, are cast to float32 and then rounded to
bf16 (nearest, ties to even).  The draw order of each workload is part of its definition.
"""

import numpy as np


def to_bf16_bits(a):
    """float -> bf16 bit patterns (round to nearest, ties to even), via float32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_float32(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_with_outliers(rng, rows, cols, frac, factor, sigma=1.0):
    """N(0, sigma^2) matrix; round(frac * rows * cols) distinct positions are multiplied by
    `factor` (activation outliers)."""
    a = rng.standard_normal((rows, cols)) * sigma
    n_out = int(round(frac * rows * cols))
    if n_out:
        pos = rng.choice(rows * cols, size=n_out, replace=False)
        a.reshape(-1)[pos] *= factor
    return a


def tiny(seed=0, m=32, k=512, n=512):
    """Tiny round trip + GEMM: A m x k ~ N(0,1) with 1% of entries x20, W n x k ~ N(0, 0.02^2).
    Draw order: A, outlier positions, W."""
    rng = np.random.default_rng(seed)
    a = normal_with_outliers(rng, m, k, 0.01, 20.0)
    w = rng.standard_normal((n, k)) * 0.02
    return {"a": to_bf16_bits(a), "w": to_bf16_bits(w)}


def activation(seed=1, rows=8192, cols=8192):
    """Activation-quantize workload: X = L * g[None, :], L ~ Laplace(0, 1) rows x cols,
    g ~ LogNormal(0, 1) per column.  Draw order: L, then g."""
    rng = np.random.default_rng(seed)
    lap = rng.laplace(0.0, 1.0, size=(rows, cols))
    g = np.exp(rng.standard_normal(cols))
    lap *= g[None, :]
    return {"x": to_bf16_bits(lap)}


def decode(seed=2, n=14336, k=4096, ms=(1, 8, 16)):
    """Decode-shaped W4A4 GEMM: W n x k ~ N(0, 0.02^2) (quantized offline with 16x16 blocks),
    then one activation A_M ~ N(0,1) of M x k for each M in `ms`, in that order."""
    rng = np.random.default_rng(seed)
    w = to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    acts = {m: to_bf16_bits(rng.standard_normal((m, k))) for m in ms}
    return {"w": w, "a": acts}


def prefill(seed=3, m=8192, k=8192, n=8192):
    """Prefill-shaped W4A4 GEMM: A m x k ~ N(0,1) with 0.5% of entries x30; W n x k ~
    N(0, 0.02^2) (quantized offline with 16x16 blocks).  Draw order: A, outlier positions, W."""
    rng = np.random.default_rng(seed)
    a = normal_with_outliers(rng, m, k, 0.005, 30.0)
    w = rng.standard_normal((n, k)) * 0.02
    return {"a": to_bf16_bits(a), "w": to_bf16_bits(w)}


def zipf_routing(rng, tokens, experts, topk, s=1.1):
    """Top-k routing: expert popularity p_e ~ (e+1)^-s; each token draws `topk` distinct experts
    with those probabilities.  Returns (row_index, offsets, counts): the routed rows grouped by
    expert, tokens in increasing id inside each group."""
    p = (np.arange(experts, dtype=np.float64) + 1.0) ** (-s)
    p /= p.sum()
    choice = np.empty((tokens, topk), dtype=np.int64)
    for t in range(tokens):
        choice[t] = rng.choice(experts, size=topk, replace=False, p=p)
    counts = np.bincount(choice.ravel(), minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_index = np.empty(tokens * topk, dtype=np.int32)
    fill = offsets[:-1].astype(np.int64).copy()
    for t in range(tokens):          # increasing token id inside each expert group
        for e in choice[t]:
            row_index[fill[e]] = t
            fill[e] += 1
    return row_index, offsets, counts.astype(np.int32)


def moe(seed=4, tokens=4096, hidden=2048, experts=128, topk=8, n=768, s=1.1):
    """MoE grouped W4A4 GEMM: routing first (zipf_routing), then A tokens x hidden ~ N(0,1),
    then each expert's W_e (n x hidden ~ N(0, 0.02^2)) in expert order.  W is returned stacked
    as (experts * n) x hidden."""
    rng = np.random.default_rng(seed)
    row_index, offsets, counts = zipf_routing(rng, tokens, experts, topk, s)
    a = to_bf16_bits(rng.standard_normal((tokens, hidden)))
    w = np.empty((experts * n, hidden), dtype=np.uint16)
    for e in range(experts):
        w[e * n:(e + 1) * n] = to_bf16_bits(rng.standard_normal((n, hidden)) * 0.02)
    return {"a": a, "w": w, "row_index": row_index, "offsets": offsets, "counts": counts,
            "n": n, "experts": experts}
