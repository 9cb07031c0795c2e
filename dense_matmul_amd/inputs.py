"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and names workloads; it holds none of
the GEMM's or the quantisers' arithmetic.  Values are N(0,1) fp32 drawn with
``numpy.random.default_rng(seed)``, row-major, the distribution the pages'
benchmarks quantise (mori PR 785 section Cost and mori PR 809 section Results
run random matrices at model-projection shapes).
"""
import numpy as np


def normal(shape, seed):
    """fp32 N(0,1) array of ``shape`` from ``default_rng(seed)``."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def stacked_normal(block_rows, blocks, cols, seeds):
    """``blocks`` row blocks of ``block_rows`` x ``cols``, block i drawn with
    seeds[i], stacked in order (one GPU's share of a gathered operand)."""
    assert len(seeds) == blocks
    out = np.empty((block_rows * blocks, cols), np.float32)
    for i, s in enumerate(seeds):
        out[i * block_rows:(i + 1) * block_rows] = normal((block_rows, cols), s)
    return out


def choice(shape, values, seed):
    """Array of ``shape`` whose entries are drawn uniformly from ``values``."""
    values = np.asarray(values)
    idx = np.random.default_rng(seed).integers(0, values.size, size=shape)
    return values.reshape(-1)[idx]


def rows_sample(m, seed, per_band=1, band=64, tile=256):
    """Row indices for sampled checks at full size: every row of the first and
    last 256-row tiles plus ``per_band`` random rows from each 64-row band."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(tile, m)))
    rows.update(range(max(0, m - tile), m))
    for b0 in range(0, m, band):
        hi = min(m, b0 + band)
        rows.update(rng.integers(b0, hi, size=per_band).tolist())
    return np.array(sorted(rows), dtype=np.int64)


# Named workloads: (mode, M, N, K, seed_a, seed_b).  Seeds for the gathered
# operand are one per 4096-row block.
WORKLOADS = {
    "ptpc_512x1024x256": ("ptpc", 512, 1024, 256, 1, 2),
    "ptpc_4096x7168x256": ("ptpc", 4096, 7168, 256, 11, 12),
    "ptpc_16384x7168x512": ("ptpc", 16384, 7168, 512, 21, 22),
    "ptpc_32768x7168x1792": ("ptpc", 32768, 7168, 1792, 31, 32),
    "blockscale_16384x7168x2048": ("blockscale", 16384, 7168, 2048, 41, 42),
    "mxfp8_32768x7168x1792": ("mxfp8", 32768, 7168, 1792, 31, 32),
    "mxfp8_16384x7168x2048": ("mxfp8", 16384, 7168, 2048, 41, 42),
    "ptpc_gathered_32768x6288x7168": ("ptpc", 32768, 6288, 7168, tuple(range(500, 508)), 510),
    "ptpc_gathered_32768x3648x7168": ("ptpc", 32768, 3648, 7168, tuple(range(500, 508)), 511),
    "bf16_4096x896x1024": ("bf16", 4096, 896, 1024, 233, 233),
    "ptpc_2048x1168x1792": ("ptpc", 2048, 1168, 1792, 61, 62),
}


def operand_a(m, k, seed):
    """fp32 A of a workload: one draw, or stacked 4096-row blocks when
    ``seed`` is a tuple of per-block seeds."""
    if isinstance(seed, tuple):
        return stacked_normal(m // len(seed), len(seed), k, seed)
    return normal((m, k), seed)


def bf16_operands(m, k, n, seed):
    """fp32 values of the bf16 GEMM's A [M,K] and B given as [K,N] (drawn
    from one generator, A first), to be cast to bf16 by the caller."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((m, k), dtype=np.float32)
    b_kn = rng.standard_normal((k, n), dtype=np.float32)
    return a, b_kn
