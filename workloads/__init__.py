"""Seeded synthetic inputs for the FP8 block-scaled GEMM workloads.

This module only draws random numbers and builds index structure (group sizes,
expert ids per row, valid-row counts, outlier rows). It contains none of the
GEMM's arithmetic: quantisation to E4M3 and the product itself live elsewhere
(the oracle on the CPU, the library on the GPU), and both consume what this
module returns.

Workloads (all fp32 N(0,1) before quantisation, K-contiguous, D = A . B^T):
  dense_small    M=128,  N=256,  K=512
  dense_skinny   M=256,  N=7168, K=7168, 1% of A's rows scaled x50 (outliers)
  contiguous     8 experts, rows per expert U{256..2048} padded up to a
                 multiple of 128, N=4096, K=7168, weights [8, 4096, 7168]
  masked         16 experts, buffer M_max=256 rows each, valid rows
                 U{0..256}, N=7168, K=2048
  dense_ffn      M=8192, N=7168, K=18432

Draw order with numpy's default_rng(seed): group sizes or masked_m first, then
A (standard_normal, float32), then B, then the outlier rows.
"""

import numpy as np

WORKLOADS = {
    "dense_small": dict(kind="dense", M=128, N=256, K=512, seed=1),
    "dense_skinny": dict(kind="dense", M=256, N=7168, K=7168, seed=2,
                         outlier_frac=0.01, outlier_scale=50.0),
    "contiguous": dict(kind="contiguous", G=8, N=4096, K=7168, seed=3,
                       m_lo=256, m_hi=2048, align=128),
    "masked": dict(kind="masked", G=16, M_max=256, N=7168, K=2048, seed=4,
                   m_lo=0, m_hi=256),
    "dense_ffn": dict(kind="dense", M=8192, N=7168, K=18432, seed=5),
}


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def dense(M, N, K, seed, outlier_frac=0.0, outlier_scale=1.0):
    """fp32 A [M, K], B [N, K]; optionally round(outlier_frac * M) rows of A
    (chosen without replacement) multiplied by outlier_scale."""
    rng = np.random.default_rng(seed)
    a = _normal(rng, (M, K))
    b = _normal(rng, (N, K))
    rows = np.zeros(0, dtype=np.int64)
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * M))
        rows = np.sort(rng.choice(M, size=n_out, replace=False))
        a[rows] *= np.float32(outlier_scale)
    return dict(kind="dense", a=a, b=b, outlier_rows=rows)


def contiguous_sizes(G, seed, m_lo, m_hi, align):
    """Per-expert row counts U{m_lo..m_hi} (inclusive) and their padded sizes."""
    rng = np.random.default_rng(seed)
    m = rng.integers(m_lo, m_hi, size=G, endpoint=True)
    padded = ((m + align - 1) // align) * align
    return rng, m.astype(np.int64), padded.astype(np.int64)


def contiguous(G, N, K, seed, m_lo=256, m_hi=2048, align=128):
    """Concatenated expert rows. Padding rows are all-zero and have expert id -1.
    Returns fp32 A [M_total, K], B [G, N, K], m_indices int32 [M_total]."""
    rng, m, padded = contiguous_sizes(G, seed, m_lo, m_hi, align)
    M = int(padded.sum())
    m_indices = np.full(M, -1, dtype=np.int32)
    a = np.zeros((M, K), dtype=np.float32)
    off = 0
    for g in range(G):
        m_indices[off:off + m[g]] = g
        off += int(padded[g])
    real = m_indices >= 0
    a[real] = _normal(rng, (int(real.sum()), K))
    b = _normal(rng, (G, N, K))
    return dict(kind="contiguous", a=a, b=b, m_indices=m_indices,
                group_m=m, group_padded=padded)


def masked(G, M_max, N, K, seed, m_lo=0, m_hi=None):
    """Per-expert fixed buffers. Every row of A is populated (also those at or
    beyond masked_m); masked_m int32 [G] ~ U{m_lo..m_hi} inclusive."""
    if m_hi is None:
        m_hi = M_max
    rng = np.random.default_rng(seed)
    masked_m = rng.integers(m_lo, m_hi, size=G, endpoint=True).astype(np.int32)
    a = _normal(rng, (G, M_max, K))
    b = _normal(rng, (G, N, K))
    return dict(kind="masked", a=a, b=b, masked_m=masked_m)


def make(name_or_cfg, **overrides):
    """Build a workload by name (``WORKLOADS``) or from an explicit dict; keyword
    overrides replace shape/seed fields, e.g. ``make("masked", N=256, K=512)``."""
    cfg = dict(WORKLOADS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "dense":
        return dense(**cfg)
    if kind == "contiguous":
        return contiguous(**cfg)
    if kind == "masked":
        return masked(**cfg)
    raise ValueError(f"unknown workload kind {kind!r}")


def useful_flop(w):
    """2 * (rows that have an output) * N * K for a generated workload."""
    b = w["b"]
    N, K = b.shape[-2], b.shape[-1]
    if w["kind"] == "dense":
        rows = w["a"].shape[0]
    elif w["kind"] == "contiguous":
        rows = int((w["m_indices"] >= 0).sum())
    else:
        rows = int(np.clip(w["masked_m"], 0, w["a"].shape[1]).sum())
    return 2.0 * rows * N * K
