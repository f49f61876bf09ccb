"""Thread-parallel drivers of the oracle's quantisers for full-size inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

An activation block (1x128) lies within one row and a weight block (128x128)
within one aligned 128-row slab of one expert, so quantising independent row
chunks and putting the pieces together gives exactly the serial result; numpy
releases the interpreter lock inside its array operations, so the chunks run
on several cores. No arithmetic of the method lives here: every code and scale
comes from ``quant.quantize_act_1x128`` / ``quant.quantize_weight_128x128``.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .quant import quantize_act_1x128, quantize_weight_128x128


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def quantize_act_1x128_par(x, pow2=False, chunk=512):
    """quantize_act_1x128 of x [M, K] (or [B, M, K], row by row) in chunks of rows."""
    x = np.asarray(x, dtype=np.float32)
    lead = x.shape[:-1]
    flat = x.reshape(-1, x.shape[-1])
    R, K = flat.shape
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((R, K // 128), np.float32)

    def one(r0):
        c, s = quantize_act_1x128(flat[r0:r0 + chunk], pow2)
        codes[r0:r0 + chunk] = c
        scales[r0:r0 + chunk] = s

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(0, R, chunk)))
    return codes.reshape(lead + (K,)), scales.reshape(lead + (K // 128,))


def quantize_weight_128x128_par(w, pow2=False, chunk=1024):
    """quantize_weight_128x128 of w [N, K] (or [G, N, K]) in slabs of 128-aligned
    rows of one expert (chunk must be a multiple of 128)."""
    if chunk % 128:
        raise ValueError("chunk must be a multiple of 128 rows")
    w = np.asarray(w, dtype=np.float32)
    w3 = w[None] if w.ndim == 2 else w
    G, N, K = w3.shape
    nb = -(-N // 128)
    codes = np.empty(w3.shape, np.uint8)
    scales = np.empty((G, nb, K // 128), np.float32)

    def one(job):
        g, r0 = job
        c, s = quantize_weight_128x128(w3[g, r0:r0 + chunk], pow2)
        codes[g, r0:r0 + chunk] = c
        scales[g, r0 // 128:r0 // 128 + s.shape[0]] = s

    jobs = [(g, r0) for g in range(G) for r0 in range(0, N, chunk)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, jobs))
    if w.ndim == 2:
        return codes[0], scales[0]
    return codes, scales
