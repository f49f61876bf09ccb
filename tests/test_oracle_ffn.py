"""Pins for the oracle's fused-epilogue reference (SiLU gate over gate/up blocks
interleaved every 128 columns).

Independent references: closed forms of silu, scipy's logistic function, a
hand-built D whose blocks are constants, and a one-hot weight that makes the
oracle GEMM copy A's columns so the activation can be written out directly.
"""
import math

import numpy as np
import scipy.special

import oracle
from oracle import silu, swiglu_blocks


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    assert silu(0.0) == 0.0
    assert math.isclose(silu(ln3), 0.75 * ln3, rel_tol=1e-15)       # sigmoid(ln 3) = 3/4
    assert math.isclose(silu(-ln3), -0.25 * ln3, rel_tol=1e-15)     # sigmoid(-ln 3) = 1/4
    assert silu(800.0) == 800.0
    big_neg = silu(-800.0)
    assert big_neg == 0.0 and math.copysign(1.0, big_neg) == -1.0  # overflow gives the signed zero


def test_silu_odd_part_identity_and_logistic():
    rng = np.random.default_rng(51)
    x = rng.standard_normal(1000) * 8
    # silu(x) - silu(-x) = x * (sigmoid(x) + sigmoid(-x)) = x
    assert np.allclose(silu(x) - silu(-x), x, rtol=1e-14, atol=1e-14)
    assert np.allclose(silu(x), x * scipy.special.expit(x), rtol=1e-14, atol=1e-300)


def test_block_interleave_map():
    """Gate block j is the constant j+1, up block j holds its column index c:
    act[:, 128j + c] = silu(j+1) * c. Swapping gate and up, or pairing block j
    with any other block, gives different values."""
    M, J = 3, 4
    d = np.zeros((M, 256 * J))
    for j in range(J):
        d[:, 256 * j:256 * j + 128] = j + 1
        d[:, 256 * j + 128:256 * j + 256] = np.arange(128)
    act = swiglu_blocks(d)
    assert act.shape == (M, 128 * J)
    for j in range(J):
        want = silu(float(j + 1)) * np.arange(128)
        assert np.array_equal(act[:, 128 * j:128 * (j + 1)], np.broadcast_to(want, (M, 128)))
    # batched (masked) shape keeps the leading axes
    assert swiglu_blocks(np.stack([d, 2 * d])).shape == (2, M, 128 * J)


def test_composition_with_the_gemm_reference():
    """B's gate row c is a one-hot on A column c and its up row c a one-hot on A
    column 128+c (code 0x38 = 1.0, unit scales), so the oracle GEMM copies A's
    columns and act must equal silu(a[:, c]) * a[:, 128 + c] of the dequantised A."""
    rng = np.random.default_rng(52)
    M, K, N = 8, 256, 256
    a = rng.standard_normal((M, K)).astype(np.float32)
    A, sa = oracle.quantize_act_1x128(a)
    B = np.zeros((N, K), np.uint8)
    for c in range(128):
        B[c, c] = 0x38
        B[128 + c, 128 + c] = 0x38
    sb = np.ones((N // 128, K // 128), np.float32)
    act = swiglu_blocks(oracle.ref_dense(A, sa, B, sb))
    ahat = oracle.dequant_act(A, sa)
    assert np.array_equal(act, silu(ahat[:, :128]) * ahat[:, 128:])
