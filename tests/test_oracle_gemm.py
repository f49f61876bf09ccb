"""Pins for the oracle GEMM (dense, grouped-contiguous, grouped-masked).

Independent references: exact rational arithmetic (pure-Python triple loop with
fractions.Fraction, decoding codes through torch's float8_e4m3fn), integer
matmul for small-integer inputs with unit scales, closed forms, and
power-of-two scale invariance.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import (ref_contiguous, ref_dense, ref_dense_twolevel, ref_entries,
                    ref_masked)


def torch_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def int_codes(values):
    """E4M3 codes of small integers via torch's cast (exact for |v| <= 16)."""
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # drop NaN codes


def brute_force(A, sa, B, sb):
    """Exact D[m][n] = sum_k dec(A[m,k]) sa[m,k//128] dec(B[n,k]) sb[n//128,k//128]."""
    da, db = torch_dec(A), torch_dec(B)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            s = Fraction(0)
            for k in range(K):
                s += (Fraction(float(da[m, k])) * Fraction(float(sa[m, k // 128]))
                      * Fraction(float(db[n, k])) * Fraction(float(sb[n // 128, k // 128])))
            out[m, n] = float(s)
    return out


def test_dense_vs_exact_rationals():
    rng = np.random.default_rng(11)
    M, N, K = 2, 256, 256                      # two N-blocks, two K-blocks
    A, B = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    sa = rng.uniform(0.01, 2.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.01, 2.0, (N // 128, K // 128)).astype(np.float32)
    exact = brute_force(A, sa, B, sb)
    ref = ref_dense(A, sa, B, sb)
    assert np.max(np.abs(ref - exact) / np.maximum(np.abs(exact), 1e-300)) < 1e-12
    two = ref_dense_twolevel(A, sa, B, sb)
    assert np.max(np.abs(two - exact) / np.maximum(np.abs(exact), 1e-300)) < 1e-12


def test_unit_scales_small_integers_equal_integer_matmul():
    rng = np.random.default_rng(12)
    M, N, K = 48, 256, 512
    ai = rng.integers(-4, 5, size=(M, K))
    bi = rng.integers(-4, 5, size=(N, K))
    ones_a = np.ones((M, K // 128), np.float32)
    ones_b = np.ones((N // 128, K // 128), np.float32)
    ref = ref_dense(int_codes(ai), ones_a, int_codes(bi), ones_b)
    assert np.array_equal(ref, (ai @ bi.T).astype(np.float64))   # exact, and B is N x K


def test_closed_form_constant_inputs():
    M, N, K = 8, 128, 1024
    alpha, beta = np.float32(0.37), np.float32(1.9)
    A = np.full((M, K), 0x38, np.uint8)          # 1.0
    B = np.full((N, K), 0x38, np.uint8)
    ref = ref_dense(A, np.full((M, K // 128), alpha), B, np.full((N // 128, K // 128), beta))
    expect = K * float(alpha) * float(beta)
    assert np.allclose(ref, expect, rtol=1e-13, atol=0)


def test_single_kblock_picks_its_own_scales():
    """Inputs nonzero only in K-block j: D = sa[:, j] * sb[nb, j] * int partial."""
    rng = np.random.default_rng(13)
    M, N, K, j = 16, 384, 640, 3
    ai = np.zeros((M, K), np.int64)
    bi = np.zeros((N, K), np.int64)
    ai[:, j * 128:(j + 1) * 128] = rng.integers(-3, 4, (M, 128))
    bi[:, j * 128:(j + 1) * 128] = rng.integers(-3, 4, (N, 128))
    sa = (2.0 ** rng.integers(-6, 6, (M, K // 128))).astype(np.float32)
    sb = (2.0 ** rng.integers(-6, 6, (N // 128, K // 128))).astype(np.float32)
    ref = ref_dense(int_codes(ai), sa, int_codes(bi), sb)
    part = (ai @ bi.T).astype(np.float64)
    expect = part * sa[:, j][:, None].astype(np.float64) * np.repeat(sb[:, j], 128)[None, :]
    assert np.array_equal(ref, expect)


def test_power_of_two_scale_invariance_is_bitwise():
    rng = np.random.default_rng(14)
    M, N, K = 32, 256, 384
    A, B = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    sa = rng.uniform(0.1, 1.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.1, 1.0, (N // 128, K // 128)).astype(np.float32)
    p = rng.integers(-5, 6, M)
    q = rng.integers(-5, 6, N // 128)
    ref = ref_dense(A, sa, B, sb)
    ref2 = ref_dense(A, (sa * (2.0 ** p)[:, None]).astype(np.float32),
                     B, (sb * (2.0 ** q)[:, None]).astype(np.float32))
    expect = ref * (2.0 ** p)[:, None] * np.repeat(2.0 ** q, 128)[None, :]
    assert np.array_equal(ref2, expect)


def test_zero_scale_gives_zero():
    rng = np.random.default_rng(15)
    A, B = random_codes(rng, (4, 256)), random_codes(rng, (128, 256))
    sa = np.ones((4, 2), np.float32)
    sa[2] = 0.0
    ref = ref_dense(A, sa, B, np.ones((1, 2), np.float32))
    assert np.all(ref[2] == 0)


def test_entries_match_full_product():
    rng = np.random.default_rng(16)
    M, N, K = 40, 384, 512
    A, B = random_codes(rng, (M, K)), random_codes(rng, (N, K))
    sa = rng.uniform(0.01, 1.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.01, 1.0, (N // 128, K // 128)).astype(np.float32)
    rows, cols = rng.integers(0, M, 50), rng.integers(0, N, 50)
    full = ref_dense(A, sa, B, sb)
    assert np.allclose(ref_entries(A, sa, B, sb, rows, cols), full[rows, cols], rtol=1e-13, atol=1e-300)


def test_contiguous_vs_exact_rationals_with_padding():
    rng = np.random.default_rng(17)
    G, N, K = 3, 128, 256
    m_indices = np.array([0, 0, -1, 2, 2, 2, -1, 1], dtype=np.int32)
    M = m_indices.size
    A, B = random_codes(rng, (M, K)), random_codes(rng, (G, N, K))
    sa = rng.uniform(0.1, 1.0, (M, K // 128)).astype(np.float32)
    sb = rng.uniform(0.1, 1.0, (G, N // 128, K // 128)).astype(np.float32)
    out, valid = ref_contiguous(A, sa, B, sb, m_indices)
    assert np.array_equal(valid, m_indices >= 0)
    for m in range(M):
        g = m_indices[m]
        if g < 0:
            assert np.all(out[m] == 0)
            continue
        exact = brute_force(A[m:m + 1], sa[m:m + 1], B[g], sb[g])[0]
        assert np.max(np.abs(out[m] - exact) / np.maximum(np.abs(exact), 1e-300)) < 1e-12


def test_contiguous_single_group_equals_dense():
    rng = np.random.default_rng(18)
    M, N, K = 64, 256, 256
    A, B = random_codes(rng, (M, K)), random_codes(rng, (1, N, K))
    sa = rng.uniform(0.1, 1.0, (M, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 1.0, (1, 2, 2)).astype(np.float32)
    out, _ = ref_contiguous(A, sa, B, sb, np.zeros(M, np.int32))
    assert np.array_equal(out, ref_dense(A, sa, B[0], sb[0]))


def test_masked_rows_and_empty_groups():
    rng = np.random.default_rng(19)
    G, Mm, N, K = 4, 8, 128, 256
    masked_m = np.array([0, 3, 8, 11], dtype=np.int32)     # 11 is clamped to 8
    A, B = random_codes(rng, (G, Mm, K)), random_codes(rng, (G, N, K))
    sa = rng.uniform(0.1, 1.0, (G, Mm, 2)).astype(np.float32)
    sb = rng.uniform(0.1, 1.0, (G, 1, 2)).astype(np.float32)
    out, valid = ref_masked(A, sa, B, sb, masked_m)
    assert valid.sum(axis=1).tolist() == [0, 3, 8, 8]
    assert np.all(out[~valid] == 0)
    exact = brute_force(A[1, :3], sa[1, :3], B[1], sb[1])
    assert np.max(np.abs(out[1, :3] - exact) / np.maximum(np.abs(exact), 1e-300)) < 1e-12
    assert np.array_equal(out[2], ref_dense(A[2], sa[2], B[2], sb[2]))


def test_oracle_is_cpu_numpy_only():
    # the oracle exposes plain numpy functions and never touches torch tensors
    assert all(hasattr(oracle, f) for f in ("ref_dense", "ref_contiguous", "ref_masked", "check"))
