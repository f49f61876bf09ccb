"""Pins for the oracle with N not a multiple of 128 (the last weight-scale block
covers the remaining N mod 128 rows).

Independent references: a block-by-block torch recipe over explicit row
ranges, the GEMM reference on the same weight padded with zero rows (whose
extra columns are discarded), the two-level form, and single-entry dot
products.
"""
import numpy as np
import torch

import oracle


def torch_weight_quant_ragged(w):
    """128x128 blocks over explicit row ranges [128j, min(128j + 128, N))."""
    t = torch.from_numpy(w)
    N, K = t.shape
    codes = torch.empty((N, K), dtype=torch.uint8)
    scales = torch.empty((-(-N // 128), K // 128), dtype=torch.float32)
    for j in range(scales.shape[0]):
        r0, r1 = 128 * j, min(128 * j + 128, N)
        for kb in range(K // 128):
            blk = t[r0:r1, kb * 128:(kb + 1) * 128]
            amax = blk.abs().max()
            s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
            scales[j, kb] = s
            y = (blk / s).clamp(-448.0, 448.0)
            codes[r0:r1, kb * 128:(kb + 1) * 128] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), scales.numpy()


def test_ragged_weight_quant_matches_blockwise_torch():
    rng = np.random.default_rng(61)
    for N in (8, 72, 200, 328):
        w = rng.standard_normal((N, 256), dtype=np.float32)
        w[-1, 3] = 40.0                      # the ragged block's maximum
        codes, sb = oracle.quantize_weight_128x128(w)
        tc, ts = torch_weight_quant_ragged(w)
        assert sb.shape == (-(-N // 128), 2)
        assert np.array_equal(sb, ts), N
        assert np.array_equal(codes, tc), N


def test_ragged_grouped_weight_quant_is_per_expert():
    rng = np.random.default_rng(62)
    w = rng.standard_normal((3, 200, 128), dtype=np.float32)
    codes, sb = oracle.quantize_weight_128x128(w)
    assert sb.shape == (3, 2, 1)
    for g in range(3):
        c, s = oracle.quantize_weight_128x128(w[g])
        assert np.array_equal(c, codes[g]) and np.array_equal(s, sb[g])


def test_ragged_gemm_equals_zero_padded_gemm():
    rng = np.random.default_rng(63)
    M, N, K = 40, 200, 384
    A, sa = oracle.quantize_act_1x128(rng.standard_normal((M, K), dtype=np.float32))
    B, sb = oracle.quantize_weight_128x128(rng.standard_normal((N, K), dtype=np.float32))
    Bp = np.zeros((256, K), np.uint8)
    Bp[:N] = B
    ref = oracle.ref_dense(A, sa, B, sb)
    assert ref.shape == (M, N)
    assert np.array_equal(ref, oracle.ref_dense(A, sa, Bp, sb)[:, :N])
    assert np.allclose(ref, oracle.ref_dense_twolevel(A, sa, B, sb), rtol=1e-12, atol=1e-9)
    rows = rng.integers(0, M, 50)
    cols = np.concatenate([rng.integers(0, N, 45), [127, 128, 199, 198, 0]])
    assert np.allclose(oracle.ref_entries(A, sa, B, sb, rows, cols), ref[rows, cols], rtol=1e-12, atol=1e-9)
