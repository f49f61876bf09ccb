"""Pins for the oracle's block quantisers (1x128 activation, 128x128 weight).

Independent references: the same recipe written with torch ops and torch's
float8_e4m3fn cast, hand-built blocks with known scales, and the format's
worst-case rounding error as a bound.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import decode_table, quantize_act_1x128, quantize_weight_128x128

DEC = decode_table()


def torch_quant(x, br, bc):
    """Block quantisation with torch ops (amax -> /448 -> divide -> clamp -> cast)."""
    t = torch.from_numpy(x)
    R, C = t.shape
    blk = t.reshape(R // br, br, C // bc, bc)
    amax = blk.abs().amax(dim=(1, 3))
    scale = amax / 448.0
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    y = (blk / scale[:, None, :, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return codes.numpy(), scale.numpy()


def test_act_quant_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512), dtype=np.float32)
    x[5] *= 50.0
    x[7, 128:256] = 0.0                      # an all-zero block
    codes, sa = quantize_act_1x128(x)
    tc, ts = torch_quant(x, 1, 128)
    assert sa.shape == (64, 4) and sa.dtype == np.float32
    assert np.array_equal(sa, ts) and np.array_equal(codes, tc)


def test_weight_quant_matches_torch():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((256, 384), dtype=np.float32) * np.float32(0.02)
    codes, sb = quantize_weight_128x128(w)
    tc, ts = torch_quant(w, 128, 128)
    assert sb.shape == (2, 3)
    assert np.array_equal(sb, ts) and np.array_equal(codes, tc)


def test_grouped_weight_quant_is_per_group():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((3, 128, 256), dtype=np.float32)
    w[1] *= 8.0
    codes, sb = quantize_weight_128x128(w)
    assert sb.shape == (3, 1, 2)
    for g in range(3):
        c, s = quantize_weight_128x128(w[g])
        assert np.array_equal(c, codes[g]) and np.array_equal(s, sb[g])


def test_scale_is_amax_over_448_and_max_maps_to_448():
    x = np.zeros((2, 256), dtype=np.float32)
    x[0, :128] = np.linspace(-3.0, 2.0, 128, dtype=np.float32)   # amax 3
    x[0, 128:] = 448.0 * 2.0 ** -5                               # amax 14, power-of-two scale
    x[1, 5] = -7.0
    codes, sa = quantize_act_1x128(x)
    assert sa[0, 0] == np.float32(3.0) / np.float32(448.0)
    assert sa[0, 1] == np.float32(2.0 ** -5)
    assert np.all(codes[0, 128:] == 0x7E)                         # exactly +448
    assert codes[0, 0] == 0xFE                                    # -3 -> -448
    assert sa[1, 0] == np.float32(7.0 / 448.0) and codes[1, 5] == 0xFE
    assert sa[1, 1] == 1.0 and np.all(codes[1, 128:] == 0)        # all-zero block


def test_block_layout_isolation():
    """A spike in one block changes only that block's scale."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 512), dtype=np.float32)
    _, sa0 = quantize_act_1x128(x)
    x[3, 300] = 1000.0
    _, sa1 = quantize_act_1x128(x)
    diff = sa0 != sa1
    assert diff.sum() == 1 and diff[3, 2]

    w = rng.standard_normal((256, 384), dtype=np.float32)
    _, sb0 = quantize_weight_128x128(w)
    w[200, 10] = 1000.0
    _, sb1 = quantize_weight_128x128(w)
    diff = sb0 != sb1
    assert diff.sum() == 1 and diff[1, 0]


def test_roundtrip_error_bound_and_no_nan():
    """|dec(code)*scale - x| <= half the E4M3 spacing at |x| (relative 2^-4 for
    normals, absolute 2^-10 * scale in the subnormal range)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((32, 1024)) * np.exp(rng.uniform(-6, 6, (32, 1)))).astype(np.float32)
    codes, sa = quantize_act_1x128(x)
    assert not np.any((codes & 0x7F) == 0x7F)
    s = np.repeat(sa.astype(np.float64), 128, axis=1)
    xr = DEC[codes] * s
    y = np.abs(x.astype(np.float64)) / s
    half_spacing = np.where(y < 2.0 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4))
    # x/scale is rounded to fp32 first; allow that one extra fp32 ulp
    assert np.all(np.abs(xr - x) <= (half_spacing * (1 + 2.0 ** -20)) * s)


@pytest.mark.parametrize("pow2", [False, True])
def test_parallel_drivers_equal_serial(pow2):
    """The chunked, thread-parallel drivers used for full-size inputs give the
    serial quantisers' codes and scales exactly (blocks never straddle a chunk),
    including a ragged last weight block and a batched activation."""
    from oracle.parallel import quantize_act_1x128_par, quantize_weight_128x128_par
    rng = np.random.default_rng(77)
    x = rng.standard_normal((1100, 384), dtype=np.float32)
    x[1099, 5] = 300.0
    c1, s1 = quantize_act_1x128_par(x, pow2, chunk=256)
    c2, s2 = oracle.quantize_act_1x128(x, pow2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    xb = rng.standard_normal((3, 70, 256), dtype=np.float32)
    c1, s1 = quantize_act_1x128_par(xb, pow2, chunk=32)
    for b in range(3):
        c2, s2 = oracle.quantize_act_1x128(xb[b], pow2)
        assert np.array_equal(c1[b], c2) and np.array_equal(s1[b], s2)
    w = rng.standard_normal((3, 584, 256), dtype=np.float32)
    w[1, 583, 7] = 50.0
    c1, s1 = quantize_weight_128x128_par(w, pow2, chunk=256)
    c2, s2 = oracle.quantize_weight_128x128(w, pow2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    c1, s1 = quantize_weight_128x128_par(w[0], pow2, chunk=128)
    c2, s2 = oracle.quantize_weight_128x128(w[0], pow2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
