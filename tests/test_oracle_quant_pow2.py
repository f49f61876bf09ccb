"""Pins for the oracle's power-of-two (E8M0) scale variant of the block quantisers.

Independent references: an exhaustive search over exponents for the scale
rule, the same recipe written with float64 log2/ceil/exp2 and torch's
float8_e4m3fn cast, lossless round trips of blocks built from E4M3 values
times a power of two, and the range the rounded-up scale guarantees.
"""
import numpy as np
import torch

from oracle import decode_table, pow2_ceil_scale, quantize_act_1x128, quantize_weight_128x128

DEC = decode_table()


def brute_pow2(s):
    """Smallest 2^e (e integer) with 2^e >= s, by scanning e upwards; floor 2^-126."""
    s = float(np.float32(s))
    e = -149
    while 2.0 ** e < s:
        e += 1
    return max(2.0 ** e, 2.0 ** -126)


def test_pow2_ceil_matches_exhaustive_search():
    rng = np.random.default_rng(41)
    vals = [np.float32(2.0 ** k) for k in range(-126, 120, 7)]                     # exact powers
    vals += [np.nextafter(np.float32(2.0 ** k), np.float32(np.inf)) for k in range(-100, 100, 9)]
    vals += [np.nextafter(np.float32(2.0 ** k), np.float32(0)) for k in range(-100, 100, 9)]
    vals += list((rng.uniform(0.5, 1.0, 200) * 2.0 ** rng.integers(-130, 120, 200)).astype(np.float32))
    vals += [np.float32(1.0e-40), np.float32(2.0 ** -149), np.float32(3.0 / 448.0)]
    vals = np.array([v for v in vals if v > 0], dtype=np.float32)
    got = pow2_ceil_scale(vals)
    want = np.array([brute_pow2(v) for v in vals], dtype=np.float32)
    assert np.array_equal(got, want)
    assert got.dtype == np.float32


def torch_quant_pow2(x, br, bc):
    """The power-of-two recipe with torch ops: amax/448 (fp32) -> 2^ceil(log2) in
    float64 -> floor 2^-126 -> exact division -> clamp -> float8 cast."""
    t = torch.from_numpy(x)
    R, C = t.shape
    blk = t.reshape(R // br, br, C // bc, bc)
    amax = blk.abs().amax(dim=(1, 3))
    scale = amax / 448.0
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    p2 = torch.exp2(torch.ceil(torch.log2(scale.double()))).clamp_min(2.0 ** -126).float()
    y = (blk / p2[:, None, :, None]).clamp(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return codes.numpy(), p2.numpy()


def test_act_quant_pow2_matches_torch():
    rng = np.random.default_rng(42)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    codes, sa = quantize_act_1x128(x, pow2=True)
    tc, ts = torch_quant_pow2(x, 1, 128)
    assert np.array_equal(sa, ts)
    assert np.array_equal(codes, tc)


def test_weight_quant_pow2_matches_torch():
    rng = np.random.default_rng(43)
    w = rng.standard_normal((384, 256), dtype=np.float32)
    codes, sb = quantize_weight_128x128(w, pow2=True)
    tc, ts = torch_quant_pow2(w, 128, 128)
    assert np.array_equal(sb, ts)
    assert np.array_equal(codes, tc)
    wg = rng.standard_normal((2, 256, 128), dtype=np.float32)
    cg, sg = quantize_weight_128x128(wg, pow2=True)
    for g in range(2):
        c, s = quantize_weight_128x128(wg[g], pow2=True)
        assert np.array_equal(c, cg[g]) and np.array_equal(s, sg[g])


def test_representable_blocks_round_trip_losslessly():
    """A block made of E4M3 values times 2^e whose largest magnitude lies in
    (224, 448] * 2^e gets scale exactly 2^e and its own codes back."""
    rng = np.random.default_rng(44)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rows = []
    exps = [-20, -7, 0, 3, 11]
    tops = [0x7E, 0x7D, 0x7A, 0x78]          # 448, 416, 352, 256: all in (224, 448]
    for e in exps:
        for top in tops:
            mags = DEC[finite] <= DEC[top]
            c = rng.choice(finite[mags & (DEC[finite] > -DEC[top])], 128)
            c[rng.integers(0, 128)] = top | (0x80 if rng.integers(0, 2) else 0)
            rows.append((c, e))
    codes_in = np.stack([c for c, _ in rows])
    x = (DEC[codes_in] * np.array([2.0 ** e for _, e in rows])[:, None]).astype(np.float32)
    codes, sa = quantize_act_1x128(x, pow2=True)
    assert np.array_equal(sa[:, 0], np.array([2.0 ** e for _, e in rows], np.float32))
    # -0 and +0 decode alike; compare values, then the nonzero codes bitwise
    assert np.array_equal(DEC[codes], DEC[codes_in])
    nz = DEC[codes_in] != 0
    assert np.array_equal(codes[nz], codes_in[nz])


def test_pow2_scale_range_and_no_saturation():
    """The rounded-up scale is a power of two in [s, 2s) of the plain scale s, so
    the block maximum lands in (224, 448] and nothing is clipped."""
    rng = np.random.default_rng(45)
    x = (rng.standard_normal((128, 1024)) * np.exp(rng.uniform(-10, 10, (128, 1)))).astype(np.float32)
    codes, sa = quantize_act_1x128(x, pow2=True)
    _, s_plain = quantize_act_1x128(x)
    m, _ = np.frexp(sa.astype(np.float64))
    assert np.all(m == 0.5)                                   # powers of two
    assert np.all(sa >= s_plain) and np.all(sa < 2 * s_plain.astype(np.float64))
    blocks = np.abs(x.astype(np.float64)).reshape(128, 8, 128).max(axis=2)
    ratio = blocks / sa
    assert np.all(ratio > 224) and np.all(ratio <= 448)
    assert not np.any((codes & 0x7F) == 0x7F)
    assert np.all(np.abs(DEC[codes]) <= 448)


def test_tiny_blocks_use_the_smallest_normal_scale():
    x = np.zeros((3, 128), dtype=np.float32)
    x[0, 0] = np.float32(1e-38)      # amax/448 is subnormal
    x[1, 7] = np.float32(-3e-36)     # amax/448 just under 2^-126 * 2
    codes, sa = quantize_act_1x128(x, pow2=True)
    assert sa[0, 0] == np.float32(2.0 ** -126)
    assert sa[1, 0] == np.float32(2.0 ** -126) or sa[1, 0] == np.float32(2.0 ** -125)
    assert sa[1, 0] == np.float32(brute_pow2(np.float32(3e-36) / np.float32(448.0)))
    assert sa[2, 0] == 1.0 and np.all(codes[2] == 0)          # all-zero block keeps scale 1
