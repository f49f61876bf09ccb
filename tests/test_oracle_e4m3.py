"""Pins for the oracle's E4M3 decode table and round-to-nearest-even encoder.

Independent references: torch's float8_e4m3fn dtype (decode and cast), an
exhaustive nearest-value search, and hand-derived landmark values of the OCP
E4M3 format (bias 7, max 448, NaN = S.1111.111).
"""
import numpy as np
import pytest
import torch

from oracle import decode_table, encode_rne


def torch_decode_all():
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_all_codes():
    ours = decode_table()
    lib = torch_decode_all()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])
    # sign of zero too
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


def test_decode_landmarks():
    t = decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0 and t[0x39] == 1.125 and t[0xB8] == -1.0
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    nan = np.isnan(t)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.all(np.diff(t[:0x7F]) > 0)  # codes 0..126 strictly increasing


def brute_force_encode(y):
    """Nearest of the 254 finite values (minimum distance, exhaustive), ties to
    the code with mantissa LSB 0; sign copied from y."""
    t = decode_table()
    pos = [(c, t[c]) for c in range(0x7F)]
    out = []
    for v in np.asarray(y, dtype=np.float32):
        a = abs(float(v))
        best = None
        for c, val in pos:
            d = abs(a - val)
            if best is None or d < best[1] or (d == best[1] and (c & 1) == 0):
                best = (c, d)
        out.append(best[0] | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_vs_bruteforce_random():
    rng = np.random.default_rng(0)
    # spread over every binade of the format, plus exact midpoints between codes
    mags = 2.0 ** rng.uniform(-12, np.log2(448.0), size=1500)
    y = (mags * rng.choice([-1, 1], size=mags.size)).astype(np.float32)
    t = decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    y = np.concatenate([y, mids, -mids, t.astype(np.float32), np.float32([0.0, -0.0, 448.0, -448.0])])
    y = np.clip(y, -448, 448).astype(np.float32)
    assert np.array_equal(encode_rne(y), brute_force_encode(y))


def test_encode_vs_torch_cast():
    rng = np.random.default_rng(1)
    y = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(60.0),
        (2.0 ** rng.uniform(-14, 8.8, 20000)).astype(np.float32),
    ])
    y = np.clip(y, -448, 448).astype(np.float32)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(encode_rne(y), lib)


@pytest.mark.parametrize("value,code", [
    (448.0, 0x7E),
    (2.0 ** -10, 0x00),          # tie between 0 and 2^-9 -> even (0)
    (1.5 * 2.0 ** -9, 0x02),     # tie between codes 1 and 2 -> even (2)
    (2.5 * 2.0 ** -9, 0x02),     # tie between codes 2 and 3 -> even (2)
    (7.5 * 2.0 ** -9, 0x08),     # tie across the subnormal/normal boundary
    (1.0625, 0x38),              # tie between 1.0 (0x38) and 1.125 (0x39)
    (1.1875, 0x3A),              # tie between 1.125 (0x39) and 1.25 (0x3A)
    (1.07, 0x39),                # nearer 1.125
    (432.0, 0x7E),               # tie between 416 (0x7D) and 448 (0x7E) -> even
    (-2.0 ** -11, 0x80),         # rounds to zero, keeps the sign
    (-3.0, 0xC4),
])
def test_encode_landmarks(value, code):
    assert encode_rne(np.float32([value]))[0] == code


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        encode_rne(np.float32([449.0]))
    with pytest.raises(ValueError):
        encode_rne(np.float32([np.nan]))
