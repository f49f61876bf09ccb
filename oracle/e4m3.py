"""OCP E4M3 ("e4m3fn") decoding and round-to-nearest-even encoding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The ruibaoantu.com page "DeepSeek open-sources DeepGEMM" (section 1, "FP8 data
type") gives E4M3 as 4 exponent bits and 3 mantissa bits; the 2kiu.com DeepGEMM
explainer (section 2.2) says E4M3 is the higher-precision, smaller-range FP8
format and is the one used for GEMM inputs, and (section 4.4) that values out of
range are clipped or saturated. The pages stop there; the reading taken is the
OCP 8-bit float "E4M3" variant: exponent bias 7, no infinities, the all-ones
pattern S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_one(code):
    """Value of one byte code s.eeee.fff (fp64; NaN for S.1111.111)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return float("nan")
    if e == 0:
        mag = f * 2.0 ** -9          # subnormal: (f/8) * 2^(1-7)
    else:
        mag = (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def decode_table():
    """All 256 E4M3 codes as fp64 values (index = byte code)."""
    return np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS = decode_table()[:0x7F]


def encode_rne(y):
    """Encode fp32 values to E4M3 codes, rounding to nearest, ties to even.

    ``y`` must already be finite and within [-448, 448] (the block quantiser
    clamps before calling). Ties go to the code whose mantissa LSB is 0; since
    the three mantissa bits are the code's low bits and the codes 0x00..0x7E are
    ordered by value, that is the even code. The sign bit is copied from y, so a
    negative value that rounds to zero gives 0x80 (negative zero).
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("encode_rne: non-finite input")
    a = np.abs(y).astype(np.float64)
    if np.any(a > E4M3_MAX):
        raise ValueError("encode_rne: input beyond 448; clamp first")
    # hi = first code whose value is >= a; lo = hi - 1.
    hi = np.searchsorted(_POS, a, side="left")
    exact = _POS[np.minimum(hi, 0x7E)] == a
    lo = np.maximum(hi - 1, 0)
    mid = (_POS[lo] + _POS[np.minimum(hi, 0x7E)]) * 0.5   # exact in fp64
    pick_hi = a > mid
    tie = a == mid
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    mag = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)
