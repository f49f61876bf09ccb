"""Block-wise FP8 quantisation with fp32 scales (DeepSeek-V3 fine-grained scaling).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The zwzgs.cn page "DeepGEMM: an open-source FP8 GEMM library" ("Features >
fine-grained scaling") says the scaling is the fine-grained scheme of
DeepSeek-V3; the 2kiu.com explainer (sections 3.3 and 4.4) says scale factors
are computed from the data's statistics so values fit the FP8 range, and that
out-of-range values are clipped/saturated. Readings taken where the pages stop:

  * granularity: one scale per 1x128 block of the activation A (a row segment
    along K) and per 128x128 block of the weight B;
  * scale = fp32(amax / 448), amax = largest |x| in the block (fp32); an
    all-zero block gets scale 1 (its codes are all zero);
  * y = fp32(x / scale), clamped to [-448, 448] before rounding (x / scale can
    land one ulp beyond 448), then rounded to nearest E4M3, ties to even.

The dequantised value of a code is decode(code) * scale.

Power-of-two scales (``pow2=True``). The 2kiu.com explainer, section 7 (where
it points beyond FP8), names MX / micro-scaling formats, whose block scales are
pure powers of two (an 8-bit exponent, E8M0). Reading taken for that variant:
the scale is the fp32 scale above rounded UP to the next power of two (so
x / scale still lies within [-448, 448] and the division is exact), and never
below 2^-126, the smallest normal fp32 value (every such scale is then an
E8M0 code 2^(e - 127) with e in 1..254).
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_rne


def pow2_ceil_scale(scale):
    """Smallest power of two >= each fp32 scale, floored at 2^-126 (fp32 out).

    frexp writes a positive s as m * 2^e with m in [0.5, 1): s is itself a power
    of two exactly when m == 0.5, otherwise the next power of two up is 2^e.
    """
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    if np.any(~(s > 0)) or np.any(~np.isfinite(s)):
        raise ValueError("pow2_ceil_scale: scales must be positive and finite")
    m, e = np.frexp(s)
    p = np.where(m == 0.5, s, np.ldexp(1.0, e))
    return np.maximum(p, 2.0 ** -126).astype(np.float32)


def quantize_blocks(x, block_rows, block_cols, pow2=False):
    """Quantise a 2-D fp32 array in (block_rows x block_cols) blocks.

    Returns (codes uint8 same shape as x, scales fp32 [R/block_rows, C/block_cols]).
    With pow2=True every scale is rounded up to a power of two first.
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if R % block_rows or C % block_cols:
        raise ValueError("quantize_blocks: shape not a multiple of the block")
    nr, nc = R // block_rows, C // block_cols
    blocks = x.reshape(nr, block_rows, nc, block_cols)
    amax = np.abs(blocks).max(axis=(1, 3))                      # fp32, exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)    # fp32 division
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    if pow2:
        scale = pow2_ceil_scale(scale)
    y = (blocks / scale[:, None, :, None]).astype(np.float32)   # fp32 division
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_rne(y).reshape(R, C)
    return codes, scale


def quantize_act_1x128(x, pow2=False):
    """Activation quantisation: x fp32 [M, K] -> codes [M, K], sa fp32 [M, K/128]."""
    return quantize_blocks(x, 1, 128, pow2)


def _quantize_weight_2d(w, pow2):
    """128x128 blocks of w [N, K]; when N is not a multiple of 128 the last row
    block holds the remaining N mod 128 rows (reading: its amax and scale come
    from those rows alone). Zero rows appended to fill the block change neither
    its amax nor its scale, so the block is quantised padded and cut back."""
    N, K = w.shape
    Np = -(-N // 128) * 128
    if Np == N:
        return quantize_blocks(w, 128, 128, pow2)
    wp = np.zeros((Np, K), dtype=np.float32)
    wp[:N] = w
    codes, scale = quantize_blocks(wp, 128, 128, pow2)
    return codes[:N], scale


def quantize_weight_128x128(w, pow2=False):
    """Weight quantisation: w fp32 [N, K] (or [G, N, K]) -> codes, sb [ceil(N/128), K/128]
    (or [G, ceil(N/128), K/128])."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim == 2:
        return _quantize_weight_2d(w, pow2)
    nb = -(-w.shape[1] // 128)
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty((w.shape[0], nb, w.shape[2] // 128), dtype=np.float32)
    for g in range(w.shape[0]):
        codes[g], scales[g] = _quantize_weight_2d(w[g], pow2)
    return codes, scales
