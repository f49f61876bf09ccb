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
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode_rne


def quantize_blocks(x, block_rows, block_cols):
    """Quantise a 2-D fp32 array in (block_rows x block_cols) blocks.

    Returns (codes uint8 same shape as x, scales fp32 [R/block_rows, C/block_cols]).
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
    y = (blocks / scale[:, None, :, None]).astype(np.float32)   # fp32 division
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_rne(y).reshape(R, C)
    return codes, scale


def quantize_act_1x128(x):
    """Activation quantisation: x fp32 [M, K] -> codes [M, K], sa fp32 [M, K/128]."""
    return quantize_blocks(x, 1, 128)


def quantize_weight_128x128(w):
    """Weight quantisation: w fp32 [N, K] (or [G, N, K]) -> codes, sb [N/128, K/128]
    (or [G, N/128, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim == 2:
        return quantize_blocks(w, 128, 128)
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty((w.shape[0], w.shape[1] // 128, w.shape[2] // 128), dtype=np.float32)
    for g in range(w.shape[0]):
        codes[g], scales[g] = quantize_blocks(w[g], 128, 128)
    return codes, scales
