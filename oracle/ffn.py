"""Reference for the fused GEMM epilogue of an MoE expert's first projection:
SiLU-gated activation of D, then FP8 re-quantisation with 1x128 scales.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. The 2kiu.com DeepGEMM explainer, section 7: a GEMM rarely stands
alone -- activation functions and normalisation come before and after it --
and fusing them with the GEMM to save memory round trips is the next
optimisation to look at. Its section 4.4 and the zwzgs.cn page ("Features >
fine-grained scaling") give the per-block quantisation the next GEMM consumes.

Readings taken where the pages stop (they name no activation and no weight
layout for one):
  * the activation is the SiLU gate of the MoE expert FFN,
        act = silu(gate) * up,   silu(x) = x / (1 + exp(-x));
  * gate and up are halves of one first-projection output D [M, N], N = 2*I,
    interleaved in 128-column blocks: D columns [256j, 256j+128) are gate
    block j and [256j+128, 256j+256) are up block j, so
        act[:, 128j + c] = silu(D[:, 256j + c]) * D[:, 256j + 128 + c];
    (a weight laid out this way lets one 256-column output tile produce
    exactly one 128-column quantisation block per row);
  * act is quantised per 1x128 block with the quantiser of ``oracle.quant``
    (fp32 scales amax/448, or powers of two), which is the next GEMM's A
    operand with K = I.
"""

import numpy as np


def silu(x):
    """x / (1 + exp(-x)) in fp64; exp(-x) overflows to inf for x < -709, where
    the quotient is the correct signed zero."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_blocks(d):
    """act [..., N/2] from D [..., N] with gate/up interleaved in 128-column blocks."""
    d = np.asarray(d, dtype=np.float64)
    N = d.shape[-1]
    if N % 256:
        raise ValueError("swiglu_blocks: N must be a multiple of 256")
    blocks = d.reshape(d.shape[:-1] + (N // 256, 2, 128))
    act = silu(blocks[..., 0, :]) * blocks[..., 1, :]
    return act.reshape(d.shape[:-1] + (N // 2,))
