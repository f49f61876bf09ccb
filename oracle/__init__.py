"""CPU oracle for the FP8 (E4M3) block-scaled GEMM: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. This package is the reference that the HIP path is
checked against. Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library itself never does, and the two
share no code, tables or constants.

What it computes (fp64 throughout, numpy):
  * ``e4m3``  -- the 256-entry OCP E4M3 decode table and a round-to-nearest-even
                 encoder with saturation at 448.
  * ``quant`` -- per 1x128 (activation) and per 128x128 (weight) block
                 quantisation with scale = amax / 448, or that scale rounded
                 up to a power of two (the E8M0 / micro-scaling variant).
  * ``gemm``  -- D = A . B^T as "dequantise, then one fp64 GEMM" for the dense,
                 grouped-contiguous and grouped-masked layouts, plus the
                 two-level (per 128-wide K-block partial, then scale and add)
                 form the method describes, and single-entry references for
                 sampling full-size outputs.
  * ``ffn``   -- the fused epilogue of an MoE expert's first projection:
                 SiLU-gated activation of D (gate/up interleaved in 128-column
                 blocks), re-quantised with the ``quant`` quantisers.
  * ``check`` -- the acceptance test (per-element and Frobenius bounds, and
                 bitwise "untouched" for rows the call must not write).

Sources: the DeepGEMM pages -- "DeepGEMM: an open-source FP8 GEMM library"
(zwzgs.cn; sections "Features > fine-grained scaling", "Features > layouts",
"Technical details > two-level accumulation"), the 2kiu.com DeepGEMM explainer
(sections 2.2 "new challenges of low precision", 3.3 "focus on FP8" and 4.4
"precision control"), and "DeepSeek open-sources DeepGEMM" (ruibaoantu.com,
section 1 "FP8 data type", which defines E4M3 as 4 exponent + 3 mantissa bits).

Parity status: every public function here is pinned by a CPU test against
something other than itself (torch's float8 cast, exhaustive search, exact
rational arithmetic, integer matmul, closed forms, invariants).
"""

from .e4m3 import decode_table, encode_rne, E4M3_MAX  # noqa: F401
from .quant import (quantize_blocks, quantize_act_1x128, quantize_weight_128x128,  # noqa: F401
                    pow2_ceil_scale)
from .gemm import (  # noqa: F401
    dequant_act,
    dequant_weight,
    ref_dense,
    ref_dense_twolevel,
    ref_contiguous,
    ref_masked,
    ref_entries,
)
from .check import check, bf16_rne, bf16_bits_to_f64  # noqa: F401
from .ffn import silu, swiglu_blocks  # noqa: F401
