"""Bitwise invariants of the GPU path, independent of any tolerance.

Every output element is computed the same way whatever tile, kernel or layout
produces it: for each 128-wide K-block, one matrix-core 16x16x128 dot product
of the same 128 code pairs (the same K placement in every lane), then, in
K-block order, fp32 promotion acc = fma(P, sa * sb, acc) (power-of-two scales:
the matrix core's scaled product added to acc). So the bf16 output must be bit
for bit the same across all compiled tiles, the dense two-shape kernel, the
contiguous layout with one expert and the masked layout with every row valid;
this pins the tiling, the scale addressing and the layouts against each other
(a wrong scale block, a transposed fragment or a tile-edge mistake anywhere
breaks it), in addition to the oracle checks of the parity tests.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_split, forced_tile
from fgtest import d_bits, dense_inputs, make_dense, make_masked, masked_inputs, new_out, to_dev

pytestmark = pytest.mark.gpu

TILES = [(256, 256), (256, 128), (128, 256), (128, 128), (64, 112), (256, 112), (256, 224)]
SCALES = [False, True]


def scale_id(pow2):
    return "pow2_scales" if pow2 else "fp32_scales"


def dense_bits(ops, M, N, pow2):
    D = new_out((M, N))
    (fg.gemm_fp8_nt_pow2 if pow2 else fg.gemm_fp8_nt)(*ops, D)
    torch.cuda.synchronize()
    return d_bits(D)


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
def test_dense_bitwise_across_tiles(pow2):
    """Ragged M and N (N = 776: a partial 128-wide scale block, no multiple of
    112, 224 or 256), K over more K-blocks than any ring holds."""
    M, N, K = 300, 776, 1152
    print(f"dense across tiles M={M} N={N} K={K} pow2={pow2}", flush=True)
    ops = dense_inputs(*make_dense(M, N, K, 700, pow2=pow2))
    ref = dense_bits(ops, M, N, pow2)
    for bm, bn in TILES:
        with forced_tile(bm, bn):
            out = dense_bits(ops, M, N, pow2)
        assert np.array_equal(out, ref), f"tile {bm}x{bn} differs from the automatic choice"
    for n_split in (256, 512):
        with forced_split(n_split):
            out = dense_bits(ops, M, N, pow2)
        assert np.array_equal(out, ref), f"split at {n_split} differs"


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
def test_contiguous_one_expert_equals_dense(pow2):
    """Contiguous with G = 1 and no padding is the dense product of the same
    operands (on the contiguous layout's own tiles and run-following kernel)."""
    M, N, K = 640, 512, 768
    print(f"contiguous one expert M={M} N={N} K={K} pow2={pow2}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, 701, pow2=pow2)
    ops = dense_inputs(A, sa, B, sb)
    ref = dense_bits(ops, M, N, pow2)
    Ad, sad, Bd, sbd = ops
    mi = to_dev(np.zeros(M, np.int32))
    fn = fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous
    for tile in (None, (256, 256), (128, 256), (128, 128)):
        D = new_out((M, N))
        if tile is None:
            fn(Ad, sad, Bd.view(1, N, K), sbd.view(1, *sbd.shape), D, mi)
        else:
            with forced_tile(*tile):
                fn(Ad, sad, Bd.view(1, N, K), sbd.view(1, *sbd.shape), D, mi)
        torch.cuda.synchronize()
        assert np.array_equal(d_bits(D), ref), f"contiguous tile {tile} differs from dense"


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
def test_masked_all_rows_equals_dense_per_expert(pow2):
    """Masked with masked_m = M_max everywhere is G dense products."""
    G, M_max, N, K = 3, 200, 384, 640
    print(f"masked all rows G={G} M_max={M_max} N={N} K={K} pow2={pow2}", flush=True)
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 702, pow2=pow2)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    (fg.grouped_masked_pow2 if pow2 else fg.grouped_masked)(Ad, sad, Bd, sbd, D,
                                                            to_dev(np.full(G, M_max, np.int32)))
    torch.cuda.synchronize()
    out = d_bits(D)
    for g in range(G):
        ref = dense_bits((Ad[g].contiguous(), sad[g].contiguous(), Bd[g].contiguous(), sbd[g].contiguous()),
                         M_max, N, pow2)
        assert np.array_equal(out[g], ref), f"expert {g} differs from its dense product"
