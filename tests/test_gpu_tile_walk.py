"""Workgroups that walk many tiles.

The dense two-shape kernel and the contiguous 256-row kernels run one
workgroup per CU, and each workgroup computes its tiles one after another:
with the direct-store epilogue the next tile's first stages are issued before
the previous tile's output stores, and its first wait counts those stores.
At the small sizes of the parity tests every workgroup gets one tile or two,
so these tests cap the grid (test library only) to make each workgroup walk
many tiles -- ragged M and N tails included -- and check against the oracle
and, bit for bit, against the automatic grid (a tile's arithmetic does not
depend on which workgroup computes it).
"""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_grid, forced_runs, forced_split, forced_tile
from fgtest import SENTINEL, d_bits, dense_inputs, make_dense, new_out, to_dev
import test_gpu_swiglu as sw

pytestmark = pytest.mark.gpu

SCALES = [False, True]


def scale_id(pow2):
    return "pow2_scales" if pow2 else "fp32_scales"


def dense_split(A, sa, B, sb, n_split, grid, pow2):
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], B.shape[0]))
    with forced_split(n_split), forced_grid(grid):
        (fg.gemm_fp8_nt_pow2 if pow2 else fg.gemm_fp8_nt)(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    return d_bits(D)


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
@pytest.mark.parametrize("K", [128, 640, 1152])
@pytest.mark.parametrize("grid", [1, 3, 7])
def test_dense_split_walk(grid, K, pow2):
    """12 tiles of 256x256 (ragged M: 1000 rows) and 16 of 256x128 (the last
    column block holds 8 columns) over 1, 3 or 7 workgroups; K from one
    K-block (fewer than the ring's stages) to an odd number of K-blocks."""
    M, N, n_split = 1000, 1160, 768
    print(f"dense split walk grid={grid} M={M} N={N} K={K} pow2={pow2}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, 300 + grid + K, pow2=pow2)
    out = dense_split(A, sa, B, sb, n_split, grid, pow2)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r
    assert np.array_equal(out, dense_split(A, sa, B, sb, n_split, 0, pow2))


def m_indices_from(segments):
    ids = []
    for e, real, padded in segments:
        ids += [e] * real + [-1] * (padded - real)
    return np.asarray(ids, np.int32)


# (expert, real rows, padded rows) in row order: odd and even runs, an expert
# in two runs, an all-padding block, a partial last block
SEGMENTS = [(2, 700, 768), (0, 100, 128), (-1, 0, 128), (1, 512, 512), (0, 300, 384), (3, 129, 256),
            (1, 250, 256)]


def contiguous_inputs(G, N, K, seed, pow2):
    mi = m_indices_from(SEGMENTS)
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((mi.shape[0], K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    A, sa = oracle.quantize_act_1x128(a, pow2)
    B, sb = oracle.quantize_weight_128x128(b, pow2)
    return A, sa, B, sb, mi


def on(kernel):
    return forced_runs() if kernel == "runs" else forced_tile(*kernel)


def contiguous_run(A, sa, B, sb, mi, kernel, grid, pow2):
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], B.shape[1]))
    with on(kernel), forced_grid(grid):
        (fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous)(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    return d_bits(D)


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
@pytest.mark.parametrize("kernel", ["runs", (256, 256), (256, 224)],
                         ids=lambda k: k if isinstance(k, str) else f"{k[0]}x{k[1]}")
@pytest.mark.parametrize("grid", [1, 5])
def test_contiguous_walk(grid, kernel, pow2):
    """The runs kernel (two-block 256x256 tiles, then 128x256 halves and single
    blocks) and the single-shape run-following kernel (256x256: direct-store
    epilogue; 256x224: staged through LDS) with 1 or 5 workgroups."""
    G, N, K = 4, 1024 if kernel != (256, 224) else 896, 384
    print(f"contiguous walk grid={grid} kernel={kernel} N={N} K={K} pow2={pow2}", flush=True)
    A, sa, B, sb, mi = contiguous_inputs(G, N, K, 310 + grid, pow2)
    out = contiguous_run(A, sa, B, sb, mi, kernel, grid, pow2)
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(out, ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r
    assert np.array_equal(out, contiguous_run(A, sa, B, sb, mi, kernel, 0, pow2))


@pytest.mark.parametrize("pow2", SCALES, ids=scale_id)
def test_contiguous_fused_walk(pow2):
    """The fused SiLU-gate epilogue on the runs kernel (staged through LDS,
    the next tile after it) with 2 workgroups: the activation against the
    oracle, codes and scales against the oracle quantiser, untouched rows
    unwritten, and every output equal to the automatic grid's."""
    G, N, K = 4, 1024, 384
    I = N // 2
    print(f"contiguous fused walk pow2={pow2}", flush=True)
    A, sa, B, sb, mi = contiguous_inputs(G, N, K, 320, pow2)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    M = A.shape[0]
    outs = []
    for grid in (2, 0):
        Q, sq, act = sw.prefilled((), M, I)
        with forced_runs(), forced_grid(grid):
            fg.grouped_contiguous_swiglu_quant(Ad, sad, Bd, sbd, to_dev(mi), Q, sq, act, pow2=pow2)
        torch.cuda.synchronize()
        outs.append((Q.cpu().numpy(), sq.cpu().numpy(), act.cpu().numpy()))
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    ref_act = np.zeros((M, I))
    ref_act[valid] = oracle.swiglu_blocks(ref[valid])
    Qh, sqh, acth = outs[0]
    sw.check_rows(Qh, sqh.T, acth, ref_act, valid, pow2)
    for x, y in zip(*outs):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
