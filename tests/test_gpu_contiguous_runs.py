"""GPU parity of the contiguous layout on 256-row tiles. Experts are padded
only to 128 rows, so those tiles follow each expert's run of 128-row blocks
from a tile list the kernel derives from m_indices: tiles start at a run's
first block and every second block after it, and the workgroups walk the list
persistently. These cases put run boundaries at odd blocks, across the 64-block
steps of the device-side scan, around all-padding blocks and partial tails, and
give an expert more than one run (more tiles than the launch has workgroups).

The same cases also run on the runs kernel ("runs"): two-block tiles of
256x256 and, for the single block at the end of an odd run and for the
two-block tiles past the last whole round, 128x256 tiles; two large cases
reach each of its two schedules (the tail split into 128-row halves, and every
two-block tile whole) on a 256-CU device."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_runs, forced_tile as forced
from fgtest import SENTINEL, d_bits, dense_inputs, new_out, to_dev

pytestmark = pytest.mark.gpu

RUN_TILES = [(256, 224), (256, 128), (256, 256), (256, 112), "runs"]


def tile_id(t):
    return t if isinstance(t, str) else f"{t[0]}x{t[1]}"


def on_tile(tile):
    return forced_runs() if tile == "runs" else forced(*tile)


def m_indices_from(segments, tail_rows=0):
    """segments: (expert, real rows, padded rows) in row order; expert -1 is a
    block of padding. tail_rows: an extra partial block of expert -1 rows."""
    ids = []
    for e, real, padded in segments:
        ids += [e] * real + [-1] * (padded - real)
    ids += [-1] * tail_rows
    return np.asarray(ids, np.int32)


def run_case(mi, G, N, K, seed, tile, pow2=False):
    rng = np.random.default_rng(seed)
    M = mi.shape[0]
    a = rng.standard_normal((M, K), dtype=np.float32)
    b = rng.standard_normal((G, N, K), dtype=np.float32)
    A, sa = oracle.quantize_act_1x128(a, pow2)
    B, sb = oracle.quantize_weight_128x128(b, pow2)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((M, N))
    with on_tile(tile):
        (fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous)(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    # ids outside [0, G) are padding: no output, not written
    mi_ref = np.where((mi >= 0) & (mi < G), mi, -1)
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi_ref)
    return oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)


CASES = {
    # odd runs, a one-block run, an all-padding block between experts, a
    # partial final block
    "odd_runs": ([(2, 300, 384), (-1, 0, 128), (0, 100, 128), (1, 256, 256), (3, 129, 256)], 77, 4),
    # one expert in several runs (5 tiles per column where 2 experts bound 3)
    "split_expert": ([(0, 128, 128), (1, 128, 128), (0, 128, 128), (1, 50, 128), (0, 128, 128)], 0, 2),
    # fewer rows than one block
    "tiny": ([(1, 5, 5)], 0, 2),
    # one expert over an odd number of blocks (G = 1)
    "one_expert": ([(0, 9 * 128 - 40, 9 * 128)], 0, 1),
    # runs that cross the scan's 64-block steps at odd offsets (141 blocks)
    "many_blocks": ([(1, 63 * 128, 63 * 128), (0, 3 * 128 - 5, 3 * 128), (2, 70 * 128, 70 * 128),
                     (0, 4 * 128, 4 * 128)], 40, 3),
}


@pytest.mark.parametrize("tile", RUN_TILES, ids=tile_id)
@pytest.mark.parametrize("case", list(CASES))
def test_contiguous_run_tiles(case, tile):
    segs, tail, G = CASES[case]
    mi = m_indices_from(segs, tail)
    N, K = (256, 256) if case == "many_blocks" else (384, 640)
    print(f"contiguous runs {case} tile {tile} M={mi.shape[0]} N={N} K={K} G={G}", flush=True)
    r = run_case(mi, G, N, K, 70 + len(mi), tile)
    assert r["ok"], r


@pytest.mark.parametrize("tile", [RUN_TILES[0], "runs"], ids=tile_id)
def test_contiguous_run_tiles_ids_out_of_range(tile):
    """Ids >= G count as padding: such rows are not written and do not decide a
    block's expert."""
    mi = m_indices_from([(0, 200, 256), (1, 128, 128)], 0)
    mi[5] = 7
    mi[130] = 99
    mi[300] = 2
    print(f"contiguous runs ids out of range tile {tile}", flush=True)
    r = run_case(mi, 2, 384, 256, 91, tile)
    assert r["ok"], r


@pytest.mark.parametrize("tile", [RUN_TILES[0], "runs"], ids=tile_id)
def test_contiguous_run_tiles_all_padding(tile):
    """No row has an expert: nothing is written."""
    mi = np.full(384, -1, np.int32)
    print(f"contiguous runs all padding tile {tile}", flush=True)
    r = run_case(mi, 2, 256, 256, 92, tile)
    assert r["ok"], r


def blocks_case(blocks):
    """Experts with the given numbers of 128-row blocks, in row order, each
    with a partial last block."""
    return m_indices_from([(e, nb * 128 - (17 * e) % 100, nb * 128) for e, nb in enumerate(blocks)])


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
@pytest.mark.parametrize("name,blocks", [
    # 31 two-block tiles x 8 columns = 248 < 256 workgroups, halves would need
    # 512 items: every two-block tile runs whole, the two single blocks as
    # 128-row tiles
    ("whole", [17, 15, 16, 16]),
    # 34 x 8 = 272: one whole round, the last 16 two-block tiles as 32 halves
    # together with 2 x 8 single-block tiles
    ("tail_halves", [18, 16, 18, 17, 1]),
])
def test_runs_kernel_schedules(name, blocks, pow2):
    mi = blocks_case(blocks)
    print(f"contiguous runs kernel {name} M={mi.shape[0]} N=2048 K=256 pow2={pow2}", flush=True)
    r = run_case(mi, len(blocks), 2048, 256, 93 + len(blocks), "runs", pow2)
    assert r["ok"], r


def test_runs_chosen_for_the_contiguous_workload():
    """The contiguous workload's shape (9472 rows in 8 experts, N 4096, K 7168)
    runs on the runs kernel: one workgroup per CU walking the work items."""
    assert fg.select_config(9472, 4096, 7168, 8, 1) == (256, 256)
    assert fg.select_grid(9472, 4096, 7168, 8, 1) == 256
