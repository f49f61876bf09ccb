"""C-ABI checks that need no GPU: the library loads, exports every function
include/fg.h declares, rejects invalid arguments before touching the device,
and the host-side tile selection is sane."""
import ctypes
import os
import re

import pytest

import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_split, forced_tile as forced, testing_lib as _testing_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fg.h")
EINVAL, OK = -1, 0


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fg_gemm_fp8_nt", "fg_grouped_contiguous", "fg_grouped_masked",
              "fg_select_config", "fg_select_grid", "fg_strerror", "fg_quant_act_1x128", "fg_quant_weight_128x128",
              "fg_gemm_fp8_nt_pow2", "fg_grouped_contiguous_pow2", "fg_grouped_masked_pow2",
              "fg_quant_act_1x128_pow2", "fg_quant_weight_128x128_pow2",
              "fg_gemm_fp8_nt_swiglu_quant", "fg_grouped_contiguous_swiglu_quant",
              "fg_grouped_masked_swiglu_quant"):
        assert n in names


def test_library_loads_and_exports_everything_declared():
    L = ctypes.CDLL(fg.LIB_PATH, mode=os.RTLD_NOW)   # unresolved symbols fail here
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror_codes():
    for c in (0, -1, -2, -3, -4, 17):
        assert isinstance(fg.strerror(c), str) and fg.strerror(c)
    assert "invalid" in fg.strerror(-1)


BAD = ctypes.c_void_p(0x1001)      # misaligned, never dereferenced
GOOD = ctypes.c_void_p(0x100000)   # aligned, never dereferenced (validation fails first)


@pytest.mark.parametrize("args", [
    (GOOD, GOOD, GOOD, GOOD, GOOD, 64, 256, 100, None),       # K not a multiple of 128
    (GOOD, GOOD, GOOD, GOOD, GOOD, 64, 196, 256, None),       # N not a multiple of 8
    (GOOD, GOOD, GOOD, GOOD, GOOD, -1, 256, 256, None),       # negative M
    (GOOD, GOOD, GOOD, GOOD, GOOD, 64, 256, 0, None),         # K < 128
    (None, GOOD, GOOD, GOOD, GOOD, 64, 256, 256, None),       # null A
    (GOOD, GOOD, GOOD, GOOD, None, 64, 256, 256, None),       # null D
    (BAD, GOOD, GOOD, GOOD, GOOD, 64, 256, 256, None),        # misaligned A
    (GOOD, GOOD, GOOD, GOOD, BAD, 64, 256, 256, None),        # misaligned D
    (GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 20, 256, 4096, None),  # M*K beyond 2^31
    (GOOD, GOOD, GOOD, GOOD, GOOD, 64, 4194304, 128, None),    # N beyond 4194296 (a 256-row tile of D past 2^31 bytes)
])
def test_dense_validation(args):
    assert fg.lib().fg_gemm_fp8_nt(*args) == EINVAL
    assert fg.lib().fg_gemm_fp8_nt_pow2(*args) == EINVAL


def test_empty_problems_are_no_ops():
    L = fg.lib()
    assert L.fg_gemm_fp8_nt(None, None, None, None, None, 0, 256, 256, None) == OK
    assert L.fg_gemm_fp8_nt(None, None, None, None, None, 64, 0, 256, None) == OK
    assert L.fg_grouped_contiguous(None, None, None, None, None, None, 0, 256, 256, 4, None) == OK
    assert L.fg_gemm_fp8_nt_pow2(None, None, None, None, None, 0, 256, 256, None) == OK
    assert L.fg_grouped_masked_pow2(None, None, None, None, None, None, 3, 0, 256, 256, None) == OK


def test_grouped_validation():
    L = fg.lib()
    # G < 1
    assert L.fg_grouped_contiguous(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 256, 256, 0, None) == EINVAL
    assert L.fg_grouped_masked(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 256, 256, None) == EINVAL
    # missing index arrays
    assert L.fg_grouped_contiguous(GOOD, GOOD, GOOD, GOOD, GOOD, None, 64, 256, 256, 2, None) == EINVAL
    assert L.fg_grouped_masked(GOOD, GOOD, GOOD, GOOD, GOOD, None, 2, 64, 256, 256, None) == EINVAL
    # misaligned masked_m
    assert L.fg_grouped_masked(GOOD, GOOD, GOOD, GOOD, GOOD, ctypes.c_void_p(0x100002), 2, 64, 256, 256,
                               None) == EINVAL
    # the power-of-two entry points validate the same way
    assert L.fg_grouped_contiguous_pow2(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 256, 256, 0, None) == EINVAL
    assert L.fg_grouped_contiguous_pow2(GOOD, GOOD, GOOD, GOOD, GOOD, None, 64, 256, 256, 2, None) == EINVAL
    assert L.fg_grouped_masked_pow2(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 256, 256, None) == EINVAL
    assert L.fg_grouped_masked_pow2(GOOD, GOOD, GOOD, GOOD, GOOD, None, 2, 64, 256, 256, None) == EINVAL


def test_quant_validation():
    L = fg.lib()
    assert L.fg_quant_act_1x128(GOOD, GOOD, GOOD, 1, 64, 100, None) == EINVAL
    assert L.fg_quant_act_1x128(BAD, GOOD, GOOD, 1, 64, 128, None) == EINVAL
    assert L.fg_quant_weight_128x128(GOOD, GOOD, GOOD, 1, 100, 100, None) == EINVAL    # K % 128
    assert L.fg_quant_weight_128x128(GOOD, GOOD, GOOD, -1, 128, 128, None) == EINVAL   # G < 0
    assert L.fg_quant_weight_128x128(BAD, GOOD, GOOD, 1, 72, 128, None) == EINVAL      # misaligned w
    assert L.fg_quant_weight_128x128(None, None, None, 2, 0, 128, None) == OK           # N = 0
    assert L.fg_quant_act_1x128(None, None, None, 1, 0, 128, None) == OK
    assert L.fg_quant_act_1x128_pow2(GOOD, GOOD, GOOD, 1, 64, 100, None) == EINVAL
    assert L.fg_quant_act_1x128_pow2(BAD, GOOD, GOOD, 1, 64, 128, None) == EINVAL
    assert L.fg_quant_weight_128x128_pow2(GOOD, GOOD, GOOD, 1, 128, 100, None) == EINVAL
    assert L.fg_quant_weight_128x128_pow2(None, None, None, 0, 128, 128, None) == OK


def test_fused_validation():
    L = fg.lib()
    # N not a multiple of 256, unknown scale kind, null or misaligned outputs
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 64, 384, 256, 0, None) == EINVAL
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, 64, 512, 256, 2, None) == EINVAL
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, None, GOOD, None, 64, 512, 256, 0, None) == EINVAL
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 64, 512, 256, 0, None) == EINVAL
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, BAD, GOOD, None, 64, 512, 256, 0, None) == EINVAL
    assert L.fg_gemm_fp8_nt_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, BAD, 64, 512, 256, 0, None) == EINVAL
    assert L.fg_grouped_contiguous_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, None, 64, 512, 256, 2,
                                                0, None) == EINVAL
    assert L.fg_grouped_masked_swiglu_quant(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 0, 64, 512, 256,
                                            0, None) == EINVAL
    # empty problems launch nothing
    assert L.fg_gemm_fp8_nt_swiglu_quant(None, None, None, None, None, None, None, 0, 512, 256, 0, None) == OK


def test_fused_select_config_uses_256_column_tiles():
    for layout, M, N, K, G in [(0, 256, 7168, 7168, 1), (0, 8192, 7168, 18432, 1), (1, 9472, 4096, 7168, 8),
                               (2, 256, 7168, 2048, 16), (0, 64, 512, 256, 1)]:
        bm, bn = fg.select_config(M, N, K, G, layout | fg.SELECT_SWIGLU_QUANT)
        assert bn == 256
        if layout == 1:
            assert 128 % bm == 0 or bm == 256


def test_select_config_argument_order():
    # int fg_select_config(M, N, K, G, layout, num_cus, *bm, *bn): the masked
    # decode problem (G = 16 experts of M_max = 256 rows) and the skinny dense
    # one give different tiles, so a swapped argument shows
    L = fg.lib()
    bm, bn = ctypes.c_int(), ctypes.c_int()
    assert L.fg_select_config(256, 7168, 7168, 1, 0, 256, ctypes.byref(bm), ctypes.byref(bn)) == OK
    assert (bm.value, bn.value) == (64, 112)
    assert L.fg_select_config(256, 7168, 2048, 16, 2, 0, ctypes.byref(bm), None) == OK
    assert bm.value == 256
    grid = ctypes.c_int()
    assert L.fg_select_grid(256, 7168, 7168, 1, 0, 256, ctypes.byref(grid)) == OK
    assert grid.value == 256
    assert L.fg_select_grid(256, 7168, 2048, 16, 2, 0, None) == OK
    # errors: unknown layout, negative size, G < 1 for a grouped layout
    assert L.fg_select_config(256, 7168, 7168, 1, 3, 0, None, None) == EINVAL
    assert L.fg_select_config(-1, 7168, 7168, 1, 0, 0, None, None) == EINVAL
    assert L.fg_select_config(256, 7168, 7168, 0, 1, 0, None, None) == EINVAL
    assert L.fg_select_grid(256, 7168, 7168, 0, 2, 0, ctypes.byref(grid)) == EINVAL
    # dense ignores G
    assert L.fg_select_config(256, 7168, 7168, 0, 0, 0, ctypes.byref(bm), None) == OK


def test_select_config_fills_the_machine():
    # every choice must be a compiled tile and give a sane grid
    for layout, M, N, K, G in [(0, 256, 7168, 7168, 1), (0, 8192, 7168, 18432, 1), (0, 128, 256, 512, 1),
                               (1, 9472, 4096, 7168, 8), (2, 256, 7168, 2048, 16)]:
        bm, bn = fg.select_config(M, N, K, G, layout)
        grid = fg.select_grid(M, N, K, G, layout)
        assert bm > 0 and bn > 0 and N % 16 == 0
        tiles = -(-M // bm) * -(-N // bn) * (G if layout == 2 else 1)
        if layout == 1 and bm == 256:
            # 256-row contiguous tiles follow the experts' runs of 128-row blocks;
            # the workgroups walk the tile list persistently, one per CU at most,
            # as many as the largest list needs (ceil((blocks + G) / 2) per column)
            blocks = -(-M // 128)
            most = min(blocks, (blocks + G + 1) // 2) * -(-N // bn)
            assert grid == min(most, 256)
        elif (layout, M, N) == (0, 8192, 7168):
            # 3.5 rounds of 256x256 tiles: the two-shape split (3 whole rounds
            # of 256x256 plus one round of 256x128), walked by one workgroup per CU
            assert (bm, bn) == (256, 256) and grid == 256
        else:
            assert grid == tiles
        if layout == 1:
            assert 128 % bm == 0 or bm == 256   # 128-row blocks, or the run-following 256-row tiles


def test_select_config_picks_the_measured_best_tiles():
    # The cost model's choices for the five workloads are the tiles that timed
    # fastest on an MI355X when every compiled tile was forced in turn: the
    # smallest tile that gives 256 workgroups for M=256, the largest tiles for
    # the big dense and masked problems (fewer re-reads of A and B; 256x224
    # splits N = 7168 into 32 whole column tiles), and for the contiguous
    # layout the runs kernel (256x256 run-following tiles, 128x256 tiles for
    # single blocks and the last round).
    assert fg.select_config(256, 7168, 7168, 1, 0) == (64, 112)
    assert fg.select_config(9472, 4096, 7168, 8, 1) == (256, 256)
    assert fg.select_config(256, 7168, 2048, 16, 2) in ((256, 224), (256, 256))
    assert fg.select_config(8192, 7168, 18432, 1, 0) in ((256, 128), (256, 256), (256, 224))


def test_dense_split_chosen_for_partial_rounds():
    """The large dense FFN shape (32 x 28 tiles of 256x256 = 3.5 rounds over
    256 CUs) runs on the two-shape kernel: 24 column tiles of 256x256 (3 whole
    rounds) and the remaining 1024 columns as one round of 256x128 tiles. The
    wide tile is the one reported; one workgroup per CU walks its tiles of
    both shapes (fewer if there are fewer tiles of either shape)."""
    assert fg.select_config(8192, 7168, 18432, 1, 0) == (256, 256)
    assert fg.select_grid(8192, 7168, 18432, 1, 0) == 256
    # a problem already in whole rounds keeps the single shape
    assert fg.select_grid(8192, 4096, 7168, 1, 0) == 512
    # not for the fused epilogue (256-column tiles only) or the grouped layouts
    assert fg.select_grid(8192, 7168, 18432, 1, fg.SELECT_SWIGLU_QUANT) == 32 * 28
    with pytest.raises(fg.FGError):
        with forced_split(100):
            pass


def test_select_config_rejects_bad_layout():
    with pytest.raises(fg.FGError):
        fg.select_config(128, 128, 128, 1, 7)


def test_product_library_has_no_tile_override():
    # the tile override is a test-build hook (libfg_testing.so), never part of
    # the product library's state
    L = ctypes.CDLL(fg.LIB_PATH)
    for name in ("fg_force_tile", "fgt_force_tile"):
        assert not hasattr(L, name), name


def test_testing_library_override_is_per_call_site():
    with forced(128, 128):
        assert fg.select_config(8192, 7168, 18432, 1, 0) == (128, 128)
    # restored on exit, and the product library never saw it
    assert fg.select_config(8192, 7168, 18432, 1, 0) != (128, 128)
    with pytest.raises(fg.FGError):
        with forced(96, 96):
            pass


def test_testing_override_is_per_thread():
    import threading
    seen = {}

    def other():
        seen["other"] = _testing_lib().fg_select_config(8192, 7168, 18432, 1, 0, 0, ctypes.byref(bm), None), bm.value

    bm = ctypes.c_int()
    with forced(128, 128):
        t = threading.Thread(target=other)
        t.start()
        t.join()
    assert seen["other"][0] == OK and seen["other"][1] != 128


def test_contiguous_256_row_tiles_only_within_the_tile_list():
    # The 256-row contiguous tiles follow a tile list each workgroup builds in
    # LDS (at most 2048 blocks of 128 rows, experts < 32768); beyond that the
    # choice falls back to tiles of at most 128 rows, and a forced 256-row tile
    # is refused.
    assert fg.select_config(2048 * 128, 4096, 7168, 8, 1)[0] == 256
    assert fg.select_config(2048 * 128 + 1, 4096, 7168, 8, 1)[0] <= 128
    assert fg.select_config(9472, 4096, 7168, 32768, 1)[0] <= 128
    with forced(256, 224):
        assert fg.select_config(9472, 4096, 7168, 8, 1) == (256, 224)
        with pytest.raises(fg.FGError):
            fg.select_config(2048 * 128 + 1, 4096, 7168, 8, 1)
        # dense and masked have no such limit
        assert fg.select_config(2048 * 128 + 1, 4096, 7168, 1, 0) == (256, 224)


def test_ceiling_helper_loads():
    """The benchmark helper bench.py loads to measure the matrix-core ceiling
    and the streaming-read rate (not part of the library) is built and exports
    its launchers, which reject bad arguments before any launch."""
    L = ctypes.CDLL(os.path.join(os.path.dirname(fg.LIB_PATH), "libfg_ceiling.so"), mode=os.RTLD_NOW)
    for name in ("fgc_src_words", "fgc_flop_per_workgroup_iteration", "fgc_mfma_loop", "fgc_stream_read"):
        assert hasattr(L, name), name
    L.fgc_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    assert L.fgc_stream_read(None, 1 << 20, None, 1, 4, None) == -1
    assert L.fgc_stream_read(ctypes.c_void_p(0x1008), 1 << 20, ctypes.c_void_p(0x2000), 1, 4, None) == -1  # misaligned
    assert L.fgc_stream_read(ctypes.c_void_p(0x1000), 100, ctypes.c_void_p(0x2000), 1, 4, None) == -1      # not whole 16 B
    assert L.fgc_stream_read(ctypes.c_void_p(0x1000), 1 << 20, ctypes.c_void_p(0x2000), 1, 5, None) == -1  # 4 or 8 in flight
    L.fgc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p]
    assert L.fgc_mfma_loop(None, None, 0, 1, 1, None) == -1        # rejected before any launch
    L.fgc_src_words.restype = ctypes.c_int
    assert L.fgc_src_words() > 0
