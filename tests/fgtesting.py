"""Test-only tile override.

The product library (libfg.so) picks every call's tile itself and holds no
state that one caller could change for another. The test suite needs to run
each compiled tile on problems the cost model would give another one, so the
build also links libfg_testing.so: the same kernel objects, with host code
built with FG_TESTING, which adds

    int fgt_force_tile(int bm, int bn);   /* per calling thread; 0, 0 = automatic */
    int fgt_force_split(int n_split);     /* dense on the two-shape kernel; -1 = automatic */
    int fgt_force_runs(int on);           /* contiguous on the runs kernel; 0 = automatic */
    int fgt_force_grid(int grid);         /* cap on the tile-walking kernels' workgroups; 0 = automatic */

``forced_tile(bm, bn)`` routes the package's calls through that library for the
duration of a ``with`` block (on this thread's override) and restores the
product library afterwards.
"""
import contextlib
import ctypes
import os

import moe_grouped_gemm_02_amd as fg

TESTING_LIB_PATH = os.path.join(os.path.dirname(fg.LIB_PATH), "libfg_testing.so")
_tlib = None


def testing_lib():
    global _tlib
    if _tlib is None:
        L = fg.load(TESTING_LIB_PATH)
        L.fgt_force_tile.argtypes = [ctypes.c_int, ctypes.c_int]
        L.fgt_force_tile.restype = ctypes.c_int
        L.fgt_force_split.argtypes = [ctypes.c_int]
        L.fgt_force_split.restype = ctypes.c_int
        L.fgt_force_runs.argtypes = [ctypes.c_int]
        L.fgt_force_runs.restype = ctypes.c_int
        L.fgt_force_grid.argtypes = [ctypes.c_int]
        L.fgt_force_grid.restype = ctypes.c_int
        _tlib = L
    return _tlib


@contextlib.contextmanager
def forced_tile(bm, bn):
    """Run the package's calls inside the block on tile bm x bn (None: the
    automatic choice, still through the testing library)."""
    L = testing_lib()
    saved = fg.lib()
    if bm is not None:
        rc = L.fgt_force_tile(bm, bn)
        if rc != 0:
            raise fg.FGError(f"fgt_force_tile({bm}, {bn}): {fg.strerror(rc)}")
    fg._lib = L
    try:
        yield
    finally:
        fg._lib = saved
        L.fgt_force_tile(0, 0)


@contextlib.contextmanager
def forced_split(n_split):
    """Run the package's dense calls inside the block on the two-shape kernel:
    columns [0, n_split) on 256x256 tiles, the rest on 256x128 tiles."""
    L = testing_lib()
    saved = fg.lib()
    rc = L.fgt_force_split(n_split)
    if rc != 0:
        raise fg.FGError(f"fgt_force_split({n_split}): {fg.strerror(rc)}")
    fg._lib = L
    try:
        yield
    finally:
        fg._lib = saved
        L.fgt_force_split(-1)


@contextlib.contextmanager
def forced_runs():
    """Run the package's contiguous calls inside the block on the runs kernel
    (256x256 run-following tiles, 128x256 single-block and tail tiles)."""
    L = testing_lib()
    saved = fg.lib()
    L.fgt_force_runs(1)
    fg._lib = L
    try:
        yield
    finally:
        fg._lib = saved
        L.fgt_force_runs(0)


@contextlib.contextmanager
def forced_grid(grid):
    """Inside the block (and inside a forced_* block of this module), launch at
    most `grid` workgroups on the kernels whose workgroups walk their tiles."""
    L = testing_lib()
    rc = L.fgt_force_grid(grid)
    if rc != 0:
        raise fg.FGError(f"fgt_force_grid({grid}): {fg.strerror(rc)}")
    try:
        yield
    finally:
        L.fgt_force_grid(0)
