"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs, element by element, at sizes spanning several tiles and ragged
tails, plus exactness and invariance properties."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_split, forced_tile as forced
from fgtest import (SENTINEL, d_bits, dense_inputs, dev, make_contiguous, make_dense,
                    make_masked, masked_inputs, new_out, to_dev)

pytestmark = pytest.mark.gpu


def run_dense(A, sa, B, sb, prefill=SENTINEL):
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], B.shape[0]), prefill)
    fg.gemm_fp8_nt(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    return d_bits(D)


@pytest.mark.parametrize("M,N,K,seed", [
    (128, 256, 512, 1),      # the small dense workload
    (16, 128, 128, 21),      # a single K-block, partial M tile
    (200, 384, 640, 22),     # ragged M, three N-blocks
    (333, 1024, 1152, 23),   # several tiles each way
])
def test_dense_parity(M, N, K, seed):
    print(f"dense M={M} N={N} K={K} seed={seed}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, seed)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    print(r)
    assert r["ok"], r


def test_dense_outlier_rows():
    A, sa, B, sb = make_dense(256, 512, 1024, 2, outlier_frac=0.01, outlier_scale=50.0)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


def int_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_dense_small_integers_bit_exact():
    """Unit scales, integer values: FP32 partial and master sums are exact, so the
    output must be the correctly rounded bf16 of the integer product."""
    rng = np.random.default_rng(31)
    M, N, K = 96, 384, 1024
    ai, bi = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    out = run_dense(int_codes(ai), sa, int_codes(bi), sb)
    exact = (ai @ bi.T).astype(np.float64)
    expect = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, expect)


def test_dense_pow2_scale_invariance_bitwise():
    rng = np.random.default_rng(32)
    A, sa, B, sb = make_dense(128, 256, 512, 33)
    base = run_dense(A, sa, B, sb)
    p = rng.integers(-4, 5, A.shape[0])
    q = rng.integers(-4, 5, B.shape[0] // 128)
    out = run_dense(A, (sa * (2.0 ** p)[:, None]).astype(np.float32),
                    B, (sb * (2.0 ** q)[:, None]).astype(np.float32))
    factor = (2.0 ** p)[:, None] * np.repeat(2.0 ** q, 128)[None, :]
    scaled = torch.from_numpy(oracle.bf16_bits_to_f64(base) * factor).to(torch.bfloat16)
    assert np.array_equal(out, scaled.view(torch.int16).numpy().view(np.uint16))


def test_dense_zero_scale_rows_are_zero():
    A, sa, B, sb = make_dense(64, 256, 256, 34)
    sa = sa.copy()
    sa[5] = 0.0
    out = run_dense(A, sa, B, sb)
    assert np.all(oracle.bf16_bits_to_f64(out[5]) == 0)


def test_dense_deterministic():
    A, sa, B, sb = make_dense(300, 512, 768, 35)
    assert np.array_equal(run_dense(A, sa, B, sb), run_dense(A, sa, B, sb))


@pytest.mark.parametrize("G,N,K,seed,m_lo,m_hi", [
    (3, 256, 512, 41, 1, 300),
    (8, 384, 384, 42, 100, 260),
])
def test_contiguous_parity(G, N, K, seed, m_lo, m_hi):
    print(f"contiguous G={G} N={N} K={K} seed={seed}", flush=True)
    A, sa, B, sb, mi = make_contiguous(G, N, K, seed, m_lo=m_lo, m_hi=m_hi)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], N))
    fg.grouped_contiguous(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    print(r)
    assert r["ok"], r


@pytest.mark.parametrize("G,M_max,N,K,seed,masked", [
    (4, 200, 256, 384, 51, [0, 37, 200, 129]),
    (6, 256, 384, 256, 52, None),
    (3, 64, 128, 128, 53, [64, 0, 300]),      # count above M_max is clamped
])
def test_masked_parity(G, M_max, N, K, seed, masked):
    print(f"masked G={G} M_max={M_max} N={N} K={K} seed={seed}", flush=True)
    A, sa, B, sb, mm = make_masked(G, M_max, N, K, seed)
    if masked is not None:
        mm = np.array(masked, np.int32)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    fg.grouped_masked(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    print(r)
    assert r["ok"], r


def test_masked_nan_rows_beyond_count_do_not_leak():
    G, M_max, N, K = 2, 128, 256, 256
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 54)
    mm = np.array([50, 77], np.int32)
    A = A.copy()
    sa = sa.copy()
    for g in range(G):
        A[g, mm[g]:] = 0x7F          # NaN codes
        sa[g, mm[g]:] = np.nan
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    fg.grouped_masked(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


TILES = [(256, 256), (256, 128), (128, 256), (128, 128), (64, 112), (256, 112), (256, 224)]


@pytest.fixture
def forced_tile(request):
    bm, bn = request.param
    with forced(bm, bn):
        yield bm, bn


@pytest.mark.parametrize("forced_tile", TILES, indirect=True, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("K", [640, 1152])
def test_every_tile_dense(forced_tile, K):
    """Ragged M and N (N=512 is not a multiple of 112 or 256), K shorter and
    longer than the deepest LDS ring."""
    print(f"tile {forced_tile} dense K={K}", flush=True)
    A, sa, B, sb = make_dense(300, 512, K, 60 + K)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("M,N,n_split,K", [(300, 520, 256, 640), (300, 776, 512, 1152), (256, 384, 256, 128),
                                           (64, 1000, 768, 256), (513, 264, 256, 384)])
def test_dense_split_kernel(M, N, n_split, K):
    """The dense two-shape kernel: columns [0, n_split) on 256x256 tiles, the
    rest (ragged N, N % 128 != 0 included) on 256x128 tiles, ragged M, K from
    one K-block to more than the deepest ring."""
    print(f"dense split M={M} N={N} n_split={n_split} K={K}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, 63 + M + N)
    with forced_split(n_split):
        out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", TILES, indirect=True, ids=lambda t: f"{t[0]}x{t[1]}")
def test_every_tile_masked(forced_tile):
    print(f"tile {forced_tile} masked", flush=True)
    G, M_max, N, K = 3, 200, 384, 768
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 61)
    mm = np.array([77, 0, 200], np.int32)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    fg.grouped_masked(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", TILES, indirect=True,
                         ids=lambda t: f"{t[0]}x{t[1]}")
def test_every_tile_contiguous(forced_tile):
    print(f"tile {forced_tile} contiguous", flush=True)
    A, sa, B, sb, mi = make_contiguous(3, 384, 640, 62, m_lo=1, m_hi=300)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], 384))
    fg.grouped_contiguous(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", TILES, indirect=True, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("K", [128, 256])
def test_every_tile_fewer_kblocks_than_stages(forced_tile, K):
    """One and two K-blocks: every LDS ring is deeper than the problem, so all
    later loads are the clamped repeats of the last K-block."""
    print(f"tile {forced_tile} dense K={K}", flush=True)
    A, sa, B, sb = make_dense(100, 256, K, 70 + K)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile,kblocks",
                         [((64, 112), kb) for kb in range(1, 14)] + [((256, 256), kb) for kb in range(1, 8)]
                         + [((256, 224), kb) for kb in range(1, 8)],
                         indirect=["forced_tile"], ids=lambda v: f"{v[0]}x{v[1]}" if isinstance(v, tuple) else f"kb{v}")
def test_every_loop_exit_phase(forced_tile, kblocks):
    """The K loop is unrolled over 12 (64x112) or 6 (256x256, 256x224) K-blocks and
    finishes the last partials in a branch per exit phase; these K lengths
    end the loop in every phase."""
    K = 128 * kblocks
    print(f"tile {forced_tile} dense K={K}", flush=True)
    A, sa, B, sb = make_dense(80, 384, K, 90 + kblocks)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


# ---------------------------------------------------------------- N not a multiple of 128

@pytest.mark.parametrize("forced_tile", TILES, indirect=True, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("N", [8, 72, 200, 328])
@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
def test_every_tile_ragged_n(forced_tile, N, pow2):
    """N a multiple of 8 only: the last weight-scale block covers N mod 128
    rows, the last column tile is partial, columns >= N are never stored."""
    print(f"tile {forced_tile} dense ragged N={N} pow2={pow2}", flush=True)
    A, sa, B, sb = make_dense(150, N, 384, 500 + N, pow2=pow2)
    assert sb.shape[0] == -(-N // 128)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((150, N))
    (fg.gemm_fp8_nt_pow2 if pow2 else fg.gemm_fp8_nt)(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    r = oracle.check(d_bits(D), oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
def test_grouped_ragged_n(pow2):
    print(f"grouped ragged N pow2={pow2}", flush=True)
    A, sa, B, sb, mi = make_contiguous(3, 200, 384, 512, pow2=pow2, m_lo=1, m_hi=300)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], 200))
    (fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous)(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r
    A, sa, B, sb, _ = make_masked(3, 150, 328, 256, 513, pow2=pow2)
    mm = np.array([150, 0, 61], np.int32)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((3, 150, 328))
    (fg.grouped_masked_pow2 if pow2 else fg.grouped_masked)(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
def test_masked_many_experts(pow2):
    """96 experts (many more groups than tiles per group), small M_max, ragged
    N, empty and full experts."""
    G, M_max, N, K = 96, 40, 264, 384
    print(f"masked many experts G={G} pow2={pow2}", flush=True)
    A, sa, B, sb, mm = make_masked(G, M_max, N, K, 90, pow2=pow2)
    mm = mm.copy()
    mm[:3] = [0, M_max, 1]
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    (fg.grouped_masked_pow2 if pow2 else fg.grouped_masked)(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
def test_contiguous_many_experts(pow2):
    """48 experts of 1..200 rows each (one or two 128-row blocks apiece: many
    short and odd runs) on the automatic choice."""
    G, N, K = 48, 256, 256
    print(f"contiguous many experts G={G} pow2={pow2}", flush=True)
    A, sa, B, sb, mi = make_contiguous(G, N, K, 91, pow2=pow2, m_lo=1, m_hi=200)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], N))
    (fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous)(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r
