"""GPU parity for the power-of-two (E8M0) scale path: the _pow2 quantisers
bit-exact against the oracle's power-of-two quantisers, and the _pow2 GEMMs
(scales applied by the matrix core, no VALU promotion) against the oracle's
fp64 reference on the same seeded inputs, for every layout and tile, plus
exactness and invariance properties."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_split, forced_tile as forced
from fgtest import (SENTINEL, d_bits, dense_inputs, make_contiguous, make_dense, make_masked,
                    masked_inputs, new_out, quant_inputs, to_dev)

pytestmark = pytest.mark.gpu

TILES = [(256, 256), (256, 128), (128, 256), (128, 128), (64, 112), (256, 112), (256, 224)]


@pytest.fixture
def forced_tile(request):
    """Force a tile shape for the test (None: the automatic choice)."""
    if request.param is None:
        yield None
        return
    bm, bn = request.param
    with forced(bm, bn):
        yield bm, bn


# ---------------------------------------------------------------- quantisers

@pytest.mark.parametrize("shape", [(16, 256), (300, 1024), (3, 40, 384)])
def test_act_quant_pow2_bit_exact(shape):
    print(f"pow2 act quant {shape}", flush=True)
    x = quant_inputs(shape, 17)
    flat = x.reshape(-1, shape[-1])
    flat[9, :128] = np.float32(1e-39)            # amax/448 is subnormal: scale floored at 2^-126
    q, sa = fg.quant_act_1x128_pow2(to_dev(x))
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_act_1x128(flat, pow2=True)
    assert np.array_equal(q.cpu().numpy().reshape(flat.shape), codes)
    if len(shape) == 3:
        b, M, K = shape
        sa_nat = np.transpose(sa.cpu().numpy(), (0, 2, 1)).reshape(b * M, K // 128)
    else:
        sa_nat = sa.cpu().numpy().T
    assert np.array_equal(sa_nat, scales)


@pytest.mark.parametrize("shape", [(128, 128), (384, 640), (2, 256, 384)])
def test_weight_quant_pow2_bit_exact(shape):
    print(f"pow2 weight quant {shape}", flush=True)
    rng = np.random.default_rng(18)
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.05)
    flat = w.reshape(-1, shape[-1])
    flat[min(130, flat.shape[0] - 1), min(200, flat.shape[1] - 1)] = 3.0
    flat[:128, :128] *= np.float32(448.0 / np.abs(flat[:128, :128]).max())   # amax exactly 448: scale 1
    q, sb = fg.quant_weight_128x128_pow2(to_dev(w))
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_weight_128x128(w, pow2=True)
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(sb.cpu().numpy(), scales)


# ---------------------------------------------------------------- GEMMs

def run_dense(A, sa, B, sb, prefill=SENTINEL):
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], B.shape[0]), prefill)
    fg.gemm_fp8_nt_pow2(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    return d_bits(D)


@pytest.mark.parametrize("M,N,K,seed", [
    (128, 256, 512, 1),
    (16, 128, 128, 121),
    (200, 384, 640, 122),
    (333, 1024, 1152, 123),
])
def test_dense_pow2_parity(M, N, K, seed):
    print(f"pow2 dense M={M} N={N} K={K} seed={seed}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, seed, pow2=True)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    print(r)
    assert r["ok"], r


def test_dense_pow2_outlier_rows():
    print("pow2 dense outliers", flush=True)
    A, sa, B, sb = make_dense(256, 512, 1024, 2, pow2=True, outlier_frac=0.01, outlier_scale=50.0)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


def int_codes(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_dense_pow2_small_integers_bit_exact():
    """Scales 2^0 and integer values: every partial and the FP32 accumulator stay
    exact, so the output is the correctly rounded bf16 of the integer product."""
    print("pow2 dense integers", flush=True)
    rng = np.random.default_rng(131)
    M, N, K = 96, 384, 1024
    ai, bi = rng.integers(-3, 4, (M, K)), rng.integers(-3, 4, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    out = run_dense(int_codes(ai), sa, int_codes(bi), sb)
    exact = (ai @ bi.T).astype(np.float64)
    expect = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, expect)


def test_dense_pow2_kblock_scales_bit_exact():
    """Integer values with a different power-of-two scale per K-block, row and
    weight block: the exact result is an integer combination of powers of two
    that FP32 holds exactly, so the output is its correctly rounded bf16."""
    print("pow2 dense per-K-block exponents", flush=True)
    rng = np.random.default_rng(132)
    M, N, K = 64, 256, 768
    KB = K // 128
    ai, bi = rng.integers(-2, 3, (M, K)), rng.integers(-2, 3, (N, K))
    ea = rng.integers(-2, 3, (M, KB))
    eb = rng.integers(-2, 3, (N // 128, KB))
    sa = (2.0 ** ea).astype(np.float32)
    sb = (2.0 ** eb).astype(np.float32)
    out = run_dense(int_codes(ai), sa, int_codes(bi), sb)
    exact = np.zeros((M, N))
    for kb in range(KB):
        ks = slice(kb * 128, (kb + 1) * 128)
        part = (ai[:, ks] @ bi[:, ks].T).astype(np.float64)
        exact += part * (2.0 ** ea[:, kb])[:, None] * np.repeat(2.0 ** eb[:, kb], 128)[None, :]
    expect = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, expect)


def test_dense_pow2_scale_invariance_bitwise():
    print("pow2 dense invariance", flush=True)
    rng = np.random.default_rng(133)
    A, sa, B, sb = make_dense(128, 256, 512, 134, pow2=True)
    base = run_dense(A, sa, B, sb)
    p = rng.integers(-4, 5, A.shape[0])
    q = rng.integers(-4, 5, B.shape[0] // 128)
    out = run_dense(A, (sa * (2.0 ** p)[:, None]).astype(np.float32),
                    B, (sb * (2.0 ** q)[:, None]).astype(np.float32))
    factor = (2.0 ** p)[:, None] * np.repeat(2.0 ** q, 128)[None, :]
    scaled = torch.from_numpy(oracle.bf16_bits_to_f64(base) * factor).to(torch.bfloat16)
    assert np.array_equal(out, scaled.view(torch.int16).numpy().view(np.uint16))


def test_dense_pow2_agrees_with_the_promotion_path():
    """Both paths on the same power-of-two-scaled operands meet the oracle bar,
    and differ from each other only by FP32 summation order."""
    print("pow2 vs promotion path", flush=True)
    A, sa, B, sb = make_dense(256, 1024, 2048, 135, pow2=True)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D1, D2 = new_out((256, 1024)), new_out((256, 1024))
    fg.gemm_fp8_nt_pow2(Ad, sad, Bd, sbd, D1)
    fg.gemm_fp8_nt(Ad, sad, Bd, sbd, D2)
    torch.cuda.synchronize()
    ref = oracle.ref_dense(A, sa, B, sb)
    for out in (d_bits(D1), d_bits(D2)):
        r = oracle.check(out, ref)
        assert r["ok"], r
    x1, x2 = oracle.bf16_bits_to_f64(d_bits(D1)), oracle.bf16_bits_to_f64(d_bits(D2))
    assert np.max(np.abs(x1 - x2)) <= 2.0 ** -7 * np.max(np.abs(ref))


def test_dense_pow2_deterministic():
    A, sa, B, sb = make_dense(300, 512, 768, 136, pow2=True)
    assert np.array_equal(run_dense(A, sa, B, sb), run_dense(A, sa, B, sb))


@pytest.mark.parametrize("M,N,n_split,K", [(300, 776, 512, 1152), (513, 264, 256, 128)])
def test_dense_split_kernel_pow2(M, N, n_split, K):
    """The dense two-shape kernel with power-of-two scales on the matrix core."""
    print(f"pow2 dense split M={M} N={N} n_split={n_split} K={K}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, 64 + M, pow2=True)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((M, N))
    with forced_split(n_split):
        fg.gemm_fp8_nt_pow2(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    r = oracle.check(d_bits(D), oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", TILES, indirect=True, ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("K", [128, 640, 1152])
def test_every_tile_dense_pow2(forced_tile, K):
    print(f"pow2 tile {forced_tile} dense K={K}", flush=True)
    A, sa, B, sb = make_dense(300, 512, K, 160 + K, pow2=True)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile,kblocks",
                         [((64, 112), kb) for kb in (2, 5, 11, 12, 13)] + [((256, 256), kb) for kb in (3, 6, 7)],
                         indirect=["forced_tile"], ids=lambda v: f"{v[0]}x{v[1]}" if isinstance(v, tuple) else f"kb{v}")
def test_loop_exit_phases_pow2(forced_tile, kblocks):
    K = 128 * kblocks
    print(f"pow2 tile {forced_tile} dense K={K}", flush=True)
    A, sa, B, sb = make_dense(80, 384, K, 190 + kblocks, pow2=True)
    out = run_dense(A, sa, B, sb)
    r = oracle.check(out, oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", [None] + TILES, indirect=True,
                         ids=lambda t: "auto" if t is None else f"{t[0]}x{t[1]}")
def test_contiguous_pow2(forced_tile):
    print(f"pow2 contiguous tile {forced_tile}", flush=True)
    A, sa, B, sb, mi = make_contiguous(3, 384, 640, 162, pow2=True, m_lo=1, m_hi=300)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D = new_out((A.shape[0], 384))
    fg.grouped_contiguous_pow2(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


@pytest.mark.parametrize("forced_tile", [None] + TILES, indirect=True,
                         ids=lambda t: "auto" if t is None else f"{t[0]}x{t[1]}")
def test_masked_pow2(forced_tile):
    print(f"pow2 masked tile {forced_tile}", flush=True)
    G, M_max, N, K = 3, 200, 384, 768
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 161, pow2=True)
    mm = np.array([77, 0, 200], np.int32)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    D = new_out((G, M_max, N))
    fg.grouped_masked_pow2(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r
