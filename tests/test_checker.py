"""The acceptance check must pass a correctly rounded bf16 result and must fail
the plausible mistakes (truncation, double rounding through fp16-ish
precision, touched rows, NaN)."""
import numpy as np
import torch

from oracle import bf16_rne, bf16_bits_to_f64, check


def f64_to_bf16_bits_rne(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-5, 5, 200000)).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_rne(x.astype(np.float64)), lib)


def test_bits_roundtrip():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x7F7F], np.uint16)
    assert bf16_bits_to_f64(bits).tolist()[:4] == [1.0, -1.0, 2.0, 0.0]


def _product(seed=0, n=512):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, n))
    y = rng.standard_normal((n, n))
    return x @ y.T


def test_rne_passes_truncation_fails():
    ref = _product()
    rne_bits = f64_to_bf16_bits_rne(ref)
    r = check(rne_bits, ref)
    assert r["ok"], r
    assert 1.5e-3 < r["frob"] < 1.8e-3
    trunc_bits = (ref.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = check(trunc_bits, ref)
    assert not r["ok"] and not r["frob_ok"], r


def test_fp16_style_intermediate_fails():
    """A result that went through a 10-bit-mantissa intermediate and then bf16
    double-rounds; a result that lost one more bit (7-bit significand) fails."""
    ref = _product(1)
    mant, e = np.frexp(ref)
    coarse = np.ldexp(np.rint(np.ldexp(mant, 7)), e - 7)      # 7 significant bits
    r = check(f64_to_bf16_bits_rne(coarse), ref)
    assert not r["ok"]


def test_touched_rows_fail_and_untouched_pass():
    ref = _product(2, 256)
    valid = np.ones(256, bool)
    valid[100:110] = False
    ref[~valid] = 0.0
    bits = f64_to_bf16_bits_rne(ref)
    bits[~valid] = 0xDEAD
    assert check(bits, ref, valid, prefill_bits=0xDEAD)["ok"]
    bits[105, 3] = 0
    r = check(bits, ref, valid, prefill_bits=0xDEAD)
    assert not r["ok"] and r["n_touched"] == 1


def test_nan_fails():
    ref = _product(3, 128)
    bits = f64_to_bf16_bits_rne(ref)
    bits[5, 5] = 0x7FC0
    assert not check(bits, ref)["ok"]


def test_single_wrong_element_fails():
    ref = _product(4, 128)
    bits = f64_to_bf16_bits_rne(ref)
    bits[7, 9] ^= 0x0010       # a few ulps off in one element
    r = check(bits, ref)
    assert not r["elem_ok"]
