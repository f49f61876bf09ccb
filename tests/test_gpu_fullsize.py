"""Full-size parity: every workload at its real size, in the launch
configuration the benchmark times (automatic tile choice), with fp32 block
scales and with power-of-two scales on the _pow2 entry points. The oracle checks
sampled outputs one dot product at a time (spread over the output plus the
tile edges); rows that must not be written are compared bitwise in full, and
the whole output must be finite."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import moe_grouped_gemm_02_amd as fg
from fgtest import SENTINEL, d_bits, dense_inputs, fullsize_contiguous, masked_inputs, new_out, to_dev

pytestmark = pytest.mark.gpu

N_SAMPLES = 768


def sample_positions(rng, rows, N, valid_rows=None):
    """Random (row, col) pairs plus the first/last row and column and points on
    128-aligned boundaries, restricted to valid rows when given."""
    cand = np.arange(rows) if valid_rows is None else np.nonzero(valid_rows)[0]
    r = rng.choice(cand, size=N_SAMPLES)
    c = rng.integers(0, N, size=N_SAMPLES)
    edges_r = np.array([cand[0], cand[-1]] + [x for x in cand if x % 128 in (0, 127)][:64])
    edges_c = np.array([0, N - 1, 111, 112, 127, 128, N // 2, N - 112])
    rr = np.concatenate([r, np.repeat(edges_r, len(edges_c))])
    cc = np.concatenate([c, np.tile(edges_c, len(edges_r))])
    return rr, cc


def assert_all_finite(bits):
    exp = (bits >> 7) & 0xFF
    assert not np.any(exp == 0xFF), "NaN/Inf in output"


POW2 = pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])


def run_dense_full(name, pow2):
    w = workloads.make(name)
    A, sa = oracle.quantize_act_1x128(w["a"], pow2)
    B, sb = oracle.quantize_weight_128x128(w["b"], pow2)
    del w
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    M, N = A.shape[0], B.shape[0]
    D = new_out((M, N))
    (fg.gemm_fp8_nt_pow2 if pow2 else fg.gemm_fp8_nt)(Ad, sad, Bd, sbd, D)
    torch.cuda.synchronize()
    bits = d_bits(D)
    assert_all_finite(bits)
    rng = np.random.default_rng(100)
    rows, cols = sample_positions(rng, M, N)
    ref = oracle.ref_entries(A, sa, B, sb, rows, cols)
    r = oracle.check(bits[rows, cols][None, :], ref[None, :])
    print(name, r)
    assert r["ok"], r


@POW2
def test_fullsize_dense_skinny(pow2):
    print(f"full dense_skinny 256x7168x7168 pow2={pow2}", flush=True)
    run_dense_full("dense_skinny", pow2)


@POW2
def test_fullsize_dense_ffn(pow2):
    print(f"full dense_ffn 8192x7168x18432 pow2={pow2}", flush=True)
    run_dense_full("dense_ffn", pow2)


@POW2
def test_fullsize_contiguous(pow2):
    print(f"full contiguous 8 experts, N=4096, K=7168 pow2={pow2}", flush=True)
    A, sa, B, sb, mi = fullsize_contiguous(pow2)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    M, N = A.shape[0], B.shape[1]
    D = new_out((M, N))
    (fg.grouped_contiguous_pow2 if pow2 else fg.grouped_contiguous)(Ad, sad, Bd, sbd, D, to_dev(mi))
    torch.cuda.synchronize()
    bits = d_bits(D)
    valid = mi >= 0
    assert np.all(bits[~valid] == SENTINEL), "padding rows were written"
    assert_all_finite(bits[valid])
    rng = np.random.default_rng(101)
    rows, cols = sample_positions(rng, M, N, valid)
    ref = np.empty(rows.size)
    for g in range(B.shape[0]):
        sel = mi[rows] == g
        if sel.any():
            ref[sel] = oracle.ref_entries(A, sa, B[g], sb[g], rows[sel], cols[sel])
    r = oracle.check(bits[rows, cols][None, :], ref[None, :])
    print(r)
    assert r["ok"], r


@POW2
def test_fullsize_masked(pow2):
    print(f"full masked 16 experts, M_max=256, N=7168, K=2048 pow2={pow2}", flush=True)
    w = workloads.make("masked")
    G, M_max, K = w["a"].shape
    A = np.empty((G, M_max, K), np.uint8)
    sa = np.empty((G, M_max, K // 128), np.float32)
    for g in range(G):
        A[g], sa[g] = oracle.quantize_act_1x128(w["a"][g], pow2)
    B, sb = oracle.quantize_weight_128x128(w["b"], pow2)
    mm = w["masked_m"]
    del w
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    N = B.shape[1]
    D = new_out((G, M_max, N))
    (fg.grouped_masked_pow2 if pow2 else fg.grouped_masked)(Ad, sad, Bd, sbd, D, to_dev(mm))
    torch.cuda.synchronize()
    bits = d_bits(D)
    valid = np.arange(M_max)[None, :] < np.clip(mm, 0, M_max)[:, None]
    assert np.all(bits[~valid] == SENTINEL), "rows beyond masked_m were written"
    assert_all_finite(bits[valid])
    rng = np.random.default_rng(102)
    flat_valid = valid.reshape(-1)
    rows, cols = sample_positions(rng, G * M_max, N, flat_valid)
    ref = np.empty(rows.size)
    for g in range(G):
        sel = rows // M_max == g
        if sel.any():
            ref[sel] = oracle.ref_entries(A[g], sa[g], B[g], sb[g], rows[sel] % M_max, cols[sel])
    r = oracle.check(bits.reshape(G * M_max, N)[rows, cols][None, :], ref[None, :])
    print(r)
    assert r["ok"], r
