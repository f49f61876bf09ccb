"""GPU parity for the fused first-projection epilogue (GEMM -> SiLU gate ->
1x128 E4M3 re-quantisation) through the C ABI, for every layout, both scale
kinds and every 256-column tile.

Each case checks
  * the fp32 activation the kernel also writes against the oracle's fp64
    silu(gate) * up of the fp64 GEMM reference, to the GEMM's own bar (per
    element |act - ref| <= 1e-2 |ref| + 1e-3 rms(ref), relative Frobenius
    <= 2e-3). Measured: ~2e-5 Frobenius and <= 4e-4 rms per element for both
    scale kinds and any K -- the error of one E4M3 matrix-core dot product of
    128 terms, which does not grow with K because every K-block is promoted
    into an FP32 accumulator (small-integer inputs, whose sums are exact, give
    1e-9);
  * the codes and scales bit for bit against the oracle's quantiser applied to
    that same fp32 activation (the quantisation decision is taken in the
    kernel's precision on both sides);
  * that rows without output keep their prefill in all three outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_runs, forced_tile as forced
from fgtest import (fullsize_contiguous, fullsize_contiguous_ref, fullsize_quantized, make_contiguous, make_dense,
                    make_masked, record_parity, to_dev)

pytestmark = pytest.mark.gpu

Q_FILL = 0x5A                          # code byte no call writes by chance into an untouched row
F_FILL = np.float32(-12345.5)          # sentinel for untouched sq / act entries
SCALES = pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])


@pytest.fixture
def forced_tile(request):
    if request.param is None:
        yield None
        return
    if request.param == "runs":
        with forced_runs():
            yield "runs"
        return
    bm, bn = request.param
    with forced(bm, bn):
        yield bm, bn


def prefilled(lead, M, I):
    dev = torch.device("cuda", 0)
    Q = torch.full(lead + (M, I), Q_FILL, dtype=torch.uint8, device=dev)
    sq = torch.full(lead + (I // 128, M), float(F_FILL), dtype=torch.float32, device=dev)
    act = torch.full(lead + (M, I), float(F_FILL), dtype=torch.float32, device=dev)
    return Q, sq, act


def check_f32(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(x - ref)
    worst = float(np.max(err / (1e-2 * np.abs(ref) + 1e-3 * rms)))
    frob = float(np.sqrt(np.sum(err * err)) / np.sqrt(np.sum(ref * ref)))
    return {"ok": bool(np.all(np.isfinite(x)) and worst <= 1.0 and frob <= 2e-3), "worst": worst, "frob": frob}


def check_rows(Q, sq_nat, act, ref_act, valid, pow2):
    """Q [M, I] codes, sq_nat [M, I/128], act [M, I] fp32 from the GPU; ref_act
    fp64 [M, I]; valid [M] bool."""
    assert np.all(Q[~valid] == Q_FILL), "Q written in a row without output"
    assert np.all(sq_nat[~valid] == F_FILL), "sq written in a row without output"
    assert np.all(act[~valid] == F_FILL), "act written in a row without output"
    if not valid.any():
        return
    r = check_f32(act[valid], ref_act[valid])
    print("act vs oracle", r)
    assert r["ok"], r
    codes, scales = oracle.quantize_act_1x128(act[valid], pow2)
    assert np.array_equal(scales, sq_nat[valid]), "scales differ from the oracle quantiser"
    assert np.array_equal(codes, Q[valid]), "codes differ from the oracle quantiser"


@pytest.mark.parametrize("forced_tile", [None, (256, 256), (128, 256)], indirect=True,
                         ids=lambda t: "auto" if t is None else f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("M,N,K,seed", [(200, 512, 640, 301), (64, 256, 128, 302), (333, 1024, 1152, 303)])
@SCALES
def test_dense_swiglu_quant(forced_tile, M, N, K, seed, pow2):
    print(f"swiglu dense tile={forced_tile} M={M} N={N} K={K} pow2={pow2}", flush=True)
    A, sa, B, sb = make_dense(M, N, K, seed, pow2=pow2)
    I = N // 2
    Q, sq, act = prefilled((), M, I)
    fg.gemm_fp8_nt_swiglu_quant(to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb),
                                Q, sq, act, pow2=pow2)
    torch.cuda.synchronize()
    ref_act = oracle.swiglu_blocks(oracle.ref_dense(A, sa, B, sb))
    check_rows(Q.cpu().numpy(), sq.cpu().numpy().T, act.cpu().numpy(), ref_act, np.ones(M, bool), pow2)


@pytest.mark.parametrize("forced_tile", [None, (128, 256), (256, 256), "runs"], indirect=True,
                         ids=lambda t: "auto" if t is None else t if isinstance(t, str) else f"{t[0]}x{t[1]}")
@SCALES
def test_contiguous_swiglu_quant(forced_tile, pow2):
    print(f"swiglu contiguous tile={forced_tile} pow2={pow2}", flush=True)
    A, sa, B, sb, mi = make_contiguous(3, 512, 640, 311, pow2=pow2, m_lo=1, m_hi=300)
    M, I = A.shape[0], 256
    Q, sq, act = prefilled((), M, I)
    fg.grouped_contiguous_swiglu_quant(to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb),
                                       to_dev(mi), Q, sq, act, pow2=pow2)
    torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
    ref_act = np.zeros((M, I))
    ref_act[valid] = oracle.swiglu_blocks(ref[valid])
    check_rows(Q.cpu().numpy(), sq.cpu().numpy().T, act.cpu().numpy(), ref_act, valid, pow2)


@pytest.mark.parametrize("forced_tile", [None, (256, 256), (128, 256)], indirect=True,
                         ids=lambda t: "auto" if t is None else f"{t[0]}x{t[1]}")
@SCALES
def test_masked_swiglu_quant(forced_tile, pow2):
    print(f"swiglu masked tile={forced_tile} pow2={pow2}", flush=True)
    G, M_max, N, K = 3, 200, 768, 384
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 321, pow2=pow2)
    mm = np.array([77, 0, 200], np.int32)
    I = N // 2
    Q, sq, act = prefilled((G,), M_max, I)
    fg.grouped_masked_swiglu_quant(to_dev(A), to_dev(np.ascontiguousarray(np.transpose(sa, (0, 2, 1)))),
                                   to_dev(B), to_dev(sb), to_dev(mm), Q, sq, act, pow2=pow2)
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    Qh, sqh, acth = Q.cpu().numpy(), sq.cpu().numpy(), act.cpu().numpy()
    for g in range(G):
        ref_act = oracle.swiglu_blocks(ref[g])
        check_rows(Qh[g], sqh[g].T, acth[g], ref_act, valid[g], pow2)


def test_without_the_activation_output():
    """act = NULL: codes and scales are the same as with it."""
    A, sa, B, sb = make_dense(128, 512, 512, 331)
    args = (to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb))
    Q1, sq1, act1 = fg.gemm_fp8_nt_swiglu_quant(*args, with_act=True)
    Q2, sq2, act2 = fg.gemm_fp8_nt_swiglu_quant(*args)
    torch.cuda.synchronize()
    assert act2 is None
    assert torch.equal(Q1, Q2) and torch.equal(sq1, sq2)


def test_fused_rejects_narrow_tiles_and_bad_n():
    A, sa, B, sb = make_dense(64, 256, 128, 332)
    args = (to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb))
    with forced(256, 128):
        with pytest.raises(fg.FGError):
            fg.gemm_fp8_nt_swiglu_quant(*args)
    A2, sa2, B2, sb2 = make_dense(64, 384, 128, 333)
    with pytest.raises(ValueError):
        fg.gemm_fp8_nt_swiglu_quant(to_dev(A2), to_dev(np.ascontiguousarray(sa2.T)), to_dev(B2), to_dev(sb2))


@SCALES
def test_fullsize_masked_swiglu_quant(pow2):
    """The masked decode workload (16 experts, M_max 256, N 7168 -> I 3584,
    K 2048) in the launch configuration the benchmark times: every act entry
    of every valid row against the oracle's silu(gate) * up of its full fp64
    GEMM, codes and scales of every valid row bit for bit, untouched rows in
    full."""
    print(f"full swiglu masked pow2={pow2}", flush=True)
    A, sa, B, sb, mm = fullsize_quantized("masked", pow2)
    G, M_max = A.shape[0], A.shape[1]
    N = B.shape[1]
    I = N // 2
    Q, sq, act = prefilled((G,), M_max, I)
    fg.grouped_masked_swiglu_quant(to_dev(A), to_dev(np.ascontiguousarray(np.transpose(sa, (0, 2, 1)))),
                                   to_dev(B), to_dev(sb), to_dev(mm), Q, sq, act, pow2=pow2)
    torch.cuda.synchronize()
    Qh, sqh, acth = Q.cpu().numpy(), sq.cpu().numpy(), act.cpu().numpy()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm)
    for g in range(G):
        v = valid[g]
        assert np.all(Qh[g][~v] == Q_FILL) and np.all(acth[g][~v] == F_FILL)
        assert np.all(sqh[g].T[~v] == F_FILL)
        if v.any():
            codes, scales = oracle.quantize_act_1x128(acth[g][v], pow2)
            assert np.array_equal(codes, Qh[g][v]) and np.array_equal(scales, sqh[g].T[v])
    r = check_f32(acth[valid], oracle.swiglu_blocks(ref[valid]))
    print(f"masked act: n_checked={int(valid.sum()) * I} {r}", flush=True)
    record_parity(f"fused masked act {'pow2' if pow2 else 'fp32'}", int(valid.sum()) * I, r["worst"], r["frob"],
                  " (codes + scales bit-exact)")
    assert r["ok"], r


@SCALES
def test_fullsize_contiguous_swiglu_quant(pow2):
    """The contiguous MoE workload (8 experts, 9472 rows with padding, N 4096 ->
    I 2048, K 7168) on the automatically chosen tile (256x256, following the
    experts' runs of 128-row blocks): codes and scales of every row with an
    expert bit for bit against the oracle quantiser of the kernel's own fp32
    activation, padding rows untouched, every act entry of every row with an
    expert against the oracle's silu(gate) * up of its full fp64 GEMM."""
    print(f"full swiglu contiguous pow2={pow2}", flush=True)
    A, sa, B, sb, mi = fullsize_contiguous(pow2)
    M, G, N = A.shape[0], B.shape[0], B.shape[1]
    I = N // 2
    Q, sq, act = prefilled((), M, I)
    fg.grouped_contiguous_swiglu_quant(to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb),
                                       to_dev(mi), Q, sq, act, pow2=pow2)
    torch.cuda.synchronize()
    Qh, sqh, acth = Q.cpu().numpy(), sq.cpu().numpy().T, act.cpu().numpy()
    valid = mi >= 0
    assert np.all(Qh[~valid] == Q_FILL) and np.all(acth[~valid] == F_FILL) and np.all(sqh[~valid] == F_FILL)
    codes, scales = oracle.quantize_act_1x128(acth[valid], pow2)
    assert np.array_equal(codes, Qh[valid]) and np.array_equal(scales, sqh[valid])
    ref, valid_ref = fullsize_contiguous_ref(pow2)
    assert np.array_equal(valid, valid_ref)
    r = check_f32(acth[valid], oracle.swiglu_blocks(ref[valid]))
    print(f"contiguous act: n_checked={int(valid.sum()) * I} {r}", flush=True)
    record_parity(f"fused contiguous act {'pow2' if pow2 else 'fp32'}", int(valid.sum()) * I, r["worst"], r["frob"],
                  " (codes + scales bit-exact)")
    assert r["ok"], r
