"""Acceptance check of a bf16 GEMM result against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The output type is bf16 (2kiu.com explainer, section 3.3: accumulate in FP32,
convert to the required type at the end). The bar, over the checked elements E
(the rows the call must write):

  (i)   every e in E:  |d - ref| <= 1e-2 * |ref| + 1e-3 * rms(ref over E)
  (ii)  ||d - ref||_F / ||ref||_F over E  <= 2e-3
  (iii) every element outside E keeps its prior bits exactly.

Why these numbers: rounding the exact result once to bf16 (8 significant bits,
round-to-nearest-even) already costs a relative Frobenius error of about
1.65e-3 on Gaussian-product data, and truncation about twice that (the checker
tests reproduce both); 2e-3 therefore admits one correctly rounded bf16
conversion of an fp32-accurate sum and rejects truncation or a second bf16
rounding. The per-element bound is a few bf16 half-ulps, relaxed by 1e-3 rms
near zero where cancellation makes the relative error meaningless.
"""

import numpy as np

REL_TOL = 1e-2
ABS_RMS_TOL = 1e-3
FROB_TOL = 2e-3


def bf16_rne(x):
    """Round fp64 values to the nearest bf16 value (ties to even), returned as
    fp64. Normal range only (the results checked here never reach bf16's
    subnormal or overflow range)."""
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)                 # x = mant * 2^exp, |mant| in [0.5, 1)
    q = np.rint(np.ldexp(mant, 8))          # 8 significant bits, half to even
    return np.ldexp(q, exp - 8)


def bf16_bits_to_f64(bits):
    """Raw bf16 bit patterns (uint16) -> fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check(d_bits, ref, valid_rows=None, prefill_bits=None,
          rel_tol=REL_TOL, abs_rms_tol=ABS_RMS_TOL, frob_tol=FROB_TOL):
    """Check a bf16 result against the oracle.

    d_bits       raw bf16 output bits (uint16), same shape as ref.
    ref          fp64 oracle result.
    valid_rows   bool mask over the leading (row) axes, True where the call must
                 write; None means every row.
    prefill_bits uint16 array (or scalar) the buffer held before the call;
                 required when some rows are not valid.
    Returns a dict; result["ok"] is the verdict.
    """
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.float64)
    if d_bits.shape != ref.shape:
        raise ValueError(f"shape mismatch {d_bits.shape} vs {ref.shape}")
    if valid_rows is None:
        valid_rows = np.ones(ref.shape[:-1], dtype=bool)
    valid_rows = np.asarray(valid_rows, dtype=bool)
    E = np.broadcast_to(valid_rows[..., None], ref.shape)

    d = bf16_bits_to_f64(d_bits)
    res = {"n_checked": int(E.sum())}
    if res["n_checked"]:
        r = ref[E]
        x = d[E]
        rms = float(np.sqrt(np.mean(r * r)))
        err = np.abs(x - r)
        bound = rel_tol * np.abs(r) + abs_rms_tol * rms
        with np.errstate(invalid="ignore", divide="ignore"):
            ratio = np.where(bound > 0, err / bound, np.where(err == 0, 0.0, np.inf))
        ratio = np.where(np.isnan(x), np.inf, ratio)
        nref = float(np.linalg.norm(r))
        frob = float(np.linalg.norm(x - r) / nref) if nref > 0 else float(np.linalg.norm(x - r))
        if np.any(np.isnan(x)):
            frob = float("inf")
        floor = float(np.linalg.norm(bf16_rne(r) - r) / nref) if nref > 0 else 0.0
        res.update(rms=rms, max_ratio=float(ratio.max()), n_bad=int((ratio > 1).sum()),
                   frob=frob, floor=floor,
                   frob_over_floor=(frob / floor) if floor > 0 else None)
        elem_ok = res["n_bad"] == 0
        frob_ok = frob <= frob_tol
    else:
        elem_ok = frob_ok = True
        res.update(rms=0.0, max_ratio=0.0, n_bad=0, frob=0.0, floor=0.0, frob_over_floor=None)

    untouched_ok = True
    n_unchecked = int((~E).sum())
    if n_unchecked:
        if prefill_bits is None:
            raise ValueError("rows outside the checked set need prefill_bits")
        pre = np.broadcast_to(np.asarray(prefill_bits, dtype=np.uint16), ref.shape)
        touched = (d_bits != pre) & ~E
        res["n_touched"] = int(touched.sum())
        untouched_ok = res["n_touched"] == 0
    res.update(elem_ok=elem_ok, frob_ok=frob_ok, untouched_ok=untouched_ok,
               ok=bool(elem_ok and frob_ok and untouched_ok))
    return res
