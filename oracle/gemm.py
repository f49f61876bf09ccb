"""Reference D = A . B^T for the three DeepGEMM layouts, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. The zwzgs.cn page "DeepGEMM: an open-source FP8 GEMM library":
"Features > layouts" (a normal layout plus two MoE layouts, contiguous and
masked), "Technical details > two-level accumulation" (FP8 matrix-core partial
sums are accumulated a second time in FP32 on the general cores) and
"Applications > MoE" (contiguous for training/prefill, masked for inference).
The 2kiu.com explainer, section 3.3: FP8 inputs, FP32 accumulation, convert to
the output type at the end. The "transB" convention (B given as N x K) is the
one the ruibaoantu.com day-3 page uses in its usage example.

Definition used as the oracle. With dec() the E4M3 decode and kb = k // 128,

    Ahat[m, k] = dec(A[m, k]) * sa[m, kb]
    Bhat[n, k] = dec(B[n, k]) * sb[n // 128, kb]
    D[m, n]    = sum_k Ahat[m, k] * Bhat[n, k]

The two-level scheme computes, per K-block, P = sum_{k in kb} dec(a) dec(b)
(exact: every E4M3 value is a multiple of 2^-9 below 2^9, so a 128-term partial
is a multiple of 2^-18 below 2^43) and then adds P * sa * sb into an FP32
master accumulator. That is the same sum regrouped, so both forms agree up to
rounding; ``ref_dense_twolevel`` keeps the pages' order for comparison.

Scale layouts here are the natural ones: sa [M, K/128] (row-major), sb
[ceil(N/128), K/128]. Grouped weights are [G, N, K] with sb [G, ceil(N/128), K/128].
N need not be a multiple of 128: the last weight-scale block then covers the
remaining N mod 128 rows.

Readings for the grouped layouts (the pages name them only):
  * contiguous: rows of all experts are concatenated along M; m_indices[m] is
    the expert of row m, -1 marks a padding row, which has no output (the
    caller's buffer keeps its prior content there);
  * masked: A is [G, M_max, K]; expert g has masked_m[g] valid rows (clamped
    to [0, M_max]); rows at or beyond masked_m[g] have no output.
"""

import numpy as np

from .e4m3 import decode_table

_DEC = decode_table()


def dequant_act(codes, sa):
    """Ahat = dec(codes) * sa broadcast over each 128-wide K-block (fp64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    return _DEC[codes] * np.repeat(sa, 128, axis=-1)


def dequant_weight(codes, sb):
    """Bhat = dec(codes) * sb broadcast over each 128x128 block (fp64); N rows need
    not fill the last block (sb has ceil(N/128) rows)."""
    codes = np.asarray(codes, dtype=np.uint8)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    N = codes.shape[-2]
    return _DEC[codes] * np.repeat(np.repeat(sb, 128, axis=-2), 128, axis=-1)[..., :N, :]


def ref_dense(A, sa, B, sb):
    """Dense layout: A [M, K] codes, sa [M, K/128], B [N, K] codes, sb [N/128, K/128]
    -> D [M, N] fp64."""
    return dequant_act(A, sa) @ dequant_weight(B, sb).T


def ref_dense_twolevel(A, sa, B, sb):
    """The same product, in the order the method describes: for every 128-wide
    K-block an exact partial of decoded values, then scaled by sa * sb and added
    into the accumulator."""
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    sb_cols = np.repeat(sb, 128, axis=0)[:N]        # [N, K/128]
    acc = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // 128):
        ks = slice(kb * 128, (kb + 1) * 128)
        partial = _DEC[A[:, ks]] @ _DEC[B[:, ks]].T   # exact
        acc += partial * (sa[:, kb][:, None] * sb_cols[:, kb][None, :])
    return acc


def ref_contiguous(A, sa, B, sb, m_indices):
    """Grouped-contiguous layout.

    A [M, K], sa [M, K/128], B [G, N, K], sb [G, N/128, K/128], m_indices [M]
    (expert id per row, -1 = padding). Returns (D [M, N] fp64 with zeros on
    rows that have no output, valid-row mask [M] bool)."""
    m_indices = np.asarray(m_indices)
    M = A.shape[0]
    G, N = B.shape[0], B.shape[1]
    out = np.zeros((M, N), dtype=np.float64)
    valid = m_indices >= 0
    for g in range(G):
        rows = np.nonzero(m_indices == g)[0]
        if rows.size:
            out[rows] = ref_dense(A[rows], sa[rows], B[g], sb[g])
    return out, valid


def ref_masked(A, sa, B, sb, masked_m):
    """Grouped-masked layout.

    A [G, M_max, K], sa [G, M_max, K/128], B [G, N, K], sb [G, N/128, K/128],
    masked_m [G]. Returns (D [G, M_max, N] fp64 with zeros on rows that have no
    output, valid-row mask [G, M_max] bool)."""
    G, M_max = A.shape[0], A.shape[1]
    N = B.shape[1]
    out = np.zeros((G, M_max, N), dtype=np.float64)
    valid = np.zeros((G, M_max), dtype=bool)
    for g in range(G):
        m = int(min(max(int(masked_m[g]), 0), M_max))
        if m:
            out[g, :m] = ref_dense(A[g, :m], sa[g, :m], B[g], sb[g])
            valid[g, :m] = True
    return out, valid


def ref_entries(A, sa, B, sb, rows, cols):
    """D[rows[i], cols[i]] for a dense problem, one dot product per entry, so
    that samples of a full-size output can be checked without the full GEMM."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = np.empty(rows.shape[0], dtype=np.float64)
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb = np.asarray(sb, dtype=np.float32).astype(np.float64)
    for i, (m, n) in enumerate(zip(rows, cols)):
        a = _DEC[A[m]] * np.repeat(sa[m], 128)          # row m of Ahat
        b = _DEC[B[n]] * np.repeat(sb[n // 128], 128)   # row n of Bhat
        out[i] = a @ b
    return out
