"""Seeded generators: reproducible, with the structure the workloads describe."""
import numpy as np

import workloads


def test_reproducible():
    a = workloads.make("dense_small")
    b = workloads.make("dense_small")
    assert np.array_equal(a["a"], b["a"]) and np.array_equal(a["b"], b["b"])
    c = workloads.make("dense_small", seed=99)
    assert not np.array_equal(a["a"], c["a"])


def test_outlier_rows():
    w = workloads.make("dense_skinny", N=256, K=256)
    assert w["outlier_rows"].size == 3          # round(0.01 * 256)
    amax = np.abs(w["a"]).max(axis=1)
    top3 = np.sort(np.argsort(amax)[-3:])
    assert np.array_equal(top3, w["outlier_rows"])


def test_contiguous_structure():
    w = workloads.make("contiguous", N=128, K=128)
    mi, m, padded = w["m_indices"], w["group_m"], w["group_padded"]
    assert np.all((m >= 256) & (m <= 2048)) and np.all(padded % 128 == 0)
    assert mi.size == padded.sum() == w["a"].shape[0]
    off = 0
    for g in range(8):
        blk = mi[off:off + padded[g]]
        assert np.all(blk[:m[g]] == g) and np.all(blk[m[g]:] == -1)
        # every 128-row block belongs to one expert (or is padding)
        for r in range(0, padded[g], 128):
            ids = set(blk[r:r + 128].tolist()) - {-1}
            assert ids == {g}
        off += padded[g]
    assert np.all(w["a"][mi < 0] == 0)
    assert w["b"].shape == (8, 128, 128)


def test_masked_structure():
    w = workloads.make("masked", N=128, K=128)
    mm = w["masked_m"]
    assert mm.dtype == np.int32 and mm.shape == (16,)
    assert np.all((mm >= 0) & (mm <= 256))
    assert w["a"].shape == (16, 256, 128)


def test_useful_flop():
    w = workloads.make("masked", N=128, K=128)
    assert workloads.useful_flop(w) == 2.0 * w["masked_m"].sum() * 128 * 128
