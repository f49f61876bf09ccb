"""GPU quantisers against the oracle's quantisers: codes and scales bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtest import quant_inputs, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(16, 256), (300, 1024), (3, 40, 384)])
def test_act_quant_bit_exact(shape):
    x = quant_inputs(shape, 7)
    q, sa = fg.quant_act_1x128(to_dev(x))
    torch.cuda.synchronize()
    flat = x.reshape(-1, shape[-1])
    codes, scales = oracle.quantize_act_1x128(flat)
    assert np.array_equal(q.cpu().numpy().reshape(flat.shape), codes)
    if len(shape) == 3:
        b, M, K = shape
        sa_nat = np.transpose(sa.cpu().numpy(), (0, 2, 1)).reshape(b * M, K // 128)
    else:
        sa_nat = sa.cpu().numpy().T
    assert np.array_equal(sa_nat, scales)


@pytest.mark.parametrize("shape", [(128, 128), (384, 640), (2, 256, 384)])
def test_weight_quant_bit_exact(shape):
    rng = np.random.default_rng(8)
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.05)
    flat = w.reshape(-1, shape[-1])
    flat[min(130, flat.shape[0] - 1), min(200, flat.shape[1] - 1)] = 3.0
    q, sb = fg.quant_weight_128x128(to_dev(w))
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_weight_128x128(w)
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(sb.cpu().numpy(), scales)


def boundary_rows():
    """Rows of 128 values whose block maximum is exactly 448 (scale 1, or 2^0 for
    power-of-two scales), so every code is the encoder's own rounding decision:
    every finite E4M3 value, every midpoint between neighbours, and the fp32
    values just below and above each midpoint, with both signs."""
    t = oracle.decode_table()[:0x7F].astype(np.float64)          # 0 .. 448, ascending
    mids = (t[:-1] + t[1:]) / 2
    vals = np.concatenate([t, mids,
                           np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                           [2.0 ** -10, 3 * 2.0 ** -11, 1e-30, 2.0 ** -126, 1e-45]]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per_row = 127
    rows = -(-vals.size // per_row)
    x = np.zeros((rows, 128), np.float32)
    for r in range(rows):
        chunk = vals[r * per_row:(r + 1) * per_row]
        x[r, :chunk.size] = chunk
        x[r, 127] = 448.0
    return x


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
def test_quant_rounding_boundaries_bit_exact(pow2):
    x = boundary_rows()
    q, sa = (fg.quant_act_1x128_pow2 if pow2 else fg.quant_act_1x128)(to_dev(x))
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_act_1x128(x, pow2)
    assert np.all(scales == 1.0)
    assert np.array_equal(sa.cpu().numpy().T, scales)
    assert np.array_equal(q.cpu().numpy(), codes)


@pytest.mark.parametrize("pow2", [False, True], ids=["fp32_scales", "pow2_scales"])
@pytest.mark.parametrize("shape", [(8, 256), (72, 384), (200, 128), (328, 640), (3, 72, 256), (2, 200, 384)])
def test_weight_quant_ragged_n_bit_exact(shape, pow2):
    """N not a multiple of 128: the last row block of each expert holds the
    remaining N mod 128 rows and takes its scale from them alone. A spike in
    the last (partial) block and a tiny-valued last block make its scale
    differ from what a full block or a neighbour would give."""
    print(f"weight quant ragged N {shape} pow2={pow2}", flush=True)
    rng = np.random.default_rng(9)
    w = rng.standard_normal(shape, dtype=np.float32)
    flat = w.reshape(-1, shape[-2], shape[-1])
    N = shape[-2]
    last = (N - 1) // 128 * 128
    flat[0, N - 1, 5] = 40.0                                  # spike in the partial block
    flat[-1, last:, 128:256] *= np.float32(2.0 ** -20)        # tiny partial block
    fn = fg.quant_weight_128x128_pow2 if pow2 else fg.quant_weight_128x128
    wd = to_dev(w)
    q = torch.full(shape, 0x5A, dtype=torch.uint8, device=wd.device)
    q, sb = fn(wd, q=q)
    torch.cuda.synchronize()
    codes, scales = oracle.quantize_weight_128x128(w, pow2)
    assert q.shape == codes.shape and sb.shape == scales.shape
    assert np.array_equal(q.cpu().numpy(), codes)
    assert np.array_equal(sb.cpu().numpy(), scales)
