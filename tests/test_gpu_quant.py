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
