"""The Python binding's argument checks: a call with a host tensor, a wrong
dtype, shape or layout, or an argument the library rejects raises before (or
instead of) any launch and leaves the output untouched."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_02_amd as fg
from fgtest import SENTINEL, d_bits, dense_inputs, make_dense, new_out

pytestmark = pytest.mark.gpu

M, N, K = 64, 256, 256


@pytest.fixture(scope="module")
def operands():
    return dense_inputs(*make_dense(M, N, K, 500))


def untouched(D):
    return np.all(d_bits(D) == SENTINEL)


def test_host_tensor_rejected(operands):
    A, sa, B, sb = operands
    D = new_out((M, N))
    with pytest.raises(ValueError, match="device tensor"):
        fg.gemm_fp8_nt(A, sa.cpu(), B, sb, D)
    with pytest.raises(ValueError, match="device tensor"):
        fg.gemm_fp8_nt(A, sa, B.cpu(), sb, D)
    assert untouched(D)


def test_wrong_dtype_rejected(operands):
    A, sa, B, sb = operands
    D = new_out((M, N))
    with pytest.raises(TypeError):
        fg.gemm_fp8_nt(A, sa.double(), B, sb, D)
    with pytest.raises(TypeError):
        fg.gemm_fp8_nt(A.to(torch.int8), sa, B, sb, D)
    with pytest.raises(TypeError):
        fg.gemm_fp8_nt(A, sa, B, sb, torch.empty((M, N), dtype=torch.float16, device=D.device))
    assert untouched(D)


def test_wrong_shape_or_layout_rejected(operands):
    A, sa, B, sb = operands
    D = new_out((M, N))
    with pytest.raises(ValueError, match="shape"):
        fg.gemm_fp8_nt(A, sa.t().contiguous(), B, sb, D)   # natural [M, K/128] instead of [K/128, M]
    with pytest.raises(ValueError, match="contiguous"):
        fg.gemm_fp8_nt(A, sa.t().contiguous().t(), B, sb, D)
    with pytest.raises(ValueError, match="shape"):
        fg.gemm_fp8_nt(A, sa, B, sb, new_out((M, N + 8)))
    assert untouched(D)


def test_float8_dtype_accepted(operands):
    """float8_e4m3fn tensors carry the same bytes as uint8 codes."""
    A, sa, B, sb = operands
    D8, Du = new_out((M, N)), new_out((M, N))
    fg.gemm_fp8_nt(A.view(torch.float8_e4m3fn), sa, B.view(torch.float8_e4m3fn), sb, D8)
    fg.gemm_fp8_nt(A, sa, B, sb, Du)
    torch.cuda.synchronize()
    assert np.array_equal(d_bits(D8), d_bits(Du))


def test_library_rejection_raises(operands):
    """A K that is not a whole number of 128-wide blocks is refused by the
    binding; a misaligned output pointer, which only the library sees, comes
    back as FGError."""
    A, sa, B, sb = operands
    with pytest.raises(ValueError):
        fg.gemm_fp8_nt(A[:, :200].contiguous(), sa, B[:, :200].contiguous(), sb, new_out((M, N)))
    buf = new_out((M * N + 1,))
    D = buf[1:].view(M, N)   # 2-byte offset: not 16-byte aligned
    with pytest.raises(fg.FGError, match="invalid argument"):
        fg.gemm_fp8_nt(A, sa, B, sb, D)
    assert np.all(d_bits(buf) == SENTINEL)
