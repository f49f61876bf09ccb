"""GPU parity at the boundary's size limits: one expert's A (and B) must stay
below 2^31 bytes, because the kernels address it with 32-bit byte offsets
(include/fg.h). These problems sit just below that limit; the operands are
random finite E4M3 codes with random positive scales, made on the device, and
the oracle checks sampled rows (the first and last 256, and 2048 more spread
over the rows) element by element."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtest import SENTINEL, d_bits, new_out

pytestmark = pytest.mark.gpu


def finite_codes(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    c = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    nan = (c & 0x7F) == 0x7F
    c[nan] ^= 1                       # 0x7f / 0xff (NaN) -> 0x7e / 0xfe
    return c


def scales(shape, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.rand(shape, dtype=torch.float32, device="cuda", generator=g) * 1.5 + 0.5


def sample_rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(256), np.arange(M - 256, M), rng.integers(0, M, 2048)])
    return np.unique(rows)


def test_dense_just_below_the_offset_limit():
    K, N = 128, 24
    M = (2**31 - 1) // K                      # M * K = 2^31 - 128
    print(f"dense limits M={M} N={N} K={K}", flush=True)
    A = finite_codes((M, K), 1)
    sa = scales((K // 128, M), 2)
    B = finite_codes((N, K), 3)
    sb = scales((1, K // 128), 4)
    D = new_out((M, N))
    fg.gemm_fp8_nt(A, sa, B, sb, D)
    torch.cuda.synchronize()
    rows = sample_rows(M, 5)
    idx = torch.from_numpy(rows).cuda()
    a = A[idx].cpu().numpy()
    s = sa[:, idx].cpu().numpy().T
    ref = oracle.ref_dense(a, s, B.cpu().numpy(), sb.cpu().numpy())
    bits = D[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    r = oracle.check(bits, ref)
    print(r, flush=True)
    assert r["ok"], r


def test_contiguous_beyond_the_run_list_near_the_offset_limit():
    """M * K just below 2^31 with more 128-row blocks than the device-side run
    list holds: the 128-row tiles, two experts in 128-row-aligned segments and
    padding rows."""
    K, N, G = 7168, 256, 2
    M = ((2**31 - 1) // K) // 128 * 128       # 299520 rows, 2340 blocks
    print(f"contiguous limits M={M} N={N} K={K} G={G}", flush=True)
    assert fg.select_config(M, N, K, G, 1)[0] <= 128
    half = (M // 2) // 128 * 128
    mi = np.full(M, -1, np.int32)
    mi[:half - 5] = 0
    mi[half:M - 77] = 1
    A = finite_codes((M, K), 11)
    sa = scales((K // 128, M), 12)
    B = finite_codes((G, N, K), 13)
    sb = scales((G, N // 128, K // 128), 14)
    D = new_out((M, N))
    fg.grouped_contiguous(A, sa, B, sb, D, torch.from_numpy(mi).cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(M, 15), np.arange(half - 8, half + 8)]))
    idx = torch.from_numpy(rows).cuda()
    a = A[idx].cpu().numpy()
    s = sa[:, idx].cpu().numpy().T
    ref, valid = oracle.ref_contiguous(a, s, B.cpu().numpy(), sb.cpu().numpy(), mi[rows])
    bits = D[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    r = oracle.check(bits, ref, valid, prefill_bits=SENTINEL)
    print(r, flush=True)
    assert r["ok"], r
