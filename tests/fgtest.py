"""Shared helpers for the GPU parity tests: seeded inputs quantised by the
oracle on the CPU, marshalled into the library's layouts, and results brought
back for the oracle's check. Nothing here computes the GEMM."""
import functools

import numpy as np
import torch

import oracle
import workloads

SENTINEL = 0x7E7E          # bf16 bits of a finite value no GEMM here produces by chance

# Whole-output parity results of the full-size tests, printed in pytest's
# terminal summary (tests/conftest.py) so that a quiet run still shows them.
PARITY = []


def record_parity(name, n_checked, max_ratio, frob, extra=""):
    PARITY.append(f"{name}: n_checked={n_checked} max_ratio={max_ratio:.3f} frob={frob:.3e}{extra}")


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch.device("cuda", 0)


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def d_bits(D):
    return D.view(torch.int16).cpu().numpy().view(np.uint16)


def new_out(shape, prefill_bits=SENTINEL):
    D = torch.empty(shape, dtype=torch.bfloat16, device=dev())
    D.view(torch.int16).fill_(np.int16(np.uint16(prefill_bits).view(np.int16)))
    return D


def quant_dense(a, b, pow2=False):
    """fp32 A [M,K], B [N,K] -> oracle codes/scales in natural layout (pow2:
    power-of-two scales)."""
    A, sa = oracle.quantize_act_1x128(a, pow2)
    B, sb = oracle.quantize_weight_128x128(b, pow2)
    return A, sa, B, sb


def dense_inputs(A, sa, B, sb):
    """Natural-layout codes/scales -> device tensors in the ABI layout
    (sa transposed to K-block-major)."""
    return (to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb))


def masked_inputs(A, sa, B, sb):
    return (to_dev(A), to_dev(np.ascontiguousarray(np.transpose(sa, (0, 2, 1)))), to_dev(B), to_dev(sb))


def make_dense(M, N, K, seed, pow2=False, **kw):
    w = workloads.dense(M, N, K, seed, **kw)
    return quant_dense(w["a"], w["b"], pow2)


def make_contiguous(G, N, K, seed, pow2=False, **kw):
    w = workloads.contiguous(G, N, K, seed, **kw)
    A, sa = oracle.quantize_act_1x128(w["a"], pow2)
    B, sb = oracle.quantize_weight_128x128(w["b"], pow2)
    return A, sa, B, sb, w["m_indices"]


def make_masked(G, M_max, N, K, seed, pow2=False, **kw):
    w = workloads.masked(G, M_max, N, K, seed, **kw)
    Gs = w["a"].shape[0]
    A = np.empty(w["a"].shape, np.uint8)
    sa = np.empty((Gs, M_max, K // 128), np.float32)
    for g in range(Gs):
        A[g], sa[g] = oracle.quantize_act_1x128(w["a"][g], pow2)
    B, sb = oracle.quantize_weight_128x128(w["b"], pow2)
    return A, sa, B, sb, w["masked_m"]


def quant_inputs(shape, seed):
    """fp32 quantiser inputs with the awkward cases: an outlier row, an all-zero
    1x128 block, a tiny-valued block, a value that rounds to -0, and exact ties
    of the E4M3 grid after scaling by amax/448 = 1."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    flat = x.reshape(-1, shape[-1])
    flat[3] *= 50.0                                   # outlier row
    flat[5, 128:256] = 0.0                            # all-zero 1x128 block
    flat[6, :128] = np.float32(2.0 ** -12) * rng.standard_normal(128).astype(np.float32)
    flat[7, 5] = -1e-30                               # rounds to -0 after scaling
    flat[8, :128] = 0.0
    flat[8, 0] = 448.0
    t = oracle.decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2)
    flat[8, 1:127] = mids[:126]
    return x


@functools.lru_cache(maxsize=1)
def workload(name):
    """The named workload's fp32 inputs (shared by consecutive full-size tests;
    treat as read-only)."""
    return workloads.make(name)


def fullsize_quantized(name, pow2=False):
    """A named workload quantised by the oracle (chunked over threads: the same
    codes and scales as the serial quantisers), natural layouts: dense
    (A, sa, B, sb), contiguous (A, sa, B, sb, m_indices), masked
    (A [G, M_max, K], sa [G, M_max, K/128], B, sb, masked_m)."""
    from oracle.parallel import quantize_act_1x128_par, quantize_weight_128x128_par
    w = workload(name)
    A, sa = quantize_act_1x128_par(w["a"], pow2)
    B, sb = quantize_weight_128x128_par(w["b"], pow2)
    if w["kind"] == "contiguous":
        return A, sa, B, sb, w["m_indices"]
    if w["kind"] == "masked":
        return A, sa, B, sb, w["masked_m"]
    return A, sa, B, sb


@functools.lru_cache(maxsize=2)
def fullsize_contiguous(pow2=False):
    """The contiguous MoE workload (8 experts, N 4096, K 7168) quantised by the
    oracle: (A, sa, B, sb, m_indices), natural layouts; computed once per scale
    kind and shared by the full-size tests (treat as read-only)."""
    return fullsize_quantized("contiguous", pow2)


@functools.lru_cache(maxsize=2)
def fullsize_contiguous_ref(pow2=False):
    """The oracle's full D of the contiguous workload and its valid-row mask."""
    A, sa, B, sb, mi = fullsize_contiguous(pow2)
    return oracle.ref_contiguous(A, sa, B, sb, mi)
