"""FP8 (OCP E4M3) block-scaled GEMM for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libfg.so`` (see ``include/fg.h``):
argument checking and marshalling only. Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and calls fail
loudly when the library is missing or the device is not gfx950.

torch is used for device memory and the current HIP stream only.

    D = A . B^T,  D[m, n] = sum_kb sa[m, kb] sb[n // 128, kb] sum_{k in kb} a[m, k] b[n, k]

Tensor conventions (all on the same CUDA/HIP device, contiguous):
    A   uint8 or float8_e4m3fn  [M, K]        (masked: [G, M_max, K])
    sa  float32                 [K/128, M]    (masked: [G, K/128, M_max])
    B   uint8 or float8_e4m3fn  [N, K]        (grouped: [G, N, K])
    sb  float32                 [ceil(N/128), K/128] (grouped: [G, ceil(N/128), K/128])
    D   bfloat16                [M, N]        (masked: [G, M_max, N])
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfg.so")

LAYOUT_DENSE, LAYOUT_CONTIGUOUS, LAYOUT_MASKED = 0, 1, 2
SELECT_SWIGLU_QUANT = 0x100      # fg_select_config: the tile of the fused SiLU-gate epilogue
SCALES_FP32, SCALES_POW2 = 0, 1

_lib = None


class FGError(RuntimeError):
    pass


def _declare(L):
    """Argument and return types of every entry point of include/fg.h."""
    vp, fp, ip, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    ipp = ctypes.POINTER(ctypes.c_int)
    L.fg_gemm_fp8_nt.argtypes = [vp, fp, vp, fp, vp, i, i, i, vp]
    L.fg_grouped_contiguous.argtypes = [vp, fp, vp, fp, vp, ip, i, i, i, i, vp]
    L.fg_grouped_masked.argtypes = [vp, fp, vp, fp, vp, ip, i, i, i, i, vp]
    L.fg_select_config.argtypes = [i, i, i, i, i, i, ipp, ipp]
    L.fg_select_grid.argtypes = [i, i, i, i, i, i, ipp]
    L.fg_quant_act_1x128.argtypes = [vp, vp, vp, i, i, i, vp]
    L.fg_quant_weight_128x128.argtypes = [vp, vp, vp, i, i, i, vp]
    L.fg_gemm_fp8_nt_pow2.argtypes = L.fg_gemm_fp8_nt.argtypes
    L.fg_grouped_contiguous_pow2.argtypes = L.fg_grouped_contiguous.argtypes
    L.fg_grouped_masked_pow2.argtypes = L.fg_grouped_masked.argtypes
    L.fg_quant_act_1x128_pow2.argtypes = L.fg_quant_act_1x128.argtypes
    L.fg_quant_weight_128x128_pow2.argtypes = L.fg_quant_weight_128x128.argtypes
    L.fg_gemm_fp8_nt_swiglu_quant.argtypes = [vp, fp, vp, fp, vp, fp, fp, i, i, i, i, vp]
    L.fg_grouped_contiguous_swiglu_quant.argtypes = [vp, fp, vp, fp, vp, fp, fp, ip, i, i, i, i, i, vp]
    L.fg_grouped_masked_swiglu_quant.argtypes = [vp, fp, vp, fp, vp, fp, fp, ip, i, i, i, i, i, vp]
    L.fg_strerror.argtypes = [i]
    L.fg_strerror.restype = ctypes.c_char_p
    for name in ENTRY_POINTS:
        if name != "fg_strerror":
            getattr(L, name).restype = ctypes.c_int
    return L


ENTRY_POINTS = ("fg_gemm_fp8_nt", "fg_grouped_contiguous", "fg_grouped_masked",
                "fg_select_config", "fg_select_grid", "fg_quant_act_1x128",
                "fg_quant_weight_128x128", "fg_gemm_fp8_nt_pow2", "fg_grouped_contiguous_pow2",
                "fg_grouped_masked_pow2", "fg_quant_act_1x128_pow2",
                "fg_quant_weight_128x128_pow2", "fg_gemm_fp8_nt_swiglu_quant",
                "fg_grouped_contiguous_swiglu_quant", "fg_grouped_masked_swiglu_quant",
                "fg_strerror")


def load(path):
    """ctypes handle of a build of the library at `path`, with its entry points
    declared (raises ImportError if the file is missing)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m moe_grouped_gemm_02_amd.build`")
    return _declare(ctypes.CDLL(path))


def lib():
    """Load libfg.so (built in-tree by ``moe_grouped_gemm_02_amd.build``)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def strerror(code):
    return lib().fg_strerror(int(code)).decode()


def _check(code, what):
    if code != 0:
        raise FGError(f"{what}: {strerror(code)} (code {code})")


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _call(fn, dev, *args):
    """Calls entry point `fn` with `dev` as the current device (the library
    launches on the current device, on the stream passed last) and raises
    FGError on a nonzero return code."""
    torch = _torch()
    with torch.cuda.device(dev):
        _check(getattr(lib(), fn)(*args), fn)


def _fp8(t, name, shape, device=None):
    torch = _torch()
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must be uint8 or float8_e4m3fn E4M3 bytes, got {t.dtype}")
    _dev(t, name, shape, device=device)


def _dev(t, name, shape, dtype=None, device=None):
    """Checks a tensor argument: on a GPU (on `device` if given), of `dtype`
    (if given), of `shape`, contiguous."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's operands on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def gemm_fp8_nt(A, sa, B, sb, D):
    """Dense D[M, N] = A[M, K] . B[N, K]^T with block scales; writes D in place."""
    return _dense("fg_gemm_fp8_nt", A, sa, B, sb, D)


def gemm_fp8_nt_pow2(A, sa, B, sb, D):
    """gemm_fp8_nt with power-of-two scales applied by the matrix core (every sa
    and sb entry must be a power of two in [2^-126, 2^127])."""
    return _dense("fg_gemm_fp8_nt_pow2", A, sa, B, sb, D)


def _dense(fn, A, sa, B, sb, D):
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    _fp8(A, "A", (M, K))
    _fp8(B, "B", (N, K), dev)
    if K % 128 or N % 8:
        raise ValueError("K must be a multiple of 128 and N of 8")
    _dev(sa, "sa", (K // 128, M), torch.float32, dev)
    _dev(sb, "sb", (-(-N // 128), K // 128), torch.float32, dev)
    _dev(D, "D", (M, N), torch.bfloat16, dev)
    _call(fn, dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), M, N, K, _stream(A))
    return D


def grouped_contiguous(A, sa, B, sb, D, m_indices):
    """MoE contiguous layout: rows of A belong to expert m_indices[row] (-1 = padding,
    not written); B is [G, N, K]."""
    return _contiguous("fg_grouped_contiguous", A, sa, B, sb, D, m_indices)


def grouped_contiguous_pow2(A, sa, B, sb, D, m_indices):
    """grouped_contiguous with power-of-two scales applied by the matrix core."""
    return _contiguous("fg_grouped_contiguous_pow2", A, sa, B, sb, D, m_indices)


def _contiguous(fn, A, sa, B, sb, D, m_indices):
    torch = _torch()
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    dev = A.device
    _fp8(A, "A", (M, K))
    _fp8(B, "B", (G, N, K), dev)
    if K % 128 or N % 8:
        raise ValueError("K must be a multiple of 128 and N of 8")
    _dev(sa, "sa", (K // 128, M), torch.float32, dev)
    _dev(sb, "sb", (G, -(-N // 128), K // 128), torch.float32, dev)
    _dev(D, "D", (M, N), torch.bfloat16, dev)
    _dev(m_indices, "m_indices", (M,), torch.int32, dev)
    _call(fn, dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), _ptr(m_indices), M, N, K, G, _stream(A))
    return D


def grouped_masked(A, sa, B, sb, D, masked_m):
    """MoE masked layout: expert g has masked_m[g] valid rows of A[g]; only those rows
    of D[g] are written. masked_m stays on the device."""
    return _masked("fg_grouped_masked", A, sa, B, sb, D, masked_m)


def grouped_masked_pow2(A, sa, B, sb, D, masked_m):
    """grouped_masked with power-of-two scales applied by the matrix core."""
    return _masked("fg_grouped_masked_pow2", A, sa, B, sb, D, masked_m)


def _masked(fn, A, sa, B, sb, D, masked_m):
    torch = _torch()
    G, M_max, K = A.shape
    N = B.shape[1]
    dev = A.device
    _fp8(A, "A", (G, M_max, K))
    _fp8(B, "B", (G, N, K), dev)
    if K % 128 or N % 8:
        raise ValueError("K must be a multiple of 128 and N of 8")
    _dev(sa, "sa", (G, K // 128, M_max), torch.float32, dev)
    _dev(sb, "sb", (G, -(-N // 128), K // 128), torch.float32, dev)
    _dev(D, "D", (G, M_max, N), torch.bfloat16, dev)
    _dev(masked_m, "masked_m", (G,), torch.int32, dev)
    _call(fn, dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(D), _ptr(masked_m), G, M_max, N, K, _stream(A))
    return D


def _fused_outputs(lead, I, M, dev, Q, sq, act, with_act):
    """Allocate (or check) the fused epilogue's outputs: Q [*lead, M, I] uint8,
    sq [*lead, I/128, M] fp32, act [*lead, M, I] fp32 or None."""
    torch = _torch()
    if Q is None:
        Q = torch.empty(lead + (M, I), dtype=torch.uint8, device=dev)
    if sq is None:
        sq = torch.empty(lead + (I // 128, M), dtype=torch.float32, device=dev)
    if act is None and with_act:
        act = torch.empty(lead + (M, I), dtype=torch.float32, device=dev)
    _fp8(Q, "Q", lead + (M, I), dev)
    _dev(sq, "sq", lead + (I // 128, M), torch.float32, dev)
    if act is not None:
        _dev(act, "act", lead + (M, I), torch.float32, dev)
    return Q, sq, act


def _opt_ptr(t):
    return ctypes.c_void_p(0) if t is None else _ptr(t)


def gemm_fp8_nt_swiglu_quant(A, sa, B, sb, Q=None, sq=None, act=None, pow2=False, with_act=False):
    """Dense first projection with the fused epilogue: H = A . B^T (B's rows
    interleave gate and up every 128), act = silu(gate) * up, quantised per 1x128
    block. Returns (Q [M, N/2] E4M3, sq [N/256, M] fp32, act [M, N/2] fp32 or None).
    pow2: power-of-two input scales and output scales."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    dev = A.device
    _fp8(A, "A", (M, K))
    _fp8(B, "B", (N, K), dev)
    if K % 128 or N % 256:
        raise ValueError("K must be a multiple of 128 and N of 256")
    _dev(sa, "sa", (K // 128, M), torch.float32, dev)
    _dev(sb, "sb", (N // 128, K // 128), torch.float32, dev)
    Q, sq, act = _fused_outputs((), N // 2, M, dev, Q, sq, act, with_act)
    _call("fg_gemm_fp8_nt_swiglu_quant", dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(Q), _ptr(sq),
          _opt_ptr(act), M, N, K, int(bool(pow2)), _stream(A))
    return Q, sq, act


def grouped_contiguous_swiglu_quant(A, sa, B, sb, m_indices, Q=None, sq=None, act=None, pow2=False,
                                    with_act=False):
    """MoE contiguous first projection with the fused epilogue (see
    gemm_fp8_nt_swiglu_quant); padding rows (m_indices = -1) are not written."""
    torch = _torch()
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    dev = A.device
    _fp8(A, "A", (M, K))
    _fp8(B, "B", (G, N, K), dev)
    if K % 128 or N % 256:
        raise ValueError("K must be a multiple of 128 and N of 256")
    _dev(sa, "sa", (K // 128, M), torch.float32, dev)
    _dev(sb, "sb", (G, N // 128, K // 128), torch.float32, dev)
    _dev(m_indices, "m_indices", (M,), torch.int32, dev)
    Q, sq, act = _fused_outputs((), N // 2, M, dev, Q, sq, act, with_act)
    _call("fg_grouped_contiguous_swiglu_quant", dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(Q), _ptr(sq),
          _opt_ptr(act), _ptr(m_indices), M, N, K, G, int(bool(pow2)), _stream(A))
    return Q, sq, act


def grouped_masked_swiglu_quant(A, sa, B, sb, masked_m, Q=None, sq=None, act=None, pow2=False,
                                with_act=False):
    """MoE masked first projection with the fused epilogue; only rows
    r < masked_m[g] of each expert are written. Q [G, M_max, N/2],
    sq [G, N/256, M_max], act [G, M_max, N/2]."""
    torch = _torch()
    G, M_max, K = A.shape
    N = B.shape[1]
    dev = A.device
    _fp8(A, "A", (G, M_max, K))
    _fp8(B, "B", (G, N, K), dev)
    if K % 128 or N % 256:
        raise ValueError("K must be a multiple of 128 and N of 256")
    _dev(sa, "sa", (G, K // 128, M_max), torch.float32, dev)
    _dev(sb, "sb", (G, N // 128, K // 128), torch.float32, dev)
    _dev(masked_m, "masked_m", (G,), torch.int32, dev)
    Q, sq, act = _fused_outputs((G,), N // 2, M_max, dev, Q, sq, act, with_act)
    _call("fg_grouped_masked_swiglu_quant", dev, _ptr(A), _ptr(sa), _ptr(B), _ptr(sb), _ptr(Q), _ptr(sq),
          _opt_ptr(act), _ptr(masked_m), G, M_max, N, K, int(bool(pow2)), _stream(A))
    return Q, sq, act


def select_config(M, N, K, G=1, layout=LAYOUT_DENSE, num_cus=0):
    """(bm, bn): the tile the library would launch for the problem (layout
    optionally | SELECT_SWIGLU_QUANT); host-only, no device access."""
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(lib().fg_select_config(M, N, K, G, layout, num_cus, ctypes.byref(bm), ctypes.byref(bn)),
           "fg_select_config")
    return bm.value, bn.value


def select_grid(M, N, K, G=1, layout=LAYOUT_DENSE, num_cus=0):
    """Workgroups the launch for the problem would use; host-only."""
    grid = ctypes.c_int()
    _check(lib().fg_select_grid(M, N, K, G, layout, num_cus, ctypes.byref(grid)), "fg_select_grid")
    return grid.value


def quant_act_1x128(x, q=None, sa=None):
    """fp32 activations [M, K] (or [batch, M, K]) -> (E4M3 codes, sa) with one scale per
    1x128 block; sa comes out in the GEMM's layout [K/128, M] ([batch, K/128, M])."""
    return _quant_act("fg_quant_act_1x128", x, q, sa)


def quant_act_1x128_pow2(x, q=None, sa=None):
    """quant_act_1x128 with each scale rounded up to a power of two (>= 2^-126)."""
    return _quant_act("fg_quant_act_1x128_pow2", x, q, sa)


def _quant_act(fn, x, q, sa):
    torch = _torch()
    if x.dim() not in (2, 3):
        raise ValueError("x must be [M, K] or [batch, M, K]")
    batch = x.shape[0] if x.dim() == 3 else 1
    M, K = x.shape[-2], x.shape[-1]
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    _dev(x, "x", tuple(x.shape), torch.float32)
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    sa_shape = (batch, K // 128, M) if x.dim() == 3 else (K // 128, M)
    if sa is None:
        sa = torch.empty(sa_shape, dtype=torch.float32, device=x.device)
    _fp8(q, "q", tuple(x.shape), x.device)
    _dev(sa, "sa", sa_shape, torch.float32, x.device)
    _call(fn, x.device, _ptr(x), _ptr(q), _ptr(sa), batch, M, K, _stream(x))
    return q, sa


def quant_weight_128x128(w, q=None, sb=None):
    """fp32 weights [N, K] (or [G, N, K]) -> (E4M3 codes, sb) with one scale per
    128x128 block; sb is [ceil(N/128), K/128] ([G, ceil(N/128), K/128]). N need
    not be a multiple of 128: the last row block then holds N mod 128 rows."""
    return _quant_weight("fg_quant_weight_128x128", w, q, sb)


def quant_weight_128x128_pow2(w, q=None, sb=None):
    """quant_weight_128x128 with each scale rounded up to a power of two (>= 2^-126)."""
    return _quant_weight("fg_quant_weight_128x128_pow2", w, q, sb)


def _quant_weight(fn, w, q, sb):
    torch = _torch()
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N, K] or [G, N, K]")
    G = w.shape[0] if w.dim() == 3 else 1
    N, K = w.shape[-2], w.shape[-1]
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    _dev(w, "w", tuple(w.shape), torch.float32)
    sb_shape = tuple(w.shape[:-2]) + (-(-N // 128), K // 128)
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if sb is None:
        sb = torch.empty(sb_shape, dtype=torch.float32, device=w.device)
    _fp8(q, "q", tuple(w.shape), w.device)
    _dev(sb, "sb", sb_shape, torch.float32, w.device)
    _call(fn, w.device, _ptr(w), _ptr(q), _ptr(sb), G, N, K, _stream(w))
    return q, sb
