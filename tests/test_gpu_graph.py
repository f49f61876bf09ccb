"""The calls inside a captured HIP graph: every entry point is asynchronous on
the caller's stream and reads nothing on the host, so it can be captured. Each
graph here is replayed several times, with eager fills, eager calls of the same
entry point into other buffers and synchronisations between the replays, and
every replay must reproduce the eager result bit for bit, including the rows the
call must leave untouched."""
import contextlib

import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_02_amd as fg
from fgtesting import forced_grid, forced_runs, forced_split, forced_tile as forced
from fgtest import (SENTINEL, d_bits, dense_inputs, make_contiguous, make_dense, make_masked,
                    masked_inputs, new_out, to_dev)

pytestmark = pytest.mark.gpu

REPLAYS = 4


def fill_sentinel(D):
    D.view(torch.int16).fill_(np.int16(np.uint16(SENTINEL).view(np.int16)))


def bits(t):
    return t.view(torch.uint8).cpu().numpy().copy()


def replay_matches_eager(call, outs, fill, other_outs):
    """call(outs) launches the op into the tensors `outs`. Runs it eagerly, then
    captures it and replays it REPLAYS times; between replays the outputs are
    refilled eagerly and the op runs eagerly into `other_outs`."""
    fill(outs)
    call(outs)
    torch.cuda.synchronize()
    eager = [bits(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    fill(outs)
    with torch.cuda.graph(g):
        call(outs)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        fill(outs)
        fill(other_outs)
        call(other_outs)                     # eager work of the same entry point
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(bits(o), e), f"replay {r} differs from the eager result"
        for o, e in zip(other_outs, eager):
            assert np.array_equal(bits(o), e), f"eager call after replay {r} differs"
    del g
    return eager


def test_graph_dense():
    print("graph dense 300x512x1152", flush=True)
    A, sa, B, sb = make_dense(300, 512, 1152, 401)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    D, D2 = new_out((300, 512)), new_out((300, 512))
    replay_matches_eager(lambda o: fg.gemm_fp8_nt(Ad, sad, Bd, sbd, o[0]), [D],
                         lambda o: [fill_sentinel(x) for x in o], [D2])
    r = oracle.check(d_bits(D), oracle.ref_dense(A, sa, B, sb))
    assert r["ok"], r


@pytest.mark.parametrize("tile", [None, (256, 224), (128, 256)],
                         ids=lambda t: "auto" if t is None else f"{t[0]}x{t[1]}")
def test_graph_contiguous(tile):
    """The 256-row tiles derive their tile list on the device from m_indices:
    a replay after m_indices changed in place must follow the new experts."""
    print(f"graph contiguous tile {tile}", flush=True)
    A, sa, B, sb, mi = make_contiguous(3, 384, 640, 402, m_lo=1, m_hi=300)
    Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
    mid = to_dev(mi)
    M = A.shape[0]
    D, D2 = new_out((M, 384)), new_out((M, 384))
    with (forced(*tile) if tile else contextlib.nullcontext()):
        replay_matches_eager(lambda o: fg.grouped_contiguous(Ad, sad, Bd, sbd, o[0], mid), [D],
                             lambda o: [fill_sentinel(x) for x in o], [D2])
        # same graph, new routing: every expert id rotated, rows stay in place
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fg.grouped_contiguous(Ad, sad, Bd, sbd, D, mid)
        mi2 = np.where(mi >= 0, (mi + 1) % 3, -1).astype(np.int32)
        mid.copy_(torch.from_numpy(mi2))
        fill_sentinel(D)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
    ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi2)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


def test_graph_masked():
    """masked_m stays on the device: a replay after masked_m changed in place
    must follow the new counts."""
    print("graph masked", flush=True)
    G, M_max, N, K = 3, 200, 384, 768
    A, sa, B, sb, _ = make_masked(G, M_max, N, K, 403)
    Ad, sad, Bd, sbd = masked_inputs(A, sa, B, sb)
    mm = to_dev(np.array([77, 0, 200], np.int32))
    D, D2 = new_out((G, M_max, N)), new_out((G, M_max, N))
    replay_matches_eager(lambda o: fg.grouped_masked(Ad, sad, Bd, sbd, o[0], mm), [D],
                         lambda o: [fill_sentinel(x) for x in o], [D2])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fg.grouped_masked(Ad, sad, Bd, sbd, D, mm)
    mm2 = np.array([5, 150, 0], np.int32)
    mm.copy_(torch.from_numpy(mm2))
    fill_sentinel(D)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ref, valid = oracle.ref_masked(A, sa, B, sb, mm2)
    r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r


def test_graph_fused_and_quantiser():
    """The fused SiLU-gate + re-quantisation call and the activation quantiser."""
    print("graph fused + quantiser", flush=True)
    A, sa, B, sb = make_dense(200, 512, 640, 404)
    Ad, sad, Bd, sbd = to_dev(A), to_dev(np.ascontiguousarray(sa.T)), to_dev(B), to_dev(sb)
    dev = torch.device("cuda", 0)

    def outs():
        return [torch.empty((200, 256), dtype=torch.uint8, device=dev),
                torch.empty((2, 200), dtype=torch.float32, device=dev)]

    def fill(o):
        o[0].fill_(0x5A)
        o[1].fill_(-1.0)

    replay_matches_eager(lambda o: fg.gemm_fp8_nt_swiglu_quant(Ad, sad, Bd, sbd, o[0], o[1]), outs(), fill,
                         outs())
    x = torch.from_numpy(np.random.default_rng(405).standard_normal((96, 512), dtype=np.float32)).to(dev)

    def qouts():
        return [torch.empty((96, 512), dtype=torch.uint8, device=dev),
                torch.empty((4, 96), dtype=torch.float32, device=dev)]

    eager = replay_matches_eager(lambda o: fg.quant_act_1x128(x, o[0], o[1]), qouts(), fill, qouts())
    codes, scales = oracle.quantize_act_1x128(x.cpu().numpy())
    assert np.array_equal(eager[0], codes)
    assert np.array_equal(eager[1].view(np.float32).reshape(4, 96), scales.T)


@pytest.mark.parametrize("kernel", ["split", "runs"])
def test_graph_tile_walk(kernel):
    """The kernels whose workgroups walk their tiles (dense two-shape, contiguous
    runs), with few workgroups so each walks several tiles, captured and
    replayed."""
    print(f"graph tile walk {kernel}", flush=True)
    if kernel == "split":
        A, sa, B, sb = make_dense(1000, 1160, 640, 406)
        Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
        D, D2 = new_out((1000, 1160)), new_out((1000, 1160))
        with forced_split(768), forced_grid(3):
            replay_matches_eager(lambda o: fg.gemm_fp8_nt(Ad, sad, Bd, sbd, o[0]), [D],
                                 lambda o: [fill_sentinel(x) for x in o], [D2])
        r = oracle.check(d_bits(D), oracle.ref_dense(A, sa, B, sb))
    else:
        A, sa, B, sb, mi = make_contiguous(3, 512, 640, 407, m_lo=200, m_hi=700)
        Ad, sad, Bd, sbd = dense_inputs(A, sa, B, sb)
        mid = to_dev(mi)
        M = A.shape[0]
        D, D2 = new_out((M, 512)), new_out((M, 512))
        with forced_runs(), forced_grid(2):
            replay_matches_eager(lambda o: fg.grouped_contiguous(Ad, sad, Bd, sbd, o[0], mid), [D],
                                 lambda o: [fill_sentinel(x) for x in o], [D2])
        ref, valid = oracle.ref_contiguous(A, sa, B, sb, mi)
        r = oracle.check(d_bits(D), ref, valid, prefill_bits=SENTINEL)
    assert r["ok"], r
