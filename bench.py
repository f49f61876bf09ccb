#!/usr/bin/env python3
"""Throughput of the FP8 (E4M3) block-scaled GEMM on one MI355X.

One step = one library call (host validation + tile choice, then the kernel:
tile scheduling, staging, E4M3 MFMA per 128-wide K-block, promotion with
sa*sb into the FP32 master accumulator, bf16 epilogue) over one batch of
seeded synthetic input that is already resident in device memory.

Headline workload (the large dense FFN GEMM, the compute-bound case): dense
D = A . B^T with M=8192, N=7168, K=18432, A and B drawn N(0,1), quantised on
the GPU to E4M3 with fp32 scales per 1x128 (A) and 128x128 (B) block, bf16
output. `--workload` names another of the five workloads instead.

The inputs are replicated into enough copies to exceed the 256 MB last-level
(MALL) cache, and consecutive steps rotate through the copies, so each launch
streams its operands from HBM instead of re-reading a cached copy.

Prints ONE JSON line. `value` is TFLOP/s of useful work (2*M*N*K over rows that
have an output) per wall-clock second over the timed steps. `roofline` is for
the GEMM kernel, from HIP events recorded on the launch stream around the timed
steps: MFMA-bound workloads against the published 5.0 PFLOP/s dense FP8 peak,
HBM-bound ones against 8 TB/s. `cpu_baseline` is the CPU oracle (dequantise +
fp64 GEMM) timed on this host on a bounded sample of the headline workload;
`cpu_baseline_per_config` does the same for every workload (the whole problem
where one oracle call takes seconds, else a stated sample). `per_workload`
repeats the GPU measurement for the other workloads (the small dense case, the
skinny dense case, MoE contiguous, MoE masked) unless --headline-only is given;
`per_workload_pow2` measures every workload again on the power-of-two-scale
entry points (E8M0 scales applied by the matrix core), with operands quantised
by the power-of-two quantisers; `moe_swiglu_quant` times the fused
first-projection calls (GEMM + SiLU gate + 1x128 E4M3 re-quantisation, fp32
scales, no activation copy) on the two MoE workloads.

Every measurement, the headline included, first runs --warmup untimed steps
and then keeps launching until at least --warmup-ms (default 400) of untimed
work has run, whatever --warmup says: the GPU's clocks take tens of
milliseconds of sustained load to settle. Non-headline entries then time
max(5, steps/10) launches. Each entry also gives `launch_us_median_min_max`
from one event pair per launch (a separate pass), and `warm_kernel_us`: the
same calls on a single input copy, resident in the MALL where it fits
(reported beside the cold numbers, never as `value`). `mfma_ceiling` is what
the matrix cores sustain on this device for the GEMM's inner loop with no
memory traffic (random and all-zero E4M3 codes), and roofline
`frac_of_measured_mfma_ceiling` the headline kernel against it;
`hbm_read_ceiling` is what a plain streaming read (16-byte nontemporal loads,
the best of three shapes of workgroups and loads in flight) pulls from HBM on
this device, and each HBM-bound workload's `frac_of_measured_hbm_read` its
algorithmic bytes per second against that. `device` names the device the line
was measured on (architecture, compute units, HBM and L2 sizes).
"""
import argparse
import ctypes
import functools
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# published MI355X dense FP8 MFMA peak (256 CUs x 2.4 GHz x 8192 FLOP/clk/CU = 5033 at the nominal clock)
PEAK_FP8_TFLOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "moe_grouped_gemm_02_amd", "csrc", f)
                  for f in ("fg_kernel.hpp", "fg_e4m3.hpp", "fg_tiles.hpp", "fg_launch.hip", "fg_host.hip")]
PEAK_HBM_GBPS = 8000.0                          # HBM3E, 8 TB/s
MALL_BYTES = 256 << 20
HEADLINE = "dense_ffn"
ORDER = ["dense_small", "dense_skinny", "contiguous", "masked", "dense_ffn"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", "--workload-warmup-ms", dest="warmup_ms", type=float, default=400.0,
                    help="minimum untimed warm-up of every measurement, the headline included "
                         "(the clocks take tens of milliseconds of sustained load to settle)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scales", choices=("fp32", "pow2"), default="fp32",
                    help="block scales of the headline run: fp32 (amax/448) or powers of two "
                         "on the _pow2 entry points")
    ap.add_argument("--no-pow2", action="store_true",
                    help="skip the per-workload measurements of the power-of-two path")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the headline's oracle baseline sample")
    ap.add_argument("--config-cpu-seconds", type=float, default=2.0,
                    help="target CPU time for each per-config oracle baseline")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="summarise rocprofv3 output under DIR (trace/, fetch/, write/ subfolders "
                         "from --kernel-trace --stats, --pmc FETCH_SIZE, --pmc WRITE_SIZE runs of "
                         "this script with --calibrate-copy-mb) and update profiles/traffic.json")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run device-to-device copies of this many MiB (a kernel of known "
                         "traffic, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# --------------------------------------------------------------------- inputs
@functools.lru_cache(maxsize=1)
def _workload(name):
    """Seeded fp32 inputs of one workload (kept while consecutive measurements
    use it; one workload at a time)."""
    import workloads
    return workloads.make(name)


def gpu_operands(name, fg, torch, pow2=False, fused=False):
    """Seeded fp32 inputs (numpy) -> device -> E4M3 + scales by the library's
    quantisers (pow2: the power-of-two-scale quantisers). Returns a dict of
    device tensors and the sizes."""
    import numpy as np
    import workloads

    w = _workload(name)
    dev = torch.device("cuda", 0)
    a = torch.from_numpy(w["a"]).to(dev)
    b = torch.from_numpy(w["b"]).to(dev)
    if pow2:
        A, sa = fg.quant_act_1x128_pow2(a)
        B, sb = fg.quant_weight_128x128_pow2(b)
    else:
        A, sa = fg.quant_act_1x128(a)
        B, sb = fg.quant_weight_128x128(b)
    del a, b
    op = dict(kind=w["kind"], A=A, sa=sa, B=B, sb=sb, pow2=pow2, fused=fused)
    N, K = w["b"].shape[-2], w["b"].shape[-1]
    op.update(N=N, K=K, flop=workloads.useful_flop(w))
    if w["kind"] == "dense":
        M = w["a"].shape[0]
        op.update(M=M, G=1, rows_out=M)
        op["D"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    elif w["kind"] == "contiguous":
        M = w["a"].shape[0]
        op.update(M=M, G=w["b"].shape[0], rows_out=int((w["m_indices"] >= 0).sum()))
        op["m_indices"] = torch.from_numpy(w["m_indices"]).to(dev)
        op["D"] = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
        op["group_m"] = w["group_m"].tolist()
    else:
        G, M_max = w["a"].shape[0], w["a"].shape[1]
        mm = np.clip(w["masked_m"], 0, M_max)
        op.update(M=M_max, G=G, rows_out=int(mm.sum()))
        op["masked_m"] = torch.from_numpy(w["masked_m"]).to(dev)
        op["D"] = torch.zeros((G, M_max, N), dtype=torch.bfloat16, device=dev)
        op["masked_m_list"] = w["masked_m"].tolist()
    if fused:
        # outputs of the fused epilogue instead of D: codes [.., M, N/2], scales [.., N/256, M]
        lead = op["D"].shape[:-2]
        M_ = op["D"].shape[-2]
        op["Q"] = torch.zeros(lead + (M_, N // 2), dtype=torch.uint8, device=dev)
        op["sq"] = torch.zeros(lead + (N // 256, M_), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    return op


def algorithmic_bytes(op):
    """Operands read once + output written once, counting only experts and rows
    that have an output (A rows with work, B of experts with work, their scales,
    D rows written)."""
    N, K = op["N"], op["K"]
    KB = K // 128
    rows = op["rows_out"]
    if op["kind"] == "masked":
        experts = sum(1 for m in op["masked_m_list"] if m > 0)
    else:
        experts = op["G"]
    a = rows * K + rows * KB * 4
    b = experts * (N * K + (N // 128) * KB * 4)
    d = rows * N * 2
    if op.get("fused"):
        d = rows * (N // 2) + rows * (N // 256) * 4     # E4M3 activation + its 1x128 scales
    return a + b + d


def replicate(op, torch):
    """Copies of the operands so that consecutive steps do not hit the MALL."""
    keys = ["A", "sa", "B", "sb"]
    foot = sum(op[k].numel() * op[k].element_size() for k in keys)
    n = max(1, min(16, math.ceil(2 * MALL_BYTES / max(foot, 1))))
    copies = [{k: op[k] for k in keys}]
    for _ in range(n - 1):
        copies.append({k: op[k].clone() for k in keys})
    torch.cuda.synchronize()
    return copies


def make_step(op, copies, fg, torch):
    """Pre-marshalled C-ABI call per copy: the timed loop pays only the ctypes
    call itself."""
    L = fg.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    D = P(op["D"])
    M, N, K, G = op["M"], op["N"], op["K"], op["G"]
    sfx = "_pow2" if op["pow2"] else ""
    calls = []
    for c in copies:
        if op["fused"]:
            Q, sq, null = P(op["Q"]), P(op["sq"]), ctypes.c_void_p(0)
            scales = 1 if op["pow2"] else 0
            if op["kind"] == "dense":
                args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), Q, sq, null, M, N, K, scales, stream)
                calls.append((L.fg_gemm_fp8_nt_swiglu_quant, args))
            elif op["kind"] == "contiguous":
                args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), Q, sq, null, P(op["m_indices"]),
                        M, N, K, G, scales, stream)
                calls.append((L.fg_grouped_contiguous_swiglu_quant, args))
            else:
                args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), Q, sq, null, P(op["masked_m"]),
                        G, M, N, K, scales, stream)
                calls.append((L.fg_grouped_masked_swiglu_quant, args))
            continue
        if op["kind"] == "dense":
            args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), D, M, N, K, stream)
            calls.append((getattr(L, "fg_gemm_fp8_nt" + sfx), args))
        elif op["kind"] == "contiguous":
            args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), D, P(op["m_indices"]),
                    M, N, K, G, stream)
            calls.append((getattr(L, "fg_grouped_contiguous" + sfx), args))
        else:
            args = (P(c["A"]), P(c["sa"]), P(c["B"]), P(c["sb"]), D, P(op["masked_m"]),
                    G, M, N, K, stream)
            calls.append((getattr(L, "fg_grouped_masked" + sfx), args))

    def step(i):
        f, a = calls[i % len(calls)]
        rc = f(*a)
        if rc != 0:
            raise RuntimeError(f"library call failed: {fg.strerror(rc)}")
    return step


def timed_steps(step, steps, warmup, torch, warmup_ms=0.0):
    """(wall ms, HIP-event ms) per step over `steps` steps after `warmup`
    untimed steps, extended until at least `warmup_ms` of them have run (the
    GPU's clocks take tens of milliseconds of sustained load to settle: the
    first launches after setup run up to ~35% slower)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    done = warmup
    if warmup_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warmup_ms:
            for _ in range(max(1, warmup)):
                step(done)
                done += 1
            torch.cuda.synchronize()
    warmup = done
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps


def time_workload(name, steps, warmup, fg, torch, pow2=False, fused=False, warm=False, warmup_ms=0.0):
    """Cold timing: steps rotate over input copies that together exceed the
    MALL, so every launch reads its operands from HBM. warm=True also times the
    same calls on one copy (operands resident in the 256 MB MALL when they fit)."""
    op = gpu_operands(name, fg, torch, pow2, fused)
    copies = replicate(op, torch)
    step = make_step(op, copies, fg, torch)
    wall_ms, kern_ms = timed_steps(step, steps, warmup, torch, warmup_ms)
    warm_ms = None
    if warm:
        warm_ms = timed_steps(make_step(op, copies[:1], fg, torch), steps, warmup, torch)[1]
    # per-launch spread: a separate pass with one event pair per launch (the
    # averaged timing above records no events between launches)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(warmup + steps + i)
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) for a, b in evs)
    layout = {"dense": 0, "contiguous": 1, "masked": 2}[op["kind"]]
    if fused:
        layout |= fg.SELECT_SWIGLU_QUANT
    bm, bn = fg.select_config(op["M"], op["N"], op["K"], op["G"], layout)
    grid = fg.select_grid(op["M"], op["N"], op["K"], op["G"], layout)
    res = dict(op=op, copies=len(copies), wall_ms=wall_ms, kern_ms=kern_ms, warm_ms=warm_ms,
               launch_ms=(per_launch[len(per_launch) // 2], per_launch[0], per_launch[-1]),
               tile=f"{bm}x{bn}", grid=grid, bytes=algorithmic_bytes(op))
    del copies
    return res


def summarize(r):
    op = r["op"]
    tflops = op["flop"] / (r["wall_ms"] * 1e-3) / 1e12
    kt = op["flop"] / (r["kern_ms"] * 1e-3) / 1e12
    out = dict(M=op["M"], N=op["N"], K=op["K"], G=op["G"], rows_out=op["rows_out"],
               tile=r["tile"], grid=r["grid"], us_per_call=round(r["wall_ms"] * 1e3, 2),
               kernel_us=round(r["kern_ms"] * 1e3, 2), tflops=round(tflops, 1),
               pct_fp8_peak=round(100 * kt / PEAK_FP8_TFLOPS, 2),
               hbm_gbps=round(r["bytes"] / (r["kern_ms"] * 1e-3) / 1e9, 1),
               input_copies=r["copies"],
               launch_us_median_min_max=[round(x * 1e3, 2) for x in r["launch_ms"]])
    if r.get("warm_ms"):
        out.update(warm_kernel_us=round(r["warm_ms"] * 1e3, 2),
                   warm_pct_fp8_peak=round(100 * op["flop"] / (r["warm_ms"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 2))
    return out


# --------------------------------------------------------------- CPU baseline
# What the oracle baseline runs per workload: None = the whole problem (one
# oracle call takes at most a few seconds); for the large dense FFN GEMM a
# block of the output -- its first `rows` rows and `cols` columns -- over the
# full K, since one call on the whole problem would take minutes of CPU time.
CPU_SAMPLES = {"dense_small": None, "dense_skinny": None, "contiguous": None, "masked": None,
               "dense_ffn": dict(rows=1024, cols=1792)}


def oracle_case(name):
    """(call, useful FLOP of one call, description) for one oracle call on the
    workload or its sample. Inputs are quantised by the oracle before any
    timing (chunked over threads; the same codes as the serial quantisers)."""
    import oracle
    from oracle.parallel import quantize_act_1x128_par, quantize_weight_128x128_par

    w = _workload(name)
    samp = CPU_SAMPLES[name]
    if w["kind"] == "dense":
        a, b = w["a"], w["b"]
        M, N, K = a.shape[0], b.shape[0], a.shape[1]
        desc = f"whole problem {M}x{N}x{K}"
        if samp:
            a, b = a[:samp["rows"]], b[:samp["cols"]]
            desc = (f"output rows 0..{a.shape[0] - 1} x columns 0..{b.shape[0] - 1} of the {M}x{N} output, "
                    f"full K = {K}")
        A, sa = quantize_act_1x128_par(a)
        B, sb = quantize_weight_128x128_par(b)
        flop = 2.0 * A.shape[0] * B.shape[0] * K
        return (lambda: oracle.ref_dense(A, sa, B, sb)), flop, desc
    import workloads
    flop = workloads.useful_flop(w)
    A, sa = quantize_act_1x128_par(w["a"])
    B, sb = quantize_weight_128x128_par(w["b"])
    if w["kind"] == "contiguous":
        mi = w["m_indices"]
        desc = f"whole problem: {B.shape[0]} experts, {int((mi >= 0).sum())} rows, N={B.shape[1]}, K={A.shape[1]}"
        return (lambda: oracle.ref_contiguous(A, sa, B, sb, mi)), flop, desc
    mm = w["masked_m"]
    desc = (f"whole problem: {B.shape[0]} experts, M_max={A.shape[1]}, {int(mm.sum())} valid rows, "
            f"N={B.shape[1]}, K={A.shape[2]}")
    return (lambda: oracle.ref_masked(A, sa, B, sb, mm)), flop, desc


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return len(os.sched_getaffinity(0))


def cpu_baseline(name, target_s):
    """The oracle as it stands (dequantise to fp64 + one fp64 numpy GEMM per
    expert), timed on this host with time.perf_counter: repeated calls until
    target_s seconds (at least one call, at most 500)."""
    call, flop, desc = oracle_case(name)
    reps, spent = 0, 0.0
    while reps == 0 or (spent < target_s and reps < 500):
        t0 = time.perf_counter()
        call()
        spent += time.perf_counter() - t0
        reps += 1
    return {"value": round(flop * reps / spent / 1e12, 5), "unit": "TFLOP/s", "cores": oracle_threads(),
            "kind": "oracle", "seconds_per_call": round(spent / reps, 4),
            "sample": f"{name}: {desc}; {reps} call(s), {spent:.1f} s; dequantise + fp64 numpy GEMM; "
                      f"host cpus {len(os.sched_getaffinity(0))}"}


def mfma_ceiling(torch, warmup_ms):
    """What the matrix cores sustain on this device for the GEMM's inner loop
    with no memory traffic (libfg_ceiling.so, a helper built beside the
    library): 8 waves per CU, each issuing its 64x128 tile's 32 E4M3 MFMAs per
    K-block on fragments held in registers -- with the fp32-scale promotion (C
    = 0, 4 FMAs per MFMA), with power-of-two accumulation, and with the
    promotion on all-zero codes. Random codes draw the matrix cores' real
    power; the gap to the zero-code figure is the power-limited clock."""
    import numpy as np
    L = ctypes.CDLL(os.path.join(ROOT, "moe_grouped_gemm_02_amd", "libfg_ceiling.so"))
    L.fgc_src_words.restype = ctypes.c_int
    L.fgc_flop_per_workgroup_iteration.restype = ctypes.c_double
    L.fgc_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p]
    L.fgc_mfma_loop.restype = ctypes.c_int
    n = L.fgc_src_words()
    codes = np.random.default_rng(11).integers(0, 256, size=4 * n, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] ^= 1          # finite codes only (no 0x7f / 0xff NaN)
    src = torch.from_numpy(codes.view(np.int32).copy()).cuda()
    zeros = torch.zeros_like(src)
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flop = L.fgc_flop_per_workgroup_iteration() * iters * grid
    res = {}
    for name, mode, data in (("random_fp32_promotion", 0, src), ("random_pow2", 1, src),
                             ("zeros_fp32_promotion", 0, zeros)):
        def launch():
            if L.fgc_mfma_loop(ctypes.c_void_p(data.data_ptr()), ctypes.c_void_p(out.data_ptr()), mode, grid,
                               iters, stream) != 0:
                raise RuntimeError("fgc_mfma_loop failed")
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warmup_ms:
            launch()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            launch()
        e1.record()
        torch.cuda.synchronize()
        tf = flop * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
    res["workgroups"] = grid
    return res


def hbm_read_ceiling(torch, warmup_ms, mb=1024):
    """HBM bytes per second a plain streaming read sustains on this device
    (libfg_ceiling.so's fgc_stream_read over a buffer 4x the MALL's size): the
    best of three shapes -- 1 workgroup of 512 threads per CU with 4 loads in
    flight per thread, 2 with 8, 8 with 8 (more bytes in flight is not faster:
    the grid-stride sweep keeps the concurrent reads compact when fewer are in
    flight)."""
    L = ctypes.CDLL(os.path.join(ROOT, "moe_grouped_gemm_02_amd", "libfg_ceiling.so"))
    L.fgc_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    L.fgc_stream_read.restype = ctypes.c_int
    nbytes = mb << 20
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 8 * 512, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for wg_per_cu, inflight in ((1, 4), (2, 8), (8, 8)):
        grid = cus * wg_per_cu

        def launch():
            if L.fgc_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()), grid,
                                 inflight, stream) != 0:
                raise RuntimeError("fgc_stream_read failed")
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < warmup_ms / 2:
            launch()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            launch()
        e1.record()
        torch.cuda.synchronize()
        gbs = nbytes * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        if best is None or gbs > best["gb_s"]:
            best = {"gb_s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBPS, 4), "bytes": nbytes,
                    "workgroups_per_cu": wg_per_cu, "loads_in_flight_per_thread": inflight}
    del buf, out
    torch.cuda.empty_cache()
    return best


def device_info(torch):
    """What the numbers were measured on: the current device's name,
    architecture, compute units, HBM and L2 sizes."""
    pr = torch.cuda.get_device_properties(torch.cuda.current_device())
    return {"name": pr.name, "arch": pr.gcnArchName, "compute_units": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2 ** 30, 1), "l2_bytes": pr.L2_cache_size}


def kernel_source_hash():
    """Hash of what defines the kernels: the kernel template with comments and
    whitespace removed, and the tile-configuration lines that instantiate it.
    Editing a comment or the host-side tile choice does not detach the
    committed counters from the code they were taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        if f.endswith(".hip"):
            text = "\n".join(re.findall(r"using Cfg\d+ = fg::TileCfg<[^>]*>;", text))
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the kernel sources as they are now; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    entry = t.get("workloads", {}).get(workload)
    return entry.get("hbm_bytes_per_launch") if entry else None


def copy_calibration(mb, torch):
    """Device-to-device copies of a known size: FETCH_SIZE / WRITE_SIZE of
    these dispatches give the counters' scale (bytes per counted KiB)."""
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    evict = torch.empty_like(src)
    src.fill_(1)
    evict.fill_(2)     # pushes src out of the 256 MB last-level cache
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, evict
    torch.cuda.empty_cache()
    return n


def summarize_profile(root, workload, copy_mb):
    """Kernel-trace statistics and HBM traffic of the GEMM kernel from rocprofv3
    CSV output. The FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) are
    scaled by the ratio of known to counted bytes of the calibration copy."""
    import csv
    import glob

    def rows(sub, name):
        out = []
        for f in glob.glob(os.path.join(root, sub, "**", name), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    stats = rows("trace", "*kernel_stats.csv")
    gemm = [r for r in stats if "fp8_bs_gemm" in r["Name"]]
    res = {"workload": workload, "kernels": {}}
    for r in gemm:
        res["kernels"][r["Name"]] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                                     "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}

    def counter(sub, cname):
        vals = {}
        for r in rows(sub, "*counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    known_kib = copy_mb * 1024.0

    def copy_factor(vals):
        best = None
        for name, v in vals.items():
            if "fp8_bs_gemm" in name or "quant_" in name:
                continue
            m = max(v)   # the copy is the largest non-GEMM dispatch
            if best is None or m > best:
                best = m
        return known_kib / best if best else None

    ff, wf = copy_factor(fetch), copy_factor(write)
    gk = [k for k in fetch if "fp8_bs_gemm" in k]
    if gk and ff and wf:
        k = gk[0]
        f_kib = sum(fetch[k]) / len(fetch[k])
        w_kib = sum(write.get(k, [0.0])) / max(1, len(write.get(k, [])))
        res.update(kernel=k, fetch_kib=f_kib, write_kib=w_kib, fetch_scale=ff, write_scale=wf,
                   hbm_bytes_per_launch=(f_kib * ff + w_kib * wf) * 1024.0)
    print(json.dumps(res, indent=1))
    if "hbm_bytes_per_launch" in res:
        try:
            with open(TRAFFIC_FILE) as fh:
                t = json.load(fh)
        except (OSError, ValueError):
            t = {}
        if t.get("source_hash") != kernel_source_hash():
            t = {"source_hash": kernel_source_hash(), "workloads": {}}
        t["workloads"][workload] = {"kernel": res["kernel"],
                                    "hbm_bytes_per_launch": round(res["hbm_bytes_per_launch"]),
                                    "fetch_kib": round(res["fetch_kib"], 1),
                                    "write_kib": round(res["write_kib"], 1),
                                    "fetch_scale": round(res["fetch_scale"], 4),
                                    "write_scale": round(res["write_scale"], 4)}
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(t, fh, indent=1)
    return res


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload, args.calibrate_copy_mb or 256)
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(nothing here uses a second GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_grouped_gemm_02_amd as fg

    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr)
        sys.exit(1)
    fg.lib()
    head_pow2 = args.scales == "pow2"
    full = not args.headline_only
    sub_steps = max(5, args.steps // 10)
    per, per_pow2, fused, cpu_cfg = {}, {}, {}, {}
    head = None
    # the headline first, then the other workloads one at a time (each
    # workload's inputs are generated once for its GPU and CPU measurements)
    for name in [args.workload] + [n for n in ORDER if n != args.workload]:
        is_head = name == args.workload
        if is_head:
            # (no warm launches in --headline-only runs: a profiler's average for
            # the kernel must be the cold launches' alone)
            head = time_workload(name, args.steps, args.warmup, fg, torch, head_pow2, warm=full,
                                 warmup_ms=args.warmup_ms)
            per[name] = summarize(head)
        elif full:
            r = time_workload(name, sub_steps, args.warmup, fg, torch, head_pow2, warm=True,
                              warmup_ms=args.warmup_ms)
            per[name] = summarize(r)
            del r
        torch.cuda.empty_cache()
        if full and not args.no_pow2:
            r = time_workload(name, sub_steps, args.warmup, fg, torch, not head_pow2, warmup_ms=args.warmup_ms)
            per_pow2[name] = summarize(r)
            del r
            torch.cuda.empty_cache()
        if full and name in ("contiguous", "masked"):
            r = time_workload(name, sub_steps, args.warmup, fg, torch, False, True, warmup_ms=args.warmup_ms)
            fused[name] = summarize(r)
            del r
            torch.cuda.empty_cache()
        if not args.no_cpu_baseline and (is_head or full):
            cpu_cfg[name] = cpu_baseline(name, args.cpu_seconds if is_head else args.config_cpu_seconds)
    _workload.cache_clear()

    hs = per[args.workload]
    op = head["op"]
    value = op["flop"] / (head["wall_ms"] * 1e-3) / 1e12
    kern_s = head["kern_ms"] * 1e-3
    achieved_gbps = head["bytes"] / kern_s / 1e9
    achieved_tflops = op["flop"] / kern_s / 1e12
    # arithmetic intensity below the FP8 ridge point -> HBM is the roof
    ridge = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    hbm_bound = op["flop"] / head["bytes"] < ridge
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_FP8_TFLOPS, 4), "traffic": None}
    roof.update(kernel_us=hs["kernel_us"], algorithmic_bytes=head["bytes"], flop=op["flop"],
                hbm_frac=round(achieved_gbps / PEAK_HBM_GBPS, 4))
    del head
    torch.cuda.empty_cache()

    if args.calibrate_copy_mb:
        copy_calibration(args.calibrate_copy_mb, torch)
    roof["traffic"] = measured_traffic(args.workload) if not head_pow2 else None
    ceiling = hbm_ceiling = None
    if full:
        ceiling = mfma_ceiling(torch, args.warmup_ms)
        hbm_ceiling = hbm_read_ceiling(torch, args.warmup_ms)
        if not hbm_bound:
            key = "random_pow2" if head_pow2 else "random_fp32_promotion"
            roof["frac_of_measured_mfma_ceiling"] = round(achieved_tflops / ceiling[key]["tflops"], 4)
        else:
            roof["frac_of_measured_hbm_read"] = round(achieved_gbps / hbm_ceiling["gb_s"], 4)
        for table in (per, per_pow2):
            for e in table.values():
                # FLOP per algorithmic byte below the ridge point: HBM is the roof
                if e["hbm_gbps"] > 0 and e["tflops"] * 1e3 / e["hbm_gbps"] < ridge:
                    e["frac_of_measured_hbm_read"] = round(e["hbm_gbps"] / hbm_ceiling["gb_s"], 4)

    line = {
        "metric": "FP8 TFLOPS (dense + grouped MoE) and % of MI355X dense FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_ms_floor": args.warmup_ms,
        "ms_per_step": round(hs["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload, "layout": op["kind"], "M": op["M"], "N": op["N"],
                   "K": op["K"], "G": op["G"],
                   "scales": "1x128 (A), 128x128 (B), " + ("powers of two (E8M0 on the matrix core)"
                                                          if head_pow2 else "fp32"),
                   "out": "bf16", "tile": hs["tile"], "input_copies": hs["input_copies"],
                   "pct_fp8_peak": round(100 * value / PEAK_FP8_TFLOPS, 2)},
        "roofline": roof,
        "device": device_info(torch),
        "mfma_ceiling": ceiling,
        "hbm_read_ceiling": hbm_ceiling,
        "cpu_baseline": cpu_cfg.get(args.workload),
        "cpu_baseline_per_config": cpu_cfg or None,
        "per_workload": per,
        ("per_workload_fp32" if head_pow2 else "per_workload_pow2"): per_pow2 or None,
        "moe_swiglu_quant": fused or None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
