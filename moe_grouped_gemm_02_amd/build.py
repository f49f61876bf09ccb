"""Ahead-of-time build of the HIP library (libfg.so) for gfx950.

Run ``python -m moe_grouped_gemm_02_amd.build`` (or call ``build()``). The
shared object is written next to this file so that it travels with the source
tree; nothing is installed elsewhere. The GEMM kernels of each layout and scale
kind are compiled as separate objects (fg_launch.hip with FG_LAUNCH_PART =
2 * layout + pow2), in parallel, then linked with the host and quantiser code.

libfg_ceiling.so (fg_ceiling.hip) is a benchmark helper that bench.py loads to
measure the matrix cores' ceiling on this device; the library does not use it.

A second library, libfg_testing.so, links the same kernel objects with the
host code built with FG_TESTING: it adds a per-thread tile override
(fgt_force_tile) that the test suite uses to run every compiled tile. The
product library carries no such state.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfg.so")
TESTING_LIB = os.path.join(HERE, "libfg_testing.so")
CEILING_LIB = os.path.join(HERE, "libfg_ceiling.so")
LAUNCH_PARTS = 6   # {dense, contiguous, masked} x {fp32 scales, power-of-two scales}
# (object name, source, extra flags)
UNITS = [("fg_host", "fg_host.hip", []), ("fg_host_testing", "fg_host.hip", ["-DFG_TESTING"]),
         ("fg_quant", "fg_quant.hip", []), ("fg_ceiling", "fg_ceiling.hip", [])] + [
    (f"fg_launch_{i}", "fg_launch.hip", [f"-DFG_LAUNCH_PART={i}"]) for i in range(LAUNCH_PARTS)]
HEADERS = ["fg_kernel.hpp", "fg_e4m3.hpp", "fg_tiles.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU forms stay off: plain v_fma_f32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results straight into VGPRs: the promotion FMA reads them there
    # (an AGPR destination would cost one v_accvgpr_read per element)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def build(verbose=False, jobs=None):
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(UNITS), max(1, len(os.sched_getaffinity(0))), 16)
    pending = list(UNITS)
    running = []
    objs = []
    failed = []
    while pending or running:
        while pending and len(running) < jobs:
            name, src, extra = pending.pop(0)
            obj = os.path.join(OBJ, name + ".o")
            cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                   text=True)))
            objs.append(obj)
        name, proc = running.pop(0)
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(name)
    if failed:
        raise RuntimeError("hipcc failed building " + ", ".join(failed))
    host = os.path.join(OBJ, "fg_host.o")
    host_t = os.path.join(OBJ, "fg_host_testing.o")
    ceiling = os.path.join(OBJ, "fg_ceiling.o")
    common = [o for o in objs if o not in (host, host_t, ceiling)]
    for out, link in ((LIB, [host, *common]), (TESTING_LIB, [host_t, *common]), (CEILING_LIB, [ceiling])):
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed linking " + os.path.basename(out))
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
