"""Builds libdrla.so (HIP kernels + C ABI) and libdrla_peaks.so (the
attainable-peak microbenchmarks the benchmark prices its roofline with) for
gfx950 with hipcc, in-tree under delta_rule_linear_chunked_amd/_build/."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD, "libdrla.so")
PEAKS_LIB = os.path.join(BUILD, "libdrla_peaks.so")
PEAKS_SRC = os.path.join(CSRC, "drla_peaks.hip")

ARCH = "gfx950"
# Packed fp32 vector ops are kept off: hipcc would otherwise form
# v_pk_{add,mul,fma}_f32 from float2 code.  MFMA accumulators are kept in
# VGPRs: the scans scale and convert them with vector ALU code every chunk,
# which in the AGPR form costs a copy in and out of the AGPR file.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return [os.path.join(CSRC, f) for f in
            ("drla_prep.hip", "drla_scan.hip", "drla_scan_lds.hip", "drla_hscan.hip", "drla_decode.hip",
             "drla_launch.hip",
             "drla_api.cpp")]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source and link libdrla.so and libdrla_peaks.so.
    Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    cmds, objs = [], []
    for src in sources() + [PEAKS_SRC]:
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [cc, *HIPFLAGS, *extra, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, "-x", "hip", *HIPFLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        cmds.append(cmd)
        objs.append(obj)
    # one compiler process per source, in parallel
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for f in [ex.submit(subprocess.check_call, c) for c in cmds]:
            f.result()
    for lib, parts in ((LIB, objs[:-1]), (PEAKS_LIB, objs[-1:])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *parts]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
