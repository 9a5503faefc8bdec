"""Build libfp4.so (the HIP library behind include/fp4.h) in-tree with hipcc for gfx950.

    python -m bit_floating_point_amd.build          # compile every source, link
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quant.hip", "gemm_w4a16.hip", "gemm_w4a4.hip", "gemm_lut.hip", "gemm_f8f6.hip", "search.hip", "fp4_api.cpp"]

# -ffp-contract=off: no silent a*b+c fusion, so every rounding is the one written
# (fused multiply-adds are explicit); packed-fp32 instructions are disabled.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


# The persistent GEMM kernels count their outstanding loads in their waits; a register
# spill would add scratch memory operations to those counts, so they must not spill.
NO_SPILL = ("gemm_w4a4.hip", "gemm_lut.hip")


def _check_no_spill(src: str, remarks: str) -> None:
    name = None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size != 0:
                raise RuntimeError(f"{src}: kernel {name} spills ({size} bytes/lane of scratch)")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SPILL else []
    cmd = [HIPCC] + CFLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if extra:
        _check_no_spill(src, r.stderr)
    return obj


# Measurement helper of bench.py (the streaming-read ceiling), a library of its own: it is
# not part of libfp4 or of include/fp4.h.
BENCH_SOURCE = "bench_read.hip"
BENCH_LIB = os.path.join(HERE, "libfp4_bench.so")


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES + [BENCH_SOURCE]))
    bench_obj = objs.pop()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", BENCH_LIB + ".tmp", bench_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed (bench helper):\n" + r.stderr)
    os.replace(BENCH_LIB + ".tmp", BENCH_LIB)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
