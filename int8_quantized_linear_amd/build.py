"""Builds libql.so (the HIP library) and libqlprobe.so (the benchmark's measurement
probes) in-tree with hipcc for gfx950.

    python int8_quantized_linear_amd/build.py

(Run as a script, not as ``-m``: importing the package would load the old library.)

Each source is compiled on its own (in parallel), then linked into one shared
library next to this file. Only gfx950 code objects are produced. Packed-fp32 VALU
instructions are disabled for all device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libql.so")
PROBE_OUT = os.path.join(HERE, "libqlprobe.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["capi.cpp", "quant.hip", "gemm_w8a8.hip", "gemm_w8a8_small.hip", "gemm_w8a8_mid.hip", "wonly.hip"]
PROBE_SOURCES = ["probes.hip"]
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    # -z defs: an undefined symbol (e.g. a kernel stub the compiler did not emit) fails the link
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libql.so and libqlprobe.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print("built", OUT, "and", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
