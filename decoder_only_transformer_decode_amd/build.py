"""Builds libdtd.so (HIP kernels + host engine) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdtd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dtd_kernels.hip", "dtd_persistent.hip", "dtd_sample.hip", "dtd_engine.cpp", "dtd_sched.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops (v_pk_*_f32).
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
         "-I" + os.path.join(ROOT, "include")]


def build(verbose: bool = True, extra=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    # the .cpp file holds host code only but includes the HIP runtime; compile it as HIP too
    cmd = [HIPCC] + FLAGS + (extra or []) + ["-x", "hip"] + srcs + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(extra=sys.argv[1:])
