"""Build step for the native library ``libmpdt.so`` (gfx950 HIP kernels and
the C ABI) and for the CPU checker under ``oracle/``.

``python -m mixed_precision_dense_tiled_amd.build`` compiles both in-tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmpdt.so")
PROBE_LIB = os.path.join(PKG, "libmpdt_probes.so")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ORACLE_LIB = os.path.join(ORACLE_DIR, "liboracle.so")

HIP_SOURCES = ["abi.hip", "gemm.hip", "gemv_w8a8.hip", "quant.hip"]

# Packed FP32 instructions are switched off for all device code (-packed-fp32-ops).
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _run(cmd, cwd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, cwd=cwd, check=True)


def build_library(extra_flags=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, *extra_flags, *srcs, "-o", tmp], cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


CLOCK_LIB = os.path.join(PKG, "libmpdt_clock.so")


def build_clock_library(extra_flags=()) -> str:
    """The same kernels with per-workgroup clock stamps (bench.py reads the
    shader clock of the timed GEMM from it; never used for results)."""
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    tmp = CLOCK_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-DMPDT_CLOCK_STAMPS", *extra_flags, *srcs, "-o", tmp], cwd=CSRC)
    os.replace(tmp, CLOCK_LIB)
    return CLOCK_LIB


def build_probes(extra_flags=()) -> str:
    """Layout-probe kernels used by the GPU tests (not part of the C ABI)."""
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, *extra_flags, os.path.join(CSRC, "probes.hip"), "-o", tmp],
         cwd=CSRC)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_oracle() -> str:
    cc = os.environ.get("CC") or "gcc"
    tmp = ORACLE_LIB + ".tmp"
    _run([cc, "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra", os.path.join(ORACLE_DIR, "oracle.c"), "-o", tmp, "-lm"],
         cwd=ORACLE_DIR)
    os.replace(tmp, ORACLE_LIB)
    return ORACLE_LIB


def build_all():
    build_oracle()
    build_library()
    build_probes()
    build_clock_library()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
