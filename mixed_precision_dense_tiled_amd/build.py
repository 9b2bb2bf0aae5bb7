"""Build step for the native library ``libmpdt.so`` (gfx950 HIP kernels and
the C ABI) and for the CPU checker under ``oracle/``.

``python -m mixed_precision_dense_tiled_amd.build`` compiles both in-tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmpdt.so")
PROBE_LIB = os.path.join(PKG, "libmpdt_probes.so")
ORACLE_DIR = os.path.join(ROOT, "oracle")
ORACLE_LIB = os.path.join(ORACLE_DIR, "liboracle.so")

HIP_SOURCES = ["abi.hip", "gemm.hip", "gemm_epi.hip", "gemm_fp8.hip", "gemm_fp8_general.hip", "gemv_w8a8.hip", "quant.hip"]

# Per-source device-compiler options.  The one-wave FP8 GEMM rescales its MFMA
# block sums with FP32 FMAs every K tile; VALU instructions cannot read AGPRs,
# so its MFMAs are built in the form that writes VGPRs.
SOURCE_FLAGS = {"gemm_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# Packed FP32 instructions are switched off for all device code (-packed-fp32-ops).
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
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


def _build_libs(specs):
    """specs: (out, sources, extra_flags) per shared library.  Every source of
    every library is compiled to its own object in one parallel pool (each
    with its own options), then each library is linked."""
    cmds, links = [], []
    for out, sources, extra_flags in specs:
        objdir = os.path.join(CSRC, "_build", os.path.basename(out))
        os.makedirs(objdir, exist_ok=True)
        objs = [os.path.join(objdir, s + ".o") for s in sources]
        cmds += [[hipcc(), *HIP_FLAGS, *SOURCE_FLAGS.get(s, []), *extra_flags, "-c",
                  os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
        links.append((out, objs))
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, CSRC), cmds))
    for out, objs in links:
        tmp = out + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], cwd=CSRC)
        os.replace(tmp, out)
    return [out for out, _ in links]


def _link(out: str, sources, extra_flags=()) -> str:
    return _build_libs([(out, sources, extra_flags)])[0]


def build_library(extra_flags=()) -> str:
    return _link(LIB, HIP_SOURCES, extra_flags)


CLOCK_LIB = os.path.join(PKG, "libmpdt_clock.so")


def build_clock_library(extra_flags=()) -> str:
    """The same kernels with per-workgroup clock stamps (bench.py reads the
    shader clock of the timed GEMM from it; never used for results)."""
    return _link(CLOCK_LIB, HIP_SOURCES, ("-DMPDT_CLOCK_STAMPS", *extra_flags))


def build_probes(extra_flags=()) -> str:
    """Layout-probe kernels used by the GPU tests (not part of the C ABI)."""
    return _link(PROBE_LIB, ["probes.hip"], extra_flags)


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
    # the three HIP libraries in one compile pool
    _build_libs([(LIB, HIP_SOURCES, ()), (PROBE_LIB, ["probes.hip"], ()),
                 (CLOCK_LIB, HIP_SOURCES, ("-DMPDT_CLOCK_STAMPS",))])


if __name__ == "__main__":
    build_all()
    sys.exit(0)
