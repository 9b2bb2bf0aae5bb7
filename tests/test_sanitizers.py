"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

  * The oracle (oracle/oracle.c) is built with gcc -fsanitize=address,undefined
    (every report fatal) and the whole CPU suite except the ABI tests runs
    against that build in a child pytest process with gcc's sanitizer runtimes
    preloaded.
  * The C ABI's host code (csrc/abi.hip: argument validation, byte spans,
    overflow and overlap arithmetic) is built host-only with clang's
    sanitizers; the kernel launchers are replaced by stubs that abort if ever
    reached -- on a machine without a GPU every valid call stops at the device
    check, so none is.  The ABI and binding tests run against that build with
    clang's runtime preloaded.

A sanitizer report aborts the child, which fails the test.  Skipped where a
GPU is visible (valid calls would reach the stubs there)."""
import os
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "csrc")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-only builds; a GPU is visible")

STUBS = """#include <cstdlib>
#include "kernels.hpp"
namespace mpdt {
hipError_t launch_gemm(Kind, const GemmArgs&, bool, hipStream_t) { std::abort(); }
hipError_t launch_fp8(const GemmArgs&, bool, hipStream_t) { std::abort(); }
hipError_t launch_gemm_epi(Kind, const GemmArgs&, bool, hipStream_t) { std::abort(); }
hipError_t launch_gemv_w8a8(const GemvArgs&, bool, hipStream_t) { std::abort(); }
hipError_t launch_gemm_w8a8(const W8A8Args&, bool, hipStream_t) { std::abort(); }
hipError_t launch_quantize_i8_rows(const QuantI8Args&, hipStream_t) { std::abort(); }
hipError_t launch_quantize_fp8_blocks(const QuantFp8Args&, hipStream_t) { std::abort(); }
}  // namespace mpdt
"""

CHECK_LOADED = """
import os, sys
import mixed_precision_dense_tiled_amd as mp, oracle
want = os.environ.get("MPDT_LIB_PATH") or os.environ.get("MPDT_ORACLE_LIB")
got = mp.lib_path() if os.environ.get("MPDT_LIB_PATH") else oracle.LIB_PATH
sys.exit(0 if got == want else 3)
"""


def _child(env_extra, args, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", OMP_NUM_THREADS="4",
               PYTHONPATH=ROOT, **env_extra)
    chk = subprocess.run([sys.executable, "-c", CHECK_LOADED], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert chk.returncode == 0, f"the sanitized build was not the one loaded: {chk.stderr[-2000:]}"
    out = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert out.returncode == 0, out.stdout[-4000:] + out.stderr[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    rt = [subprocess.run([gcc, f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
          for n in ("libasan.so", "libubsan.so")]
    tests = [os.path.join("tests", f) for f in sorted(os.listdir(os.path.join(ROOT, "tests")))
             if f.startswith("test_oracle_")]
    _child({"MPDT_ORACLE_LIB": lib, "LD_PRELOAD": " ".join(rt)}, tests, tmp_path)


def test_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    stubs = tmp_path / "stubs.hip"
    stubs.write_text(STUBS)
    lib = str(tmp_path / "libmpdt_san.so")
    # host-only build: every sanitizer flag is for the host compiler
    subprocess.run([hipcc, "--offload-arch=gfx950", "--offload-host-only", "-O1", "-g", "-fPIC", "-std=c++17",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-shared",
                    os.path.join(CSRC, "abi.hip"), str(stubs), "-o", lib], check=True)
    rt = subprocess.run([hipcc, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        import glob
        found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not found:
            pytest.skip("clang's ASan runtime not found")
        rt = found[0]
    _child({"MPDT_LIB_PATH": lib, "LD_PRELOAD": rt},
           ["tests/test_abi.py", "tests/test_binding_shapes.py"], tmp_path)
