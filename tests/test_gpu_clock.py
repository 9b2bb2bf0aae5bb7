"""The instrumented build (libmpdt_clock.so) that bench.py reads the GEMM's
shader clock from must compute exactly what the product library computes,
and its stamps must be ordered and give a plausible clock."""
import ctypes
import os

import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
from helpers import dev
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

PKG = os.path.dirname(mp.__file__)


def test_clock_library_same_bits_and_sane_stamps(gpu_ok):
    L = ctypes.CDLL(os.path.join(PKG, "libmpdt_clock.so"))
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.gemm_bf16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    L.gemm_bf16.restype = ctypes.c_int
    L.mpdt_clock_stamps.argtypes = [vp, ctypes.c_int]
    L.mpdt_clock_stamps.restype = ctypes.c_int
    M, N, K = 512, 768, 1024
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16", seeds=(41, 42, 43))
    tA, tB, tC = dev(A), dev(B), dev(C)
    ref = mp.gemm_bf16(tA, tB, tC)
    out = torch.empty_like(ref)
    s = torch.cuda.current_stream().cuda_stream
    assert L.gemm_bf16(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N,
                       out.data_ptr(), N, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    wgs = (M // 256) * (N // 256)
    buf = np.zeros(wgs * 6, dtype=np.uint64)
    assert L.mpdt_clock_stamps(buf.ctypes.data, wgs) == 0
    q = buf.reshape(wgs, 6).astype(np.float64)
    assert (q[:, 0] < q[:, 1]).all() and (q[:, 1] < q[:, 2]).all()
    assert (q[:, 3] <= q[:, 4]).all() and (q[:, 4] <= q[:, 5]).all() and (q[:, 5] > q[:, 3]).all()
    ghz = (q[:, 2] - q[:, 0]) / ((q[:, 5] - q[:, 3]) / 100e6) / 1e9
    assert ((ghz > 0.3) & (ghz < 3.5)).all(), ghz
