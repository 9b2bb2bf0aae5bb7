"""Parity at the workload's full sizes, through the same entry points and
launch configuration the benchmark times, on EVERY output element: the
oracle computes the whole reference R and the bound matrix S = sum |a * b|
(FP64, OpenMP over the host's cores), each element is held to its bound and
the relative Frobenius error is taken over the whole of D.

  * BF16 4096 x 4096 x 4096, N(0,1) inputs, FP32 C;
  * FP16 8191 x 8193 x 4099 with tight leading dimensions and C = 0 (and
    C = NULL giving identical bits);
  * FP8 E4M3 block-scaled 4096 x 7168 x 7168, BF16 output: the per-element
    bound |D - R| <= 1e-3 S + 1e-6 taken literally, the BF16 rounding of D
    included (at K = 7168, S is tens of times |R| -- about 68 times on
    average, above 10 even at five standard deviations of R -- so the one
    output rounding, at most 2^-8 |R|, fits inside 1e-3 S with room);
  * INT8 4096 x 4096 x 4096, bit-exact.
(The full 4096 x 14336 W8A8 layer is compared in full in test_gpu_gemv.)"""
import os

import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

# the oracle's OpenMP pool takes every core this process may use
os.environ.setdefault("OMP_NUM_THREADS", str(len(os.sched_getaffinity(0))))


def test_bf16_4096(gpu_ok):
    M = N = K = 4096
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16")
    D = host(mp.gemm_bf16(dev(A), dev(B), dev(C)))
    R, S = oracle.gemm_bf16(A, B, C)
    check_fp(D, R, S, 1e-5, "bf16 4096^3 (every element)")


def test_f16_ragged_8191_8193_4099(gpu_ok):
    M, N, K = 8191, 8193, 4099
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt="f16", c_zero=True)
    tA, tB = dev(A), dev(B)
    D0 = mp.gemm_f16(tA, tB, dev(C))
    Dn = mp.gemm_f16(tA, tB, None)
    assert torch.equal(D0.view(torch.int32), Dn.view(torch.int32))
    del Dn, tA, tB
    D = host(D0)
    del D0
    R, S = oracle.gemm_f16(A, B, C)
    check_fp(D, R, S, 1e-5, "f16 ragged (every element)")


def test_fp8_4096_7168_7168(gpu_ok):
    M, N, K = 4096, 7168, 7168
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K)
    D = mp.gemm_fp8_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb))
    got = oracle.bf16_to_f64(host(D).view(np.uint16))
    del D
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    # no allowance for the output rounding at this K: the bound as stated
    check_fp(got, R, S, 1e-2, "fp8 4096x7168x7168 (every element)")


def test_i8_4096(gpu_ok):
    M = N = K = 4096
    A, B, C = inputs.i8_operands(M, N, K)
    D = host(mp.gemm_i8_i32(dev(A), dev(B), dev(C)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C))
