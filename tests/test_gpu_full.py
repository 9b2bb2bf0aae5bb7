"""Parity at the workload's full sizes, through the same entry points and
launch configuration the benchmark times, on sampled outputs the oracle
computes one at a time (random positions plus the first and last rows and
columns and the 256-boundaries of the workgroup tiles):

  * BF16 4096 x 4096 x 4096, N(0,1) inputs, FP32 C;
  * FP16 8191 x 8193 x 4099 with tight leading dimensions and C = 0 (and
    C = NULL giving identical bits), with every row of the last column;
  * FP8 E4M3 block-scaled 4096 x 7168 x 7168, BF16 output;
  * INT8 4096 x 4096 x 4096, bit-exact.
(The full 4096 x 14336 W8A8 layer is compared in full in test_gpu_gemv.)"""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu


def sample_positions(M, N, n=6000, seed=0):
    r = np.random.default_rng(seed)
    ii = list(r.integers(0, M, n))
    jj = list(r.integers(0, N, n))
    edge_r = sorted({0, 1, M - 1, M - 2, 255 % M, 256 % M, (M // 256) * 256 % M})
    edge_c = sorted({0, 1, N - 1, N - 2, 255 % N, 256 % N, (N // 256) * 256 % N})
    for a in edge_r:
        for b in edge_c:
            ii.append(a)
            jj.append(b)
    return np.array(ii, np.int64), np.array(jj, np.int64)


def test_bf16_4096(gpu_ok):
    M = N = K = 4096
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16")
    D = host(mp.gemm_bf16(dev(A), dev(B), dev(C)))
    ii, jj = sample_positions(M, N)
    R, S = oracle.gemm_bf16_at(A, B, C, ii, jj)
    check_fp(D[ii, jj], R, S, 1e-5, "bf16 4096^3")


def test_f16_ragged_8191_8193_4099(gpu_ok):
    M, N, K = 8191, 8193, 4099
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt="f16", c_zero=True)
    tA, tB = dev(A), dev(B)
    D0 = mp.gemm_f16(tA, tB, dev(C))
    Dn = mp.gemm_f16(tA, tB, None)
    assert torch.equal(D0.view(torch.int32), Dn.view(torch.int32))
    del Dn
    D = host(D0)
    ii, jj = sample_positions(M, N, seed=1)
    # the whole last column: the N-edge strip kernel writes it
    ii = np.concatenate([ii, np.arange(M)])
    jj = np.concatenate([jj, np.full(M, N - 1)])
    R, S = oracle.gemm_f16_at(A, B, C, ii, jj)
    check_fp(D[ii, jj], R, S, 1e-5, "f16 ragged")


def test_fp8_4096_7168_7168(gpu_ok):
    M, N, K = 4096, 7168, 7168
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K)
    D = mp.gemm_fp8_blockscaled(dev(qa), dev(sa), dev(qb), dev(sb))
    got = oracle.bf16_to_f64(host(D).view(np.uint16))
    ii, jj = sample_positions(M, N, n=3000, seed=2)
    R, S = oracle.gemm_fp8_blockscaled_at(qa, sa, qb, sb, ii, jj)
    check_fp(got[ii, jj], R, S, 1e-2, "fp8 4096x7168x7168", bf16_out=True)


def test_i8_4096(gpu_ok):
    M = N = K = 4096
    A, B, C = inputs.i8_operands(M, N, K)
    D = host(mp.gemm_i8_i32(dev(A), dev(B), dev(C)))
    ii, jj = sample_positions(M, N, seed=3)
    assert np.array_equal(D[ii, jj], oracle.gemm_i8_i32_at(A, B, C, ii, jj))
