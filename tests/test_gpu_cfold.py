"""The one-wave GEMM's in-loop C: on full 256 x 256 tiles with at least 50 K
tiles (16-bit: K >= 1568 + 32; INT8: K >= 3136 + 64) each wave brings C into
its accumulators during the K loop instead of adding it after the last MFMA.

  * integer-valued A, B and C keep every FP32 partial sum exact, so D must
    equal the oracle's exact result bit for bit whatever the order of the
    adds -- at K just below the threshold (C added after the loop), at it,
    past it with a partial last K tile, and with edge tiles beside the
    interior ones;
  * D written in place over C gives the same bits as a separate D;
  * C = 0 gives the same bits as C = NULL (adding +0 to a sum that started
    at +0 changes nothing);
  * random operands: the per-element bound and Frobenius <= 1e-5;
  * INT8: bit-exact, also in place."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

GPU = {"f16": mp.gemm_f16, "bf16": mp.gemm_bf16}
ORC = {"f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16}


def int_c(M, N, seed):
    """C with integer values in [-16, 16]: exact in FP32 and in every sum here."""
    return np.round(inputs.uniform_f32((M, N), seed) * 16.0).astype(np.float32)


# 16-bit K tiles hold 32 elements: 1568 = 49 tiles (C after the loop), 1600 =
# 50 (in-loop C, the smallest case), 1601 (a partial 51st tile), 4160 = 130
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(512, 512, 1568), (512, 512, 1600), (512, 512, 1601),
                                   (520, 776, 1632), (256, 256, 4160), (768, 512, 2111)])
def test_integer_operands_bit_exact(gpu_ok, fmt, M, N, K):
    A, B, _ = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, with_c=False, seeds=(M, N, K))
    C = int_c(M, N, K + 7)
    D = host(GPU[fmt](dev(A), dev(B), dev(C)))
    R, _ = ORC[fmt](A, B, C)      # integer products and sums: exact
    assert np.array_equal(D.astype(np.float64), R), f"{fmt} {M}x{N}x{K}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_in_place_equals_separate_d(gpu_ok, fmt):
    M, N, K = 520, 776, 2048
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt=fmt, seeds=(21, 22, 23))
    tA, tB = dev(A), dev(B)
    D1 = GPU[fmt](tA, tB, dev(C))
    tC = dev(C)
    D2 = GPU[fmt](tA, tB, tC, out=tC)
    assert D2.data_ptr() == tC.data_ptr()
    assert torch.equal(D1.view(torch.int32), D2.view(torch.int32))
    R, S = ORC[fmt](A, B, C)
    check_fp(host(D2), R, S, 1e-5, f"{fmt} in place, in-loop C")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_zero_c_equals_null_c(gpu_ok, fmt):
    M, N, K = 512, 768, 2048
    A, B, _ = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, with_c=False, seeds=(31, 32, 33))
    tA, tB = dev(A), dev(B)
    Dn = GPU[fmt](tA, tB, None)
    Dz = GPU[fmt](tA, tB, torch.zeros(M, N, device=gpu_ok))
    assert torch.equal(Dn.view(torch.int32), Dz.view(torch.int32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_random_operands_bound(gpu_ok, fmt):
    M, N, K = 768, 520, 3000
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(41, 42, 43))
    D = host(GPU[fmt](dev(A), dev(B), dev(C)))
    R, S = ORC[fmt](A, B, C)
    check_fp(D, R, S, 1e-5, f"{fmt} {M}x{N}x{K} in-loop C")


# INT8 K tiles hold 64 elements: 3136 = 49 tiles, 3200 = 50, 3264 = 51
@pytest.mark.parametrize("M,N,K", [(512, 512, 3136), (512, 512, 3200), (520, 776, 3264), (256, 512, 4100)])
def test_i8_bit_exact_and_in_place(gpu_ok, M, N, K):
    A, B, C = inputs.i8_operands(M, N, K, seeds=(M + 5, N + 6, K + 7))
    want = oracle.gemm_i8_i32(A, B, C)
    tA, tB = dev(A), dev(B)
    assert np.array_equal(host(mp.gemm_i8_i32(tA, tB, dev(C))), want)
    tC = dev(C)
    D = mp.gemm_i8_i32(tA, tB, tC, out=tC)
    assert D.data_ptr() == tC.data_ptr()
    assert np.array_equal(host(D), want)
