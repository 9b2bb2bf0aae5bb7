"""The oracle's FP16/BF16/INT8 GEMMs pinned to things other than themselves:
exact rational brute force on tiny rectangular inputs, identity and
permutation matrices, small-integer matrices (exact in every order), an
independent FP64 BLAS product at a moderate size, and agreement of the
element-at-a-time and full-matrix forms.  The definition is the textbook
D = A x B + C of the "Tensor Core" handbook page (section on what a Tensor
Core does), with A and B row-major as its wmma_gemm.cu program indexes them."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_dense_tiled_amd import inputs


def _as_float(bits, fmt):
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _exact(Af, Bf, Cf):
    M, K = Af.shape
    N = Bf.shape[1]
    R = [[None] * N for _ in range(M)]
    S = [[None] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            bnd = Fraction(0)
            for k in range(K):
                p = Fraction(float(Af[i, k])) * Fraction(float(Bf[k, j]))
                acc += p
                bnd += abs(p)
            if Cf is not None:
                acc += Fraction(float(Cf[i, j]))
            R[i][j] = acc
            S[i][j] = bnd
    return R, S


SHAPES = [(1, 1, 1), (2, 3, 5), (3, 7, 2), (5, 1, 7), (7, 5, 3), (16, 17, 33), (17, 16, 1),
          (3, 33, 17)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_brute_force_exact(fmt, M, N, K):
    seed = M * 10000 + N * 100 + K
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt=fmt,
                                     seeds=(seed, seed + 1, seed + 2))
    # random leading dimensions wider than the rows
    lda, ldb, ldc = K + (seed % 5), N + (seed % 3), N + 2
    A2, B2, C2 = inputs.with_ld(A, lda), inputs.with_ld(B, ldb), inputs.with_ld(C, ldc)
    fn = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    R, S = fn(A2, B2, C2)
    Re, Se = _exact(_as_float(A, fmt), _as_float(B, fmt), C.astype(np.float64))
    for i in range(M):
        for j in range(N):
            # FP64 accumulation: |R - exact| <= (K + 1) * 2^-52 * (S + |C|)
            tol = Fraction(K + 1) * Fraction(2) ** -52 * (Se[i][j] + abs(Fraction(float(C[i, j]))))
            assert abs(Fraction(R[i, j]) - Re[i][j]) <= tol
            assert abs(Fraction(S[i, j]) - Se[i][j]) <= Fraction(K + 1) * Fraction(2) ** -52 * Se[i][j]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identity_and_permutation_exact(fmt):
    n = 24
    A, B, _ = inputs.gemm16_operands(n, n, n, dist="uniform", fmt=fmt, with_c=False,
                                     seeds=(11, 12, 13))
    conv = inputs.to_f16_bits if fmt == "f16" else inputs.to_bf16_bits
    fn = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    eye = conv(np.eye(n, dtype=np.float32))
    R, _ = fn(A, eye)
    assert np.array_equal(R, _as_float(A, fmt))
    perm = np.random.default_rng(5).permutation(n)
    P = conv(np.eye(n, dtype=np.float32)[perm])
    R, _ = fn(P, B)
    assert np.array_equal(R, _as_float(B, fmt)[perm])
    # A . P^T permutes columns of A
    R, _ = fn(A, conv(np.eye(n, dtype=np.float32)[perm].T.copy()))
    assert np.array_equal(R, _as_float(A, fmt)[:, perm])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_small_integers_exact(fmt):
    M, N, K = 37, 29, 41
    A, B, _ = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, with_c=False,
                                     seeds=(21, 22, 23))
    Ai = _as_float(A, fmt).astype(np.int64)
    Bi = _as_float(B, fmt).astype(np.int64)
    C = np.random.default_rng(24).integers(-100, 100, (M, N)).astype(np.float32)
    fn = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    R, S = fn(A, B, C)
    assert np.array_equal(R, (Ai @ Bi + C.astype(np.int64)).astype(np.float64))
    assert np.array_equal(S, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_against_blas_fp64(fmt):
    M, N, K = 96, 80, 200
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(31, 32, 33))
    fn = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    R, S = fn(A, B, C)
    Af, Bf = _as_float(A, fmt), _as_float(B, fmt)
    ref = Af @ Bf + C.astype(np.float64)
    assert np.max(np.abs(R - ref) / (S + 1.0)) < 1e-12
    assert np.allclose(S, np.abs(Af) @ np.abs(Bf), rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_sampled_equals_full(fmt):
    M, N, K = 40, 70, 130
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt=fmt, seeds=(41, 42, 43))
    A2, B2 = inputs.with_ld(A, K + 3), inputs.with_ld(B, N + 1)
    full = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    at = oracle.gemm_f16_at if fmt == "f16" else oracle.gemm_bf16_at
    R, S = full(A2, B2, C)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Rp, Sp = at(A2, B2, C, ii.ravel(), jj.ravel())
    assert np.array_equal(Rp.reshape(M, N), R)
    assert np.array_equal(Sp.reshape(M, N), S)


def test_c_none_is_zero():
    A, B, C = inputs.gemm16_operands(9, 11, 13, seeds=(51, 52, 53))
    R0, _ = oracle.gemm_f16(A, B, None)
    Rz, _ = oracle.gemm_f16(A, B, np.zeros_like(C))
    assert np.array_equal(R0, Rz)


def test_k_zero_gives_c():
    A = np.zeros((4, 0), np.uint16)
    B = np.zeros((0, 5), np.uint16)
    C = inputs.uniform_f32((4, 5), 3)
    R, S = oracle.gemm_f16(A, B, C)
    assert np.array_equal(R, C.astype(np.float64)) and not S.any()


def test_intexact_single_rounding():
    M = N = K = 64
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt="f16", seeds=(1, 2, 3))
    D = oracle.gemm_f16_intexact(A, B, C)
    Ai = A.view(np.float16).astype(np.int64)
    Bi = B.view(np.float16).astype(np.int64)
    sums = (Ai @ Bi).astype(np.float32)       # exact: |sum| <= 1024
    assert np.array_equal(D.view(np.uint32), (sums + C).view(np.uint32))  # one fp32 add
    # and it is the FP32 rounding of the exact (FP64-representable here) value
    R, _ = oracle.gemm_f16(A, B, C)
    assert np.array_equal(D, R.astype(np.float32))


def test_intexact_rejects_fractions():
    A, B, C = inputs.gemm16_operands(4, 4, 4, dist="uniform", fmt="f16", seeds=(1, 2, 3))
    with pytest.raises(oracle.OracleError):
        oracle.gemm_f16_intexact(A, B, C)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (13, 7, 29), (64, 64, 64), (33, 65, 127)])
def test_i8_against_int64_matmul(M, N, K):
    A, B, C = inputs.i8_operands(M, N, K, seeds=(M, N + 100, K + 200))
    A2, B2 = inputs.with_ld(A, K + 5), inputs.with_ld(B, N + 7)
    D = oracle.gemm_i8_i32(A2, B2, C)
    ref = A.astype(np.int64) @ B.astype(np.int64) + C.astype(np.int64)
    assert np.array_equal(D.astype(np.int64), ref)
    ii = np.random.default_rng(0).integers(0, M, 50)
    jj = np.random.default_rng(1).integers(0, N, 50)
    assert np.array_equal(oracle.gemm_i8_i32_at(A2, B2, C, ii, jj), D[ii, jj])


def test_i8_extremes_and_overflow_detection():
    K = 4096
    A = np.full((2, K), -128, np.int8)
    B = np.full((K, 3), -128, np.int8)
    D = oracle.gemm_i8_i32(A, B, None)
    assert (D == K * 128 * 128).all()
    C = np.full((2, 3), 2 ** 31 - 1 - K * 128 * 128, np.int32)
    assert (oracle.gemm_i8_i32(A, B, C) == 2 ** 31 - 1).all()
    C = C + 1
    with pytest.raises(oracle.OracleError):
        oracle.gemm_i8_i32(A, B, C)
