"""The oracle's block-scaled FP8 GEMM pinned by special cases and invariants:
unit scales reduce it to a plain E4M3 GEMM; power-of-two scales scale the
result exactly; a single K block is sA * sB * (qA . qB); every element checked
against exact rational brute force on tiny ragged shapes (partial 128-blocks in
K and N).  The scaled-FP8 idea is the one named in the "Tensor Core" handbook
page's precision section (FP8 needs per-tensor, per-row or per-block scale
factors); the 1x128 / 128x128 block shapes are the workload's."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_dense_tiled_amd import inputs


def _e4m3_float(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _random_e4m3(shape, seed):
    r = np.random.default_rng(seed)
    q = r.integers(0, 256, size=shape).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return q


def test_unit_scales_is_plain_e4m3_gemm():
    M, N, K = 33, 150, 300
    qa, qb = _random_e4m3((M, K), 1), _random_e4m3((K, N), 2)
    sa = np.ones((M, 3), np.float32)
    sb = np.ones((3, 2), np.float32)
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    a, b = _e4m3_float(qa), _e4m3_float(qb)
    ref = a @ b
    assert np.max(np.abs(R - ref) / (S + 1e-300)) < 1e-12
    assert np.allclose(S, np.abs(a) @ np.abs(b), rtol=1e-12, atol=0)


def test_power_of_two_scales_are_exact_scaling():
    M, N, K = 8, 130, 256
    qa, qb = _random_e4m3((M, K), 3), _random_e4m3((K, N), 4)
    ones_a, ones_b = np.ones((M, 2), np.float32), np.ones((2, 2), np.float32)
    R1, S1 = oracle.gemm_fp8_blockscaled(qa, ones_a, qb, ones_b)
    # the same power of two on every block of A: the whole result scales exactly
    Rp, Sp = oracle.gemm_fp8_blockscaled(qa, ones_a * np.float32(0.25), qb, ones_b * 8)
    assert np.array_equal(Rp, R1 * 2.0) and np.array_equal(Sp, S1 * 2.0)


def test_single_block_is_scale_product_times_raw_gemm():
    M, N, K = 5, 128, 128
    qa, qb = _random_e4m3((M, K), 5), _random_e4m3((K, N), 6)
    sa = np.random.default_rng(7).uniform(0.001, 0.01, (M, 1)).astype(np.float32)
    sb = np.array([[0.0037]], np.float32)
    R, _ = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    raw = _e4m3_float(qa) @ _e4m3_float(qb)   # exact: small products, K=128
    ref = (sa.astype(np.float64) * np.float64(sb[0, 0])) * raw
    assert np.array_equal(R, ref)


@pytest.mark.parametrize("M,N,K", [(2, 3, 5), (3, 130, 131), (4, 129, 257)])
def test_brute_force_exact_ragged_blocks(M, N, K):
    qa, qb = _random_e4m3((M, K), M + 10), _random_e4m3((K, N), N + 20)
    kb, nb = (K + 127) // 128, (N + 127) // 128
    r = np.random.default_rng(K)
    sa = r.uniform(0.01, 2.0, (M, kb)).astype(np.float32)
    sb = r.uniform(0.01, 2.0, (kb, nb)).astype(np.float32)
    R, S = oracle.gemm_fp8_blockscaled(inputs.with_ld(qa, K + 1), inputs.with_ld(sa, kb + 2),
                                       inputs.with_ld(qb, N + 3), sb)
    a, b = _e4m3_float(qa), _e4m3_float(qb)
    for i in range(M):
        for j in range(N):
            acc = Fraction(0)
            bnd = Fraction(0)
            for k in range(K):
                fa = Fraction(float(a[i, k])) * Fraction(float(sa[i, k // 128]))
                fb = Fraction(float(b[k, j])) * Fraction(float(sb[k // 128, j // 128]))
                acc += fa * fb
                bnd += abs(fa * fb)
            tol = Fraction(K + 4) * Fraction(2) ** -52 * bnd
            assert abs(Fraction(R[i, j]) - acc) <= tol
            assert abs(Fraction(S[i, j]) - bnd) <= tol


def test_sampled_equals_full_and_workload_generator():
    M, N, K = 70, 300, 384
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(8, 9))
    assert sa.shape == (M, 3) and sb.shape == (3, 3)
    # generator puts each block's largest magnitude at (or next to) 448
    assert np.abs(_e4m3_float(qa)).max() == 448.0
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Rp, Sp = oracle.gemm_fp8_blockscaled_at(qa, sa, qb, sb, ii.ravel(), jj.ravel())
    assert np.array_equal(Rp.reshape(M, N), R) and np.array_equal(Sp.reshape(M, N), S)
