"""Pins of the oracle's FP8 variants: the E5M2 format, each operand's format
in the block-scaled GEMM, the per-row / per-tensor scaled GEMM and the
quantiser into either format.  The "Tensor Core" page's precision section
names both FP8 formats (E4M3, and E5M2 with its wider range) and scale factors
per tensor, per row or per block.

  * E5M2 decode: every code against numpy's IEEE half (E5M2 is exactly the
    top byte of an FP16 code) and against torch's CPU float8_e5m2;
  * E5M2 encode: the round trip of every finite code, ties to the even code
    (midpoints between neighbours), subnormals, saturation at 57344, and
    torch's CPU cast on in-range values;
  * block-scaled GEMM with formats: unit scales give the plain product of the
    decoded operands (numpy FP64), mixed formats included;
  * row-scaled GEMM: unit scales equal the block-scaled GEMM with unit scales
    (both exact sums of exact products for E4M3), power-of-two per-tensor
    scales scale exactly, exact rational brute force on tiny shapes with
    random per-row / per-column scales;
  * quantiser: per-row (1 x C blocks) and per-tensor (R x C) scales, E5M2
    codes recovered exactly for on-grid data."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_dense_tiled_amd import inputs

E4, E5 = oracle.E4M3, oracle.E5M2


def _random_fp8(shape, seed, fmt):
    r = np.random.default_rng(seed)
    q = r.integers(0, 256, size=shape).astype(np.uint8)
    if fmt == E4:
        q[(q & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    else:
        q[(q & 0x7C) == 0x7C] = 0x3C                 # no infinities / NaNs
    return q


def test_e5m2_decode_every_code():
    q = np.arange(256, dtype=np.uint8)
    got = oracle.e5m2_to_f64(q)
    half = (q.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    same = np.isnan(got) == np.isnan(half)
    assert same.all()
    fin = ~np.isnan(got)
    assert np.array_equal(got[fin], half[fin])
    tt = torch.from_numpy(q).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(got[fin], tt[fin])
    assert got[0x7B] == 57344.0 and np.isinf(got[0x7C]) and got[0x01] == 2.0 ** -16


def test_e5m2_encode_round_trip_ties_and_saturation():
    q = np.arange(256, dtype=np.uint8)
    v = oracle.e5m2_to_f64(q)
    fin = np.isfinite(v)
    back = oracle.f32_to_e5m2_rne_sat(v[fin].astype(np.float32))
    want = q[fin].copy()
    assert np.array_equal(back, want)
    # midpoints between consecutive positive codes go to the even code
    pos = v[:0x7C]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    enc = oracle.f32_to_e5m2_rne_sat(mid)
    lo = np.arange(0x7B, dtype=np.uint8)
    assert np.array_equal(enc, np.where(lo % 2 == 0, lo, lo + 1))
    big = oracle.f32_to_e5m2_rne_sat(np.array([57344, 61439, 61440, 1e30, -1e30], np.float32))
    assert big.tolist() == [0x7B, 0x7B, 0x7B, 0x7B, 0xFB]
    # torch's CPU cast on in-range values
    r = np.random.default_rng(3)
    x = (r.standard_normal(4000) * 2.0 ** r.integers(-18, 15, 4000)).astype(np.float32)
    x = x[np.abs(x) < 57344]
    tq = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.f32_to_e5m2_rne_sat(x), tq)


@pytest.mark.parametrize("fa,fb", [(E4, E5), (E5, E4), (E5, E5)])
def test_blockscaled_formats_unit_scales_is_plain_product(fa, fb):
    M, N, K = 20, 140, 300
    qa, qb = _random_fp8((M, K), 1, fa), _random_fp8((K, N), 2, fb)
    sa = np.ones((M, 3), np.float32)
    sb = np.ones((3, 2), np.float32)
    R, S = oracle.gemm_fp8_blockscaled_fmt(qa, fa, sa, qb, fb, sb)
    a, b = oracle.fp8_to_f64(qa, fa), oracle.fp8_to_f64(qb, fb)
    assert np.max(np.abs(R - a @ b) / (S + 1e-300)) < 1e-12
    assert np.allclose(S, np.abs(a) @ np.abs(b), rtol=1e-12, atol=0)
    if fa == E4 and fb == E4:
        R0, _ = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
        assert np.array_equal(R, R0)


def test_rowscaled_unit_equals_blockscaled_and_tensor_scales_exact():
    M, N, K = 17, 130, 260
    qa, qb = _random_fp8((M, K), 4, E4), _random_fp8((K, N), 5, E4)
    R1, S1 = oracle.gemm_fp8_rowscaled(qa, E4, np.ones(M, np.float32), qb, E4, np.ones(N, np.float32))
    R2, S2 = oracle.gemm_fp8_blockscaled(qa, np.ones((M, 3), np.float32), qb, np.ones((3, 2), np.float32))
    assert np.array_equal(R1, R2) and np.allclose(S1, S2, rtol=1e-15, atol=0)
    Rt, St = oracle.gemm_fp8_rowscaled(qa, E4, np.float32([2.0 ** -5]), qb, E4, np.float32([8.0]))
    assert np.array_equal(Rt, R1 * 2.0 ** -2) and np.array_equal(St, S1 * 2.0 ** -2)
    ii = np.array([0, 16, 3, 9])
    jj = np.array([0, 129, 64, 7])
    sa = np.random.default_rng(6).uniform(0.1, 2, M).astype(np.float32)
    sb = np.random.default_rng(7).uniform(0.1, 2, N).astype(np.float32)
    R, S = oracle.gemm_fp8_rowscaled(qa, E4, sa, qb, E4, sb)
    Ra, Sa = oracle.gemm_fp8_rowscaled_at(qa, E4, sa, qb, E4, sb, ii, jj)
    assert np.array_equal(Ra, R[ii, jj]) and np.array_equal(Sa, S[ii, jj])


@pytest.mark.parametrize("fa,fb", [(E4, E4), (E5, E4), (E4, E5), (E5, E5)])
@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (2, 9, 131)])
def test_rowscaled_brute_force(fa, fb, M, N, K):
    qa, qb = _random_fp8((M, K), M + K, fa), _random_fp8((K, N), N + K, fb)
    r = np.random.default_rng(M * N * K)
    sa = r.uniform(0.01, 3, M).astype(np.float32)
    sb = r.uniform(0.01, 3, N).astype(np.float32)
    R, _ = oracle.gemm_fp8_rowscaled(qa, fa, sa, qb, fb, sb)
    a, b = oracle.fp8_to_f64(qa, fa), oracle.fp8_to_f64(qb, fb)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K))
            exact *= Fraction(float(sa[i])) * Fraction(float(sb[j]))
            assert abs(Fraction(R[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


@pytest.mark.parametrize("fmt,qmax", [(E4, 448.0), (E5, 57344.0)])
def test_quantiser_per_row_and_per_tensor(fmt, qmax):
    # on-grid rows: values are codes times 2^e, the row's largest element is
    # qmax * 2^e, so the scale is exactly 2^e and the codes come back
    r = np.random.default_rng(11)
    R, Cc = 6, 300
    codes = _random_fp8((R, Cc), 12, fmt)
    v = oracle.fp8_to_f64(codes, fmt)
    e = r.integers(-6, 6, R).astype(np.float64)
    v[:, 0] = qmax
    X = (v * 2.0 ** e[:, None]).astype(np.float32)
    Q, S = oracle.quantize_fp8_blocks_fmt(X, fmt, 1, Cc)          # one scale per row
    assert S.shape == (R, 1) and np.array_equal(S[:, 0], (2.0 ** e).astype(np.float32))
    want = codes.copy()
    want[:, 0] = 0x7E if fmt == E4 else 0x7B
    assert np.array_equal(oracle.fp8_to_f64(Q, fmt), oracle.fp8_to_f64(want, fmt))
    Qt, St = oracle.quantize_fp8_blocks_fmt(X, fmt, R, Cc)         # one per tensor
    assert St.shape == (1, 1) and St[0, 0] == np.float32(np.abs(X).max() / np.float32(qmax))
    assert np.abs(oracle.fp8_to_f64(Qt, fmt)).max() == qmax
    with pytest.raises(oracle.OracleError):
        oracle.quantize_fp8_blocks_fmt(X, 2, 1, Cc)


@pytest.mark.parametrize("fa,fb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(3, 130, 131), (5, 257, 300), (2, 128, 128)])
def test_blockscaled_full_matrix_equals_element_by_element(fa, fb, M, N, K):
    """The whole-matrix form walks B by rows; each element must still get
    exactly the operations of the one-element form, in the same order: bit
    for bit the same R and S (ragged blocks, padded leading dimensions)."""
    r = np.random.default_rng(M * 1000 + N + K)
    qa = r.integers(0, 256, (M, K)).astype(np.uint8)
    qb = r.integers(0, 256, (K, N)).astype(np.uint8)
    for q, f in ((qa, fa), (qb, fb)):     # finite codes only
        if f == 0:
            q[(q & 0x7F) == 0x7F] = 0x38
        else:
            q[(q & 0x7C) == 0x7C] = 0x3C
    kb, nb = (K + 127) // 128, (N + 127) // 128
    sa = r.uniform(0.01, 2.0, (M, kb)).astype(np.float32)
    sb = r.uniform(0.01, 2.0, (kb, nb)).astype(np.float32)
    A, B, SA = inputs.with_ld(qa, K + 5), inputs.with_ld(qb, N + 3), inputs.with_ld(sa, kb + 1)
    R, S = oracle.gemm_fp8_blockscaled_fmt(A, fa, SA, B, fb, sb)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Rp, Sp = oracle.gemm_fp8_blockscaled_fmt_at(A, fa, SA, B, fb, sb, ii.ravel(), jj.ravel())
    assert np.array_equal(Rp.reshape(M, N), R) and np.array_equal(Sp.reshape(M, N), S)
