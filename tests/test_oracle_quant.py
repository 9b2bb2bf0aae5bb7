"""Pins of the oracle's encoders, quantisers and M-token W8A8 layer against
what the formats and the mathematics fix (not against a retyped formula):

  * FP32 -> FP16: numpy's IEEE half conversion on values across the whole
    range (subnormals, ties, overflow) and the round trip of every finite
    FP16 code;
  * FP32 -> E4M3FN: the round trip of every finite code, ties between
    neighbouring codes going to the even code, saturation at 448, and
    torch's CPU float8_e4m3fn cast on in-range values;
  * INT8 per-token quantiser: rows on an exact grid (q recovered exactly),
    exact halfway ties (to even), the all-zero row (s = 1), invariance under
    power-of-two scaling;
  * FP8 block quantiser: blocks of on-grid values whose largest element is
    448 * 2^e (scale 2^e exactly, codes recovered), every block's largest
    element on the largest code, partial edge blocks with their own scale;
  * M-token W8A8: M = 1 is the pinned batch-1 layer, Z is the exact integer
    product, the bias with unit scales is an exact integer sum rounded once;
  * the requantising W8A8 epilogue: a worked example in exact binary
    arithmetic (saturation and a tie), unit scales against numpy's integer
    product clipped, and agreement with the BF16 layer within half an output
    step.
"""
import numpy as np
import pytest
import torch

import oracle


def test_f16_encoder_matches_ieee_half_conversion():
    r = np.random.default_rng(7)
    parts = [r.standard_normal(50000).astype(np.float32),
             (r.standard_normal(20000) * 6e4).astype(np.float32),           # near overflow
             (r.standard_normal(20000) * 1e-5).astype(np.float32),          # subnormal range
             (r.uniform(-1, 1, 20000) * 2.0 ** r.integers(-30, 20, 20000)).astype(np.float32),
             np.array([65504, 65519.99, 65520, 7e4, 5.96e-8, 2.98e-8, 2.99e-8, 0.0, -0.0],
                      np.float32)]
    x = np.concatenate(parts)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = oracle.f32_to_f16_rne(x)
    assert np.array_equal(got, want)


def test_f16_encoder_round_trips_every_finite_code_and_ties_go_even():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.f16_to_f64(codes)
    fin = np.isfinite(vals)
    got = oracle.f32_to_f16_rne(vals[fin].astype(np.float32))
    assert np.array_equal(got, codes[fin])
    # midpoint between consecutive positive finite codes (exact in FP32)
    lo = np.arange(0, 0x7bff, dtype=np.uint16)
    mid = ((oracle.f16_to_f64(lo) + oracle.f16_to_f64(lo + 1)) / 2).astype(np.float32)
    got = oracle.f32_to_f16_rne(mid)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, even)


def test_e4m3_encoder_round_trip_ties_and_saturation():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    fin = np.isfinite(vals)
    got = oracle.f32_to_e4m3_rne_sat(vals[fin].astype(np.float32))
    assert np.array_equal(got, codes[fin])
    # ties between neighbouring positive codes 0x00..0x7e go to the even code
    lo = np.arange(0, 0x7e, dtype=np.uint16).astype(np.uint8)
    mid = ((oracle.e4m3_to_f64(lo) + oracle.e4m3_to_f64(lo + 1)) / 2).astype(np.float32)
    got = oracle.f32_to_e4m3_rne_sat(mid)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
    big = np.array([448, 449, 463.9, 464, 480, 1e6, -500, -448.5], np.float32)
    assert np.array_equal(oracle.f32_to_e4m3_rne_sat(big),
                          np.array([0x7e] * 6 + [0xfe, 0xfe], np.uint8))
    assert oracle.f32_to_e4m3_rne_sat(np.array([np.nan], np.float32))[0] & 0x7f == 0x7f


def test_e4m3_encoder_matches_torch_cast_in_range():
    r = np.random.default_rng(8)
    x = np.concatenate([r.uniform(-447, 447, 40000),
                        r.standard_normal(40000) * 2.0 ** r.integers(-12, 6, 40000)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.f32_to_e4m3_rne_sat(x), want)


def bf16_bits(x):
    """exact BF16 bit patterns of FP32 values that are on the BF16 grid"""
    u = np.asarray(x, np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any(), "value not representable in BF16"
    return (u >> 16).astype(np.uint16)


def test_i8_quantiser_on_grid_ties_zero_and_scaling():
    r = np.random.default_rng(9)
    n = r.integers(-127, 128, (6, 256))
    n[:, 7] = np.where(np.arange(6) % 2 == 0, 127, -127)       # amax element = 127 steps
    for e in (-3, 0, 5):
        X = bf16_bits(n * 2.0 ** e)
        Q, S = oracle.quantize_i8_rows(X)
        assert np.array_equal(Q, n.astype(np.int8))
        assert np.array_equal(S, np.full(6, 127 * 2.0 ** e / 127, np.float32))
    # exact ties (s = 1): halves go to the even integer
    row = np.array([127, 2.5, 3.5, -0.5, -1.5, 126.5, 0.5, -2.5], np.float32)
    Q, S = oracle.quantize_i8_rows(bf16_bits(row)[None])
    assert S[0] == 1.0
    assert Q[0].tolist() == [127, 2, 4, 0, -2, 126, 0, -2]
    # all-zero row: scale 1, codes 0
    Q, S = oracle.quantize_i8_rows(np.zeros((2, 40), np.uint16))
    assert (Q == 0).all() and (S == 1.0).all()
    # power-of-two scaling leaves the codes alone and scales s exactly
    Xf = (r.standard_normal((3, 100)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    X = bf16_bits(Xf)
    Q1, S1 = oracle.quantize_i8_rows(X)
    Q2, S2 = oracle.quantize_i8_rows(bf16_bits(Xf * 8.0))
    assert np.array_equal(Q1, Q2) and np.array_equal(S2, S1 * 8)


def test_fp8_block_quantiser_recovers_on_grid_blocks():
    r = np.random.default_rng(10)
    codes = r.integers(0, 0x7e, (256, 384)).astype(np.uint8) | (r.integers(0, 2, (256, 384)) << 7).astype(np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    for br in (1, 128):
        c = codes.copy()
        v = vals.copy()
        nbr, nbc = 256 // br, 3
        e = r.integers(-8, 8, (nbr, nbc))
        for bi in range(nbr):
            for bj in range(nbc):
                c[bi * br, bj * 128] = 0x7e                    # block amax = 448
                v[bi * br, bj * 128] = 448.0
                v[bi * br:(bi + 1) * br, bj * 128:(bj + 1) * 128] *= 2.0 ** e[bi, bj]
        Q, S = oracle.quantize_fp8_blocks(v.astype(np.float32), br)
        assert np.array_equal(S, (2.0 ** e).astype(np.float32))
        assert np.array_equal(Q, c)


def test_fp8_block_quantiser_partial_blocks_and_zero_block():
    r = np.random.default_rng(11)
    X = r.standard_normal((130, 200)).astype(np.float32)
    X[128:, 128:] *= 100.0                      # the corner block has its own scale
    X[:128, 128:] = 0.0                         # an all-zero block
    Q, S = oracle.quantize_fp8_blocks(X, 128)
    assert S.shape == (2, 2)
    assert S[0, 1] == 1.0 and (Q[:128, 128:] == 0).all()
    for (i0, i1, j0, j1), s in zip([(0, 128, 0, 128), (128, 130, 0, 128), (128, 130, 128, 200)],
                                   [S[0, 0], S[1, 0], S[1, 1]]):
        blk = X[i0:i1, j0:j1]
        assert s == np.float32(np.abs(blk).max()) / np.float32(448)
        amax_at = np.unravel_index(np.abs(blk).argmax(), blk.shape)
        assert Q[i0:i1, j0:j1][amax_at] & 0x7f == 0x7e      # largest element on 448


def test_w8a8_m_tokens_pins():
    r = np.random.default_rng(12)
    M, N, K = 5, 300, 1000
    X = r.integers(-128, 128, (M, K)).astype(np.int8)
    W = r.integers(-128, 128, (N, K)).astype(np.int8)
    sx = r.uniform(0.01, 0.1, M).astype(np.float32)
    sw = r.uniform(0.001, 0.01, N).astype(np.float32)
    Z, Y = oracle.gemm_w8a8(X, sx, W, sw)
    assert np.array_equal(Z, X.astype(np.int64) @ W.astype(np.int64).T)
    for m in range(M):                                   # each token is the batch-1 layer
        z1, y1 = oracle.gemv_w8a8(X[m].copy(), sx[m], W, sw)
        assert np.array_equal(Z[m], z1) and np.array_equal(Y[m], y1)
    # unit scales and an integer bias: y = bf16(z + bias), an exact integer sum rounded once
    bias = r.integers(-1000, 1000, N).astype(np.float32)
    Zb, Yb = oracle.gemm_w8a8(X, np.ones(M, np.float32), W, np.ones(N, np.float32), bias)
    assert np.array_equal(Zb, Z)
    want = oracle.f32_to_bf16_rne((Z.astype(np.int64) + bias.astype(np.int64)).astype(np.float32))
    assert np.array_equal(Yb, want)


def test_w8a8_requant_pins():
    # (1) a worked example in exact binary arithmetic: X = [[1, 2]],
    # W = [[3, 4], [-5, 6], [40, 40], [-40, -40], [1, 0]]: z = [11, 7, 120, -120, 1];
    # s_x = 0.5, s_w = [0.25, 1, 1, 1, 0.3125], bias = [0.125, -0.25, 0, 0, 0],
    # s_out = 1/16: t = [1.5, 3.25, 60, -60, 0.15625] -> t / s_out =
    # [24, 52, 960, -960, 2.5] -> q = [24, 52, 127, -127, 2] (saturation, a tie to even)
    X = np.array([[1, 2]], np.int8)
    W = np.array([[3, 4], [-5, 6], [40, 40], [-40, -40], [1, 0]], np.int8)
    sx = np.array([0.5], np.float32)
    sw = np.array([0.25, 1, 1, 1, 0.3125], np.float32)
    bias = np.array([0.125, -0.25, 0, 0, 0], np.float32)
    Z, Q = oracle.gemm_w8a8_requant(X, sx, W, sw, bias, 0.0625)
    assert Z.tolist() == [[11, 7, 120, -120, 1]]
    assert Q.tolist() == [[24, 52, 127, -127, 2]]
    # (2) unit scales, s_out = 1: Q = clip(X . W^T, -127, 127) from numpy's
    # integer product
    r = np.random.default_rng(13)
    M, N, K = 4, 200, 400
    X = r.integers(-3, 4, (M, K)).astype(np.int8)
    W = r.integers(-3, 4, (N, K)).astype(np.int8)
    Z, Q = oracle.gemm_w8a8_requant(X, np.ones(M, np.float32), W, np.ones(N, np.float32), None, 1.0)
    ref = X.astype(np.int64) @ W.astype(np.int64).T
    assert np.array_equal(Z, ref) and np.array_equal(Q, np.clip(ref, -127, 127))
    assert (np.abs(ref) > 127).any() and (np.abs(ref) < 127).any()
    # (3) against the pinned BF16 layer: |Q s_out - t| <= s_out / 2 unless
    # saturated, with t within half a BF16 ulp of Y
    X = r.integers(-128, 128, (M, 1000)).astype(np.int8)
    W = r.integers(-128, 128, (N, 1000)).astype(np.int8)
    sx = r.uniform(0.01, 0.1, M).astype(np.float32)
    sw = r.uniform(0.001, 0.01, N).astype(np.float32)
    bias = r.standard_normal(N).astype(np.float32)
    s_out = np.float32(0.5)
    Z, Q = oracle.gemm_w8a8_requant(X, sx, W, sw, bias, s_out)
    _, Y = oracle.gemm_w8a8(X, sx, W, sw, bias)
    y = oracle.bf16_to_f64(Y)
    inside = np.abs(Q) < 127
    assert inside.mean() > 0.5 and (~inside).any()
    err = np.abs(Q.astype(np.float64) * s_out - y)
    assert (err[inside] <= s_out / 2 * (1 + 1e-6) + 2.0 ** -8 * np.abs(y[inside])).all()
    assert (np.sign(Q[~inside]) == np.sign(y[~inside])).all()
    assert (np.abs(y[~inside]) >= 126.5 * s_out * (1 - 2.0 ** -8)).all()
    # (4) s_out must be finite and positive
    for bad in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(oracle.OracleError):
            oracle.gemm_w8a8_requant(X, sx, W, sw, None, bad)
