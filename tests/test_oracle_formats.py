"""The oracle's number-format decoders and BF16 rounding, pinned to library
casts (numpy float16, torch bfloat16 / float8_e4m3fn on the CPU) over every
bit pattern and to the closed-form definitions of the formats (the format
table of the "Tensor Core" handbook page, section on FP16/BF16/TF32/FP8
precision: FP16 1/5/10, BF16 1/8/7, E4M3 1/4/3 sign/exponent/fraction bits)."""
import numpy as np
import pytest
import torch

import oracle


def test_f16_every_pattern_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_bf16_every_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())
    ours = oracle.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_every_pattern_matches_torch_and_closed_form():
    bits = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]  # only S.1111.111 is NaN
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed forms of the OCP E4M3FN encoding
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and ours[0x00] == 0.0


def test_f16_closed_forms():
    vals = oracle.f16_to_f64(np.array([0x3C00, 0x0001, 0x0400, 0x7BFF, 0xC000, 0x7C00],
                                      np.uint16))
    assert list(vals[:5]) == [1.0, 2.0 ** -24, 2.0 ** -14, 65504.0, -2.0]
    assert np.isinf(vals[5])


def _torch_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_random_and_crafted():
    r = np.random.default_rng(123)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32),
        (r.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormals
        (r.standard_normal(20000) * 1.5e38).astype(np.float32),       # near overflow
    ])
    # exact ties: lower 16 bits == 0x8000 with both parities of the kept part
    ties = (np.arange(0x3F800000, 0x3F800000 + (1 << 20), 1 << 16, dtype=np.uint32)
            | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([3.4028235e38, -3.4028235e38, 0.0, -0.0],
                                                 np.float32)])
    assert np.array_equal(oracle.f32_to_bf16_rne(x), _torch_bf16(x))


def test_bf16_rounding_closed_forms():
    f = lambda u: np.array([u], np.uint32).view(np.float32)  # noqa: E731
    # 1 + 2^-8 is half an ulp above 1.0 (ulp 2^-7): tie -> even (1.0)
    assert oracle.f32_to_bf16_rne(f(0x3F808000))[0] == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even) -> 0x3F82
    assert oracle.f32_to_bf16_rne(f(0x3F818000))[0] == 0x3F82
    # just above a tie rounds up, just below rounds down
    assert oracle.f32_to_bf16_rne(f(0x3F808001))[0] == 0x3F81
    assert oracle.f32_to_bf16_rne(f(0x3F807FFF))[0] == 0x3F80
    # the largest FP32 rounds past the largest BF16 to infinity
    assert oracle.f32_to_bf16_rne(f(0x7F7FFFFF))[0] == 0x7F80
    assert oracle.f32_to_bf16_rne(np.array([np.nan], np.float32))[0] & 0x7FC0 == 0x7FC0


@pytest.mark.parametrize("bits", [0x7F, 0xFF])
def test_e4m3_nan_is_rejected_by_gemm(bits):
    A = np.full((1, 1), bits, np.uint8)
    B = np.full((1, 1), 0x38, np.uint8)
    s = np.ones((1, 1), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_fp8_blockscaled(A, s, B, s)
