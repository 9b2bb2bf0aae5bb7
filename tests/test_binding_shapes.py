"""The Python binding checks every tensor's shape against the problem size
(and that all tensors share one device) before it calls the C ABI: the C
entry points see only pointers and leading dimensions, so a buffer too small
for the problem -- a one-row D, a short B, a one-row scale grid -- would be
read or written past its end.  These checks raise ValueError before anything
is launched; here they run on CPU tensors, so no GPU and no native call is
involved (a well-shaped CPU tensor is then refused as not on the GPU)."""
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp

i16, u8, i8, f32, i32 = torch.int16, torch.uint8, torch.int8, torch.float32, torch.int32


def z(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def raises_shape(fn, *a, match=None, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


@pytest.mark.parametrize("gemm", [mp.gemm_f16, mp.gemm_bf16, mp.gemm_f16_f16out, mp.gemm_bf16_bf16out])
def test_gemm16_shapes(gemm):
    M, N, K = 64, 48, 32
    A, B = z(M, K, dtype=i16), z(K, N, dtype=i16)
    raises_shape(gemm, A, z(K + 1, N, dtype=i16), match="inner")
    raises_shape(gemm, A, B, z(1, N), match="C must have shape")
    raises_shape(gemm, A, B, z(M, N + 1), match="C must have shape")
    raises_shape(gemm, A, B, None, out=z(1, N), match="out must have shape")
    raises_shape(gemm, A, B, None, out=z(M, N - 1), match="out must have shape")
    raises_shape(gemm, z(M, K, K, dtype=i16), B, match="2-D")
    raises_shape(gemm, A, B, z(M, N), match="GPU")          # right shapes, CPU tensors


@pytest.mark.parametrize("gemm", [mp.gemm_f16_bias_act, mp.gemm_bf16_bias_act])
def test_gemm16_bias_act_shapes(gemm):
    M, N, K = 64, 48, 32
    A, B = z(M, K, dtype=i16), z(K, N, dtype=i16)
    raises_shape(gemm, A, B, z(M, N), z(N - 1), match="bias must have shape")
    raises_shape(gemm, A, B, z(1, N), z(N), match="C must have shape")
    raises_shape(gemm, A, B, None, z(N), out=z(1, N), match="out must have shape")


def test_i8_shapes():
    M, N, K = 64, 48, 32
    A, B = z(M, K, dtype=i8), z(K, N, dtype=i8)
    raises_shape(mp.gemm_i8_i32, A, z(K - 1, N, dtype=i8), match="inner")
    raises_shape(mp.gemm_i8_i32, A, B, z(M, 1, dtype=i32), match="C must have shape")
    raises_shape(mp.gemm_i8_i32, A, B, None, out=z(1, N, dtype=i32), match="out must have shape")


@pytest.mark.parametrize("fmt", [False, True])
def test_fp8_blockscaled_shapes(fmt):
    M, N, K = 300, 520, 400           # ceil(K/128) = 4, ceil(N/128) = 5
    A, B = z(M, K, dtype=u8), z(K, N, dtype=u8)
    sa, sb = z(M, 4), z(4, 5)

    def call(A, sa, B, sb, out=None):
        if fmt:
            return mp.gemm_fp8_blockscaled_fmt(A, mp.FP8_E4M3, sa, B, mp.FP8_E5M2, sb, out=out)
        return mp.gemm_fp8_blockscaled(A, sa, B, sb, out=out)

    raises_shape(call, A, sa, z(K + 1, N, dtype=u8), sb, match="inner")
    raises_shape(call, A, z(1, 4), B, sb, match="scale_a must have shape")
    raises_shape(call, A, z(M, 3), B, sb, match="scale_a must have shape")
    raises_shape(call, A, sa, B, z(4, 4), match="scale_b must have shape")
    raises_shape(call, A, sa, B, z(1, 5), match="scale_b must have shape")
    raises_shape(call, A, sa, B, sb, out=z(1, N, dtype=i16), match="out must have shape")
    raises_shape(call, A, sa, B, sb, match="GPU")


def test_fp8_rowscaled_shapes():
    M, N, K = 64, 48, 32
    A, B = z(M, K, dtype=u8), z(K, N, dtype=u8)
    raises_shape(mp.gemm_fp8_rowscaled, A, 0, z(M), z(K + 2, N, dtype=u8), 0, z(N), match="inner")
    raises_shape(mp.gemm_fp8_rowscaled, A, 0, z(M), B, 0, z(N), out=z(M, 1, dtype=i16),
                 match="out must have shape")


def test_gemv_shapes():
    N, K = 100, 64
    x, W, sw = z(K, dtype=i8), z(N, K, dtype=i8), z(N)
    raises_shape(mp.gemv_w8a8, z(K + 1, dtype=i8), 0.5, W, sw, match=r"W must be \[N, K\]")
    raises_shape(mp.gemv_w8a8, z(1, K, dtype=i8), 0.5, W, sw, match="1-D")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, z(N - 1), match="w_scale must have shape")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, sw, out=z(N - 1, dtype=i16), match="out must have shape")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, sw, out=z(1, N, dtype=i16), match="out must have shape")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, sw, z_out=z(N // 2, dtype=i32), match="z_out must have shape")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, sw, out=z(N, dtype=f32), match="2-byte")
    raises_shape(mp.gemv_w8a8, x, 0.5, W, sw, match="GPU")


@pytest.mark.parametrize("which", ["nk", "kn", "requant"])
def test_w8a8_token_shapes(which):
    M, N, K = 5, 100, 64
    X, sx, sw = z(M, K, dtype=i8), z(M), z(N)
    W = z(K, N, dtype=i8) if which == "kn" else z(N, K, dtype=i8)

    def call(X, W, out=None, z_out=None):
        if which == "nk":
            return mp.gemm_w8a8(X, sx, W, sw, None, out=out, z_out=z_out)
        if which == "kn":
            return mp.gemm_w8a8_kn(X, sx, W, sw, None, out=out, z_out=z_out)
        return mp.gemm_w8a8_requant(X, sx, W, sw, None, 0.1, out=out, z_out=z_out)

    raises_shape(call, z(M, K + 1, dtype=i8), W, match="W must be")
    raises_shape(call, X, W, out=z(1, N, dtype=i8 if which == "requant" else i16), match="out must have shape")
    raises_shape(call, X, W, z_out=z(M, N - 1, dtype=i32), match="z_out must have shape")


def test_quantiser_shapes():
    M, K = 4, 300
    X16 = z(M, K, dtype=i16)
    raises_shape(mp.quantize_i8_rows, X16, q_out=z(M, K - 1, dtype=i8), match="q_out must have shape")
    raises_shape(mp.quantize_i8_rows, X16, scales_out=z(M - 1), match="scales_out must have shape")
    X = z(257, 300)
    raises_shape(mp.quantize_fp8_blocks, X, 128, scales_out=z(2, 2), match="scales_out must have shape")
    raises_shape(mp.quantize_fp8_blocks, X, 1, q_out=z(257, 299, dtype=u8), match="q_out must have shape")
    raises_shape(mp.quantize_fp8_blocks, X, 64, match="block_rows")
    raises_shape(mp.quantize_fp8, X, mp.FP8_E4M3, 1, 128, scales_out=z(257, 2), match="scales_out must have shape")
    raises_shape(mp.quantize_fp8, X, mp.FP8_E4M3, 257, 300, scales_out=z(2, 1), match="scales_out must have shape")
