"""GPU parity of the 16-bit-output GEMMs (gemm_f16_f16out, gemm_bf16_bf16out):
D = round16(A . B + C) with the sum formed in FP32 and rounded once.

  * integer-valued inputs keep the FP32 sum exact, so D must equal the
    oracle's exact result rounded to FP32 and then to the 16-bit format
    (bit-exact), on the general kernel and on the interior + edge split;
  * random inputs: per element |D - R| <= 1e-3 * S + 1e-6 plus half an ulp of
    the output format, relative Frobenius error <= 1e-3 (FP16) / 1e-2 (BF16);
  * FP16 overflow gives infinity; the guard band around a padded D stays
    untouched; C = NULL equals C = 0; an FP32 C may not alias the 16-bit D."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

GPU = {"f16": mp.gemm_f16_f16out, "bf16": mp.gemm_bf16_bf16out}
ORC = {"f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16}
ROUND = {"f16": oracle.f32_to_f16_rne, "bf16": oracle.f32_to_bf16_rne}
DEC = {"f16": oracle.f16_to_f64, "bf16": oracle.bf16_to_f64}


def bits16(t):
    return host(t.view(torch.int16)).view(np.uint16)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 520, 400), (600, 776, 512), (64, 64, 64), (257, 31, 129)])
def test_out16_integer_inputs_bit_exact(gpu_ok, fmt, M, N, K):
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, seeds=(M, N, K))
    D = GPU[fmt](dev(A), dev(B), dev(C))
    R, _ = ORC[fmt](A, B, C)             # exact: integer products, FP64 sum
    want = ROUND[fmt](R.astype(np.float32))
    assert np.array_equal(bits16(D), want), f"{fmt} {M}x{N}x{K}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,dist", [(384, 640, 512, "normal"), (513, 257, 300, "uniform"),
                                        (1024, 1024, 1024, "normal")])
def test_out16_parity(gpu_ok, fmt, M, N, K, dist):
    A, B, C = inputs.gemm16_operands(M, N, K, dist=dist, fmt=fmt, seeds=(M + 5, N + 6, K + 7))
    D = DEC[fmt](bits16(GPU[fmt](dev(A), dev(B), dev(C))))
    R, S = ORC[fmt](A, B, C)
    check_fp(D, R, S, 1e-3 if fmt == "f16" else 1e-2, f"{fmt} out16 {M}x{N}x{K}",
             bf16_out=(fmt == "bf16"), f16_out=(fmt == "f16"))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_out16_c_null_guard_band_and_aliasing(gpu_ok, fmt):
    M, N, K = 259, 300, 128
    A, B, _ = inputs.gemm16_operands(M, N, K, fmt=fmt, seeds=(51, 52, 53), with_c=False)
    d0 = GPU[fmt](dev(A), dev(B), None)
    dz = GPU[fmt](dev(A), dev(B), torch.zeros(M, N, device=gpu_ok))
    assert torch.equal(d0.view(torch.int16), dz.view(torch.int16))
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    buf = torch.full((M + 4, N + 10), 3.0, dtype=dt, device=gpu_ok)
    out = buf[2:2 + M, 5:5 + N]
    GPU[fmt](dev(A), dev(B), None, out=out)
    h = bits16(buf)
    assert np.array_equal(h[2:2 + M, 5:5 + N], bits16(d0))
    mask = np.ones_like(h, bool)
    mask[2:2 + M, 5:5 + N] = False
    three = bits16(torch.tensor([3.0], dtype=dt))[0]
    assert (h[mask] == three).all()
    c32 = torch.zeros(M, N, dtype=torch.float32, device=gpu_ok)
    with pytest.raises(mp.MpdtError):
        GPU[fmt](dev(A), dev(B), c32, out=c32.view(dt)[:, :N])


def test_f16_out_overflow_is_infinity(gpu_ok):
    A = np.full((32, 8), 0x5C00, np.uint16)          # 256.0
    B = np.full((8, 32), 0x5C00, np.uint16)          # 256.0 -> sums of 8 * 65536
    D = bits16(mp.gemm_f16_f16out(dev(A), dev(B), None))
    assert (D == 0x7C00).all()
