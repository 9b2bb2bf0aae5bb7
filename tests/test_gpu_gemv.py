"""GPU parity of the batch-1 W8A8 layer against the oracle: the INT32 sums and
the BF16 outputs are bit-exact (the dequantisation order (float(z) * s_x) *
s_w is fixed).  Covers the full 1 x 4096 . 4096 x 14336 layer, N not a
multiple of the rows a workgroup owns, K not a multiple of 16 or 1024, -128
weights and activations at the INT32 bound, misaligned x / W and a padded
leading dimension, and K = 0.  y and z are written into guard-banded buffers:
nothing outside the N outputs may change."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

GUARD = 64


def run(x, s_x, W, s_w, ldw=None, x_shift=0):
    N, K = W.shape
    if x_shift:
        tx = dev(np.concatenate([np.zeros(x_shift, np.int8), x]))[x_shift:]
    else:
        tx = dev(x)
    # y and z sit inside guard bands of GUARD elements on each side, filled
    # with a pattern no output takes; a write outside [0, N) changes them
    ybuf = torch.full((N + 2 * GUARD,), -21846, dtype=torch.int16, device="cuda:0")   # 0xAAAA
    zbuf = torch.full((N + 2 * GUARD,), -0x55555556, dtype=torch.int32, device="cuda:0")
    y = ybuf[GUARD:GUARD + N].view(torch.bfloat16)
    z = zbuf[GUARD:GUARD + N]
    mp.gemv_w8a8(tx, float(s_x), dev(W, ldw, pad=77), dev(s_w), out=y, z_out=z)
    torch.cuda.synchronize()
    yb, zb = host(ybuf).view(np.uint16), host(zbuf)
    for name, b, fill in (("y", yb, 0xAAAA), ("z", zb, -0x55555556)):
        assert (b[:GUARD] == fill).all() and (b[GUARD + N:] == fill).all(), f"{name} written outside [0, N)"
    zr, yr = oracle.gemv_w8a8(x, s_x, W, s_w)
    return zb[GUARD:GUARD + N], yb[GUARD:GUARD + N], zr, yr


def test_full_layer_bit_exact(gpu_ok):
    x, s_x, W, s_w = inputs.w8a8_operands(14336, 4096)
    z, y, zr, yr = run(x, s_x, W, s_w)
    assert np.array_equal(z, zr)
    assert np.array_equal(y, yr)


@pytest.mark.parametrize("N,K", [(1, 1), (17, 4096), (1000, 4095), (333, 1000), (20, 5000),
                                 (4097, 64), (15, 8193),
                                 # around the 28 rows of a workgroup, whole passes of 4096 bytes
                                 (27, 8192), (28, 4096), (29, 12288), (57, 4096), (85, 8192)])
def test_shapes_bit_exact(gpu_ok, N, K):
    x, s_x, W, s_w = inputs.w8a8_operands(N, K, seeds=(N, K, 3, 4))
    z, y, zr, yr = run(x, s_x, W, s_w)
    assert np.array_equal(z, zr) and np.array_equal(y, yr)


def test_int32_bound_and_minus_128(gpu_ok):
    K, N = 4096, 70
    x = np.full(K, -128, np.int8)
    W = np.full((N, K), -128, np.int8)
    W[1::2] = 127
    s_w = np.full(N, 0.001, np.float32)
    z, y, zr, yr = run(x, np.float32(0.05), W, s_w)
    assert z[0] == 4096 * 128 * 128 and np.array_equal(z, zr) and np.array_equal(y, yr)


@pytest.mark.parametrize("ldw,shift", [(4096 + 1, 0), (4096 + 16, 3), (4100, 8)])
def test_unaligned_and_padded(gpu_ok, ldw, shift):
    x, s_x, W, s_w = inputs.w8a8_operands(500, 4096, seeds=(1, 2, 3, 4))
    z, y, zr, yr = run(x, s_x, W, s_w, ldw=ldw, x_shift=shift)
    assert np.array_equal(z, zr) and np.array_equal(y, yr)


def test_k_zero(gpu_ok):
    x = torch.zeros(0, dtype=torch.int8, device=gpu_ok)
    W = torch.zeros((40, 0), dtype=torch.int8, device=gpu_ok)
    y, z = mp.gemv_w8a8(x, 0.5, W, torch.ones(40, device=gpu_ok), return_z=True)
    assert not host(z).any() and not host(y).any()
