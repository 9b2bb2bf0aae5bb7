"""GPU parity of the W8A8 layer for M tokens (with and without bias) and of
the two quantisers, against the oracle, bit-exact (every step is an integer
sum or a fixed sequence of IEEE FP32 operations, then one rounding):

  * gemm_w8a8_kn: the same layer with the weights stored K x N (ragged N,
    padded ldw, K = 1, 4 tokens x the 4096 x 14336 layer);
  * gemm_w8a8_requant: the same layer requantised to INT8 (saturation,
    exact ties to even, a padded output, K = 0);
  * gemm_w8a8: M = 1, 2, 3, 5, 8, 16, 17, 31, 32, 33, 40, 65 tokens (groups of
    32 per launch),
    N not a multiple of a workgroup's 32 channels, K not a multiple of the
    wave slices, with and without bias, padded and misaligned operands, -128 at the
    INT32 bound, K = 0, and the full 4096 x 14336 layer for 4 tokens; the
    streaming path of up to 16 tokens over whole 4096-byte passes (ragged N
    around its 28-channel workgroups, one to three passes, guard-banded
    outputs, the full layer at 16 tokens, requantised);
  * quantize_i8_rows: random BF16 rows, exact ties, zero rows, K tails;
  * quantize_fp8_blocks: 1 x 128 and 128 x 128 blocks, ragged edges, a zero
    block, the FP8 workload's operand sizes, and the result fed to
    gemm_fp8_blockscaled."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host

pytestmark = pytest.mark.gpu


def w8a8_inputs(M, N, K, seed):
    r = np.random.default_rng(seed)
    X = r.integers(-127, 128, (M, K)).astype(np.int8)
    W = r.integers(-127, 128, (N, K)).astype(np.int8)
    sx = r.uniform(0.01, 0.1, M).astype(np.float32)
    sw = r.uniform(0.001, 0.01, N).astype(np.float32)
    bias = r.standard_normal(N).astype(np.float32)
    return X, sx, W, sw, bias


def run_w8a8(X, sx, W, sw, bias, ldx=None, ldw=None, shift=0):
    tX = dev(X, ldx, pad=55)
    if shift:
        M, K = X.shape
        base = dev(np.concatenate([np.zeros(shift, np.int8), X.ravel()]))
        tX = base[shift:].view(M, K)
    y, z = mp.gemm_w8a8(tX, dev(sx), dev(W, ldw, pad=-66), dev(sw),
                        None if bias is None else dev(bias), return_z=True)
    torch.cuda.synchronize()
    zr, yr = oracle.gemm_w8a8(X, sx, W, sw, bias)
    return host(z), host(y).view(np.uint16), zr, yr


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16, 17, 31, 32, 33, 40, 65])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_tokens_bit_exact(gpu_ok, M, with_bias):
    X, sx, W, sw, bias = w8a8_inputs(M, 1000, 4500, seed=M)
    z, y, zr, yr = run_w8a8(X, sx, W, sw, bias if with_bias else None)
    assert np.array_equal(z, zr) and np.array_equal(y, yr)


@pytest.mark.parametrize("M,N,K,ldx,ldw,shift", [(4, 333, 1000, 1003, 1001, 0), (6, 17, 64, None, 80, 3),
                                                 (16, 9, 8193, None, None, 0), (2, 1, 1, None, None, 1),
                                                 (5, 40, 4196, None, 4211, 1), (20, 70, 8192, None, None, 2)])
def test_w8a8_tokens_shapes_padded_unaligned(gpu_ok, M, N, K, ldx, ldw, shift):
    X, sx, W, sw, bias = w8a8_inputs(M, N, K, seed=N + K)
    z, y, zr, yr = run_w8a8(X, sx, W, sw, bias, ldx=ldx, ldw=ldw, shift=shift)
    assert np.array_equal(z, zr) and np.array_equal(y, yr)


def test_w8a8_tokens_int32_bound_full_layer_and_k_zero(gpu_ok):
    K, N = 4096, 64
    X = np.full((3, K), -128, np.int8)
    W = np.full((N, K), -128, np.int8)
    W[1::2] = 127
    sx = np.full(3, 0.05, np.float32)
    sw = np.full(N, 0.001, np.float32)
    z, y, zr, yr = run_w8a8(X, sx, W, sw, None)
    assert z[0, 0] == K * 128 * 128 and np.array_equal(z, zr) and np.array_equal(y, yr)
    X, sx, W, sw, bias = w8a8_inputs(4, 14336, 4096, seed=99)
    z, y, zr, yr = run_w8a8(X, sx, W, sw, bias)
    assert np.array_equal(z, zr) and np.array_equal(y, yr)
    bias = np.linspace(-2, 2, 30).astype(np.float32)
    y, z = mp.gemm_w8a8(torch.zeros((5, 0), dtype=torch.int8, device=gpu_ok), dev(np.ones(5, np.float32)),
                        torch.zeros((30, 0), dtype=torch.int8, device=gpu_ok), dev(np.ones(30, np.float32)),
                        dev(bias), return_z=True)
    assert not host(z).any()
    assert np.array_equal(host(y).view(np.uint16), np.tile(oracle.f32_to_bf16_rne(bias), (5, 1)))


# Up to 16 tokens over whole 4096-byte passes with 16-byte aligned rows: the
# streaming kernel (14 waves of two weight rows, 28 channels per workgroup,
# the sums of several passes carried through LDS).  N around and across the
# 28-channel workgroups, padded rows, one to three passes, the full layer at
# 16 tokens; Y and Z written into guard-banded buffers that must keep their
# padding.
@pytest.mark.parametrize("M,N,K,ldx,ldw", [(1, 1, 4096, None, None), (2, 27, 4096, 4112, None),
                                           (5, 28, 8192, None, 8208), (8, 29, 4096, None, None),
                                           (13, 57, 12288, 12304, 12320), (14, 1000, 4096, None, None),
                                           (15, 85, 8192, None, None), (16, 300, 4096, 4160, 4128),
                                           (16, 14336, 4096, None, None)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_stream_path_bit_exact_guarded(gpu_ok, M, N, K, ldx, ldw, with_bias):
    X, sx, W, sw, bias = w8a8_inputs(M, N, K, seed=7 * M + N)
    b = bias if with_bias else None
    ybuf = torch.empty((M + 1, N + 9), dtype=torch.bfloat16, device=gpu_ok)
    ybuf.view(torch.int16).fill_(0x7FC1)
    zbuf = torch.full((M + 1, N + 9), -7, dtype=torch.int32, device=gpu_ok)
    mp.gemm_w8a8(dev(X, ldx, pad=55), dev(sx), dev(W, ldw, pad=-66), dev(sw), None if b is None else dev(b),
                 out=ybuf[:M, :N], z_out=zbuf[:M, :N])
    torch.cuda.synchronize()
    zr, yr = oracle.gemm_w8a8(X, sx, W, sw, b)
    y, z = host(ybuf).view(np.uint16), host(zbuf)
    assert np.array_equal(z[:M, :N], zr) and np.array_equal(y[:M, :N], yr)
    assert (z[M:] == -7).all() and (z[:, N:] == -7).all()
    assert (y[M:] == 0x7FC1).all() and (y[:, N:] == 0x7FC1).all()


@pytest.mark.parametrize("M,N,K", [(16, 100, 4096), (3, 57, 8192)])
def test_w8a8_stream_path_requant_bit_exact(gpu_ok, M, N, K):
    X, sx, W, sw, bias = w8a8_inputs(M, N, K, seed=M + N + K)
    s_out = np.float32(0.6)
    Q, Z = mp.gemm_w8a8_requant(dev(X), dev(sx), dev(W), dev(sw), dev(bias), float(s_out), return_z=True)
    torch.cuda.synchronize()
    Zr, Qr = oracle.gemm_w8a8_requant(X, sx, W, sw, bias, s_out)
    assert np.array_equal(host(Z), Zr) and np.array_equal(host(Q), Qr)


@pytest.mark.parametrize("M", [1, 3, 17, 33, 40])
@pytest.mark.parametrize("with_bias", [False, True])
def test_w8a8_requant_bit_exact(gpu_ok, M, with_bias):
    X, sx, W, sw, bias = w8a8_inputs(M, 1000, 4500, seed=M + 100)
    b = bias if with_bias else None
    s_out = np.float32(0.6)                        # most codes inside +-127, some saturated
    Q, Z = mp.gemm_w8a8_requant(dev(X), dev(sx), dev(W, 4501, pad=-7), dev(sw),
                                None if b is None else dev(b), float(s_out), return_z=True)
    torch.cuda.synchronize()
    Zr, Qr = oracle.gemm_w8a8_requant(X, sx, W, sw, b, s_out)
    q = host(Q)
    assert np.array_equal(host(Z), Zr) and np.array_equal(q, Qr)
    assert (np.abs(q) == 127).any() and (np.abs(q) < 127).mean() > 0.5


def test_w8a8_requant_padded_output_ties_and_k_zero(gpu_ok):
    M, N, K = 6, 333, 1000
    X, sx, W, sw, bias = w8a8_inputs(M, N, K, seed=7)
    buf = torch.full((M, N + 5), 99, dtype=torch.int8, device=gpu_ok)
    mp.gemm_w8a8_requant(dev(X, K + 3), dev(sx), dev(W), dev(sw), dev(bias), 0.25, out=buf[:, :N])
    _, Qr = oracle.gemm_w8a8_requant(X, sx, W, sw, bias, np.float32(0.25))
    h = host(buf)
    assert np.array_equal(h[:, :N], Qr) and (h[:, N:] == 99).all()
    # exact ties: unit scales, s_out = 2, odd integer sums -> t / 2 = k + 1/2 -> even
    X = np.array([[1, 0], [3, 0], [5, 0], [-1, 0], [-3, 0]], np.int8)
    W = np.array([[1, 0]], np.int8)
    Q = mp.gemm_w8a8_requant(dev(X), dev(np.ones(5, np.float32)), dev(W), dev(np.ones(1, np.float32)),
                             None, 2.0)
    assert host(Q).ravel().tolist() == [0, 2, 2, 0, -2]
    # K = 0: Q = rne(bias / s_out)
    bias = np.array([0.3, -0.7, 100.0, 1e3], np.float32)
    Q = mp.gemm_w8a8_requant(torch.zeros((2, 0), dtype=torch.int8, device=gpu_ok), dev(np.ones(2, np.float32)),
                             torch.zeros((4, 0), dtype=torch.int8, device=gpu_ok), dev(np.ones(4, np.float32)),
                             dev(bias), 0.5)
    assert host(Q).tolist() == [[1, -1, 127, 127]] * 2


@pytest.mark.parametrize("M,N,K,ldw,with_bias", [(1, 1000, 4500, None, True), (4, 14336, 4096, None, True),
                                                 (17, 333, 1000, 347, False), (33, 70, 300, None, True),
                                                 (16, 5, 1, 9, True), (2, 64, 513, 100, False)])
def test_w8a8_kn_weights_bit_exact(gpu_ok, M, N, K, ldw, with_bias):
    X, sx, W, sw, bias = w8a8_inputs(M, N, K, seed=M * 7 + N + K)
    b = bias if with_bias else None
    Wkn = np.ascontiguousarray(W.T)                # the same weights stored K x N
    y, z = mp.gemm_w8a8_kn(dev(X, K + 1, pad=3) if M > 1 else dev(X), dev(sx), dev(Wkn, ldw, pad=-9),
                           dev(sw), None if b is None else dev(b), return_z=True)
    torch.cuda.synchronize()
    zr, yr = oracle.gemm_w8a8(X, sx, W, sw, b)
    assert np.array_equal(host(z), zr) and np.array_equal(host(y).view(np.uint16), yr)


def bf16_matrix(shape, seed, scale=1.0):
    r = np.random.default_rng(seed)
    v = (r.standard_normal(shape) * scale).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,K", [(1, 4096), (7, 4096), (3, 1000), (2, 1), (64, 4099)])
def test_quantize_i8_rows_bit_exact(gpu_ok, M, K):
    X = bf16_matrix((M, K), seed=M * 7 + K, scale=3.0)
    q, s = mp.quantize_i8_rows(dev(X))
    qr, sr = oracle.quantize_i8_rows(X)
    assert np.array_equal(host(q), qr) and np.array_equal(host(s), sr)


def test_quantize_i8_rows_ties_zero_rows_padding(gpu_ok):
    row = np.array([127, 2.5, 3.5, -0.5, -1.5, 126.5, 0.5, -2.5], np.float32)
    X = np.zeros((3, 8), np.uint16)
    X[0] = (row.view(np.uint32) >> 16).astype(np.uint16)
    X[2] = bf16_matrix((1, 8), 5)[0]
    tX = dev(X, 13, pad=0x7FC0)                      # NaN padding must not be read
    q_out = dev(np.full((3, 8), 99, np.int8), 11, pad=77)
    q, s = mp.quantize_i8_rows(tX, q_out=q_out)
    qr, sr = oracle.quantize_i8_rows(X)
    assert np.array_equal(host(q), qr) and np.array_equal(host(s), sr)
    assert host(q)[0].tolist() == [127, 2, 4, 0, -2, 126, 0, -2] and host(s)[1] == 1.0
    full = host(q_out.as_strided((3, 11), (11, 1)))
    assert (full[:, 8:] == 77).all()                 # padding of Q untouched


@pytest.mark.parametrize("M,K,ldx,ldq", [(5, 1003, 1008, 1016), (3, 8192, 8192, 8192), (2, 8193, 8200, 8200),
                                         (4, 17, 24, 24)])
def test_quantize_i8_rows_aligned_padded_tails(gpu_ok, M, K, ldx, ldq):
    """Rows 16-byte aligned (X) and 8-byte aligned (Q), with a partial last
    group of eight at the end of K, padding that holds BF16 NaN codes in X and
    a marker in Q (neither may be read or written), and K past the 8192
    elements one pass of registers holds."""
    X = bf16_matrix((M, K), seed=M + K, scale=2.0)
    tX = dev(X, ldx, pad=0x7FC0)
    q_out = dev(np.zeros((M, K), np.int8), ldq, pad=77)
    q, s = mp.quantize_i8_rows(tX, q_out=q_out)
    qr, sr = oracle.quantize_i8_rows(X)
    assert np.array_equal(host(q), qr) and np.array_equal(host(s), sr)
    full = host(q_out.as_strided((M, ldq), (ldq, 1)))
    assert (full[:, K:] == 77).all()


@pytest.mark.parametrize("R,C,br", [(256, 384, 128), (130, 200, 128), (5, 300, 1), (129, 257, 1),
                                    (1, 1, 1), (1, 1, 128)])
def test_quantize_fp8_blocks_bit_exact(gpu_ok, R, C, br):
    r = np.random.default_rng(R * C + br)
    X = (r.standard_normal((R, C)) * 2.0 ** r.integers(-10, 10, (R, 1))).astype(np.float32)
    if R > 128 and C > 128:
        X[:128, 128:256] = 0.0                        # an all-zero block
    q, s = mp.quantize_fp8_blocks(dev(X), br)
    qr, sr = oracle.quantize_fp8_blocks(X, br)
    assert np.array_equal(host(s), sr)
    assert np.array_equal(host(q), qr)


def test_quantize_fp8_workload_sizes_feed_the_fp8_gemm(gpu_ok):
    M, N, K = 512, 768, 1024
    r = np.random.default_rng(3)
    A = r.standard_normal((M, K)).astype(np.float32)
    B = r.standard_normal((K, N)).astype(np.float32)
    qa, sa = mp.quantize_fp8_blocks(dev(A), 1)
    qb, sb = mp.quantize_fp8_blocks(dev(B), 128)
    qar, sar = oracle.quantize_fp8_blocks(A, 1)
    qbr, sbr = oracle.quantize_fp8_blocks(B, 128)
    assert np.array_equal(host(qa), qar) and np.array_equal(host(sa), sar)
    assert np.array_equal(host(qb), qbr) and np.array_equal(host(sb), sbr)
    D = mp.gemm_fp8_blockscaled(qa, sa, qb, sb)
    got = oracle.bf16_to_f64(host(D).view(np.uint16))
    R_, S_ = oracle.gemm_fp8_blockscaled(qar, sar, qbr, sbr)
    check_fp(got, R_, S_, 1e-2, "quantised fp8 gemm", bf16_out=True)
    # and the quantised product approximates the FP32 product of the originals
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 0.1
