"""GPU parity of the GEMM entry points against the CPU oracle, element by
element, at sizes that span several 256x256 workgroup tiles with ragged M, N
and K tails, plus the edge cases: odd leading dimensions, base pointers off
16-byte alignment, C = NULL, in-place D == C, K = 0, M = 0, tiny shapes, and
guard bands around D that must stay untouched.

Bars: FP16/BF16 |D - R| <= 1e-3 * S + 1e-6 per element and relative Frobenius
error <= 1e-5; integer-valued FP16 inputs bit-exact; INT8 bit-exact; FP8 the
same per-element bound against the unrounded result and Frobenius <= 1e-2."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import check_fp, dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}
FN16 = {"f16": (mp.gemm_f16, oracle.gemm_f16), "bf16": (mp.gemm_bf16, oracle.gemm_bf16)}


def run16(fmt, A, B, C, lda=None, ldb=None, ldc=None, ldd=None, dist_check=True):
    M, K = A.shape
    N = B.shape[1]
    gpu, orc = FN16[fmt]
    tA = dev(A, lda, pad=NAN16[fmt])
    tB = dev(B, ldb, pad=NAN16[fmt])
    tC = None if C is None else dev(C, ldc, pad=np.float32(np.nan))
    out = None
    if ldd is not None:
        out = dev(np.zeros((M, N), np.float32), ldd, pad=np.float32(-7.0))
    D = gpu(tA, tB, tC, out=out)
    torch.cuda.synchronize()
    Dh = host(D)
    R, S = orc(A, B, C)
    return Dh, R, S, D


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 520, 200), (513, 257, 129),
                                   (256, 256, 256), (1, 1, 1), (17, 300, 65), (260, 31, 1000)])
def test_gemm16_parity(gpu_ok, fmt, M, N, K):
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt=fmt,
                                     seeds=(M + 1, N + 2, K + 3))
    D, R, S, _ = run16(fmt, A, B, C)
    check_fp(D, R, S, 1e-5, f"{fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm16_normal_inputs(gpu_ok, fmt):
    A, B, C = inputs.gemm16_operands(384, 640, 512, dist="normal", fmt=fmt)
    D, R, S, _ = run16(fmt, A, B, C)
    check_fp(D, R, S, 1e-5, fmt)


def test_f16_64_integer_variant_bit_exact(gpu_ok):
    A, B, C = inputs.gemm16_operands(64, 64, 64, dist="int4", fmt="f16")
    D, _, _, _ = run16("f16", A, B, C)
    ref = oracle.gemm_f16_intexact(A, B, C)
    assert np.array_equal(D.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_integer_variant_bit_exact_multi_tile(gpu_ok, fmt):
    # integer inputs keep every partial sum exact: D must be bit-exact at any size
    A, B, C = inputs.gemm16_operands(300, 520, 400, dist="int4", fmt=fmt, seeds=(4, 5, 6))
    D, R, _, _ = run16(fmt, A, B, C)
    # R = exact integer sum + C in FP64 (exact here: |sum| <= 6400, C in [-1, 1])
    assert np.array_equal(D, R.astype(np.float32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_unaligned_leading_dims_and_nan_padding(gpu_ok, fmt):
    M, N, K = 301, 333, 203
    A, B, C = inputs.gemm16_operands(M, N, K, fmt=fmt, seeds=(7, 8, 9))
    D, R, S, _ = run16(fmt, A, B, C, lda=K + 1, ldb=N + 3, ldc=N + 5, ldd=N + 7)
    check_fp(D, R, S, 1e-5, "odd ld")


@pytest.mark.parametrize("shift", [2, 4, 8])
def test_base_pointer_offsets(gpu_ok, shift):
    M, N, K = 200, 300, 150
    A, B, C = inputs.gemm16_operands(M, N, K, fmt="f16", seeds=(10, 11, 12))
    e = shift // 2
    tA = dev(np.concatenate([np.zeros(e, np.uint16), A.ravel()]))[e:].view(M, K)
    tB = dev(np.concatenate([np.zeros(e, np.uint16), B.ravel()]))[e:].view(K, N)
    ce = max(shift // 4, 1)
    tC = dev(np.concatenate([np.zeros(ce, np.float32), C.ravel()]))[ce:].view(M, N)
    D = host(mp.gemm_f16(tA, tB, tC))
    R, S = oracle.gemm_f16(A, B, C)
    check_fp(D, R, S, 1e-5, f"shift {shift}")


def test_c_null_equals_zero_c_bitwise(gpu_ok):
    A, B, _ = inputs.gemm16_operands(300, 270, 310, fmt="f16", with_c=False)
    t0 = mp.gemm_f16(dev(A), dev(B), None)
    tz = mp.gemm_f16(dev(A), dev(B), torch.zeros(300, 270, device=gpu_ok))
    assert torch.equal(t0.view(torch.int32), tz.view(torch.int32))


def test_in_place_d_equals_c(gpu_ok):
    A, B, C = inputs.gemm16_operands(280, 290, 130, fmt="bf16", seeds=(13, 14, 15))
    tC = dev(C)
    D = mp.gemm_bf16(dev(A), dev(B), tC, out=tC)
    assert D.data_ptr() == tC.data_ptr()
    R, S = oracle.gemm_bf16(A, B, C)
    check_fp(host(D), R, S, 1e-5, "in place")


def test_k_zero_and_m_zero(gpu_ok):
    C = inputs.uniform_f32((70, 90), 3)
    A = torch.zeros((70, 0), dtype=torch.int16, device=gpu_ok)
    B = torch.zeros((0, 90), dtype=torch.int16, device=gpu_ok)
    D = host(mp.gemm_f16(A, B, dev(C)))
    assert np.array_equal(D, C)
    D = host(mp.gemm_f16(A, B, None))
    assert not D.any()
    e = torch.zeros((0, 90), dtype=torch.float32, device=gpu_ok)
    mp.gemm_f16(torch.zeros((0, 5), dtype=torch.int16, device=gpu_ok),
                torch.zeros((5, 90), dtype=torch.int16, device=gpu_ok), None, out=e)


def test_guard_bands_untouched(gpu_ok):
    M, N, K = 257, 259, 70
    A, B, C = inputs.gemm16_operands(M, N, K, fmt="f16", seeds=(16, 17, 18))
    ldd = N + 16
    buf = torch.full((M + 8, ldd), -3.25, dtype=torch.float32, device=gpu_ok)
    out = buf[4:4 + M, 3:3 + N]
    mp.gemm_f16(dev(A), dev(B), dev(C), out=out)
    h = host(buf)
    R, S = oracle.gemm_f16(A, B, C)
    check_fp(h[4:4 + M, 3:3 + N], R, S, 1e-5, "guarded")
    mask = np.ones_like(h, bool)
    mask[4:4 + M, 3:3 + N] = False
    assert (h[mask] == -3.25).all()


# Aligned rows with whole 32-element K tiles: full 256 x 256 tiles run the
# one-wave interior kernel, the rest the general kernel in a second launch.
# K = 96 (three K tiles) is below the interior kernel's minimum and runs
# the general kernel alone; K = 128 is its minimum.
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(600, 776, 512), (512, 512, 128), (768, 264, 96),
                                   (256, 1024, 1056), (264, 256, 160)])
def test_interior_and_edge_tiles_integer_bit_exact(gpu_ok, fmt, M, N, K):
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, seeds=(M, N, K))
    D, R, _, _ = run16(fmt, A, B, C)
    assert np.array_equal(D, R.astype(np.float32)), f"{fmt} {M}x{N}x{K}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_interior_and_edge_tiles_uniform_in_place(gpu_ok, fmt):
    M, N, K = 520, 780, 640
    A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt=fmt, seeds=(31, 32, 33))
    tC = dev(C)
    fn = mp.gemm_f16 if fmt == "f16" else mp.gemm_bf16
    D = fn(dev(A), dev(B), tC, out=tC)
    R, S = FN16[fmt][1](A, B, C)
    check_fp(host(D), R, S, 1e-5, f"{fmt} interior+edge in place")
    t0 = fn(dev(A), dev(B), None)
    tz = fn(dev(A), dev(B), torch.zeros(M, N, device=gpu_ok))
    assert torch.equal(t0.view(torch.int32), tz.view(torch.int32))


# The one-wave kernel takes every tile of a problem with at least four K
# tiles: its last K tile is read as a 64-byte window ending on the 16-byte
# boundary at or after K (the bytes before the previous tile's end and from K
# on cleared in the fragments), and the last tile column of B is loaded from
# column N - 256 when B's rows end inside a 16-byte chunk.  Every residue of
# K modulo 32 elements that exercises a different window offset, rows padded
# with NaN, integer inputs: bit-exact.
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("K", [129, 131, 135, 136, 137, 143, 144, 145, 159, 160])
def test_one_wave_k_window_bit_exact(gpu_ok, fmt, K):
    M, N = 300, 272
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, seeds=(K, M, N))
    D, R, _, _ = run16(fmt, A, B, C, lda=K + 5, ldb=N + 3)
    assert np.array_equal(D, R.astype(np.float32)), f"{fmt} K={K}"


# B rows that end inside a 16-byte chunk (N * 2 bytes not a multiple of 16)
# with N >= 256: the shifted last tile column must store only its own columns,
# also in place (D == C, where a second write of a column would add A.B twice).
@pytest.mark.parametrize("N", [257, 263, 511, 777])
def test_one_wave_shifted_last_column_in_place(gpu_ok, N):
    M, K = 264, 200
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt="f16", seeds=(N, 1, 2))
    tC = dev(C)
    D = mp.gemm_f16(dev(A), dev(B, N + 1, pad=NAN16["f16"]), tC, out=tC)
    R, _ = oracle.gemm_f16(A, B, C)
    assert np.array_equal(host(D), R.astype(np.float32)), f"N={N}"


EDGE = [1, 15, 16, 17, 31, 33, 127, 128, 129, 255, 257]


def test_edge_sweep(gpu_ok):
    r = np.random.default_rng(2024)
    cases = [(m, n, k) for m in EDGE for n in EDGE for k in EDGE]
    pick = [cases[i] for i in r.choice(len(cases), 60, replace=False)]
    pick += [(257, 257, 257), (1, 257, 1), (257, 1, 129), (129, 129, 1)]
    for (M, N, K) in pick:
        for fmt in ("f16", "bf16"):
            A, B, C = inputs.gemm16_operands(M, N, K, fmt=fmt, seeds=(M, N, K))
            D, R, S, _ = run16(fmt, A, B, C, lda=K + (M % 3), ldb=N + (K % 2))
            check_fp(D, R, S, 1e-5, f"{fmt} {M}x{N}x{K}")


# ------------------------------------------------------------------ INT8 --
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 520, 200), (513, 257, 129), (1, 1, 1),
                                   (256, 256, 512), (600, 776, 512), (512, 272, 256),
                                   (256, 512, 192)])
def test_i8_bit_exact(gpu_ok, M, N, K):
    A, B, C = inputs.i8_operands(M, N, K, seeds=(M, N, K))
    D = host(mp.gemm_i8_i32(dev(A), dev(B), dev(C)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C))


# INT8 through the one-wave kernel: K tails of every 16-byte residue class,
# rows of B ending inside a 16-byte chunk (N % 16 != 0), unaligned rows.
@pytest.mark.parametrize("M,N,K", [(260, 263, 257), (300, 300, 263), (256, 511, 300),
                                   (257, 270, 321), (129, 777, 399)])
def test_i8_one_wave_edges_bit_exact(gpu_ok, M, N, K):
    A, B, C = inputs.i8_operands(M, N, K, seeds=(M, N, K))
    D = host(mp.gemm_i8_i32(dev(A, K + 3, pad=-128), dev(B, N + 7, pad=127), dev(C)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C))


@pytest.mark.parametrize("pad", [0, 3])
def test_i8_sums_beyond_2_24_exact(gpu_ok, pad):
    # A, B in [100, 127] and K = 4096 give sums near 5e7, past 2^24: most
    # are not FP32 values, so the INT32 path must never pass through FP32
    # (pad 0: one-wave kernel; pad 3: rows not 16-byte aligned, general kernel)
    M, N, K = 300, 260, 4096
    r = np.random.default_rng(17 + pad)
    A = r.integers(100, 128, (M, K)).astype(np.int8)
    B = r.integers(100, 128, (K, N)).astype(np.int8)
    C = r.integers(-1000, 1000, (M, N)).astype(np.int32)
    D = host(mp.gemm_i8_i32(dev(A, K + pad), dev(B), dev(C)))
    want = oracle.gemm_i8_i32(A, B, C)
    assert (np.abs(want) > 2 ** 25).mean() > 0.9 and (want % 4 != 0).mean() > 0.5
    assert np.array_equal(D, want)


def test_i8_extremes_unaligned_and_null_c(gpu_ok):
    M, N, K = 130, 270, 1031
    A = np.full((M, K), -128, np.int8)
    B = np.full((K, N), -128, np.int8)
    B[:, ::3] = 127
    D = host(mp.gemm_i8_i32(dev(A, K + 5, pad=99), dev(B, N + 3, pad=-99), None))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, None))
    A, B, C = inputs.i8_operands(M, N, K, seeds=(1, 2, 3))
    D = host(mp.gemm_i8_i32(dev(A, K + 7, pad=5), dev(B, N + 1, pad=5), dev(C, N + 2)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C))


# ------------------------------------------------------------------- FP8 --
def run_fp8(qa, sa, qb, sb, lda=None, ldb=None):
    D = mp.gemm_fp8_blockscaled(dev(qa, lda, pad=0x7F), dev(sa), dev(qb, ldb, pad=0x7F), dev(sb))
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(host(D).view(np.uint16))
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    return got, R, S


# Full 128 x 256 tiles with whole 128-wide K blocks (at least three) go to the
# one-wavefront kernel, and so do the edge tiles when N is a multiple of 16
# and M >= 128; the rest (short or ragged K, edge tiles of other shapes) go to
# the general one: (256, 512, 384) and (384, 768, 512) are all one-wave tiles
# with the fewest K blocks it takes, (300, 600, 768) mixes both kernels in one
# call (N = 600 is not a multiple of 16).
@pytest.mark.parametrize("M,N,K", [(128, 256, 256), (300, 520, 400), (129, 130, 131),
                                   (1, 1, 1), (256, 512, 1024), (256, 512, 384),
                                   (384, 768, 512), (300, 600, 768)])
def test_fp8_parity(gpu_ok, M, N, K):
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(M, N))
    got, R, S = run_fp8(qa, sa, qb, sb)
    check_fp(got, R, S, 1e-2, f"fp8 {M}x{N}x{K}", bf16_out=True)


# Edge tiles on the one-wavefront kernel: with M >= 128, N a multiple of 16 and
# whole 128-wide K blocks (at least three), every tile of a block-scaled
# problem runs there in one launch -- the last row tile moves up to end at row
# M - 1 (its rows shared with the tile above are stored once), B's columns past
# N read zeros and D's are not stored.  (129, 272): one stored row and 16
# columns in the edge tiles; (1000, 1040): a last column tile with 16 columns
# and no second B scale block; (128, 48) with B rows padded to 256 bytes: a
# single tile 48 columns wide; (128, 16) with tight B rows (16 bytes, under
# the 256 the one-wave kernel's B loads need): the general kernel.
@pytest.mark.parametrize("M,N,K,ldb", [(200, 400, 1024, None), (1000, 1040, 384, None),
                                       (129, 272, 512, None), (128, 48, 384, 256), (128, 16, 384, None),
                                       (2000, 2000, 2048, None)])
def test_fp8_edge_tiles_one_wave(gpu_ok, M, N, K, ldb):
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(M + 1, N + 2))
    got, R, S = run_fp8(qa, sa, qb, sb, ldb=ldb)
    # (the output's rounding is admitted on top of the bound only up to K = 1024)
    check_fp(got, R, S, 1e-2, f"fp8 edge tiles {M}x{N}x{K} ldb={ldb}", bf16_out=K <= 1024)


# Wide one-wave grids with a partly filled last round (8 x 33 and 8 x 34
# tiles on 256 CUs); (1000, 8432): the row shift and a partial last column.
@pytest.mark.parametrize("M,N,K", [(1024, 8448, 384), (1024, 8576, 512), (1000, 8432, 768)])
def test_fp8_wide_grids(gpu_ok, M, N, K):
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(M + 3, N + 4))
    got, R, S = run_fp8(qa, sa, qb, sb)
    check_fp(got, R, S, 1e-2, f"fp8 wide grid {M}x{N}x{K}", bf16_out=True)


def test_fp8_edge_tiles_guard_band(gpu_ok):
    """Edge tiles with padded rows everywhere: A and B padded with E4M3 NaN
    codes, D inside a larger buffer.  No NaN reaches D, and nothing right of
    column N or below row M of the buffer is written."""
    M, N, K = 200, 400, 768
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(41, 42))
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    buf = torch.full((M + 3, N + 16), -1, dtype=torch.int16, device=gpu_ok).view(torch.bfloat16)
    mp.gemm_fp8_blockscaled(dev(qa, K + 16, pad=0x7F), dev(sa), dev(qb, N + 16, pad=0x7F), dev(sb),
                            out=buf[:M, :N])
    torch.cuda.synchronize()
    whole = host(buf).view(np.uint16)
    assert (whole[:, N:] == 0xFFFF).all() and (whole[M:] == 0xFFFF).all(), "D written outside M x N"
    check_fp(oracle.bf16_to_f64(whole[:M, :N]), R, S, 1e-2, "fp8 edge tiles, padded", bf16_out=True)


def test_fp8_shape_sweep(gpu_ok):
    """Seeded random shapes around the one-wave kernel's conditions: M on
    both sides of 128, N multiples of 16 (one-wave edge tiles) and not (edge
    tiles on the general kernel), K whole scale blocks from three up, and
    padded leading dimensions (A and B rows padded with E4M3 NaN codes, D
    inside a buffer whose padding must stay untouched)."""
    r = np.random.default_rng(4242)
    for case in range(24):
        M = int(r.integers(100, 700))
        N = int(r.integers(1, 50)) * 16 + (0 if case % 4 else int(r.integers(1, 16)))
        K = 128 * int(r.integers(3, 12))
        lda = K + 16 * int(r.integers(0, 3))
        ldb = N + (16 * int(r.integers(0, 3)) if N % 16 == 0 else int(r.integers(0, 9)))
        ldd = N + 8 * int(r.integers(0, 3))
        qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(case, M + N + K))
        R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
        buf = torch.full((M + 2, ldd), -1, dtype=torch.int16, device=gpu_ok).view(torch.bfloat16)
        mp.gemm_fp8_blockscaled(dev(qa, lda, pad=0x7F), dev(sa), dev(qb, ldb, pad=0x7F), dev(sb),
                                out=buf[:M, :N])
        torch.cuda.synchronize()
        whole = host(buf).view(np.uint16)
        what = f"fp8 sweep case {case}: {M}x{N}x{K} lda={lda} ldb={ldb} ldd={ldd}"
        assert (whole[:, N:] == 0xFFFF).all() and (whole[M:] == 0xFFFF).all(), what + ": padding written"
        check_fp(oracle.bf16_to_f64(whole[:M, :N]), R, S, 1e-2, what, bf16_out=K <= 1024)


def test_fp8_unaligned_and_unit_scales(gpu_ok):
    M, N, K = 200, 300, 333
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(21, 22))
    got, R, S = run_fp8(qa, sa, qb, sb, lda=K + 3, ldb=N + 5)
    check_fp(got, R, S, 1e-2, "fp8 unaligned", bf16_out=True)
    ones_a, ones_b = np.ones_like(sa), np.ones_like(sb)
    got, R, S = run_fp8(qa, ones_a, qb, ones_b)
    check_fp(got, R, S, 1e-2, "fp8 unit scales", bf16_out=True)


def test_fp8_padded_scales_and_output(gpu_ok):
    """Scale matrices and D with leading dimensions wider than their rows.  A
    16-byte aligned D (ldd a multiple of 8) keeps the interior tiles on the
    one-wavefront kernel; an odd ldd sends the whole problem to the general
    kernel.  Both must agree with the oracle."""
    M, N, K = 256, 768, 640
    qa, sa, qb, sb = inputs.fp8_operands(M, N, K, seeds=(31, 32))
    R, S = oracle.gemm_fp8_blockscaled(qa, sa, qb, sb)
    ta, tb = dev(qa), dev(qb)
    tsa = dev(sa, sa.shape[1] + 3, pad=np.float32(1e30))
    tsb = dev(sb, sb.shape[1] + 2, pad=np.float32(-1e30))
    for ldd in (N + 8, N + 3):
        buf = torch.full((M, ldd), -1, dtype=torch.int16, device=gpu_ok).view(torch.bfloat16)
        out = buf[:, :N]
        mp.gemm_fp8_blockscaled(ta, tsa, tb, tsb, out=out)
        torch.cuda.synchronize()
        whole = host(buf).view(np.uint16)
        assert (whole[:, N:] == 0xFFFF).all(), f"ldd {ldd}: padding of D was written"
        got = oracle.bf16_to_f64(whole[:, :N])
        check_fp(got, R, S, 1e-2, f"fp8 padded ldd={ldd}", bf16_out=True)


def test_fp8_k_zero(gpu_ok):
    D = mp.gemm_fp8_blockscaled(torch.zeros((40, 0), dtype=torch.uint8, device=gpu_ok),
                                torch.zeros((40, 0), device=gpu_ok),
                                torch.zeros((0, 50), dtype=torch.uint8, device=gpu_ok),
                                torch.zeros((0, 1), device=gpu_ok))
    assert not host(D).any()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(300, 257, 200), (513, 520, 300), (1000, 784, 4099), (260, 265, 1),
                                   (17, 512 + 13, 1500), (2049, 1024 + 16, 700),
                                   # the 4-column strip with K = 1, with a last chunk of B's
                                   # final row alone (4097 = 4096 + 1), over three chunks
                                   (300, 258, 1), (260, 257, 4097), (130, 259, 8193), (64, 261, 2049)])
def test_narrow_last_column_strip(gpu_ok, fmt, M, N, K):
    """N a few columns past a multiple of 256: the tiles take the whole
    256-column blocks and the strip kernel the rest.  Integer-valued inputs:
    bit-exact for FP32 and for 16-bit D, C in place; random inputs: the
    bound; bias + activation of the fused epilogue on the strip too."""
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, seeds=(M, N, K))
    C = np.round(C * 8).astype(np.float32)                # integer-valued C
    gemm = mp.gemm_f16 if fmt == "f16" else mp.gemm_bf16
    tc = dev(C)
    gemm(dev(A), dev(B), tc, out=tc)                       # in place
    R, _ = (oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16)(A, B, C)
    assert np.array_equal(host(tc), R.astype(np.float32)), f"{fmt} {M}x{N}x{K} in place"
    out16 = mp.gemm_f16_f16out if fmt == "f16" else mp.gemm_bf16_bf16out
    D16 = host(out16(dev(A), dev(B), dev(C)).view(torch.int16)).view(np.uint16)
    rnd = oracle.f32_to_f16_rne if fmt == "f16" else oracle.f32_to_bf16_rne
    assert np.array_equal(D16, rnd(R.astype(np.float32))), f"{fmt} {M}x{N}x{K} 16-bit"
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(M + 1, N + 1, K + 1))
    D = host(gemm(dev(A), dev(B), dev(C)))
    R, S = (oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16)(A, B, C)
    check_fp(D, R, S, 1e-5, f"{fmt} {M}x{N}x{K} strip")
    bias = inputs.normal_f32((N,), N)
    ba = mp.gemm_f16_bias_act if fmt == "f16" else mp.gemm_bf16_bias_act
    dec = oracle.f16_to_f64 if fmt == "f16" else oracle.bf16_to_f64
    ulp = 2.0 ** -11 if fmt == "f16" else 2.0 ** -8
    for act in (mp.ACT_RELU, mp.ACT_GELU):
        Rg, Sg, Pg = oracle.gemm16_bias_act(fmt, A, B, C, bias, act)
        bound = 1.13 * (1e-3 * Sg + 1e-6 + 2.0 ** -22 * np.abs(Pg)) + 2.0 ** -20 * (np.abs(Pg) + np.abs(Rg))
        Dg = host(ba(dev(A), dev(B), dev(C), dev(bias), act))
        assert (np.abs(Dg - Rg) <= bound).all(), f"{fmt} {M}x{N}x{K} act {act}"
        # 16-bit D: the same bound plus half an ulp of the output format
        Dh = dec(host(ba(dev(A), dev(B), dev(C), dev(bias), act, d16=True).view(torch.int16)).view(np.uint16))
        bound16 = bound + ulp * np.maximum(np.abs(Rg), np.abs(Dh)) + 2.0 ** -25
        assert (np.abs(Dh - Rg) <= bound16).all(), f"{fmt} {M}x{N}x{K} act {act} 16-bit"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,pad", [(64, 64, 64, 0), (1, 1, 1, 0), (256, 256, 256, 0), (33, 200, 17, 3),
                                       (200, 33, 255, 1), (5, 7, 16, 0), (64, 64, 0, 0), (257, 64, 64, 0)])
def test_small_problems(gpu_ok, fmt, M, N, K, pad):
    """M, N and K at most 256 take the small-problem kernel (one round trip
    of loads into the MFMA fragments); 257 rows take the tiles.  Integer-
    valued inputs: bit-exact FP32 D in place and 16-bit D, A rows not
    16-byte aligned when padded; random inputs: the bound, also through the
    fused bias + GELU epilogue with 16-bit D."""
    A, B, C = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, seeds=(M + 7, N + 7, K + 7))
    C = np.round(C * 8).astype(np.float32)
    gemm = mp.gemm_f16 if fmt == "f16" else mp.gemm_bf16
    ref = oracle.gemm_f16 if fmt == "f16" else oracle.gemm_bf16
    tA = dev(A, K + pad, pad=0x7C00) if pad else dev(A)     # padding: never read
    tc = dev(C)
    gemm(tA, dev(B), tc, out=tc)
    R, _ = ref(A, B, C)
    assert np.array_equal(host(tc), R.astype(np.float32)), f"{fmt} {M}x{N}x{K} in place"
    out16 = mp.gemm_f16_f16out if fmt == "f16" else mp.gemm_bf16_bf16out
    rnd = oracle.f32_to_f16_rne if fmt == "f16" else oracle.f32_to_bf16_rne
    D16 = host(out16(tA, dev(B), dev(C)).view(torch.int16)).view(np.uint16)
    assert np.array_equal(D16, rnd(R.astype(np.float32))), f"{fmt} {M}x{N}x{K} 16-bit"
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(M + 8, N + 8, K + 8))
    R, S = ref(A, B, C)
    check_fp(host(gemm(dev(A), dev(B), dev(C))), R, S, 1e-5, f"{fmt} {M}x{N}x{K} small")
    check_fp(host(gemm(dev(A), dev(B), None)), R - C, S, 1e-5, f"{fmt} {M}x{N}x{K} no C")
    bias = inputs.normal_f32((N,), N + 9)
    ba = mp.gemm_f16_bias_act if fmt == "f16" else mp.gemm_bf16_bias_act
    dec = oracle.f16_to_f64 if fmt == "f16" else oracle.bf16_to_f64
    ulp = 2.0 ** -11 if fmt == "f16" else 2.0 ** -8
    Rg, Sg, Pg = oracle.gemm16_bias_act(fmt, A, B, C, bias, mp.ACT_GELU)
    Dh = dec(host(ba(dev(A), dev(B), dev(C), dev(bias), mp.ACT_GELU, d16=True).view(torch.int16)).view(np.uint16))
    bound = (1.13 * (1e-3 * Sg + 1e-6 + 2.0 ** -22 * np.abs(Pg)) + 2.0 ** -20 * (np.abs(Pg) + np.abs(Rg))
             + ulp * np.maximum(np.abs(Rg), np.abs(Dh)) + 2.0 ** -25)
    assert (np.abs(Dh - Rg) <= bound).all(), f"{fmt} {M}x{N}x{K} bias + GELU 16-bit"


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (256, 256, 256), (1, 1, 1), (33, 200, 33), (200, 17, 255),
                                   (40, 50, 0), (256, 257, 100)])
def test_i8_small_problems_bit_exact(gpu_ok, M, N, K):
    """INT8 problems with M, N and K at most 256 take the small-problem
    kernel (exact INT32): extremes -128 / 127 over the whole of K, rows not
    16-byte aligned with guard values in the padding, C NULL, K = 0, K
    tails; 257 columns take the tiles."""
    A = np.full((M, K), -128, np.int8)
    B = np.full((K, N), -128, np.int8)
    C = inputs.i8_operands(M, N, K, seeds=(M + 1, N + 1, K + 1))[2]
    D = host(mp.gemm_i8_i32(dev(A), dev(B), dev(C)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C)), "extremes"
    A, B, C = inputs.i8_operands(M, N, K, seeds=(M + 2, N + 2, K + 2))
    D = host(mp.gemm_i8_i32(dev(A, K + 5, pad=99), dev(B, N + 3, pad=-99), None))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, None)), "unaligned, C NULL"
    D = host(mp.gemm_i8_i32(dev(A), dev(B), dev(C)))
    assert np.array_equal(D, oracle.gemm_i8_i32(A, B, C)), "random"


def test_random_shape_sweep_bit_exact(gpu_ok):
    """Seeded random shapes up to ~1100 x 1100 x 3300 through every 16-bit
    and INT8 path (small-problem, tile, strip and general kernels, K tails,
    the in-loop C of long K), with padded leading dimensions (NaN or marker
    padding), C absent, given or overwritten in place, and a guard band
    around D.  Integer-valued 16-bit inputs keep every FP32 partial sum
    exact, so D must equal the oracle bit for bit in every case."""
    r = np.random.default_rng(777)
    for case in range(60):
        fmt = ("f16", "bf16", "i8")[case % 3]
        M, N = int(r.integers(1, 1100)), int(r.integers(1, 1100))
        K = int(r.integers(1, 3300)) if case % 5 else int(r.integers(1600, 3300))
        pa, pb, pd = (int(x) for x in r.integers(0, 9, 3))
        cmode = ("none", "given", "inplace")[int(r.integers(0, 3))]
        what = f"case {case}: {fmt} {M}x{N}x{K} pads {pa},{pb},{pd} C {cmode}"
        if fmt == "i8":
            A, B, C = inputs.i8_operands(M, N, K, seeds=(case, M, N))
            if cmode == "none":
                C = None
            want = oracle.gemm_i8_i32(A, B, C)
            tA, tB = dev(A, K + pa, pad=-128), dev(B, N + pb, pad=127)
            gpu, dt, marker = mp.gemm_i8_i32, np.int32, -7
        else:
            A, B, _ = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, with_c=False, seeds=(case, M, N))
            C = None if cmode == "none" else np.round(inputs.uniform_f32((M, N), case + 99) * 16.0).astype(np.float32)
            want, _ = FN16[fmt][1](A, B, C)
            tA, tB = dev(A, K + pa, pad=NAN16[fmt]), dev(B, N + pb, pad=NAN16[fmt])
            gpu, dt, marker = FN16[fmt][0], np.float32, -7.0
        buf = dev(np.zeros((M + 2, N + pd), dt), pad=0)
        buf.fill_(marker)
        if cmode == "inplace":
            buf[:M, :N] = torch.from_numpy(C).to(buf.device)
            out = buf[:M, :N]
            D = gpu(tA, tB, out, out=out)
        else:
            out = buf[:M, :N]
            D = gpu(tA, tB, None if C is None else dev(C), out=out)
        torch.cuda.synchronize()
        assert D.data_ptr() == out.data_ptr(), what
        whole = host(buf)
        assert np.array_equal(whole[:M, :N].astype(np.float64), np.asarray(want, np.float64)), what + ": D differs"
        assert (whole[:, N:] == marker).all() and (whole[M:] == marker).all(), what + ": guard band written"
