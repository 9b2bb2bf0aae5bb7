"""The C ABI without a GPU: libmpdt.so loads, exports every function that
include/mpdt.h declares, and validates arguments on the host before touching
any device (invalid calls return their status and launch nothing; valid calls
on a machine with no GPU return MPDT_ERROR_NO_DEVICE)."""
import ctypes
import os
import re

import pytest
import torch

import mixed_precision_dense_tiled_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpdt.h")

SUCCESS, INVALID, MISALIGNED, ALIASING, NO_DEVICE, UNSUPPORTED, LAUNCH = range(7)

gpu_present = torch.cuda.is_available()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_five_operations():
    names = declared_functions()
    for op in ("gemm_f16", "gemm_bf16", "gemm_i8_i32", "gemm_fp8_blockscaled", "gemv_w8a8"):
        assert op in names


def test_library_exports_every_declared_symbol():
    L = mp.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert mp.version() == 100
    assert L.mpdt_status_string(0) == b"success"
    assert b"gfx950" in L.mpdt_status_string(UNSUPPORTED)


# Fake, never-dereferenced "device" addresses: validation must reject or
# accept them without any device access.
P = 1 << 40          # 16-byte aligned base
Q = P + (1 << 32)    # far away from P
R = P + (2 << 32)
R_ = P + (3 << 32)


def g16(M, N, K, A=P, lda=None, B=Q, ldb=None, C=None, ldc=None, D=R, ldd=None, fn="gemm_f16"):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    ldd = N if ldd is None else ldd
    return getattr(mp.lib(), fn)(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, None)


@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16"])
def test_gemm16_validation(fn):
    assert g16(-1, 4, 4, fn=fn) == INVALID
    assert g16(4, 4, (1 << 30) + 1, fn=fn) == INVALID
    assert g16(4, 4, 4, A=None, fn=fn) == INVALID
    assert g16(4, 4, 4, B=None, fn=fn) == INVALID
    assert g16(4, 4, 4, D=None, fn=fn) == INVALID
    assert g16(4, 4, 8, lda=7, fn=fn) == INVALID
    assert g16(4, 8, 4, ldb=7, fn=fn) == INVALID
    assert g16(4, 8, 4, ldd=7, fn=fn) == INVALID
    assert g16(4, 8, 4, C=P + (3 << 32), ldc=7, fn=fn) == INVALID
    assert g16(4, 4, 4, A=P + 1, fn=fn) == MISALIGNED
    assert g16(4, 4, 4, D=R + 2, fn=fn) == MISALIGNED
    # D overlapping A or B
    assert g16(4, 4, 4, D=P, fn=fn) == ALIASING
    assert g16(64, 64, 64, D=Q + 100 * 4, fn=fn) == ALIASING
    # C overlapping D other than exactly
    assert g16(8, 8, 8, C=R + 4, fn=fn) == ALIASING
    assert g16(8, 8, 8, C=R, ldc=9, ldd=8, fn=fn) == ALIASING
    # zero-size outputs are a no-op success, even with no device
    assert g16(0, 8, 8, fn=fn) == SUCCESS
    assert g16(8, 0, 8, fn=fn) == SUCCESS
    assert g16(0, 0, 0, A=None, B=None, D=None, fn=fn) == SUCCESS
    assert b"gemm" in mp.lib().mpdt_last_error()


@pytest.mark.skipif(gpu_present, reason="checks the no-device path")
def test_valid_calls_report_no_device():
    assert g16(8, 8, 8) == NO_DEVICE
    assert g16(8, 8, 8, C=R) == NO_DEVICE            # in place D == C is allowed
    assert g16(8, 8, 0, A=None, B=None) == NO_DEVICE  # K == 0 needs no A/B
    L = mp.lib()
    assert L.gemm_i8_i32(8, 8, 8, P + 1, 8, Q + 3, 8, None, 8, R, 8, None) == NO_DEVICE
    assert L.gemm_fp8_blockscaled(8, 8, 8, P, 8, Q, 1, P + 4096, 8, Q + 4096, 1, R, 8,
                                  None) == NO_DEVICE
    assert L.gemv_w8a8(1, 16, 64, P, ctypes.c_float(0.5), Q, 64, P + 4096, R, None,
                       None) == NO_DEVICE
    assert b"no HIP device" in L.mpdt_last_error()


@pytest.mark.parametrize("fn", ["gemm_f16_bias_act", "gemm_bf16_bias_act"])
def test_bias_act_validation(fn):
    L = mp.lib()
    S = R + (1 << 30)    # a bias array far from everything else

    def call(M=8, N=8, K=8, A=P, lda=8, B=Q, ldb=8, C=None, ldc=8, bias=S, act=2, D=R, ldd=8, d16=0):
        return getattr(L, fn)(M, N, K, A, lda, B, ldb, C, ldc, bias, act, D, ldd, d16, None)

    assert call(act=4) == INVALID
    assert call(act=-1) == INVALID
    assert call(d16=2) == INVALID
    assert call(lda=7) == INVALID
    assert call(bias=S + 2) == MISALIGNED
    assert call(D=R + 2) == MISALIGNED
    assert call(D=R + 2, d16=1) != MISALIGNED
    assert call(D=S) == ALIASING             # D over the bias
    assert call(D=S - 8 * 4 + 4) == ALIASING  # the last row of D over the bias's first value
    assert call(C=R, d16=1) == ALIASING       # a 16-bit D cannot be C
    assert call(M=0) == SUCCESS
    assert call(N=0, act=1) == SUCCESS
    if not gpu_present:
        assert call() == NO_DEVICE
        assert call(bias=None, act=0, C=R) == NO_DEVICE     # in place, no bias
        assert call(d16=1) == NO_DEVICE


def test_i8_validation():
    L = mp.lib()
    assert L.gemm_i8_i32(4, 4, 4, P, 4, Q, 4, None, 4, R + 1, 4, None) == MISALIGNED
    assert L.gemm_i8_i32(4, 4, 4, P, 4, Q, 4, P + 3, 4, R, 4, None) == MISALIGNED
    assert L.gemm_i8_i32(4, 4, 4, P, 3, Q, 4, None, 4, R, 4, None) == INVALID
    assert L.gemm_i8_i32(4, 4, 4, P, 4, Q, 4, None, 4, P, 4, None) == ALIASING


def test_fp8_validation():
    L = mp.lib()
    S1, S2 = P + 65536, Q + 65536
    ok = dict(M=256, N=300, K=260)
    kb, nb = 3, 3

    def call(M=256, N=300, K=260, A=P, lda=260, sa=S1, ldsa=kb, B=Q, ldb=300, sb=S2, ldsb=nb,
             D=R, ldd=300):
        return L.gemm_fp8_blockscaled(M, N, K, A, lda, sa, ldsa, B, ldb, sb, ldsb, D, ldd, None)

    assert call(ldsa=2) == INVALID
    assert call(ldsb=2) == INVALID
    assert call(sa=None) == INVALID
    assert call(sb=S2 + 2) == MISALIGNED
    assert call(D=R + 1) == MISALIGNED
    assert call(D=S1) == ALIASING          # D over the A scales
    assert call(M=0) == SUCCESS
    assert ok


def test_fp8_format_and_rowscaled_validation():
    L = mp.lib()
    S1, S2 = P + 65536, Q + 65536

    def blk(fa=0, fb=1, D=R):
        return L.gemm_fp8_blockscaled_fmt(256, 300, 260, P, 260, fa, S1, 3, Q, 300, fb, S2, 3, D, 300, None)

    def row(fa=1, fb=1, sa=S1, ia=1, sb=S2, ib=0, K=260, D=R):
        return L.gemm_fp8_rowscaled(256, 300, K, P, 260, fa, sa, ia, Q, 300, fb, sb, ib, D, 300, None)

    assert blk(fa=2) == INVALID and blk(fb=-1) == INVALID
    assert row(fa=3) == INVALID
    assert row(ia=2) == INVALID and row(ib=-1) == INVALID
    assert row(sa=None) == INVALID and row(sb=None, K=0) == INVALID   # read even for K = 0
    assert row(sb=S2 + 2) == MISALIGNED
    assert row(D=S1 - 2 * 300 * 255) == ALIASING                    # D's last row over scale_a
    assert row(D=S1 + 4 * 255 - 2 * 300 * 255 - 2) == ALIASING
    if not gpu_present:
        assert blk() == NO_DEVICE and row() == NO_DEVICE and row(ia=0, ib=1, K=0) == NO_DEVICE


def test_quantize_fp8_validation():
    L = mp.lib()

    def call(R=300, C=500, fmt=1, br=1, bc=500, S=Q, lds=1, Qo=R_):
        return L.quantize_fp8(R, C, P, 500, fmt, br, bc, Qo, 500, S, lds, None)

    assert call(fmt=2) == INVALID
    assert call(br=2, bc=64) == INVALID         # unsupported block shape
    assert call(br=0) == INVALID
    assert call(br=1, bc=128, lds=3) == INVALID  # lds < ceil(500/128)
    assert call(S=Q + 2) == MISALIGNED
    assert call(Qo=P + 100) == ALIASING
    assert call(R=0) == SUCCESS
    if not gpu_present:
        for br, bc, lds in ((1, 500, 1), (300, 1, 500), (300, 500, 1), (1, 128, 4), (128, 128, 4)):
            assert call(br=br, bc=bc, lds=lds) == NO_DEVICE


def test_gemv_validation():
    L = mp.lib()
    f = ctypes.c_float(0.25)
    assert L.gemv_w8a8(2, 16, 64, P, f, Q, 64, R, R + 4096, None, None) == INVALID  # M != 1
    assert L.gemv_w8a8(1, 16, 64, None, f, Q, 64, R, R + 4096, None, None) == INVALID
    assert L.gemv_w8a8(1, 16, 64, P, f, Q, 63, R, R + 4096, None, None) == INVALID
    assert L.gemv_w8a8(1, 16, 64, P, f, Q, 64, R + 2, R + 4096, None, None) == MISALIGNED
    assert L.gemv_w8a8(1, 16, 64, P, f, Q, 64, R, R + 4097, None, None) == MISALIGNED
    assert L.gemv_w8a8(1, 16, 64, P, f, Q, 64, R, Q + 32, None, None) == ALIASING    # y over W
    assert L.gemv_w8a8(1, 16, 64, P, f, Q, 64, R, R + 4096, R + 4100, None) == ALIASING
    assert L.gemv_w8a8(1, 0, 64, P, f, Q, 64, R, R + 4096, None, None) == SUCCESS


def test_w8a8_kn_validation():
    L = mp.lib()

    def call(M=4, N=16, K=64, ldw=16, Y=R, W=Q):
        return L.gemm_w8a8_kn(M, N, K, P, 64, P + 4096, W, ldw, Q + 65536, None, Y, 16, None, 16, None)

    assert call(ldw=15) == INVALID                     # K x N: ldw >= N
    assert call(Y=Q + 16 * 63) == ALIASING             # Y over the last row of W (K x N)
    assert call(Y=Q + 16 * 64) != ALIASING
    if not gpu_present:
        assert call() == NO_DEVICE and call(ldw=20) == NO_DEVICE


def test_w8a8_requant_validation():
    L = mp.lib()
    f = ctypes.c_float

    def call(M=4, N=16, K=64, X=P, ldx=64, sx=P + 4096, W=Q, ldw=64, sw=Q + 65536, bias=None,
             s=f(0.5), Qo=R, ldq=16, Z=None, ldz=16):
        return L.gemm_w8a8_requant(M, N, K, X, ldx, sx, W, ldw, sw, bias, s, Qo, ldq, Z, ldz, None)

    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert call(s=f(bad)) == INVALID
    assert call(ldq=15) == INVALID
    assert call(Qo=None) == INVALID
    assert call(sw=Q + 65538) == MISALIGNED
    assert call(Qo=R + 1) != MISALIGNED               # INT8 output: any byte address
    assert call(Qo=Q + 64) == ALIASING                # Q over W
    assert call(Z=R + 8, ldz=16) == ALIASING          # Z over Q
    assert call(M=0) == SUCCESS
    if not gpu_present:
        assert call() == NO_DEVICE


def test_binding_raises_on_status():
    with pytest.raises((mp.MpdtError, ValueError, RuntimeError)):
        mp.gemm_f16(torch.zeros(4, 4, dtype=torch.float16), torch.zeros(4, 4, dtype=torch.float16))
