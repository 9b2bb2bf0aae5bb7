"""ctypes front of the plain CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the HIP
library and its binding) never imports this package.

Arrays are numpy arrays.  Two-dimensional operands may be row-strided views
(leading dimension = ``strides[0] / itemsize``) but must have unit element
stride.  Each wrapper names the C function it forwards to; the C source states
the definition each one follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MPDT_ORACLE_LIB names another build of oracle.c (the test-suite's sanitizer
# build); by default the in-tree one.
LIB_PATH = os.environ.get("MPDT_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"oracle library missing: {LIB_PATH}; build it with __graft_entry__.build()")
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.oracle_f16_to_f64.restype = ctypes.c_double
        _lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        _lib.oracle_bf16_to_f64.restype = ctypes.c_double
        _lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        _lib.oracle_e4m3_to_f64.restype = ctypes.c_double
        _lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        _lib.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
        _lib.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        for name in ("oracle_decode_f16", "oracle_decode_bf16", "oracle_decode_e4m3", "oracle_decode_e5m2",
                     "oracle_round_bf16"):
            fn = getattr(_lib, name)
            fn.restype = None
            fn.argtypes = [_vp, _vp, _c_i64]
        for name in ("oracle_gemm_f16", "oracle_gemm_bf16"):
            fn = getattr(_lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [_c_i64] * 3 + [_vp, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp, _vp]
        for name in ("oracle_gemm_f16_at", "oracle_gemm_bf16_at"):
            fn = getattr(_lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = ([_c_i64] * 3 + [_vp, _c_i64, _vp, _c_i64, _vp, _c_i64]
                           + [_c_i64, _vp, _vp, _vp, _vp])
        _lib.oracle_gemm_f16_intexact.restype = ctypes.c_int
        _lib.oracle_gemm_f16_intexact.argtypes = ([_c_i64] * 3
                                                  + [_vp, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp])
        _lib.oracle_gemm_i8_i32.restype = ctypes.c_int
        _lib.oracle_gemm_i8_i32.argtypes = [_c_i64] * 3 + [_vp, _c_i64, _vp, _c_i64, _vp, _c_i64,
                                                           _vp]
        _lib.oracle_gemm_i8_i32_at.restype = ctypes.c_int
        _lib.oracle_gemm_i8_i32_at.argtypes = ([_c_i64] * 3
                                               + [_vp, _c_i64, _vp, _c_i64, _vp, _c_i64]
                                               + [_c_i64, _vp, _vp, _vp])
        _lib.oracle_gemm_fp8_blockscaled.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_blockscaled.argtypes = ([_c_i64] * 3
                                                     + [_vp, _c_i64, _vp, _c_i64]
                                                     + [_vp, _c_i64, _vp, _c_i64, _vp, _vp])
        _lib.oracle_gemm_fp8_blockscaled_at.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_blockscaled_at.argtypes = ([_c_i64] * 3
                                                        + [_vp, _c_i64, _vp, _c_i64]
                                                        + [_vp, _c_i64, _vp, _c_i64]
                                                        + [_c_i64, _vp, _vp, _vp, _vp])
        _lib.oracle_f32_to_f16_rne.restype = ctypes.c_uint16
        _lib.oracle_f32_to_f16_rne.argtypes = [ctypes.c_float]
        _lib.oracle_f32_to_e5m2_rne_sat.restype = ctypes.c_uint8
        _lib.oracle_f32_to_e5m2_rne_sat.argtypes = [ctypes.c_float]
        _lib.oracle_e5m2_to_f64.restype = ctypes.c_double
        _lib.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
        _lib.oracle_gemm_fp8_blockscaled_fmt.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_blockscaled_fmt.argtypes = ([_c_i64] * 3
                                                         + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
                                                         + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
                                                         + [_vp, _vp])
        _lib.oracle_gemm_fp8_blockscaled_fmt_at.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_blockscaled_fmt_at.argtypes = (
            [_c_i64] * 3 + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
            + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64] + [_c_i64, _vp, _vp, _vp, _vp])
        _lib.oracle_gemm_fp8_rowscaled.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_rowscaled.argtypes = ([_c_i64] * 3
                                                   + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
                                                   + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
                                                   + [_vp, _vp])
        _lib.oracle_gemm_fp8_rowscaled_at.restype = ctypes.c_int
        _lib.oracle_gemm_fp8_rowscaled_at.argtypes = (
            [_c_i64] * 3 + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64]
            + [_vp, _c_i64, ctypes.c_int, _vp, _c_i64] + [_c_i64, _vp, _vp, _vp, _vp])
        _lib.oracle_quantize_fp8_blocks_fmt.restype = ctypes.c_int
        _lib.oracle_quantize_fp8_blocks_fmt.argtypes = ([_c_i64, _c_i64, _vp, _c_i64, ctypes.c_int]
                                                        + [_c_i64, _c_i64, _vp, _c_i64, _vp, _c_i64])
        _lib.oracle_f32_to_e4m3_rne_sat.restype = ctypes.c_uint8
        _lib.oracle_f32_to_e4m3_rne_sat.argtypes = [ctypes.c_float]
        _lib.oracle_gemm_w8a8.restype = ctypes.c_int
        _lib.oracle_gemm_w8a8.argtypes = ([_c_i64] * 3 + [_vp, _c_i64, _vp, _vp, _c_i64, _vp, _vp]
                                          + [_vp, _c_i64, _vp, _c_i64])
        _lib.oracle_gemm_w8a8_requant.restype = ctypes.c_int
        _lib.oracle_gemm_w8a8_requant.argtypes = ([_c_i64] * 3
                                                  + [_vp, _c_i64, _vp, _vp, _c_i64, _vp, _vp]
                                                  + [ctypes.c_float, _vp, _c_i64, _vp, _c_i64])
        _lib.oracle_quantize_i8_rows.restype = ctypes.c_int
        _lib.oracle_quantize_i8_rows.argtypes = [_c_i64, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp]
        _lib.oracle_quantize_fp8_blocks.restype = ctypes.c_int
        _lib.oracle_quantize_fp8_blocks.argtypes = ([_c_i64, _c_i64, _vp, _c_i64, _c_i64, _c_i64]
                                                    + [_vp, _c_i64, _vp, _c_i64])
        _lib.oracle_bias_act.restype = ctypes.c_int
        _lib.oracle_bias_act.argtypes = [_c_i64, _c_i64, _vp, _c_i64, _vp, ctypes.c_int]
        _lib.oracle_gemv_w8a8.restype = ctypes.c_int
        _lib.oracle_gemv_w8a8.argtypes = [_c_i64, _c_i64, _vp, ctypes.c_float, _vp, _c_i64, _vp,
                                          _vp, _vp]
    return _lib


class OracleError(RuntimeError):
    pass


_ERRORS = {1: "invalid argument", 2: "non-finite input", 3: "INT32 overflow",
           4: "non-integer input"}


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERRORS.get(rc, rc)}")


def _mat(x: np.ndarray, dtype) -> tuple[int, int]:
    """Pointer and leading dimension (elements) of a row-major 2-D operand."""
    if x.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {x.dtype}")
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    item = x.itemsize
    if x.size == 0:
        return x.ctypes.data, max(int(x.shape[1]), 1)
    if x.shape[1] > 1 and x.strides[1] != item:
        raise ValueError("unit element stride required")
    ld = x.strides[0] // item if x.shape[0] > 1 else max(x.shape[1], 1)
    if x.shape[0] > 1 and x.strides[0] % item:
        raise ValueError("row stride must be a whole number of elements")
    return x.ctypes.data, int(ld)


def _ptr(x):
    return None if x is None else x.ctypes.data


# ---------------------------------------------------------------- formats --
def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_f16(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_bf16(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def e4m3_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_e4m3(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def e5m2_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_decode_e5m2(bits.ctypes.data, out.ctypes.data, bits.size)
    return out


E4M3, E5M2 = 0, 1


def fp8_to_f64(bits, fmt):
    return e4m3_to_f64(bits) if fmt == E4M3 else e5m2_to_f64(bits)


def f32_to_e5m2_rne_sat(x: np.ndarray) -> np.ndarray:
    """oracle_f32_to_e5m2_rne_sat elementwise (E5M2 codes)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().oracle_f32_to_e5m2_rne_sat
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def f32_to_f16_rne(x: np.ndarray) -> np.ndarray:
    """oracle_f32_to_f16_rne elementwise (FP16 bit patterns)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().oracle_f32_to_f16_rne
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f32_to_e4m3_rne_sat(x: np.ndarray) -> np.ndarray:
    """oracle_f32_to_e4m3_rne_sat elementwise (E4M3FN codes)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().oracle_f32_to_e4m3_rne_sat
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


# ------------------------------------------------------------------ GEMMs --
def _gemm16(fn_name, A, B, C):
    lib = _load()
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    pa, lda = _mat(A, np.uint16)
    pb, ldb = _mat(B, np.uint16)
    pc, ldc = (None, 0) if C is None else _mat(C, np.float32)
    R = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _check(getattr(lib, fn_name)(M, N, K, pa, lda, pb, ldb, pc, ldc, R.ctypes.data,
                                 S.ctypes.data), fn_name)
    return R, S


def gemm_f16(A, B, C=None):
    """``oracle_gemm_f16``: (R, S) with R = A.B + C in FP64 and S = sum |a.b|."""
    return _gemm16("oracle_gemm_f16", A, B, C)


def gemm_bf16(A, B, C=None):
    """``oracle_gemm_bf16``: (R, S) as :func:`gemm_f16` for BF16 bit patterns."""
    return _gemm16("oracle_gemm_bf16", A, B, C)


def _gemm16_at(fn_name, A, B, C, ii, jj):
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint16)
    pb, ldb = _mat(B, np.uint16)
    pc, ldc = (None, 0) if C is None else _mat(C, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    R = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(getattr(lib, fn_name)(M, N, K, pa, lda, pb, ldb, pc, ldc, ii.size, ii.ctypes.data,
                                 jj.ctypes.data, R.ctypes.data, S.ctypes.data), fn_name)
    return R, S


def gemm_f16_at(A, B, C, ii, jj):
    """``oracle_gemm_f16_at``: R, S at output positions (ii[p], jj[p])."""
    return _gemm16_at("oracle_gemm_f16_at", A, B, C, ii, jj)


def gemm_bf16_at(A, B, C, ii, jj):
    """``oracle_gemm_bf16_at``: R, S at output positions (ii[p], jj[p])."""
    return _gemm16_at("oracle_gemm_bf16_at", A, B, C, ii, jj)


def gemm_f16_intexact(A, B, C=None):
    """``oracle_gemm_f16_intexact``: FP32 D = fl32(exact integer sum + C)."""
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint16)
    pb, ldb = _mat(B, np.uint16)
    pc, ldc = (None, 0) if C is None else _mat(C, np.float32)
    D = np.empty((M, N), np.float32)
    _check(lib.oracle_gemm_f16_intexact(M, N, K, pa, lda, pb, ldb, pc, ldc, D.ctypes.data),
           "oracle_gemm_f16_intexact")
    return D


def gemm_i8_i32(A, B, C=None):
    """``oracle_gemm_i8_i32``: exact INT32 D = A.B + C."""
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.int8)
    pb, ldb = _mat(B, np.int8)
    pc, ldc = (None, 0) if C is None else _mat(C, np.int32)
    D = np.empty((M, N), np.int32)
    _check(lib.oracle_gemm_i8_i32(M, N, K, pa, lda, pb, ldb, pc, ldc, D.ctypes.data),
           "oracle_gemm_i8_i32")
    return D


def gemm_i8_i32_at(A, B, C, ii, jj):
    """``oracle_gemm_i8_i32_at``: exact INT32 D at output positions (ii[p], jj[p])."""
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.int8)
    pb, ldb = _mat(B, np.int8)
    pc, ldc = (None, 0) if C is None else _mat(C, np.int32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    D = np.empty(ii.shape, np.int32)
    _check(lib.oracle_gemm_i8_i32_at(M, N, K, pa, lda, pb, ldb, pc, ldc, ii.size,
                                     ii.ctypes.data, jj.ctypes.data, D.ctypes.data),
           "oracle_gemm_i8_i32_at")
    return D


def gemm_fp8_blockscaled(A, sA, B, sB):
    """``oracle_gemm_fp8_blockscaled``: (R, S) in FP64 for E4M3 bytes with
    1x128 A scales and 128x128 B scales."""
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    psa, ldsa = _mat(sA, np.float32)
    psb, ldsb = _mat(sB, np.float32)
    R = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _check(lib.oracle_gemm_fp8_blockscaled(M, N, K, pa, lda, psa, ldsa, pb, ldb, psb, ldsb,
                                           R.ctypes.data, S.ctypes.data),
           "oracle_gemm_fp8_blockscaled")
    return R, S


def gemm_fp8_blockscaled_fmt(A, fmt_a, sA, B, fmt_b, sB):
    """``oracle_gemm_fp8_blockscaled_fmt``: as gemm_fp8_blockscaled with each
    operand's format given (E4M3 or E5M2)."""
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    psa, ldsa = _mat(sA, np.float32)
    psb, ldsb = _mat(sB, np.float32)
    R = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _check(_load().oracle_gemm_fp8_blockscaled_fmt(M, N, K, pa, lda, int(fmt_a), psa, ldsa, pb, ldb,
                                                   int(fmt_b), psb, ldsb, R.ctypes.data, S.ctypes.data),
           "oracle_gemm_fp8_blockscaled_fmt")
    return R, S


def gemm_fp8_blockscaled_fmt_at(A, fmt_a, sA, B, fmt_b, sB, ii, jj):
    """``oracle_gemm_fp8_blockscaled_fmt_at``: R, S at (ii[p], jj[p])."""
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    psa, ldsa = _mat(sA, np.float32)
    psb, ldsb = _mat(sB, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    R = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(_load().oracle_gemm_fp8_blockscaled_fmt_at(M, N, K, pa, lda, int(fmt_a), psa, ldsa, pb, ldb,
                                                      int(fmt_b), psb, ldsb, ii.size, ii.ctypes.data,
                                                      jj.ctypes.data, R.ctypes.data, S.ctypes.data),
           "oracle_gemm_fp8_blockscaled_fmt_at")
    return R, S


def gemm_fp8_rowscaled(A, fmt_a, sA, B, fmt_b, sB):
    """``oracle_gemm_fp8_rowscaled``: (R, S) with R = sA[i] sB[j] sum_k a b in
    FP64; sA holds M values (or 1: per tensor), sB N values (or 1)."""
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    sA = np.ascontiguousarray(sA, np.float32).ravel()
    sB = np.ascontiguousarray(sB, np.float32).ravel()
    inc_a = 0 if sA.size == 1 and M != 1 else 1
    inc_b = 0 if sB.size == 1 and N != 1 else 1
    R = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _check(_load().oracle_gemm_fp8_rowscaled(M, N, K, pa, lda, int(fmt_a), sA.ctypes.data, inc_a, pb,
                                             ldb, int(fmt_b), sB.ctypes.data, inc_b, R.ctypes.data,
                                             S.ctypes.data),
           "oracle_gemm_fp8_rowscaled")
    return R, S


def gemm_fp8_rowscaled_at(A, fmt_a, sA, B, fmt_b, sB, ii, jj):
    """``oracle_gemm_fp8_rowscaled_at``: R, S at (ii[p], jj[p])."""
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    sA = np.ascontiguousarray(sA, np.float32).ravel()
    sB = np.ascontiguousarray(sB, np.float32).ravel()
    inc_a = 0 if sA.size == 1 and M != 1 else 1
    inc_b = 0 if sB.size == 1 and N != 1 else 1
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    R = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(_load().oracle_gemm_fp8_rowscaled_at(M, N, K, pa, lda, int(fmt_a), sA.ctypes.data, inc_a,
                                                pb, ldb, int(fmt_b), sB.ctypes.data, inc_b, ii.size,
                                                ii.ctypes.data, jj.ctypes.data, R.ctypes.data,
                                                S.ctypes.data),
           "oracle_gemm_fp8_rowscaled_at")
    return R, S


def gemm_fp8_blockscaled_at(A, sA, B, sB, ii, jj):
    """``oracle_gemm_fp8_blockscaled_at``: R, S at output positions (ii[p], jj[p])."""
    lib = _load()
    M, K = A.shape
    N = B.shape[1]
    pa, lda = _mat(A, np.uint8)
    pb, ldb = _mat(B, np.uint8)
    psa, ldsa = _mat(sA, np.float32)
    psb, ldsb = _mat(sB, np.float32)
    ii = np.ascontiguousarray(ii, np.int64)
    jj = np.ascontiguousarray(jj, np.int64)
    R = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _check(lib.oracle_gemm_fp8_blockscaled_at(M, N, K, pa, lda, psa, ldsa, pb, ldb, psb, ldsb,
                                              ii.size, ii.ctypes.data, jj.ctypes.data,
                                              R.ctypes.data, S.ctypes.data),
           "oracle_gemm_fp8_blockscaled_at")
    return R, S


def gemv_w8a8(x, s_x, W, s_w):
    """``oracle_gemv_w8a8``: (z INT32 [N], y BF16 bits [N]) for W stored N x K."""
    lib = _load()
    N, K = W.shape
    x = np.ascontiguousarray(x, np.int8)
    assert x.size == K
    pw, ldw = _mat(W, np.int8)
    s_w = np.ascontiguousarray(s_w, np.float32)
    z = np.empty(N, np.int32)
    y = np.empty(N, np.uint16)
    _check(lib.oracle_gemv_w8a8(N, K, x.ctypes.data, float(np.float32(s_x)), pw, ldw,
                                s_w.ctypes.data, z.ctypes.data, y.ctypes.data),
           "oracle_gemv_w8a8")
    return z, y


# ------------------------------------------------------ W8A8, M tokens --
def gemm_w8a8(X, s_x, W, s_w, bias=None):
    """oracle_gemm_w8a8: X int8 [M, K], s_x FP32 [M], W int8 [N, K] (one
    output channel per row), s_w FP32 [N], bias FP32 [N] or None.
    Returns (Z int32 [M, N], Y BF16 bits [M, N])."""
    M, K = X.shape
    N = W.shape[0]
    px, ldx = _mat(X, np.int8)
    pw, ldw = _mat(W, np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    Z = np.empty((M, N), np.int32)
    Y = np.empty((M, N), np.uint16)
    _check(_load().oracle_gemm_w8a8(M, N, K, px, ldx, s_x.ctypes.data, pw, ldw, s_w.ctypes.data,
                                    _ptr(b), Z.ctypes.data, max(N, 1), Y.ctypes.data, max(N, 1)),
           "gemm_w8a8")
    return Z, Y


# ------------------------------------------------- bias + activation --
ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3


def bias_act(R, bias, act):
    """oracle_bias_act on a copy of the FP64 matrix R: act(R + bias[j])."""
    R = np.array(R, dtype=np.float64, order="C", copy=True)
    M, N = R.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(_load().oracle_bias_act(M, N, R.ctypes.data, max(N, 1), _ptr(b), int(act)),
           "oracle_bias_act")
    return R


def gemm16_bias_act(fmt, A, B, C, bias, act):
    """FP16 ("f16") / BF16 ("bf16") GEMM followed by the bias and activation
    epilogue.  Returns (R, S, P): R = act(A.B + C + bias) in FP64, S the
    GEMM's sum |a.b| and P = A.B + C + bias (the value the activation sees)."""
    R0, S = (gemm_f16 if fmt == "f16" else gemm_bf16)(A, B, C)
    return bias_act(R0, bias, act), S, bias_act(R0, bias, ACT_NONE)


def gemm16_bias_act_at(fmt, A, B, C, bias, act, ii, jj):
    """gemm16_bias_act at output positions (ii[p], jj[p]) only."""
    R0, S = (gemm_f16_at if fmt == "f16" else gemm_bf16_at)(A, B, C, ii, jj)
    bj = None if bias is None else np.asarray(bias, np.float32)[np.asarray(jj)]
    # one row of P sampled points, each with its own column's bias
    row = R0.reshape(1, -1)
    bb = None if bj is None else bj.reshape(-1)
    return (bias_act(row, bb, act).reshape(R0.shape), S,
            bias_act(row, bb, ACT_NONE).reshape(R0.shape))


def gemm_w8a8_requant(X, s_x, W, s_w, bias, s_out):
    """oracle_gemm_w8a8_requant: as gemm_w8a8, with the FP32 value requantised
    to INT8 by one output scale.  Returns (Z int32 [M, N], Q int8 [M, N])."""
    M, K = X.shape
    N = W.shape[0]
    px, ldx = _mat(X, np.int8)
    pw, ldw = _mat(W, np.int8)
    s_x = np.ascontiguousarray(s_x, dtype=np.float32)
    s_w = np.ascontiguousarray(s_w, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    Z = np.empty((M, N), np.int32)
    Q = np.empty((M, N), np.int8)
    _check(_load().oracle_gemm_w8a8_requant(M, N, K, px, ldx, s_x.ctypes.data, pw, ldw,
                                            s_w.ctypes.data, _ptr(b), float(np.float32(s_out)),
                                            Z.ctypes.data, max(N, 1), Q.ctypes.data, max(N, 1)),
           "gemm_w8a8_requant")
    return Z, Q


# ------------------------------------------------------------ quantisers --
def quantize_i8_rows(X):
    """oracle_quantize_i8_rows: X BF16 bits [M, K] -> (Q int8 [M, K], S FP32 [M])."""
    M, K = X.shape
    px, ldx = _mat(X, np.uint16)
    Q = np.empty((M, K), np.int8)
    S = np.empty(M, np.float32)
    _check(_load().oracle_quantize_i8_rows(M, K, px, ldx, Q.ctypes.data, max(K, 1), S.ctypes.data),
           "quantize_i8_rows")
    return Q, S


def quantize_fp8_blocks_fmt(X, fmt, br, bc):
    """oracle_quantize_fp8_blocks_fmt: X FP32 [R, C] in br x bc blocks, into
    E4M3 (fmt 0) or E5M2 (fmt 1) -> (Q codes [R, C], S FP32 [ceil(R/br), ceil(C/bc)])."""
    R, Cc = X.shape
    px, ldx = _mat(X, np.float32)
    Q = np.empty((R, Cc), np.uint8)
    nbr, nbc = -(-R // br), -(-Cc // bc)
    S = np.empty((nbr, nbc), np.float32)
    _check(_load().oracle_quantize_fp8_blocks_fmt(R, Cc, px, ldx, int(fmt), br, bc, Q.ctypes.data,
                                                  max(Cc, 1), S.ctypes.data, max(nbc, 1)),
           "quantize_fp8_blocks_fmt")
    return Q, S


def quantize_fp8_blocks(X, br, bc=128):
    """oracle_quantize_fp8_blocks: X FP32 [R, C] in br x bc blocks ->
    (Q E4M3 codes [R, C], S FP32 [ceil(R/br), ceil(C/bc)])."""
    R, Cc = X.shape
    px, ldx = _mat(X, np.float32)
    Q = np.empty((R, Cc), np.uint8)
    nbr, nbc = -(-R // br), -(-Cc // bc)
    S = np.empty((nbr, nbc), np.float32)
    _check(_load().oracle_quantize_fp8_blocks(R, Cc, px, ldx, br, bc, Q.ctypes.data, max(Cc, 1),
                                              S.ctypes.data, max(nbc, 1)),
           "quantize_fp8_blocks")
    return Q, S
