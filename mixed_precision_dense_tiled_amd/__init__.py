"""Python binding of libmpdt.so, the gfx950 library of tiled mixed-precision
multiply-accumulate kernels (see include/mpdt.h for the C ABI).

The functions here only marshal arguments: they take torch tensors that live
on the GPU, read their data pointers and leading dimensions, allocate outputs
with torch when none is given, and call the C entry point of the same name on
torch's current stream.  All arithmetic runs in the HIP kernels; there is no
fallback of any kind.  If the native library is missing, every call raises.

Bit-pattern operands may be passed with any 2-byte dtype (float16, bfloat16,
int16, uint16) for the 16-bit GEMMs and any 1-byte dtype (uint8, int8,
float8_e4m3fn) for FP8; only the bytes are used.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gemm_f16", "gemm_bf16", "gemm_f16_f16out", "gemm_bf16_bf16out", "gemm_f16_bias_act",
           "gemm_bf16_bias_act", "ACT_NONE", "ACT_RELU", "ACT_GELU", "ACT_SILU", "gemm_i8_i32",
           "gemm_fp8_blockscaled", "gemm_fp8_blockscaled_fmt", "gemm_fp8_rowscaled", "FP8_E4M3",
           "FP8_E5M2", "gemv_w8a8", "gemm_w8a8", "gemm_w8a8_kn", "gemm_w8a8_requant", "quantize_i8_rows",
           "quantize_fp8_blocks", "quantize_fp8",
           "MpdtError", "lib", "lib_path", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# MPDT_LIB_PATH names another build of the same library (the test-suite's
# sanitizer build of the host code, for one); by default the in-tree one.
_LIB_PATH = os.environ.get("MPDT_LIB_PATH") or os.path.join(_HERE, "libmpdt.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class MpdtError(RuntimeError):
    """Raised when a libmpdt entry point returns a non-success status."""

    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded native library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"native library not built: {_LIB_PATH} is missing "
                "(run `python -m mixed_precision_dense_tiled_amd.build`)")
        L = ctypes.CDLL(_LIB_PATH)
        gemm_args = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
        for name in ("gemm_f16", "gemm_bf16", "gemm_i8_i32", "gemm_f16_f16out",
                     "gemm_bf16_bf16out"):
            getattr(L, name).argtypes = gemm_args
            getattr(L, name).restype = ctypes.c_int
        for name in ("gemm_f16_bias_act", "gemm_bf16_bias_act"):
            getattr(L, name).argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                         ctypes.c_int, _vp, _i64, ctypes.c_int, _vp]
            getattr(L, name).restype = ctypes.c_int
        L.gemm_fp8_blockscaled.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                           _i64, _vp, _i64, _vp]
        L.gemm_fp8_blockscaled.restype = ctypes.c_int
        L.gemm_fp8_blockscaled_fmt.argtypes = [_i64, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _i64,
                                               _vp, _i64, ctypes.c_int, _vp, _i64, _vp, _i64, _vp]
        L.gemm_fp8_blockscaled_fmt.restype = ctypes.c_int
        L.gemm_fp8_rowscaled.argtypes = [_i64, _i64, _i64, _vp, _i64, ctypes.c_int, _vp, _i64,
                                         _vp, _i64, ctypes.c_int, _vp, _i64, _vp, _i64, _vp]
        L.gemm_fp8_rowscaled.restype = ctypes.c_int
        L.gemv_w8a8.argtypes = [_i64, _i64, _i64, _vp, ctypes.c_float, _vp, _i64, _vp, _vp, _vp,
                                _vp]
        L.gemv_w8a8.restype = ctypes.c_int
        L.gemm_w8a8.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _i64,
                                _vp, _i64, _vp]
        L.gemm_w8a8.restype = ctypes.c_int
        L.gemm_w8a8_kn.argtypes = L.gemm_w8a8.argtypes
        L.gemm_w8a8_kn.restype = ctypes.c_int
        L.gemm_w8a8_requant.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp,
                                         ctypes.c_float, _vp, _i64, _vp, _i64, _vp]
        L.gemm_w8a8_requant.restype = ctypes.c_int
        L.quantize_i8_rows.argtypes = [_i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]
        L.quantize_i8_rows.restype = ctypes.c_int
        L.quantize_fp8_blocks.argtypes = [_i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]
        L.quantize_fp8_blocks.restype = ctypes.c_int
        L.quantize_fp8.argtypes = [_i64, _i64, _vp, _i64, ctypes.c_int, _i64, _i64, _vp, _i64, _vp,
                                   _i64, _vp]
        L.quantize_fp8.restype = ctypes.c_int
        L.mpdt_status_string.argtypes = [ctypes.c_int]
        L.mpdt_status_string.restype = ctypes.c_char_p
        L.mpdt_last_error.argtypes = []
        L.mpdt_last_error.restype = ctypes.c_char_p
        L.mpdt_version.argtypes = []
        L.mpdt_version.restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> int:
    return lib().mpdt_version()


def _check(fn: str, status: int):
    if status != 0:
        raise MpdtError(fn, status, lib().mpdt_last_error().decode())


# torch's current stream on a device, as the raw HIP stream handle: the
# direct accessor where this torch has it (a tenth of the public route's host
# time), else the public one.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _mat(t: torch.Tensor, itemsize: int, name: str):
    """(pointer, leading dimension in elements) of a row-major 2-D tensor."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.element_size() != itemsize:
        raise TypeError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    rows, cols = t.shape
    if rows == 0 or cols == 0:
        # an empty operand: nothing is read or written through it
        return t.data_ptr(), max(cols, 1)
    s0, s1 = t.stride()
    if cols > 1 and s1 != 1:
        raise ValueError(f"{name} must have unit stride along its rows")
    return t.data_ptr(), s0 if rows > 1 else max(cols, 1)


def _shape(t, shape, name):
    """Raise ValueError unless tensor t (or None) has exactly this shape.
    The C ABI sees only pointers and leading dimensions, so this is the one
    place where a buffer too small for the problem can be caught before a
    kernel reads or writes past it."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(ref, *ts):
    d = ref.get_device()
    for name, t in ts:
        if t is not None and t.get_device() != d:
            raise ValueError(f"{name} is on {t.device}, the operands on {ref.device}")


def _dims2(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return tuple(t.shape)


def _cdiv(a, b):
    return -(-a // b)


def _gemm16(fn, A, B, C, out, out_dtype=torch.float32):
    M, K = _dims2(A, "A")
    K2, N = _dims2(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _shape(C, (M, N), "C")
    _shape(out, (M, N), "out")
    _same_device(A, ("B", B), ("C", C), ("out", out))
    pa, lda = _mat(A, 2, "A")
    pb, ldb = _mat(B, 2, "B")
    pc, ldc = (None, N) if C is None else _mat(C, 4, "C")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    pd, ldd = _mat(out, out_dtype.itemsize, "out")
    _check(fn, getattr(lib(), fn)(M, N, K, pa, lda, pb, ldb, pc, ldc, pd, ldd, _stream(A)))
    return out


def gemm_f16(A, B, C=None, out=None):
    """D = A . B + C; A [M,K], B [K,N] FP16 bits, C/D [M,N] FP32 (C optional)."""
    return _gemm16("gemm_f16", A, B, C, out)


def gemm_bf16(A, B, C=None, out=None):
    """D = A . B + C; A [M,K], B [K,N] BF16 bits, C/D [M,N] FP32 (C optional)."""
    return _gemm16("gemm_bf16", A, B, C, out)


def gemm_f16_f16out(A, B, C=None, out=None):
    """D = fp16(A . B + C); A [M,K], B [K,N] FP16 bits, C [M,N] FP32 (optional);
    returns D as a float16 tensor."""
    return _gemm16("gemm_f16_f16out", A, B, C, out, torch.float16)


def gemm_bf16_bf16out(A, B, C=None, out=None):
    """D = bf16(A . B + C); A [M,K], B [K,N] BF16 bits, C [M,N] FP32 (optional);
    returns D as a bfloat16 tensor."""
    return _gemm16("gemm_bf16_bf16out", A, B, C, out, torch.bfloat16)


# activations of the fused epilogue (mpdt_act)
ACT_NONE, ACT_RELU, ACT_GELU, ACT_SILU = 0, 1, 2, 3


def _gemm16_bias_act(fn, A, B, C, bias, act, out, out_dtype):
    M, K = _dims2(A, "A")
    K2, N = _dims2(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _shape(C, (M, N), "C")
    _shape(bias, (N,), "bias")
    _shape(out, (M, N), "out")
    _same_device(A, ("B", B), ("C", C), ("bias", bias), ("out", out))
    pa, lda = _mat(A, 2, "A")
    pb, ldb = _mat(B, 2, "B")
    pc, ldc = (None, N) if C is None else _mat(C, 4, "C")
    if bias is not None:
        if bias.dim() != 1 or bias.numel() != N or bias.element_size() != 4 or not bias.is_cuda:
            raise ValueError("bias must be a GPU tensor of N 4-byte values")
        if N > 1 and bias.stride(0) != 1:
            raise ValueError("bias must be contiguous")
    pbias = None if bias is None else bias.data_ptr()
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    d16 = out.element_size() == 2
    pd, ldd = _mat(out, 2 if d16 else 4, "out")
    _check(fn, getattr(lib(), fn)(M, N, K, pa, lda, pb, ldb, pc, ldc, pbias, int(act), pd, ldd,
                                  int(d16), _stream(A)))
    return out


def gemm_f16_bias_act(A, B, C=None, bias=None, act=ACT_NONE, out=None, d16=False):
    """D = act(A . B + C + bias); A [M,K], B [K,N] FP16 bits, C [M,N] FP32 and
    bias [N] FP32 (both optional); D FP32, or FP16 with d16 (or a 2-byte out)."""
    return _gemm16_bias_act("gemm_f16_bias_act", A, B, C, bias, act, out,
                            torch.float16 if d16 else torch.float32)


def gemm_bf16_bias_act(A, B, C=None, bias=None, act=ACT_NONE, out=None, d16=False):
    """D = act(A . B + C + bias); A [M,K], B [K,N] BF16 bits, C [M,N] FP32 and
    bias [N] FP32 (both optional); D FP32, or BF16 with d16 (or a 2-byte out)."""
    return _gemm16_bias_act("gemm_bf16_bias_act", A, B, C, bias, act, out,
                            torch.bfloat16 if d16 else torch.float32)


def gemm_i8_i32(A, B, C=None, out=None):
    """D = A . B + C; A [M,K], B [K,N] INT8, C/D [M,N] INT32 (C optional)."""
    M, K = _dims2(A, "A")
    K2, N = _dims2(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _shape(C, (M, N), "C")
    _shape(out, (M, N), "out")
    _same_device(A, ("B", B), ("C", C), ("out", out))
    pa, lda = _mat(A, 1, "A")
    pb, ldb = _mat(B, 1, "B")
    pc, ldc = (None, N) if C is None else _mat(C, 4, "C")
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=A.device)
    pd, ldd = _mat(out, 4, "out")
    _check("gemm_i8_i32", lib().gemm_i8_i32(M, N, K, pa, lda, pb, ldb, pc, ldc, pd, ldd,
                                            _stream(A)))
    return out


def _fp8_blockscaled_shapes(A, scale_a, B, scale_b, out):
    """(M, N, K) of a block-scaled FP8 call; the scale grids must be exactly
    [M, ceil(K/128)] and [ceil(K/128), ceil(N/128)]."""
    M, K = _dims2(A, "A")
    K2, N = _dims2(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _shape(scale_a, (M, _cdiv(K, 128)), "scale_a")
    _shape(scale_b, (_cdiv(K, 128), _cdiv(N, 128)), "scale_b")
    _shape(out, (M, N), "out")
    _same_device(A, ("B", B), ("scale_a", scale_a), ("scale_b", scale_b), ("out", out))
    return M, N, K


def gemm_fp8_blockscaled(A, scale_a, B, scale_b, out=None):
    """BF16 D = block-scaled E4M3 A [M,K] . B [K,N]; scale_a [M, ceil(K/128)],
    scale_b [ceil(K/128), ceil(N/128)] FP32.  Returns D as a bfloat16 tensor."""
    M, N, K = _fp8_blockscaled_shapes(A, scale_a, B, scale_b, out)
    pa, lda = _mat(A, 1, "A")
    pb, ldb = _mat(B, 1, "B")
    psa, ldsa = _mat(scale_a, 4, "scale_a")
    psb, ldsb = _mat(scale_b, 4, "scale_b")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    pd, ldd = _mat(out, 2, "out")
    _check("gemm_fp8_blockscaled",
           lib().gemm_fp8_blockscaled(M, N, K, pa, lda, psa, ldsa, pb, ldb, psb, ldsb, pd, ldd,
                                      _stream(A)))
    return out


# FP8 operand formats (mpdt_fp8_format)
FP8_E4M3, FP8_E5M2 = 0, 1


def gemm_fp8_blockscaled_fmt(A, fmt_a, scale_a, B, fmt_b, scale_b, out=None):
    """gemm_fp8_blockscaled with each operand's format (FP8_E4M3 / FP8_E5M2)."""
    M, N, K = _fp8_blockscaled_shapes(A, scale_a, B, scale_b, out)
    pa, lda = _mat(A, 1, "A")
    pb, ldb = _mat(B, 1, "B")
    psa, ldsa = _mat(scale_a, 4, "scale_a")
    psb, ldsb = _mat(scale_b, 4, "scale_b")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    pd, ldd = _mat(out, 2, "out")
    _check("gemm_fp8_blockscaled_fmt",
           lib().gemm_fp8_blockscaled_fmt(M, N, K, pa, lda, int(fmt_a), psa, ldsa, pb, ldb, int(fmt_b),
                                          psb, ldsb, pd, ldd, _stream(A)))
    return out


def gemm_fp8_rowscaled(A, fmt_a, scale_a, B, fmt_b, scale_b, out=None):
    """BF16 D = (A . B) * scale_a[i] * scale_b[j]: FP8 A [M,K], B [K,N];
    scale_a FP32 with M values (per row) or 1 (per tensor), scale_b with N
    values (per column) or 1."""
    M, K = _dims2(A, "A")
    K2, N = _dims2(B, "B")
    if K2 != K:
        raise ValueError("inner dimensions differ")
    _shape(out, (M, N), "out")
    _same_device(A, ("B", B), ("scale_a", scale_a), ("scale_b", scale_b), ("out", out))
    pa, lda = _mat(A, 1, "A")
    pb, ldb = _mat(B, 1, "B")
    inc = []
    for t, n, name in ((scale_a, M, "scale_a"), (scale_b, N, "scale_b")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() not in (1, n):
            raise ValueError(f"{name} must be a contiguous FP32 GPU tensor of 1 or {n} values")
        inc.append(0 if t.numel() == 1 and n != 1 else 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    pd, ldd = _mat(out, 2, "out")
    _check("gemm_fp8_rowscaled",
           lib().gemm_fp8_rowscaled(M, N, K, pa, lda, int(fmt_a), scale_a.data_ptr(), inc[0], pb, ldb,
                                    int(fmt_b), scale_b.data_ptr(), inc[1], pd, ldd, _stream(A)))
    return out


def gemv_w8a8(x, x_scale, W, w_scale, out=None, z_out=None, return_z=False):
    """Batch-1 W8A8 layer: x INT8 [K], W INT8 [N, K] (one output channel per
    row), w_scale FP32 [N]; returns y BF16 [N] (and the INT32 sums when
    return_z or z_out is given)."""
    if x.dim() != 1:
        raise ValueError("x must be 1-D")
    K = x.numel()
    N, K2 = _dims2(W, "W")
    if K2 != K:
        raise ValueError("W must be [N, K]")
    _shape(w_scale, (N,), "w_scale")
    _shape(out, (N,), "out")
    _shape(z_out, (N,), "z_out")
    _same_device(W, ("x", x), ("w_scale", w_scale), ("out", out), ("z_out", z_out))
    if out is not None and (out.element_size() != 2 or not out.is_contiguous()):
        raise ValueError("out must be a contiguous 2-byte (BF16) tensor")
    if z_out is not None and (z_out.dtype != torch.int32 or not z_out.is_contiguous()):
        raise ValueError("z_out must be a contiguous INT32 tensor")
    pw, ldw = _mat(W, 1, "W")
    if x.element_size() != 1 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous 1-byte GPU tensor")
    if w_scale.dtype != torch.float32 or not w_scale.is_contiguous():
        raise ValueError("w_scale must be a contiguous FP32 tensor of N entries")
    if out is None:
        out = torch.empty(N, dtype=torch.bfloat16, device=W.device)
    if z_out is None and return_z:
        z_out = torch.empty(N, dtype=torch.int32, device=W.device)
    pz = None if z_out is None else z_out.data_ptr()
    _check("gemv_w8a8", lib().gemv_w8a8(1, N, K, x.data_ptr(), float(x_scale), pw, ldw,
                                        w_scale.data_ptr(), out.data_ptr(), pz, _stream(W)))
    if return_z or z_out is not None:
        return out, z_out
    return out


def _vec(t, n, dtype, name):
    if t.dim() != 1 or t.dtype != dtype or t.numel() != n or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor of {n} entries")
    return t.data_ptr()


def _w8a8_shapes(M, N, X, W, out, z_out):
    _shape(out, (M, N), "out")
    _shape(z_out, (M, N), "z_out")
    _same_device(W, ("X", X), ("out", out), ("z_out", z_out))


def gemm_w8a8(X, x_scale, W, w_scale, bias=None, out=None, z_out=None, return_z=False):
    """W8A8 layer for M tokens: X INT8 [M, K], x_scale FP32 [M], W INT8 [N, K]
    (one output channel per row), w_scale FP32 [N], bias FP32 [N] or None;
    returns Y BF16 [M, N] (and the INT32 sums when return_z or z_out is given)."""
    M, K = _dims2(X, "X")
    N, K2 = _dims2(W, "W")
    if K2 != K:
        raise ValueError("W must be [N, K]")
    _w8a8_shapes(M, N, X, W, out, z_out)
    px, ldx = _mat(X, 1, "X")
    pw, ldw = _mat(W, 1, "W")
    psx = _vec(x_scale, M, torch.float32, "x_scale")
    psw = _vec(w_scale, N, torch.float32, "w_scale")
    pb = None if bias is None else _vec(bias, N, torch.float32, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=W.device)
    py, ldy = _mat(out, 2, "out")
    if z_out is None and return_z:
        z_out = torch.empty((M, N), dtype=torch.int32, device=W.device)
    pz, ldz = (None, N) if z_out is None else _mat(z_out, 4, "z_out")
    _check("gemm_w8a8", lib().gemm_w8a8(M, N, K, px, ldx, psx, pw, ldw, psw, pb, py, ldy, pz, ldz,
                                        _stream(W)))
    if return_z or z_out is not None:
        return out, z_out
    return out


def gemm_w8a8_kn(X, x_scale, W, w_scale, bias=None, out=None, z_out=None, return_z=False):
    """gemm_w8a8 with W INT8 stored [K, N] (row k holds input k of every
    output channel); returns Y BF16 [M, N] (and the INT32 sums on request)."""
    M, K = _dims2(X, "X")
    K2, N = _dims2(W, "W")
    if K2 != K:
        raise ValueError("W must be [K, N]")
    _w8a8_shapes(M, N, X, W, out, z_out)
    px, ldx = _mat(X, 1, "X")
    pw, ldw = _mat(W, 1, "W")
    psx = _vec(x_scale, M, torch.float32, "x_scale")
    psw = _vec(w_scale, N, torch.float32, "w_scale")
    pb = None if bias is None else _vec(bias, N, torch.float32, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=W.device)
    py, ldy = _mat(out, 2, "out")
    if z_out is None and return_z:
        z_out = torch.empty((M, N), dtype=torch.int32, device=W.device)
    pz, ldz = (None, N) if z_out is None else _mat(z_out, 4, "z_out")
    _check("gemm_w8a8_kn", lib().gemm_w8a8_kn(M, N, K, px, ldx, psx, pw, ldw, psw, pb, py, ldy, pz, ldz,
                                              _stream(W)))
    if return_z or z_out is not None:
        return out, z_out
    return out


def gemm_w8a8_requant(X, x_scale, W, w_scale, bias, out_scale, out=None, z_out=None,
                      return_z=False):
    """The W8A8 layer requantised for a next INT8 layer: as gemm_w8a8, then
    Q = clamp(rne(value / out_scale), -127, 127); returns Q INT8 [M, N] (and
    the INT32 sums when return_z or z_out is given)."""
    M, K = _dims2(X, "X")
    N, K2 = _dims2(W, "W")
    if K2 != K:
        raise ValueError("W must be [N, K]")
    _w8a8_shapes(M, N, X, W, out, z_out)
    px, ldx = _mat(X, 1, "X")
    pw, ldw = _mat(W, 1, "W")
    psx = _vec(x_scale, M, torch.float32, "x_scale")
    psw = _vec(w_scale, N, torch.float32, "w_scale")
    pb = None if bias is None else _vec(bias, N, torch.float32, "bias")
    if out is None:
        out = torch.empty((M, N), dtype=torch.int8, device=W.device)
    pq, ldq = _mat(out, 1, "out")
    if z_out is None and return_z:
        z_out = torch.empty((M, N), dtype=torch.int32, device=W.device)
    pz, ldz = (None, N) if z_out is None else _mat(z_out, 4, "z_out")
    _check("gemm_w8a8_requant",
           lib().gemm_w8a8_requant(M, N, K, px, ldx, psx, pw, ldw, psw, pb, float(out_scale), pq, ldq,
                                   pz, ldz, _stream(W)))
    if return_z or z_out is not None:
        return out, z_out
    return out


def quantize_i8_rows(X, q_out=None, scales_out=None):
    """Per-token INT8 quantisation of BF16 activations X [M, K] (any 2-byte
    dtype holding BF16 bits); returns (Q INT8 [M, K], scales FP32 [M])."""
    M, K = _dims2(X, "X")
    _shape(q_out, (M, K), "q_out")
    _shape(scales_out, (M,), "scales_out")
    _same_device(X, ("q_out", q_out), ("scales_out", scales_out))
    px, ldx = _mat(X, 2, "X")
    if q_out is None:
        q_out = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if scales_out is None:
        scales_out = torch.empty(M, dtype=torch.float32, device=X.device)
    pq, ldq = _mat(q_out, 1, "q_out")
    ps = _vec(scales_out, M, torch.float32, "scales_out")
    _check("quantize_i8_rows", lib().quantize_i8_rows(M, K, px, ldx, pq, ldq, ps, _stream(X)))
    return q_out, scales_out


def quantize_fp8_blocks(X, block_rows, q_out=None, scales_out=None):
    """FP8 E4M3 block quantisation of an FP32 matrix X [R, C] in
    block_rows x 128 blocks (block_rows 1 or 128); returns (Q uint8 [R, C],
    scales FP32 [ceil(R/block_rows), ceil(C/128)])."""
    R, Cc = _dims2(X, "X")
    if block_rows not in (1, 128):
        raise ValueError("block_rows must be 1 or 128")
    nbr, nbc = -(-R // block_rows), -(-Cc // 128)
    _shape(q_out, (R, Cc), "q_out")
    _shape(scales_out, (nbr, nbc), "scales_out")
    _same_device(X, ("q_out", q_out), ("scales_out", scales_out))
    px, ldx = _mat(X, 4, "X")
    if q_out is None:
        q_out = torch.empty((R, Cc), dtype=torch.uint8, device=X.device)
    if scales_out is None:
        scales_out = torch.empty((nbr, nbc), dtype=torch.float32, device=X.device)
    pq, ldq = _mat(q_out, 1, "q_out")
    ps, lds = _mat(scales_out, 4, "scales_out")
    _check("quantize_fp8_blocks", lib().quantize_fp8_blocks(R, Cc, px, ldx, block_rows, pq, ldq, ps,
                                                            lds, _stream(X)))
    return q_out, scales_out


def quantize_fp8(X, fmt, block_rows, block_cols, q_out=None, scales_out=None):
    """FP8 quantisation of an FP32 matrix X [R, C] into fmt (FP8_E4M3 or
    FP8_E5M2) with block_rows x block_cols blocks: 1 x 128, 128 x 128, whole
    rows (1 x C), whole columns (R x 1) or the whole tensor (R x C); returns
    (Q uint8 [R, C], scales FP32 [ceil(R/block_rows), ceil(C/block_cols)])."""
    R, Cc = _dims2(X, "X")
    if block_rows <= 0 or block_cols <= 0:
        raise ValueError("block_rows and block_cols must be positive")
    nbr, nbc = -(-R // block_rows), -(-Cc // block_cols)
    _shape(q_out, (R, Cc), "q_out")
    _shape(scales_out, (max(nbr, 1), max(nbc, 1)), "scales_out")
    _same_device(X, ("q_out", q_out), ("scales_out", scales_out))
    px, ldx = _mat(X, 4, "X")
    if q_out is None:
        q_out = torch.empty((R, Cc), dtype=torch.uint8, device=X.device)
    if scales_out is None:
        scales_out = torch.empty((max(nbr, 1), max(nbc, 1)), dtype=torch.float32, device=X.device)
    pq, ldq = _mat(q_out, 1, "q_out")
    ps, lds = _mat(scales_out, 4, "scales_out")
    _check("quantize_fp8", lib().quantize_fp8(R, Cc, px, ldx, int(fmt), int(block_rows), int(block_cols),
                                              pq, ldq, ps, lds, _stream(X)))
    return q_out, scales_out
