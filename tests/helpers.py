"""Shared helpers of the GPU tests: host <-> device copies of bit-pattern
operands and the acceptance checks (per-element bound |D - R| <= 1e-3 * S +
1e-6 with S = sum_k |a_ik * b_kj|, relative Frobenius error, bit-exactness)."""
import ctypes
import os

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_VIEW = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}


def dev(x: np.ndarray, ld=None, pad=0, device="cuda:0") -> torch.Tensor:
    """Copy a numpy array to the GPU.  With ``ld``, a 2-D array is placed in
    a wider row-major buffer (leading dimension ld, padding filled with the
    bit pattern ``pad``) and the returned tensor is the row-strided view."""
    x = np.asarray(x)
    if x.dtype in _VIEW:
        x = x.view(_VIEW[x.dtype])
    if ld is None or x.ndim != 2:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    rows, cols = x.shape
    buf = np.empty((rows, ld), x.dtype)
    buf.view(np.uint8)[...] = 0
    buf[...] = np.array(pad).astype(np.int64).astype(x.dtype) if x.dtype.kind in "iu" else pad
    buf[:, :cols] = x
    return torch.from_numpy(buf).to(device)[:, :cols]


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    a = a.numpy()
    return a.view(dtype) if dtype is not None else a


def check_fp(D, R, S, frob_max, what="", bf16_out=False, f16_out=False):
    """Per-element bound and relative Frobenius error; returns (worst margin, frob).

    bf16_out / f16_out: the output was rounded to BF16 / FP16 after
    accumulation; the bound then also admits that one rounding (half an ulp:
    at most 2^-8 |value| for BF16, 2^-11 |value| for FP16, plus half the
    smallest FP16 subnormal)."""
    D = np.asarray(D, np.float64)
    assert np.isfinite(D).all(), f"{what}: non-finite output"
    err = np.abs(D - R)
    bound = 1e-3 * S + 1e-6
    if bf16_out:
        bound = bound + 2.0 ** -8 * np.maximum(np.abs(R), np.abs(D))
    if f16_out:
        bound = bound + 2.0 ** -11 * np.maximum(np.abs(R), np.abs(D)) + 2.0 ** -25
    margin = float((err / bound).max()) if err.size else 0.0
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements over the bound, first at {bad[:5].tolist()}, "
                           f"worst margin {margin:.3g}")
    nr = np.linalg.norm(R)
    frob = float(np.linalg.norm(D - R) / nr) if nr > 0 else float(np.linalg.norm(D))
    assert frob <= frob_max, f"{what}: relative Frobenius error {frob:.3g} > {frob_max}"
    return margin, frob


def probes():
    L = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "libmpdt_probes.so"))
    L.mpdt_probe_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    L.mpdt_probe_mfma_peak.restype = ctypes.c_int
    L.mpdt_probe_tr.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    L.mpdt_probe_tr.restype = ctypes.c_int
    L.mpdt_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.mpdt_probe_mfma.restype = ctypes.c_int
    L.mpdt_probe_unaligned.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.mpdt_probe_unaligned.restype = ctypes.c_int
    return L
