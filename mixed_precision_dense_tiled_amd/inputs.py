"""Seeded synthetic inputs for the GEMM and W8A8 workloads.

This module only draws random numbers and stores them in the operand formats
(FP16 / BF16 / FP8 E4M3 bit patterns, INT8, FP32).  It holds none of the
multiply-accumulate arithmetic and none of the kernels' or the oracle's code;
both sides receive the same bytes from here.

Distributions and seeds (numpy PCG64 ``default_rng``): A=1, B=2, C=3, x=4, W=5,
s_x=6, s_w=7, FP8 A=8, FP8 B=9; values are drawn in FP32 and then stored in the
operand format with library casts (numpy float16 and torch bfloat16 /
float8_e4m3fn, all round-to-nearest-even).  FP8 operands are scaled per block
(1x128 rows of A, 128x128 tiles of B) by s = amax/448 before the cast, with the
quotient clamped to +-448, and s is returned as the block's dequantisation
multiplier (s = 1 for an all-zero block).
"""
from __future__ import annotations

import numpy as np
import torch

SEED_A, SEED_B, SEED_C, SEED_X, SEED_W, SEED_SX, SEED_SW, SEED_QA, SEED_QB, SEED_BIAS = range(1, 11)
FP8_BLOCK = 128
E4M3_MAX = 448.0


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ------------------------------------------------------------ raw draws --
def uniform_f32(shape, seed, lo=-1.0, hi=1.0) -> np.ndarray:
    return rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def normal_f32(shape, seed) -> np.ndarray:
    return rng(seed).standard_normal(size=shape, dtype=np.float32)


def int_uniform(shape, seed, lo, hi_inclusive, dtype) -> np.ndarray:
    return rng(seed).integers(lo, hi_inclusive + 1, size=shape).astype(dtype)


# ----------------------------------------------------------- storage ----
def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    x = np.clip(np.ascontiguousarray(x, np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def with_ld(x: np.ndarray, ld: int, fill=0) -> np.ndarray:
    """The same matrix inside a wider row-major buffer (leading dimension ld):
    returns a view whose rows are ld elements apart."""
    rows, cols = x.shape
    assert ld >= cols
    buf = np.full((rows, ld), fill, dtype=x.dtype)
    buf[:, :cols] = x
    return buf[:, :cols]


# --------------------------------------------------------- FP8 blocks ---
def _block_scale(amax: np.ndarray) -> np.ndarray:
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def fp8_quantize_rows(v: np.ndarray):
    """A-side: one scale per (row, 128-wide K block). Returns (bytes, scales)."""
    M, K = v.shape
    kb = (K + FP8_BLOCK - 1) // FP8_BLOCK
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, kb), np.float32)
    for b in range(kb):
        blk = v[:, b * FP8_BLOCK:(b + 1) * FP8_BLOCK]
        sb = _block_scale(np.abs(blk).max(axis=1))
        s[:, b] = sb
        q[:, b * FP8_BLOCK:(b + 1) * FP8_BLOCK] = to_e4m3_bits(blk / sb[:, None])
    return q, s


def fp8_quantize_tiles(v: np.ndarray):
    """B-side: one scale per 128x128 tile. Returns (bytes, scales)."""
    K, N = v.shape
    kb = (K + FP8_BLOCK - 1) // FP8_BLOCK
    nb = (N + FP8_BLOCK - 1) // FP8_BLOCK
    q = np.empty((K, N), np.uint8)
    s = np.empty((kb, nb), np.float32)
    for b in range(kb):
        rows = slice(b * FP8_BLOCK, (b + 1) * FP8_BLOCK)
        for c in range(nb):
            cols = slice(c * FP8_BLOCK, (c + 1) * FP8_BLOCK)
            blk = v[rows, cols]
            sb = _block_scale(np.float32(np.abs(blk).max()))
            s[b, c] = sb
            q[rows, cols] = to_e4m3_bits(blk / sb)
    return q, s


# ------------------------------------------------------- the workloads --
def gemm16_operands(M, N, K, dist="uniform", fmt="f16", with_c=True, c_zero=False,
                    seeds=(SEED_A, SEED_B, SEED_C)):
    """A (M x K) and B (K x N) bit patterns plus an FP32 C (or None).

    dist: "uniform" (U[-1,1]), "normal" (N(0,1)) or "int4" (integers in [-4, 4])."""
    sa, sb, sc = seeds
    if dist == "uniform":
        a, b = uniform_f32((M, K), sa), uniform_f32((K, N), sb)
    elif dist == "normal":
        a, b = normal_f32((M, K), sa), normal_f32((K, N), sb)
    elif dist == "int4":
        a = int_uniform((M, K), sa, -4, 4, np.float32)
        b = int_uniform((K, N), sb, -4, 4, np.float32)
    else:
        raise ValueError(dist)
    conv = to_f16_bits if fmt == "f16" else to_bf16_bits
    C = None
    if with_c:
        if c_zero:
            C = np.zeros((M, N), np.float32)
        elif dist == "normal":
            C = normal_f32((M, N), sc)
        else:
            C = uniform_f32((M, N), sc)
    return conv(a), conv(b), C


def i8_operands(M, N, K, with_c=True, seeds=(SEED_A, SEED_B, SEED_C)):
    sa, sb, sc = seeds
    A = int_uniform((M, K), sa, -128, 127, np.int8)
    B = int_uniform((K, N), sb, -128, 127, np.int8)
    C = int_uniform((M, N), sc, -(1 << 20), 1 << 20, np.int32) if with_c else None
    return A, B, C


def fp8_operands(M, N, K, seeds=(SEED_QA, SEED_QB)):
    qa, sa = fp8_quantize_rows(normal_f32((M, K), seeds[0]))
    qb, sb = fp8_quantize_tiles(normal_f32((K, N), seeds[1]))
    return qa, sa, qb, sb


def w8a8_operands(N, K, seeds=(SEED_X, SEED_W, SEED_SX, SEED_SW)):
    """x int8 [K], W int8 stored N x K, s_x FP32 scalar, s_w FP32 [N]."""
    x = int_uniform((K,), seeds[0], -127, 127, np.int8)
    W = int_uniform((N, K), seeds[1], -127, 127, np.int8)
    s_x = np.float32(rng(seeds[2]).uniform(0.01, 0.1))
    s_w = rng(seeds[3]).uniform(0.001, 0.01, size=N).astype(np.float32)
    return x, s_x, W, s_w
