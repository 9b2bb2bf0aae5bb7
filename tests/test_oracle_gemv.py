"""The oracle's batch-1 W8A8 linear layer ("NVIDIA A100: from chip to SIMT",
sections 5.1-5.2): exact INT32 dot products per output channel with weights
stored [N][K] row-major, then (float(z) * s_x) * s_w[o] in FP32, rounded to
BF16.  Pinned to an int64 numpy dot, to numpy FP32 steps plus torch's BF16
cast, and to the page's INT32 bound at K = 4096."""
import json
import os

import numpy as np
import torch

import oracle
from mixed_precision_dense_tiled_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_closed_forms.json")))


def _torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_gemv_against_numpy_steps():
    N, K = 1000, 4096
    x, s_x, W, s_w = inputs.w8a8_operands(N, K)
    z, y = oracle.gemv_w8a8(x, s_x, inputs.with_ld(W, K + 64), s_w)
    zr = W.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(z.astype(np.int64), zr)
    t = zr.astype(np.float32) * np.float32(s_x)      # first FP32 multiply
    t = t * s_w                                      # second FP32 multiply
    assert np.array_equal(y, _torch_bf16_bits(t))


def test_gemv_order_matters_and_is_pinned():
    # Multiplying s_x * s_w first can round to a different BF16; find such
    # channels (deterministic search) and check the oracle takes
    # float(z) * s_x first, then * s_w.
    r = np.random.default_rng(99)
    N, K = 4096, 64
    for _ in range(200):
        x = r.integers(-127, 128, K).astype(np.int8)
        W = r.integers(-127, 128, (N, K)).astype(np.int8)
        s_x = np.float32(r.uniform(0.01, 0.1))
        s_w = r.uniform(0.001, 0.01, N).astype(np.float32)
        zf = (W.astype(np.int64) @ x.astype(np.int64)).astype(np.float32)
        mine = _torch_bf16_bits((zf * s_x) * s_w)
        other = _torch_bf16_bits(zf * (s_x * s_w))
        if (mine != other).any():
            break
    assert (mine != other).any()
    _, y = oracle.gemv_w8a8(x, s_x, W, s_w)
    assert np.array_equal(y, mine)


def test_page_int32_bound():
    K = 4096
    x = np.full(K, -128, np.int8)
    W = np.full((3, K), -128, np.int8)
    z, _ = oracle.gemv_w8a8(x, np.float32(1.0), W, np.ones(3, np.float32))
    assert (z == GOLD["int32_bound_k4096"]["value"]).all()
    assert GOLD["int32_bound_k4096"]["value"] < 2 ** 31
    W[1] = 127
    z, _ = oracle.gemv_w8a8(x, np.float32(1.0), W, np.ones(3, np.float32))
    assert z[1] == -128 * 127 * K


def test_page_counts_k4096():
    # useful MACs = K * N, weight bytes = K * N, activation K bytes, FP32 scales 4 N bytes
    K = N = 4096
    assert K * N == GOLD["w8a8_useful_macs_k4096_n4096"]["value"]
    assert K * N * 1 == GOLD["w8a8_weight_bytes_k4096_n4096"]["value"]
    assert K * 1 == GOLD["w8a8_activation_bytes_k4096"]["value"]
    assert N * 4 == GOLD["w8a8_weight_scale_bytes_n4096"]["value"]
    assert 2 * 16 * 16 * 16 == GOLD["flop_per_16x16x16_mma"]["value"]


def test_gemv_k_zero_and_small():
    x = np.zeros(0, np.int8)
    W = np.zeros((5, 0), np.int8)
    z, y = oracle.gemv_w8a8(x, np.float32(0.5), W, np.ones(5, np.float32))
    assert (z == 0).all() and (y == 0).all()
    x = np.array([3, -2], np.int8)
    W = np.array([[1, 1], [2, 5], [-7, 0]], np.int8)
    z, y = oracle.gemv_w8a8(x, np.float32(0.5), W, np.array([2.0, 1.0, 0.25], np.float32))
    assert list(z) == [1, -4, -21]
    assert list(oracle.bf16_to_f64(y)) == [1.0, -2.0, -2.625]
