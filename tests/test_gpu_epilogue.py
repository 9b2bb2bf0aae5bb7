"""GPU parity of the FP16 / BF16 GEMMs with the fused bias + activation
epilogue (gemm_f16_bias_act, gemm_bf16_bias_act): D = act(A . B + C + bias),
the sum in FP32, C then the bias added as FP32 steps, the activation in FP32,
then D in FP32 or rounded once to the input format.

  * integer-valued A, B, C and bias keep every step exact, so with no
    activation or ReLU, D equals the oracle's exact result (rounded once to
    the 16-bit format for d16) bit for bit -- on the one-wave kernel (aligned
    rows, also ragged edges and the K window) and on the general kernel
    (unaligned rows, short K);
  * random inputs, every activation: per element
        |D - R| <= L (1e-3 S + 1e-6 + 2^-22 |P|) + 2^-20 (|P| + |R|) [+ half an ulp of D]
    with R = act(P) and P = A.B + C + bias from the oracle in FP64, S the
    GEMM's sum |a.b|.  The first term is the GEMM's own bound plus the two
    FP32 additions (each at most 2^-24 |value|), carried through the
    activation's Lipschitz constant L (1 for none / ReLU; max GELU' = 1.129,
    max SiLU' = 1.100, so L = 1.13); the second covers the FP32 evaluation
    of the activation (erfcf / expf / an IEEE division: a few ulps of the
    result, and of |P| where erfc's argument is rounded deep in the tail);
  * the full 4096^3 BF16 workload with bias, C and GELU into BF16, sampled;
  * bias NULL, C NULL, C == D in place, a padded D's guard band."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_tiled_amd as mp
import oracle
from helpers import dev, host
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu

GPU = {"f16": mp.gemm_f16_bias_act, "bf16": mp.gemm_bf16_bias_act}
ROUND = {"f16": oracle.f32_to_f16_rne, "bf16": oracle.f32_to_bf16_rne}
DEC = {"f16": oracle.f16_to_f64, "bf16": oracle.bf16_to_f64}
ACTS = [mp.ACT_NONE, mp.ACT_RELU, mp.ACT_GELU, mp.ACT_SILU]
LIP = {mp.ACT_NONE: 1.0, mp.ACT_RELU: 1.0, mp.ACT_GELU: 1.13, mp.ACT_SILU: 1.13}


def out_values(D, fmt, d16):
    if not d16:
        return host(D).astype(np.float64)
    return DEC[fmt](host(D.view(torch.int16)).view(np.uint16))


def check_act(D, R, S, P, act, fmt, d16, frob_max, what):
    D = np.asarray(D, np.float64)
    assert np.isfinite(D).all(), f"{what}: non-finite output"
    bound = (LIP[act] * (1e-3 * S + 1e-6 + 2.0 ** -22 * np.abs(P))
             + 2.0 ** -20 * (np.abs(P) + np.abs(R)))
    if d16 and fmt == "bf16":
        bound = bound + 2.0 ** -8 * np.maximum(np.abs(R), np.abs(D))
    if d16 and fmt == "f16":
        bound = bound + 2.0 ** -11 * np.maximum(np.abs(R), np.abs(D)) + 2.0 ** -25
    err = np.abs(D - R)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements over the bound, first at {bad[:5].tolist()}, "
                           f"worst margin {float((err / bound).max()):.3g}")
    nr = np.linalg.norm(R)
    frob = float(np.linalg.norm(D - R) / nr) if nr > 0 else float(np.linalg.norm(D))
    assert frob <= frob_max, f"{what}: relative Frobenius error {frob:.3g} > {frob_max}"


def int_operands(M, N, K, fmt, seed):
    A, B, _ = inputs.gemm16_operands(M, N, K, dist="int4", fmt=fmt, with_c=False,
                                     seeds=(seed, seed + 1, seed + 2))
    C = inputs.int_uniform((M, N), seed + 3, -8, 8, np.float32)
    bias = inputs.int_uniform((N,), seed + 4, -8, 8, np.float32)
    return A, B, C, bias


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("d16", [False, True])
@pytest.mark.parametrize("act", [mp.ACT_NONE, mp.ACT_RELU])
@pytest.mark.parametrize("M,N,K,pad", [(300, 520, 200, 0), (257, 31, 129, 0), (512, 512, 256, 0),
                                       (300, 520, 200, 3), (130, 70, 40, 0)])
def test_integer_inputs_bit_exact(gpu_ok, fmt, d16, act, M, N, K, pad):
    A, B, C, bias = int_operands(M, N, K, fmt, seed=M + N + K + pad)
    tA = dev(A, K + pad, pad=0x7C00) if pad else dev(A)      # pad: rows not 16-byte aligned
    D = GPU[fmt](tA, dev(B), dev(C), dev(bias), act, d16=d16)
    torch.cuda.synchronize()
    R, _, _ = oracle.gemm16_bias_act(fmt, A, B, C, bias, act)  # exact: small integers
    r32 = R.astype(np.float32)
    if d16:
        assert np.array_equal(host(D.view(torch.int16)).view(np.uint16), ROUND[fmt](r32)), what(fmt, M, N, K)
    else:
        assert np.array_equal(host(D), r32), what(fmt, M, N, K)


def what(fmt, M, N, K):
    return f"{fmt} {M}x{N}x{K}"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("d16", [False, True])
@pytest.mark.parametrize("M,N,K", [(384, 640, 512), (513, 257, 300), (64, 96, 64)])
def test_random_inputs_every_activation(gpu_ok, fmt, act, d16, M, N, K):
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(M + 1, N + 2, K + 3))
    C = (C * 4.0).astype(np.float32)          # spread P over the activations' curved range
    bias = inputs.normal_f32((N,), M + N)
    D = GPU[fmt](dev(A), dev(B), dev(C), dev(bias), act, d16=d16)
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, C, bias, act)
    frob = 1e-2 if (d16 and fmt == "bf16") else 1e-3
    check_act(out_values(D, fmt, d16), R, S, P, act, fmt, d16, frob, f"{what(fmt, M, N, K)} act {act}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_null_bias_null_c_in_place_and_guard_band(gpu_ok, fmt):
    M, N, K = 259, 300, 128
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(61, 62, 63))
    bias = inputs.normal_f32((N,), 64)
    # no bias: act(A.B + C)
    D = GPU[fmt](dev(A), dev(B), dev(C), None, mp.ACT_GELU)
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, C, None, mp.ACT_GELU)
    check_act(host(D), R, S, P, mp.ACT_GELU, fmt, False, 1e-3, "no bias")
    # no C: act(A.B + bias)
    D = GPU[fmt](dev(A), dev(B), None, dev(bias), mp.ACT_SILU)
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, None, bias, mp.ACT_SILU)
    check_act(host(D), R, S, P, mp.ACT_SILU, fmt, False, 1e-3, "no C")
    # C == D in place (FP32 D)
    tc = dev(C)
    out = GPU[fmt](dev(A), dev(B), tc, dev(bias), mp.ACT_RELU, out=tc)
    assert out.data_ptr() == tc.data_ptr()
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, C, bias, mp.ACT_RELU)
    check_act(host(tc), R, S, P, mp.ACT_RELU, fmt, False, 1e-3, "in place")
    # a padded 16-bit D: the guard band stays untouched
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    buf = torch.full((M + 4, N + 10), 3.0, dtype=dt, device=gpu_ok)
    o16 = buf[2:2 + M, 5:5 + N]
    GPU[fmt](dev(A), dev(B), dev(C), dev(bias), mp.ACT_GELU, out=o16)
    h = host(buf.view(torch.int16)).view(np.uint16)
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, C, bias, mp.ACT_GELU)
    check_act(DEC[fmt](h[2:2 + M, 5:5 + N]), R, S, P, mp.ACT_GELU, fmt, True,
              1e-2 if fmt == "bf16" else 1e-3, "padded d16")
    mask = np.ones_like(h, bool)
    mask[2:2 + M, 5:5 + N] = False
    three = host(torch.tensor([3.0], dtype=dt).view(torch.int16)).view(np.uint16)[0]
    assert (h[mask] == three).all()


def test_full_size_bf16_gelu_sampled(gpu_ok):
    """The 4096^3 BF16 workload with a bias, C and GELU into BF16, in the
    launch configuration the benchmark times: 4096 sampled outputs against
    the oracle element by element, every output finite."""
    M = N = K = 4096
    A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16", seeds=(71, 72, 73))
    bias = inputs.normal_f32((N,), 74)
    D = mp.gemm_bf16_bias_act(dev(A), dev(B), dev(C), dev(bias), mp.ACT_GELU, d16=True)
    d = DEC["bf16"](host(D.view(torch.int16)).view(np.uint16))
    assert np.isfinite(d).all()
    r = np.random.default_rng(75)
    ii = np.concatenate([r.integers(0, M, 4000), [0, M - 1, 0, M - 1]])
    jj = np.concatenate([r.integers(0, N, 4000), [0, 0, N - 1, N - 1]])
    R, S, P = oracle.gemm16_bias_act_at("bf16", A, B, C, bias, mp.ACT_GELU, ii, jj)
    check_act(d[ii, jj], R, S, P, mp.ACT_GELU, "bf16", True, 1e-2, "4096^3 sampled")


def test_random_shape_sweep(gpu_ok):
    """Seeded random shapes through the fused epilogue: with no activation
    or ReLU, integer-valued inputs and D checked bit for bit (FP32 or 16-bit,
    long K included, where C joins inside the K loop, and unaligned A rows);
    with GELU or SiLU, random inputs against the bound above."""
    r = np.random.default_rng(31337)
    for case in range(36):
        fmt = ("f16", "bf16")[case % 2]
        d16 = bool((case // 2) % 2)
        M, N = int(r.integers(1, 900)), int(r.integers(1, 900))
        K = int(r.integers(1, 2100)) if case % 3 else int(r.integers(1600, 2100))
        pad = int(r.integers(0, 4))
        name = f"case {case}: {fmt} {M}x{N}x{K} d16={d16} pad={pad}"
        if case < 24:
            act = (mp.ACT_NONE, mp.ACT_RELU)[(case // 4) % 2]
            A, B, C, bias = int_operands(M, N, K, fmt, seed=case * 10)
            tA = dev(A, K + pad, pad=0x7C00) if pad else dev(A)
            D = GPU[fmt](tA, dev(B), dev(C), dev(bias), act, d16=d16)
            torch.cuda.synchronize()
            R, _, _ = oracle.gemm16_bias_act(fmt, A, B, C, bias, act)
            r32 = R.astype(np.float32)
            if d16:
                assert np.array_equal(host(D.view(torch.int16)).view(np.uint16), ROUND[fmt](r32)), name
            else:
                assert np.array_equal(host(D), r32), name
        else:
            act = (mp.ACT_GELU, mp.ACT_SILU)[case % 2]
            A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt=fmt, seeds=(case, M, N))
            C = (C * 4.0).astype(np.float32)
            bias = inputs.normal_f32((N,), case + 5)
            D = GPU[fmt](dev(A), dev(B), dev(C), dev(bias), act, d16=d16)
            R, S, P = oracle.gemm16_bias_act(fmt, A, B, C, bias, act)
            frob = 1e-2 if (d16 and fmt == "bf16") else 1e-3
            check_act(out_values(D, fmt, d16), R, S, P, act, fmt, d16, frob, f"{name} act {act}")
