"""The oracle's bias + activation epilogue pinned to things other than
itself: textbook values of the standard normal CDF and of the logistic
function, library routines of another form (x * Phi(x) through scipy's
normal CDF, x * logistic(x) through scipy's expit), the odd-part identity
act(x) - act(-x) = x that all three activations satisfy, and the identity
matrix, which turns the GEMM into its B operand so that the bias must land
per output column.  The bias belongs in the floating-point epilogue
("NVIDIA A100: from chip to SIMT", section 5.1); the activations are the
usual ReLU, GELU (erf form) and SiLU."""
import numpy as np
import pytest
from scipy.special import expit
from scipy.stats import norm

import oracle

ACTS = [oracle.ACT_RELU, oracle.ACT_GELU, oracle.ACT_SILU]


def _row(x):
    return np.asarray(x, np.float64).reshape(1, -1)


@pytest.mark.parametrize("act", ACTS)
def test_odd_part_identity(act):
    # relu, x Phi(x) and x sigma(x) all satisfy f(x) - f(-x) = x, because
    # Phi(x) + Phi(-x) = 1 and sigma(x) + sigma(-x) = 1; a dropped factor,
    # a sign error inside erf / exp or a wrong scale of the erf argument
    # breaks it
    x = np.linspace(-9.0, 9.0, 361)
    d = oracle.bias_act(_row(x), None, act)[0] - oracle.bias_act(_row(-x), None, act)[0]
    assert np.allclose(d, x, rtol=0, atol=4e-15)


def test_textbook_values():
    x = _row([1.0, -1.0, 2.0, 0.0])
    g = oracle.bias_act(x, None, oracle.ACT_GELU)[0]
    s = oracle.bias_act(x, None, oracle.ACT_SILU)[0]
    # Phi(1) = 0.841344746068543, Phi(2) = 0.977249868051821 (normal table);
    # sigma(1) = e / (1 + e) = 0.731058578630005
    assert np.allclose(g, [0.841344746068543, -0.158655253931457, 2 * 0.977249868051821, 0.0],
                       rtol=1e-14, atol=0)
    assert np.allclose(s, [0.731058578630005, -0.268941421369995, 2 * 0.880797077977882, 0.0],
                       rtol=1e-14, atol=0)
    r = oracle.bias_act(_row([-3.0, -0.0, 0.5, 7.0]), None, oracle.ACT_RELU)[0]
    assert r.tolist() == [0.0, 0.0, 0.5, 7.0]


def test_against_library_forms():
    x = np.linspace(-30.0, 30.0, 2001)
    g = oracle.bias_act(_row(x), None, oracle.ACT_GELU)[0]
    s = oracle.bias_act(_row(x), None, oracle.ACT_SILU)[0]
    gl = x * norm.cdf(x)
    sl = x * expit(x)
    assert np.all(np.abs(g - gl) <= 1e-14 * np.abs(x) + 1e-300)
    assert np.all(np.abs(s - sl) <= 1e-14 * np.abs(x) + 1e-300)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("act", [oracle.ACT_NONE] + ACTS)
def test_identity_gemm_puts_bias_on_columns(fmt, act):
    # A = I (M = K = 5), B 5 x 7 small integers: A.B = B exactly, so
    # R = act(B + C + bias[j]); with M != N a bias taken per row, or from
    # the wrong end, gives other values
    M = K = 5
    N = 7
    r = np.random.default_rng(act)
    Bv = r.integers(-6, 7, (K, N)).astype(np.float32)
    Cv = r.integers(-3, 4, (M, N)).astype(np.float32)
    bias = np.arange(N, dtype=np.float32) * 3 - 10
    one = 0x3C00 if fmt == "f16" else 0x3F80
    A = np.zeros((M, K), np.uint16)
    A[np.arange(M), np.arange(K)] = one
    if fmt == "f16":
        B = Bv.astype(np.float16).view(np.uint16)
    else:
        B = (Bv.view(np.uint32) >> 16).astype(np.uint16)
    R, S, P = oracle.gemm16_bias_act(fmt, A, B, Cv, bias, act)
    pre = Bv.astype(np.float64) + Cv + bias[None, :]
    assert np.array_equal(P, pre)
    want = {oracle.ACT_NONE: pre, oracle.ACT_RELU: np.maximum(pre, 0.0),
            oracle.ACT_GELU: pre * norm.cdf(pre), oracle.ACT_SILU: pre * expit(pre)}[act]
    assert np.allclose(R, want, rtol=1e-12, atol=1e-300)   # erfc and ndtr deep in the tail
    assert np.array_equal(S, np.abs(Bv).astype(np.float64))


def test_no_bias_no_activation_is_the_gemm_and_sampled_form_agrees():
    r = np.random.default_rng(5)
    A = (r.standard_normal((9, 33)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    B = (r.standard_normal((33, 11)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    C = r.standard_normal((9, 11)).astype(np.float32)
    bias = r.standard_normal(11).astype(np.float32)
    R0, S0 = oracle.gemm_bf16(A, B, C)
    R, S, P = oracle.gemm16_bias_act("bf16", A, B, C, None, oracle.ACT_NONE)
    assert np.array_equal(R, R0) and np.array_equal(S, S0) and np.array_equal(P, R0)
    for act in ACTS:
        R, S, P = oracle.gemm16_bias_act("bf16", A, B, C, bias, act)
        ii, jj = np.meshgrid(np.arange(9), np.arange(11), indexing="ij")
        Ra, Sa, Pa = oracle.gemm16_bias_act_at("bf16", A, B, C, bias, act, ii.ravel(), jj.ravel())
        assert np.array_equal(Ra, R.ravel()) and np.array_equal(Pa, P.ravel())


def test_rejects_unknown_activation_and_non_finite_bias():
    with pytest.raises(oracle.OracleError):
        oracle.bias_act(_row([1.0]), None, 4)
    with pytest.raises(oracle.OracleError):
        oracle.bias_act(_row([1.0]), np.array([np.inf], np.float32), 0)
