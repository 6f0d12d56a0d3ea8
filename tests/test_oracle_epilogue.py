"""Pins for the oracle's fused epilogue (no GPU).

Kernel Tuning Guide §6 names the fused epilogues bias, bias+ReLU, bias+SiLU
and bias+GELU. The oracle adds an fp32 bias per output column and applies
relu(x) = max(x, 0), silu(x) = x / (1 + e^-x), gelu(x) = x Phi(x) (the erf
form). These are checked against routes that share nothing with the
oracle's own formulas: the odd-part identity f(x) - f(-x) = x that all three
satisfy, SiLU through tanh, the normal CDF by numerical integration of the
density (Simpson's rule) and its textbook table values, e / (1 + e) for
sigmoid(1), and the broadcast of the bias along columns.
"""
import math

import numpy as np
import pytest

import oracle

X = np.linspace(-9.0, 9.0, 721)


@pytest.mark.parametrize("act", ["relu", "silu", "gelu"])
def test_odd_part_is_identity(act):
    f = oracle.activation(X, act)
    g = oracle.activation(-X, act)
    assert np.allclose(f - g, X, rtol=0, atol=1e-13)


def test_relu_values():
    assert oracle.activation(np.array([-2.0, -0.0, 0.0, 3.5]), "relu").tolist() == [0.0, 0.0, 0.0, 3.5]


def test_silu_through_tanh_and_sigmoid_one():
    ref = 0.5 * X * (1.0 + np.tanh(0.5 * X))
    assert np.allclose(oracle.activation(X, "silu"), ref, rtol=1e-14, atol=1e-15)
    assert abs(oracle.activation(np.array([1.0]), "silu")[0] - math.e / (1 + math.e)) < 1e-15
    assert oracle.activation(np.array([0.0]), "silu")[0] == 0.0


def _phi_simpson(x, n=20000):
    """Standard normal CDF by Simpson's rule on the density over [-12, x]."""
    lo = -12.0
    h = (x - lo) / n
    t = lo + h * np.arange(n + 1)
    w = np.ones(n + 1)
    w[1:-1:2] = 4
    w[2:-1:2] = 2
    dens = np.exp(-0.5 * t * t) / math.sqrt(2 * math.pi)
    return float(h / 3 * np.sum(w * dens))


@pytest.mark.parametrize("x", [-3.0, -1.0, -0.25, 0.5, 1.0, 2.0, 4.0])
def test_gelu_against_integrated_normal_cdf(x):
    assert abs(oracle.activation(np.array([x]), "gelu")[0] - x * _phi_simpson(x)) < 1e-12


def test_gelu_table_values():
    # standard normal table: Phi(1) = 0.8413, Phi(1.96) = 0.9750, Phi(-0.5) = 0.3085
    for x, phi in [(1.0, 0.8413), (1.96, 0.9750), (-0.5, 0.3085)]:
        assert abs(oracle.activation(np.array([x]), "gelu")[0] / x - phi) < 5e-5


def test_bias_added_per_column_then_activation():
    import workloads

    M, N, K = 16, 48, 128
    h = workloads.make_inputs("fp8", M, N, K, 3, bias=True)
    h0 = workloads.make_inputs("fp8", M, N, K, 3)
    for k in ("a", "b", "scale_a", "scale_b"):
        assert np.array_equal(h[k], h0[k])          # the bias is drawn after A and B
    r = oracle.gemm("fp8", h)
    for act in ("none", "relu", "silu", "gelu"):
        out = oracle.gemm("fp8", h, act=act)
        ref = oracle.activation(r + h["bias"].astype(np.float64)[None, :], act)
        assert np.array_equal(out, ref)
    # A = 0: the output is the activation of the bias in every row
    hz = dict(h, a=np.zeros_like(h["a"]))
    out = oracle.gemm("fp8", hz, act="gelu")
    assert np.array_equal(out, np.repeat(oracle.activation(h["bias"].astype(np.float64), "gelu")[None, :], M, 0))
    # column subsets take the matching bias entries
    cols = [5, 0, 47]
    assert np.array_equal(oracle.gemm("fp8", h, cols=cols, act="silu"), oracle.gemm("fp8", h, act="silu")[:, cols])


def test_int8_has_no_epilogue():
    import workloads

    h = workloads.make_inputs("int8", 16, 16, 64, 1)
    with pytest.raises(ValueError):
        oracle.gemm("int8", h, act="relu")
