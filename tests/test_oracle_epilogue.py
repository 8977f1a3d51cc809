"""Pins for the oracle's epilogue: bias and the tanh form of GELU.

No page prints a GELU value, so the activation is pinned by what the
mathematics fixes: GELU(0) = 0 and GELU(x) - GELU(-x) = x exactly in real
arithmetic (the tanh argument is odd and the prefactor is x/2), the limits x
and 0 for large |x|, torch's CPU float64 tanh-form GELU (a library routine
for exactly this function), and the distance to the exact erf form, which the
tanh form approximates to a few parts in 10^4.  A wrong constant in the tanh
argument moves the value by more than that.
"""
import math

import numpy as np
import torch

import oracle
from dense_gemm_engineering_amd import inputs


def test_gelu_special_values():
    assert oracle.gelu_tanh(0.0) == 0.0
    for x in (30.0, 100.0, 1e3):
        assert oracle.gelu_tanh(x) == x
        assert oracle.gelu_tanh(-x) == 0.0 or abs(oracle.gelu_tanh(-x)) < 1e-300


def test_gelu_odd_identity():
    for x in np.linspace(-6, 6, 1201):
        g = oracle.gelu_tanh(x) - oracle.gelu_tanh(-x)
        assert abs(g - x) <= 4e-16 * max(1.0, abs(x))


def test_gelu_matches_torch_tanh_form():
    xs = np.concatenate([np.linspace(-8, 8, 4001), [1e-8, -1e-8, 0.5, -0.5]])
    want = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(x) for x in xs])
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)


def test_gelu_close_to_erf_form():
    worst = 0.0
    for x in np.linspace(-6, 6, 2401):
        exact = 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))
        worst = max(worst, abs(oracle.gelu_tanh(x) - exact))
    assert 1e-5 < worst < 5e-4


def test_bias_integer_exact():
    M, N, K = 9, 14, 50
    r = np.random.Generator(np.random.PCG64(600))
    Ai, Bi = r.integers(-4, 5, (M, K)), r.integers(-4, 5, (K, N))
    bi = r.integers(-20, 21, N)
    A = inputs.to_bits(Ai.astype(float), "f16")
    B = inputs.to_bits(Bi.astype(float), "f16")
    T, _ = oracle.gemm(A, B, "f16", epi="bias", bias=bi.astype(float), alpha=2.0)
    assert np.array_equal(T, (2 * (Ai @ Bi) + bi[None, :]).astype(float))


def test_bias_gelu_applies_after_bias():
    M, N, K = 4, 6, 8
    A = inputs.to_bits(np.zeros((M, K)), "f16")
    B = inputs.to_bits(np.zeros((K, N)), "f16")
    bias = np.array([-3.0, -1.0, 0.0, 0.5, 1.0, 3.0])
    T, _ = oracle.gemm(A, B, "f16", epi="bias_gelu", bias=bias)
    want = torch.nn.functional.gelu(torch.from_numpy(bias), approximate="tanh").numpy()
    assert np.allclose(T, np.broadcast_to(want, (M, N)), rtol=1e-14)
