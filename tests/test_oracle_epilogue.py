"""Pins of the fused-epilogue oracle (oracle/epilogue.py) against facts that do
not come from the oracle itself: hand-computed small cases, the standard normal
CDF, algebraic identities of the activations, and planted mistakes."""
import math

import numpy as np
import pytest
from scipy.stats import norm

from oracle import epilogue as epi
from oracle.gemm import ref_gemm

# Phi(x) to 9 decimals, as printed in standard normal tables.
PHI_TABLE = [(-2.0, 0.022750132), (-1.0, 0.158655254), (-0.5, 0.308537539), (0.0, 0.5),
             (0.5, 0.691462461), (1.0, 0.841344746), (2.0, 0.977249868)]


def _hand_case():
    # A = [[1, 2], [3, 4]], B = [[5, 6], [7, 8]]: A.B = [[19, 22], [43, 50]]
    P = np.array([[19.0, 22.0], [43.0, 50.0]])
    C0 = np.ones((2, 2))
    bias = np.array([0.5, -0.5])
    return P, C0, bias


def _pins_pass(mutation: int) -> bool:
    checks = []
    P, C0, bias = _hand_case()
    # 2 P - C0 + bias, worked by hand
    D, _ = epi.epilogue_ref(P, C0, 2.0, -1.0, bias, "none", mutation)
    checks.append(np.array_equal(D, [[37.5, 42.5], [85.5, 98.5]]))
    # ReLU of -P + 30: [[11, 8], [-13, -20]] -> [[11, 8], [0, 0]]
    D, _ = epi.epilogue_ref(P, np.full((2, 2), 30.0), -1.0, 1.0, None, "relu", mutation)
    checks.append(np.array_equal(D, [[11.0, 8.0], [0.0, 0.0]]))
    # GELU at table points: x Phi(x)
    xs = np.array([[x for x, _ in PHI_TABLE]])
    D, _ = epi.epilogue_ref(xs, None, 1.0, 0.0, None, "gelu", mutation)
    want = np.array([[x * ph for x, ph in PHI_TABLE]])
    checks.append(np.allclose(D, want, rtol=0, atol=2e-9))
    # bias on a taller-than-wide output: row i, column j gets bias[j]
    P3 = np.zeros((3, 2))
    D, _ = epi.epilogue_ref(P3, None, 1.0, 0.0, np.array([1.0, 2.0]), "none", mutation)
    checks.append(np.array_equal(D, [[1.0, 2.0]] * 3))
    return all(checks)


def test_pins_pass_on_the_oracle():
    assert _pins_pass(0)


@pytest.mark.parametrize("mutation", [1, 2, 3, 4])
def test_planted_mistakes_are_caught(mutation):
    assert not _pins_pass(mutation), f"planted mistake {mutation} slipped through the pins"


def test_identity_epilogue_is_the_product():
    rng = np.random.default_rng(3)
    P = rng.standard_normal((5, 7))
    D, Y = epi.epilogue_ref(P, None)
    assert np.array_equal(D, P) and np.array_equal(Y, P)


def test_identity_epilogue_over_the_gemm_oracle():
    # small integers in bf16: the product is exact, so alpha = 2, beta = -3 and an
    # integer bias give exact integers computed here by numpy int64 arithmetic
    rng = np.random.default_rng(5)
    M, N, K = 6, 8, 16
    ai = rng.integers(-4, 5, size=(M, K))
    bi = rng.integers(-4, 5, size=(K, N))
    to_bf16 = lambda x: (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    P, _ = ref_gemm(to_bf16(ai), to_bf16(bi), M, N, K, "kn", "bf16")
    c0 = rng.integers(-9, 10, size=(M, N))
    bias = rng.integers(-9, 10, size=N)
    D, _ = epi.epilogue_ref(P, c0.astype(np.float64), 2.0, -3.0, bias.astype(np.float64), "none")
    assert np.array_equal(D, (2 * (ai @ bi) - 3 * c0 + bias[None, :]).astype(np.float64))


def test_gelu_matches_normal_cdf():
    x = np.linspace(-6, 6, 241)[None, :]
    D, _ = epi.epilogue_ref(x, None, act="gelu")
    assert np.allclose(D, x * norm.cdf(x), rtol=1e-13, atol=1e-15)


def test_gelu_symmetry_and_limits():
    x = np.linspace(-8, 8, 321)[None, :]
    g = epi.activation(x, "gelu")
    gn = epi.activation(-x, "gelu")
    assert np.allclose(g - gn, x, rtol=0, atol=1e-14)     # Phi(-x) = 1 - Phi(x)
    assert epi.activation(np.array([0.0]), "gelu")[0] == 0.0
    assert abs(epi.activation(np.array([30.0]), "gelu")[0] - 30.0) < 1e-12
    assert abs(epi.activation(np.array([-30.0]), "gelu")[0]) < 1e-12


def test_gelu_lipschitz_constant():
    # derivative Phi(x) + x phi(x); its extremes are at x = +-sqrt(2)
    x = np.linspace(-10, 10, 2_000_001)
    d = norm.cdf(x) + x * norm.pdf(x)
    peak = float(np.max(np.abs(d)))
    r2 = math.sqrt(2.0)
    assert abs(peak - (norm.cdf(r2) + r2 * norm.pdf(r2))) < 1e-9
    assert peak <= epi.GELU_LIPSCHITZ < peak + 1e-3


def test_relu_invariants():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((4, 9))
    r = epi.activation(y, "relu")
    assert (r >= 0).all()
    assert np.array_equal(r - epi.activation(-y, "relu"), y)
    assert np.array_equal(epi.activation(r, "relu"), r)


def test_beta_zero_ignores_prior_output():
    P = np.array([[1.0, -2.0]])
    C0 = np.array([[np.nan, np.inf]])
    D, _ = epi.epilogue_ref(P, C0, 3.0, 0.0, None, "none")
    assert np.array_equal(D, [[3.0, -6.0]])


def test_bound_scales_and_covers_rounding():
    P = np.array([[1.0, -2.0]])
    S = np.array([[10.0, 20.0]])
    b0 = epi.epilogue_bound(S, P, None, 1.0, 0.0, None, "none")
    b2 = epi.epilogue_bound(S, P, None, -2.0, 0.0, None, "none")
    assert np.all(b2 > 1.9 * b0)
    # an fp32 evaluation of the epilogue on exact inputs stays inside the bound
    rng = np.random.default_rng(11)
    P = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    C0 = rng.standard_normal((64, 64)).astype(np.float32).astype(np.float64)
    bias = rng.standard_normal(64).astype(np.float32).astype(np.float64)
    alpha, beta = np.float32(0.7), np.float32(-1.3)
    y32 = (alpha * P.astype(np.float32) + beta * C0.astype(np.float32)) + bias.astype(np.float32)[None, :]
    D, _ = epi.epilogue_ref(P, C0, float(alpha), float(beta), bias, "none")
    bound = epi.epilogue_bound(np.zeros_like(P), P, C0, float(alpha), float(beta), bias, "none")
    ok, worst, _ = epi.within_bound(y32, D, bound)
    assert ok, worst
