"""fp64 reference of the fused GEMM epilogue.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the library.  It shares
no code with the HIP path.

What it computes (CUTLASS optimisation guide, "Epilogue Optimization": the
epilogue forms D = alpha.AB + beta.C, and "Fused Epilogue Operations": a bias
addition and a ReLU or GELU activation fused into it):

    D[i,j] = act(alpha * P[i,j] + beta * C0[i,j] + bias[j])

where P = A.B is the fp64 product from ``oracle.gemm.ref_gemm`` and C0 is the
prior content of the output.  Readings where the page leaves a step open:

* the bias is one value per output column j (broadcast over rows) and is added
  before the activation;
* GELU is the exact form x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), Phi the
  standard normal CDF;
* with beta == 0 the prior output is not read at all (a NaN there does not
  propagate), as in BLAS.

``epilogue_bound`` gives the elementwise tolerance: the GEMM bound scaled by
|alpha|, the epilogue's own fp32 roundings, all multiplied by the activation's
Lipschitz constant.

Pins (tests/test_oracle_epilogue.py): the identity epilogue equals the plain
product, hand-computed small cases, standard normal CDF table values for GELU,
the symmetry gelu(x) - gelu(-x) = x, ReLU invariants, beta = 0 ignoring NaN, and
planted mistakes (``mutation``) that the pins must catch.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
from scipy.special import erf

from .gemm import TOLERANCE

ACTS = ("none", "relu", "gelu")

# fp32 rounding allowance of the epilogue arithmetic: beta*c, the fused
# alpha*acc + beta*c and the bias addition each round once (unit 2^-24), with
# margin for the activation's own steps.
EPI_EPS = 2.0 ** -21

# sup |d/dx x Phi(x)| = sup |Phi(x) + x phi(x)|: the derivative peaks at
# x = sqrt(2) (where its own derivative phi(x) (2 - x^2) vanishes) with
# Phi(sqrt 2) + sqrt(2) phi(sqrt 2) = 1.12880...; the test recomputes it.
GELU_LIPSCHITZ = 1.1290


def _gelu(x: np.ndarray, mutation: int = 0) -> np.ndarray:
    if mutation == 3:   # planted: wrong scaling of the erf argument
        return 0.5 * x * (1.0 + erf(x / 2.0))
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def activation(y: np.ndarray, act: str, mutation: int = 0) -> np.ndarray:
    if act == "none":
        return y
    if act == "relu":
        if mutation == 4:   # planted: leaky negative side
            return np.where(y > 0, y, 0.01 * y)
        return np.maximum(y, 0.0)
    if act == "gelu":
        return _gelu(y, mutation)
    raise ValueError(f"unknown activation {act!r}")


def epilogue_ref(P: np.ndarray, C0: Optional[np.ndarray], alpha: float = 1.0, beta: float = 0.0,
                 bias: Optional[np.ndarray] = None, act: str = "none", mutation: int = 0):
    """Returns (D, Y): the epilogue output and its pre-activation value, fp64."""
    P = np.asarray(P, dtype=np.float64)
    y = float(alpha) * P
    if beta != 0.0:
        if C0 is None:
            raise ValueError("beta != 0 needs the prior output C0")
        c0 = np.asarray(C0, dtype=np.float64)
        if mutation == 1:   # planted: beta applied to the product instead of C0
            y = y + float(beta) * P
        else:
            y = y + float(beta) * c0
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        if mutation == 2:   # planted: bias indexed by row instead of column
            y = y + b[np.arange(y.shape[0]) % b.size][:, None]
        else:
            y = y + b[None, :]
    return activation(y, act, mutation), y


def epilogue_bound(S: np.ndarray, P: np.ndarray, C0: Optional[np.ndarray], alpha: float, beta: float,
                   bias: Optional[np.ndarray], act: str, tol: float = TOLERANCE) -> np.ndarray:
    """Elementwise bound on |D_gpu - D| for an fp32 epilogue over an fp32 product."""
    S = np.asarray(S, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    mag = np.abs(float(alpha) * P)
    if beta != 0.0:
        mag = mag + np.abs(float(beta) * np.asarray(C0, dtype=np.float64))
    if bias is not None:
        mag = mag + np.abs(np.asarray(bias, dtype=np.float64))[None, :]
    lin = tol * abs(float(alpha)) * S + EPI_EPS * mag
    if act == "gelu":
        return GELU_LIPSCHITZ * lin + EPI_EPS * mag
    return lin


def within_bound(d_test: np.ndarray, d_ref: np.ndarray, bound: np.ndarray):
    """``|d_test - d_ref| <= bound`` elementwise; returns (ok, worst ratio, index)."""
    d_test = np.asarray(d_test, dtype=np.float64)
    err = np.abs(d_test - d_ref)
    bad = ~(err <= bound)
    if err.size == 0:
        return True, 0.0, None
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err == 0, 0.0, np.inf))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return (not bool(bad.any())), float(ratio[idx]), idx
