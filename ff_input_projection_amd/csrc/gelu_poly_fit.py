"""Coefficients of the polynomial GELU used by the HIP kernels (gelu_erf_poly in
device_common.h).

Exact-erf GELU is gelu(y) = y * Phi(y) with Phi the standard normal CDF. Writing
q(a) = Phi(-a) = erfc(a / sqrt(2)) / 2 for a = |y| >= 0 gives

    gelu(y) = max(y, 0) - |y| * q(|y|),

and log2 q(a) is smooth on [0, A] (it tends to -a^2 / (2 ln 2) minus a slowly growing
logarithm), so it is approximated by one polynomial P of degree 6 in a. The kernel
clamps a to A = 6 in both places it is used (past 6, |y| * q(|y|) < 1e-8, and
6 * q(6) stands for it).

The fit is a weighted least-squares fit on Chebyshev nodes with iteratively
reweighted errors (a near-minimax fit). Run this file to print the coefficients and
the error bound that tests/test_gelu_poly.py checks.
"""
import numpy as np
from scipy.special import erf, erfc

A = 6.0
DEG = 6


def fit(deg=DEG, a_max=A, nodes=4000, iters=40):
    x = np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes) * a_max / 2 + a_max / 2
    f = np.log2(0.5 * erfc(x / np.sqrt(2)))
    w = np.ones_like(x)
    V = np.vander(x, deg + 1)
    for _ in range(iters):
        c, *_ = np.linalg.lstsq(V * w[:, None], f * w, rcond=None)
        e = np.abs(V @ c - f)
        w = w * (e / e.max() + 0.05) ** 0.5
    return c  # highest degree first


def gelu_poly_f32(y, c):
    """The kernel's sequence in float32 (exp2 modelled as correctly rounded)."""
    y = np.asarray(y, np.float32)
    a = np.minimum(np.abs(y), np.float32(A))
    p = np.float32(c[0])
    for ci in c[1:]:
        p = (p * a + np.float32(ci)).astype(np.float32)
    e = np.exp2(p.astype(np.float64)).astype(np.float32)
    return (np.maximum(y, np.float32(0)) - a * e).astype(np.float32)


def gelu_exact(y):
    y = np.asarray(y, np.float64)
    return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))


if __name__ == "__main__":
    c = fit()
    print(f"coefficients (a^{DEG} .. a^0):")
    for ci in c:
        print(f"    {float(np.float32(ci))!r}f")
    y = np.linspace(-12, 12, 2_000_001)
    err = np.abs(gelu_poly_f32(y, c).astype(np.float64) - gelu_exact(y))
    print(f"max |gelu_poly - gelu| on [-12, 12]: {err.max():.3e}")
