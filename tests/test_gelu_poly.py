"""The polynomial GELU of the fast kernel (gelu_erf_poly in device_common.h), checked on
the CPU: its coefficients are read from the header and its instruction sequence is
evaluated in float32 against exact-erf GELU (scipy's erf in float64). This pins the
formula; the GPU parity tests pin its execution."""
import os
import re

import numpy as np
from scipy.special import erf

from ff_input_projection_amd import build as fpbuild


def _coefficients():
    src = open(os.path.join(fpbuild.CSRC, "device_common.h")).read()
    body = src[src.index("float gelu_erf_poly(float y)"):]
    body = body[: body.index("\n}\n")]
    first = re.search(r"float p = ([-+0-9.e]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, a, ([-+0-9.e]+)f\);", body)
    clamp = float(re.search(r"fmed3f\(fabsf\(y\), 0\.0f, ([0-9.]+)f\)", body).group(1))
    # the positive part max(y, 0) is (y + |y|) / 2
    assert "0.5f * (y + fabsf(y))" in body
    return [np.float32(first)] + [np.float32(c) for c in rest], np.float32(clamp)


def _gelu_poly_f32(y, coef, clamp):
    y = np.asarray(y, np.float32)
    a = np.minimum(np.abs(y), clamp)
    p = np.full_like(a, coef[0])
    for c in coef[1:]:
        # fmaf: one rounding of the exact p * a + c
        p = (p.astype(np.float64) * a.astype(np.float64) + np.float64(c)).astype(np.float32)
    e = np.exp2(p.astype(np.float64)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        pos = np.float32(0.5) * (y + np.abs(y))                                 # (y + |y|) / 2, exact
    with np.errstate(invalid="ignore"):
        out = -a.astype(np.float64) * e.astype(np.float64) + pos.astype(np.float64)
    return out.astype(np.float32)


def _gelu_exact(y):
    y = np.asarray(y, np.float64)
    return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))


def test_polynomial_gelu_within_1e5_of_exact_erf_gelu():
    coef, clamp = _coefficients()
    assert len(coef) == 7 and clamp == 6.0
    y = np.concatenate([np.linspace(-12, 12, 1_200_001), [-1e4, -50.0, 0.0, 50.0, 1e4]]).astype(np.float32)
    err = np.abs(_gelu_poly_f32(y, coef, clamp).astype(np.float64) - _gelu_exact(y))
    assert err.max() < 1e-5, err.max()


def test_polynomial_gelu_special_values():
    coef, clamp = _coefficients()
    y = np.array([0.0, 1.0, -1.0, 3.0, -3.0], np.float32)
    got = _gelu_poly_f32(y, coef, clamp).astype(np.float64)
    # gelu(0) = 0; gelu(y) - gelu(-y) = y (Phi(y) + Phi(-y) = 1)
    assert abs(got[0]) < 1e-9
    assert abs((got[1] - got[2]) - 1.0) < 2e-5 and abs((got[3] - got[4]) - 3.0) < 2e-5


def test_polynomial_gelu_non_finite_values_follow_the_definition():
    """y Phi(y) in IEEE arithmetic (the oracle's and torch's float64 GELU): NaN stays NaN,
    +inf stays +inf, and -inf gives -inf * 0 = NaN. A min / max / med3 positive part would
    turn NaN into a finite value."""
    import torch
    coef, clamp = _coefficients()
    y = np.array([np.nan, np.inf, -np.inf], np.float32)
    got = _gelu_poly_f32(y, coef, clamp)
    ref = torch.nn.functional.gelu(torch.from_numpy(y.astype(np.float64))).numpy()
    assert np.isnan(got[0]) and np.isnan(ref[0])
    assert got[1] == np.inf and ref[1] == np.inf
    assert np.isnan(got[2]) and np.isnan(ref[2])


def _grad_coefficients():
    src = open(os.path.join(fpbuild.CSRC, "device_common.h")).read()
    body = src[src.index("float gelu_erf_grad_poly(float y)"):]
    body = body[: body.index("\n}\n")]
    first = re.search(r"float p = ([-+0-9.e]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, a, ([-+0-9.e]+)f\);", body)
    pdf_k = float(re.search(r"exp2f\(([-0-9.e]+)f \* \(y \* y\)\)", body).group(1))
    pdf_c = float(re.search(r"const float pdf = ([0-9.e]+)f \*", body).group(1))
    return [np.float32(first)] + [np.float32(c) for c in rest], np.float32(pdf_k), np.float32(pdf_c)


def test_polynomial_gelu_derivative_within_3e5_of_exact():
    """gelu_erf_grad_poly (the backward pass's dy = d_ff * GELU'(y) on the fast kernel): its
    coefficients read from the header (the forward's Phi(-a) polynomial and the normal
    density's constants), evaluated in float32, against Phi(y) + y phi(y) in float64."""
    coef, pdf_k, pdf_c = _grad_coefficients()
    fwd, _ = _coefficients()
    assert [float(c) for c in coef] == [float(c) for c in fwd]
    y = np.concatenate([np.linspace(-12, 12, 1_200_001), [-1e4, -50.0, 0.0, 50.0, 1e4]]).astype(np.float32)
    a = np.minimum(np.abs(y), np.float32(6))
    p = np.full_like(a, coef[0])
    for c in coef[1:]:
        p = (p.astype(np.float64) * a.astype(np.float64) + np.float64(c)).astype(np.float32)
    q = np.exp2(p.astype(np.float64)).astype(np.float32)
    cdf = np.where(y >= 0, (np.float32(1) - q).astype(np.float32), q)
    arg = (pdf_k * (y * y).astype(np.float32)).astype(np.float32)
    pdf = (pdf_c * np.exp2(arg.astype(np.float64)).astype(np.float32)).astype(np.float32)
    got = (y.astype(np.float64) * pdf.astype(np.float64) + cdf.astype(np.float64)).astype(np.float32)
    yd = y.astype(np.float64)
    exact = 0.5 * (1 + erf(yd / np.sqrt(2))) + yd * np.exp(-0.5 * yd * yd) / np.sqrt(2 * np.pi)
    err = np.abs(got.astype(np.float64) - exact)
    assert err.max() < 3e-5, err.max()
    # GELU'(y) + GELU'(-y) = Phi(y) + Phi(-y) = 1
    pos = np.linspace(0.01, 8, 800).astype(np.float32)
    def g(v):
        a = np.minimum(np.abs(v), np.float32(6))
        p = np.full_like(a, coef[0])
        for c in coef[1:]:
            p = (p.astype(np.float64) * a.astype(np.float64) + np.float64(c)).astype(np.float32)
        q = np.exp2(p.astype(np.float64)).astype(np.float32)
        cdf = np.where(v >= 0, (np.float32(1) - q).astype(np.float32), q)
        pdf = (pdf_c * np.exp2((pdf_k * (v * v).astype(np.float32)).astype(np.float64)).astype(np.float32))
        return v.astype(np.float64) * pdf.astype(np.float64) + cdf.astype(np.float64)
    assert np.abs(g(pos) + g(-pos) - 1.0).max() < 1e-6
