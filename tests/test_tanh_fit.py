"""The small-argument tanh polynomial of the soft-capped kernels
(varlen_sliding_window_amd/csrc/device.h, tanh_narrow): for |x| < 0.55 the
kernels use tanh(x) = x + x^3 g(x^2) with a quartic g fitted by weighted
least squares to (tanh(x) - x) / x^3.  This test reads the five coefficients
out of the source, refits them from that definition (weights chosen so the
residual is the relative error of tanh), and checks that

- the source's polynomial has a relative error below 2.5e-7 on |x| < 0.55
  (evaluated in fp64, and in fp32 with the kernels' Horner order and fmas);
- the refit and the source coefficients agree to a few units in the last
  printed place of each, and their error curves are equally good.
"""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEVICE_H = os.path.join(ROOT, "varlen_sliding_window_amd", "csrc", "device.h")
NARROW = 0.55


def source_coefficients():
    text = open(DEVICE_H).read()
    body = text[text.index("float tanh_narrow(float x)"):]
    body = body[:body.index("}")]
    start = float(re.search(r"float g = (-?[0-9.e-]+)f;", body).group(1))
    steps = [float(v) for v in re.findall(r"g = fmaf\(g, y, (-?[0-9.e-]+)f\);", body)]
    # Horner from the highest power: returns g's coefficients c0 .. c4 (ascending powers of y)
    return np.array(list(reversed([start] + steps)), dtype=np.float64)


def refit():
    x = np.linspace(1e-4, NARROW, 20001)
    target = (np.tanh(x) - x) / x ** 3
    w = x ** 3 / np.tanh(x)            # residual in g times w = relative error of tanh
    y = x * x
    a = np.stack([y ** k for k in range(5)], axis=1) * w[:, None]
    coef, *_ = np.linalg.lstsq(a, target * w, rcond=None)
    return coef


def rel_err_f64(c, x):
    y = x * x
    g = np.polynomial.polynomial.polyval(y, c)
    return np.abs((x + x ** 3 * g) - np.tanh(x)) / np.abs(np.tanh(x))


def tanh_narrow_f32(c, x):
    x = x.astype(np.float32)
    y = (x * x).astype(np.float32)
    c32 = c.astype(np.float32)
    g = np.full_like(x, c32[4])
    for k in (3, 2, 1, 0):
        g = (g.astype(np.float64) * y + c32[k]).astype(np.float32)   # one rounding: an fma
    return ((x * y).astype(np.float64) * g + x).astype(np.float32)


def test_source_polynomial_is_accurate():
    c = source_coefficients()
    assert len(c) == 5
    x = np.linspace(1e-6, NARROW, 200001)
    assert rel_err_f64(c, x).max() < 2.5e-7
    got = tanh_narrow_f32(c, x).astype(np.float64)
    assert (np.abs(got - np.tanh(x)) / np.tanh(x)).max() < 4e-7


def test_source_coefficients_are_the_weighted_least_squares_fit():
    c = source_coefficients()
    r = refit()
    # leading coefficient -1/3 (Taylor) and the rest close to the refit
    assert abs(c[0] + 1.0 / 3.0) < 2e-7
    np.testing.assert_allclose(c, r, rtol=2e-3, atol=2e-6)
    x = np.linspace(1e-6, NARROW, 200001)
    assert rel_err_f64(c, x).max() <= 1.5 * rel_err_f64(r, x).max() + 1e-9
