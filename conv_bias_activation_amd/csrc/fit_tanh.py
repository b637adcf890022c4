"""Coefficients of the small-argument branch of the device tanh.

For |x| < 0.625 the kernels evaluate tanh(x) = x * P(x^2), P of degree 5.
P is the least-squares fit of tanh(x)/x on 400 Chebyshev nodes of
x^2 in [0, 0.625^2], with the constant term then fixed at 1.  Run this script
to reprint the constants used in device_common.hpp and the maximum relative
error of the float32 evaluation (Horner with fused multiply-adds) against
float64 numpy.tanh.
"""
import numpy as np

TH, DEG, NODES = 0.625, 5, 400


def fit():
    k = np.arange(NODES)
    t = (np.cos((2 * k + 1) * np.pi / (2 * NODES)) + 1) / 2 * TH * TH
    x = np.sqrt(t)
    f = np.tanh(x) / x
    c, *_ = np.linalg.lstsq(np.vander(t, DEG + 1, increasing=True), f, rcond=None)
    c = c.astype(np.float32)
    c[0] = np.float32(1.0)
    return c


def max_rel_error(c):
    xs = np.linspace(1e-6, TH, 400001).astype(np.float32)
    t = (xs * xs).astype(np.float32)
    p = np.full_like(xs, c[-1])
    for ci in c[-2::-1]:
        p = (p.astype(np.float64) * t + ci).astype(np.float32)    # one rounding per fma
    y = (xs * p).astype(np.float32)
    ref = np.tanh(xs.astype(np.float64))
    return float(np.max(np.abs(y - ref) / ref))


if __name__ == "__main__":
    c = fit()
    for i, v in enumerate(c):
        print(f"c{i} = {float(v):.9e}f")
    print(f"max relative error on (0, {TH}): {max_rel_error(c):.3e}")
