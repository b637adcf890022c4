"""Coefficients of the device erfc used by the GELU epilogue.

For x >= 0 the kernels evaluate erfc(x) = t * exp(-x^2 + P(t)) with
t = 1 / (1 + x/2) and P a polynomial of degree 9: the functional form of the
Chebyshev-fitted erfc of Press, Teukolsky, Vetterling and Flannery
(Numerical Recipes, section 6.2), whose exponent is smooth in t on the whole
half-line.  The coefficients here are this script's own least-squares fit of
P(t) = ln(erfc(x) / t) + x^2 on Chebyshev nodes of t in [1/6, 1]
(x in [0, 10]; past x = 10 erfc is below the float32 range); negative
arguments use erfc(-x) = 2 - erfc(x).  Run it to reprint the constants used
in device_common.hpp and the maximum relative error of the float32
evaluation (Horner with fused multiply-adds, exp through exp2) against
scipy.special.erfc in float64.
"""
import numpy as np
from scipy.special import erfc

DEG, NODES, XMAX = 9, 800, 10.0
LOG2E = 1.4426950408889634


def fit():
    tmin = 1.0 / (1.0 + XMAX / 2.0)
    k = np.arange(NODES)
    t = tmin + (np.cos((2 * k + 1) * np.pi / (2 * NODES)) + 1) / 2 * (1.0 - tmin)
    x = 2.0 * (1.0 / t - 1.0)
    f = np.log(erfc(x) / t) + x * x
    c, *_ = np.linalg.lstsq(np.vander(t, DEG + 1, increasing=True), f, rcond=None)
    return c.astype(np.float32)


def eval_f32(c, xs):
    """The device's evaluation order, one float32 rounding per operation."""
    f32 = np.float32
    xs = xs.astype(f32)
    t = (f32(1.0) / (f32(1.0) + f32(0.5) * xs)).astype(f32)
    p = np.full_like(xs, c[-1])
    for ci in c[-2::-1]:
        p = (p.astype(np.float64) * t + ci).astype(f32)              # fma
    e = (p.astype(np.float64) - xs.astype(np.float64) * xs).astype(f32)   # fma(-x, x, p)
    y = (t * np.exp2((e * f32(LOG2E)).astype(f32).astype(np.float64)).astype(f32)).astype(f32)
    return y


def max_rel_error(c, lo=0.0, hi=9.0):
    xs = np.linspace(lo, hi, 900001).astype(np.float32)
    ref = erfc(xs.astype(np.float64))
    y = eval_f32(c, xs).astype(np.float64)
    return float(np.max(np.abs(y - ref) / ref))


if __name__ == "__main__":
    c = fit()
    for i, v in enumerate(c):
        print(f"c{i} = {float(v):.9e}f")
    for lo, hi in ((0.0, 1.0), (1.0, 4.0), (4.0, 9.0)):
        print(f"max relative error of the float32 evaluation on [{lo}, {hi}]: {max_rel_error(c, lo, hi):.3e}")
