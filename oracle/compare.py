"""Acceptance rule for comparing a device result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The rule, per output element with oracle value ref:

  * fp32 output, fp16/bf16 inputs:   |y - ref| <= 1e-3 * (1 + |ref|)
    (the scale of the rtol = atol = 1e-3 acceptance check of the
    MatmulLeakyRelu sample, "CANN pyasc MatmulLeakyRelu 融合算子实战",
    section 编译执行);
  * fp32 output, fp32 inputs:        |y - ref| <= 1e-5 * (1 + |ref|), with no
    allowance for the fp32 accumulation error: a shape whose accumulation
    error exceeds it fails and the report carries the element's gamma_K
    bound;
  * fp32 output, int8 operands: the fp32-input rule (the integer sum is
    exact; only its conversion to fp32 and the activation round);
  * int32 output (int8 operands, int32 bias; every sum exact): bit-exact;
  * fp16 / bf16 output: one output ulp,
        |y - ref| <= max(ulp(ref), ulp(|ref| + d) / 2 + d),
    where d bounds how far the device's fp32 activation value can sit from
    ref before its single rounding to the output format:
        d = L * E + ETA_ACT * |ref|.
    E = gamma_n * S bounds the fp32 accumulation error of the pre-activation
    z (Higham's bound: S = sum_k |a_k b_k| + |bias| (+ |R|), n the number of
    terms, gamma_n = n u / (1 - n u), u = 2^-24); L is the largest slope
    |act'| anywhere in [z - E, z + E] (ReLU past zero and LeakyReLU's
    negative side pass on none or alpha of it; tanh and Sigmoid at most
    1 - tanh^2 and s(1 - s) at the interval's point nearest 0); ETA_ACT
    bounds the relative error of an fp32 activation evaluation.  A rounding
    to nearest of a value within d of ref is within ulp(|ref| + d) / 2 + d of
    it, so a correct fp32-accumulate kernel always passes; where d is below
    half an ulp the rule is plain "one output ulp".
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

# (precision p incl. the implicit bit, smallest normal exponent, subnormal spacing)
_FMT = {
    "f16": (11, -14, 2.0 ** -24),
    "bf16": (8, -126, 2.0 ** -133),
    "f32": (24, -126, 2.0 ** -149),
}

# relative error allowed to one fp32 evaluation of an activation
ETA_ACT = 2.0 ** -15


def ulp(v: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of the `fmt` grid at |v| (2^(floor(log2|v|) - p + 1), or the
    subnormal spacing below the smallest normal)."""
    p, emin, sub = _FMT[fmt]
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)                   # a = m * 2^e, m in [0.5, 1)  => floor(log2 a) = e - 1
    u = np.ldexp(1.0, (e - 1) - p + 1)
    return np.where(a < 2.0 ** emin, sub, u)


def gamma(n: int, u: float = 2.0 ** -24) -> float:
    """Higham's gamma_n = n u / (1 - n u)."""
    return n * u / (1.0 - n * u)


def _phi(t):
    return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)


def _Phi(t):
    from scipy.special import ndtr         # the standard normal CDF
    return ndtr(np.asarray(t, dtype=np.float64))


def slope_bound(z: np.ndarray, e: np.ndarray, act: str, alpha: float = 0.0) -> np.ndarray:
    """sup |act'(t)| over t in [z - e, z + e], elementwise."""
    z = np.asarray(z, dtype=np.float64)
    e = np.broadcast_to(np.asarray(e, dtype=np.float64), z.shape)
    if act == "none":
        return np.ones_like(z)
    if act == "relu":
        return np.where(z + e > 0.0, 1.0, 0.0)
    if act == "leaky_relu":
        return np.where(z + e >= 0.0, 1.0, abs(alpha))
    near = np.maximum(np.abs(z) - e, 0.0)       # |t| nearest 0 within the interval
    if act == "tanh":
        t = np.tanh(near)
        return 1.0 - t * t
    if act == "sigmoid":
        s = 0.5 * (1.0 + np.tanh(0.5 * near))
        return s * (1.0 - s)
    if act == "gelu":
        # GELU'(t) = Phi(t) + t phi(t); its extrema sit at t = +-sqrt(2)
        lo, hi = z - e, z + e
        d = lambda t: np.abs(_Phi(t) + t * _phi(t))
        out = np.maximum(d(lo), d(hi))
        r2 = math.sqrt(2.0)
        for c in (-r2, r2):
            inside = (lo <= c) & (c <= hi)
            if np.any(inside):
                out = np.where(inside, np.maximum(out, float(d(np.array(c)))), out)
        return out
    raise ValueError(f"unknown activation {act!r}")


def propagated_bound(z: np.ndarray, abs_sum: np.ndarray, n_terms: int, act: str,
                     alpha: float = 0.0) -> np.ndarray:
    """L * E: the accumulation bound E = gamma_n * abs_sum carried through the
    activation at pre-activation z."""
    E = gamma(n_terms) * np.asarray(abs_sum, dtype=np.float64)
    return slope_bound(z, E, act, alpha) * E


def tolerance(ref: np.ndarray, in_dtype: str, out_dtype: str,
              acc: Optional[np.ndarray] = None) -> np.ndarray:
    """Allowed |y - ref| per element; `acc` is the propagated accumulation
    bound L * E (used for 16-bit outputs only)."""
    ref = np.asarray(ref, dtype=np.float64)
    if out_dtype == "i32":
        return np.zeros_like(ref)
    if out_dtype == "f32":
        rel = 1e-5 if in_dtype in ("f32", "i8") else 1e-3
        return rel * (1.0 + np.abs(ref))
    a = np.abs(ref)
    d = ETA_ACT * a
    if acc is not None:
        d = d + np.asarray(acc, dtype=np.float64)
    return np.maximum(ulp(a, out_dtype), 0.5 * ulp(a + d, out_dtype) + d)


def decode_out(words: np.ndarray, out_dtype: str) -> np.ndarray:
    """Device output words -> float64 (numpy's own conversions; the oracle's
    decoders are kept for the oracle side)."""
    w = np.ascontiguousarray(words)
    if out_dtype == "f32":
        return w.view(np.float32).astype(np.float64)
    if out_dtype == "f16":
        return w.view(np.float16).astype(np.float64)
    if out_dtype == "bf16":
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if out_dtype == "i32":
        return w.view(np.int32).astype(np.float64)
    raise ValueError(out_dtype)


def compare(y: np.ndarray, ref: np.ndarray, in_dtype: str, out_dtype: str,
            acc: Optional[np.ndarray] = None, abs_sum: Optional[np.ndarray] = None,
            n_terms: Optional[int] = None) -> dict:
    """Element-by-element report.  `abs_sum` / `n_terms`, when given, only
    add each failing element's gamma_K accumulation bound to the report."""
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    acc = None if acc is None else np.asarray(acc, dtype=np.float64).ravel()
    tol = tolerance(ref, in_dtype, out_dtype, acc)
    err = np.abs(y - ref)
    bad = ~(err <= tol)                   # NaN counts as bad
    n_bad = int(bad.sum())
    rep = {
        "n": int(y.size),
        "n_bad": n_bad,
        "max_abs_err": float(np.nanmax(err)) if y.size else 0.0,
        # an exact (zero) tolerance: any error is infinitely over it
        "max_err_over_tol": float(np.nanmax(np.where(tol > 0, err / np.where(tol > 0, tol, 1.0),
                                                     np.where(err > 0, np.inf, 0.0))))
        if y.size else 0.0,
        "n_nonfinite": int((~np.isfinite(y)).sum()),
    }
    if out_dtype in ("f16", "bf16") and y.size:
        in_ulps = err / ulp(ref, out_dtype)
        rep["max_err_ulp"] = float(np.nanmax(in_ulps))
        rep["n_within_1ulp"] = int((in_ulps <= 1.0).sum())
        rep["frac_within_1ulp"] = rep["n_within_1ulp"] / y.size
        if acc is not None:
            rep["max_acc_bound_ulp"] = float(np.nanmax(acc / ulp(ref, out_dtype)))
    if n_bad:
        k = int(np.argmax(np.where(bad, err / np.where(tol > 0, tol, 1e-300), -1)))
        worst = {"index": k, "y": float(y[k]), "ref": float(ref[k]), "tol": float(tol[k])}
        if abs_sum is not None and n_terms is not None:
            worst["gamma_K_bound"] = float(gamma(n_terms) * np.asarray(abs_sum).ravel()[k])
        rep["worst"] = worst
    rep["ok"] = n_bad == 0
    return rep


def merge(reports) -> dict:
    """One report over several compare() reports of disjoint chunks."""
    reports = list(reports)
    out = {"n": sum(r["n"] for r in reports), "n_bad": sum(r["n_bad"] for r in reports),
           "n_nonfinite": sum(r["n_nonfinite"] for r in reports)}
    for key in ("max_abs_err", "max_err_over_tol", "max_err_ulp", "max_acc_bound_ulp"):
        vals = [r[key] for r in reports if key in r]
        if vals:
            out[key] = max(vals)
    if any("n_within_1ulp" in r for r in reports):
        out["n_within_1ulp"] = sum(r.get("n_within_1ulp", 0) for r in reports)
        out["frac_within_1ulp"] = out["n_within_1ulp"] / max(out["n"], 1)
    worst = [r["worst"] for r in reports if "worst" in r]
    if worst:
        out["worst"] = worst[0]
    out["ok"] = out["n_bad"] == 0
    return out
