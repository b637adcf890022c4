"""Acceptance rule for comparing a device result with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The rule:
  * fp32 output, fp16/bf16 inputs:   |y - ref| <= 1e-3 * (1 + |ref|)
    (the same scale as the rtol = atol = 1e-3 allclose check that the
    MatmulLeakyRelu sample of "CANN pyasc MatmulLeakyRelu 融合算子实战" runs
    in its 编译执行 section);
  * fp32 output, fp32 inputs:        |y - ref| <= 1e-5 * (1 + |ref|);
  * fp16 / bf16 output:              |y - ref| <= ulp_out(ref) + E, one ulp
    of the output format at |ref| plus E, a bound on the device's fp32
    accumulation error (Higham: gamma_n * (sum_k |a_k b_k| + |bias|) with
    n = K + 1 terms, gamma_n = n u / (1 - n u), u = 2^-24).  The device
    result is round(z) with |z - ref| <= E, so |y - ref| <= ulp/2 + E; without
    E an output whose exact value is tiny next to sum |a_k b_k| would demand
    an fp32 sum far more accurate than fp32 itself.
  * int32 output (int8 operands, int32 bias; every sum exact): bit-exact;
  * fp32 output, int8 operands: the fp32-input rule (the integer sum is
    exact; only its conversion to fp32 and the activation round);
  * fp32 output with an error bound E given (used only for shapes outside
    the named workloads, e.g. fp32 inputs with K > 512, where fp32 summation
    error alone exceeds 1e-5 * (1 + |ref|)): max(rule, E).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

# (precision p incl. the implicit bit, smallest normal exponent, subnormal spacing)
_FMT = {
    "f16": (11, -14, 2.0 ** -24),
    "bf16": (8, -126, 2.0 ** -133),
    "f32": (24, -126, 2.0 ** -149),
}


def ulp(v: np.ndarray, fmt: str) -> np.ndarray:
    """Spacing of the `fmt` grid at |v| (2^(floor(log2|v|) - p + 1), or the
    subnormal spacing below the smallest normal)."""
    p, emin, sub = _FMT[fmt]
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(a)                   # a = m * 2^e, m in [0.5, 1)  => floor(log2 a) = e - 1
    u = np.ldexp(1.0, (e - 1) - p + 1)
    return np.where(a < 2.0 ** emin, sub, u)


def gamma(K: int, u: float = 2.0 ** -24) -> float:
    return K * u / (1.0 - K * u)


def tolerance(ref: np.ndarray, in_dtype: str, out_dtype: str,
              err_floor: Optional[np.ndarray] = None) -> np.ndarray:
    ref = np.asarray(ref, dtype=np.float64)
    e = 0.0 if err_floor is None else np.asarray(err_floor, dtype=np.float64)
    if out_dtype == "i32":
        return np.zeros_like(ref)
    if out_dtype == "f32":
        rel = 1e-5 if in_dtype in ("f32", "i8") else 1e-3
        return np.maximum(rel * (1.0 + np.abs(ref)), e)
    return ulp(np.abs(ref), out_dtype) + e


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
            err_floor: Optional[np.ndarray] = None) -> dict:
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    floor = None if err_floor is None else np.asarray(err_floor, dtype=np.float64).ravel()
    tol = tolerance(ref, in_dtype, out_dtype, floor)
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
    if floor is not None:
        rep["max_floor"] = float(floor.max()) if floor.size else 0.0
    if n_bad:
        k = int(np.argmax(np.where(bad, err / np.where(tol > 0, tol, 1e-300), -1)))
        rep["worst"] = {"index": k, "y": float(y[k]), "ref": float(ref[k]), "tol": float(tol[k])}
    rep["ok"] = n_bad == 0
    return rep
