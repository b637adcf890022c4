"""Shared helpers of the GPU tests: move encoded inputs to the device, run the
library through its binding, and compute the oracle's reference for the same
bits."""
from __future__ import annotations

import numpy as np

import oracle as orc
from oracle.compare import compare, decode_out, merge, propagated_bound
import workloads as wl

_O = None


def O():
    global _O
    if _O is None:
        _O = orc.Oracle()
    return _O


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
            "i32": torch.int32}[dt]


def to_dev(words: np.ndarray, dt: str, guard: int = 0, fill_word=None):
    """Encoded words -> contiguous device tensor.  With guard > 0 the tensor is
    a view into a larger buffer with `guard` canary elements on each side;
    returns (tensor, buffer)."""
    import torch
    words = np.ascontiguousarray(words)
    if dt == "f32":
        host = torch.from_numpy(words.view(np.float32).copy())
    elif dt in ("i8", "i32"):
        host = torch.from_numpy(words.view(np.int8 if dt == "i8" else np.int32).copy())
    else:
        host = torch.from_numpy(words.view(np.int16).copy()).view(torch_dtype(dt))
    if not guard:
        return host.cuda(), None
    n = words.size
    buf = torch.empty(n + 2 * guard, dtype=torch_dtype(dt), device="cuda")
    if fill_word is not None:
        _fill_words(buf, fill_word, dt)
    view = buf[guard:guard + n].view(words.shape)
    view.copy_(host.cuda())
    return view, buf


def _fill_words(t, word, dt):
    import torch
    if dt == "f32":
        t.view(torch.int32).fill_(np.int32(np.uint32(word).view(np.int32)))
    else:
        t.view(torch.int16).fill_(int(np.uint16(word).view(np.int16)))


def empty_out(shape, dt: str, guard: int = 0, canary: int | None = None):
    import torch
    n = int(np.prod(shape))
    if not guard:
        t = torch.empty(shape, dtype=torch_dtype(dt), device="cuda")
        if canary is not None:
            _fill_words(t, canary, dt)
        return t, None
    buf = torch.empty(n + 2 * guard, dtype=torch_dtype(dt), device="cuda")
    _fill_words(buf, canary if canary is not None else 0x7FC0, dt)
    return buf[guard:guard + n].view(shape), buf


def words_of(t, dt: str) -> np.ndarray:
    """Flat output words of a device tensor."""
    import torch
    c = t.detach().cpu().contiguous().reshape(-1)
    if dt in ("f32", "i32"):
        return c.view(torch.int32).numpy().view(np.uint32).copy()
    return c.view(torch.int16).numpy().view(np.uint16).copy()


def values_of(t, dt: str) -> np.ndarray:
    """Flat float64 values of a device tensor."""
    return decode_out(words_of(t, dt), dt).ravel()


def guard_intact(buf, guard: int, dt: str, canary: int) -> bool:
    w = words_of(buf, dt)
    return bool(np.all(w[:guard] == canary) and np.all(w[-guard:] == canary))


# ---------------------------------------------------------------------------
# reference computation on the oracle
# ---------------------------------------------------------------------------

def acc_bound(out_dtype, n_terms, z, abs_sum, act, alpha):
    """The accumulation-error allowance of the acceptance rule
    (oracle/compare.py): for 16-bit outputs, gamma_n * abs_sum carried
    through the activation's largest slope near the pre-activation z; None
    for fp32 and int32 outputs, whose rules take no such allowance."""
    if out_dtype in ("f32", "i32"):
        return None
    return propagated_bound(z, abs_sum, n_terms, act, alpha)


def gemm_reference(case: wl.GemmCase, inp, idx=None, rows=None):
    """Oracle values and the accumulation allowance for all outputs, for the
    flat indices `idx`, or for the output rows `rows` (a slice)."""
    o = O()
    A = o.decode(inp["A"], case.in_dtype).reshape(case.M, case.K)
    B = o.decode(inp["B"], case.in_dtype).reshape(case.K, case.N)
    bias = o.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
    alpha = orc.f32(case.alpha)
    need = case.out_dtype not in ("f32", "i32")
    absb = None if bias is None else np.abs(bias)
    R = None if inp.get("R") is None else o.decode(inp["R"].ravel(), case.out_dtype)
    n_terms = case.K + 1 + (R is not None)
    s = None
    if idx is None:
        if rows is not None:
            A = A[rows]
            if R is not None:
                R = R.reshape(case.M, case.N)[rows].ravel()
        z = o.gemm(A, B, bias, "none").ravel()
        if need:
            s = o.gemm(np.abs(A), np.abs(B), absb, "none").ravel()
    else:
        ii, jj = idx // case.N, idx % case.N
        z = o.gemm_elems(A, B, bias, ii, jj, "none")
        if need:
            s = o.gemm_elems(np.abs(A), np.abs(B), absb, ii, jj, "none")
        if R is not None:
            R = R[idx]
    if R is not None:
        z = z + R
        if s is not None:
            s = s + np.abs(R)
    ref = o.act(z, case.act, alpha)
    return ref, acc_bound(case.out_dtype, n_terms, z, s, case.act, alpha)


def conv_reference(case: wl.ConvCase, inp, idx=None):
    o = O()
    x = o.decode(inp["x"], case.in_dtype).reshape(case.N, case.C, case.H, case.W)
    w = o.decode(inp["w"], case.in_dtype).reshape(case.Co, case.C, case.kh, case.kw)
    bias = o.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
    args = (case.strides, case.pads, case.dilations)
    alpha = orc.f32(case.alpha)
    need = case.out_dtype not in ("f32", "i32")
    absb = None if bias is None else np.abs(bias)
    R = None if inp.get("R") is None else o.decode(inp["R"].ravel(), case.out_dtype)
    n_terms = case.C * case.kh * case.kw + 1 + (R is not None)
    s = None
    if idx is None:
        z = o.conv2d(x, w, bias, *args, "none").ravel()
        if need:
            s = o.conv2d(np.abs(x), np.abs(w), absb, *args, "none").ravel()
    else:
        z = o.conv2d_elems(x, w, bias, *args, idx, "none")
        if need:
            s = o.conv2d_elems(np.abs(x), np.abs(w), absb, *args, idx, "none")
        if R is not None:
            R = R[idx]
    if R is not None:
        z = z + R
        if s is not None:
            s = s + np.abs(R)
    ref = o.act(z, case.act, alpha)
    return ref, acc_bound(case.out_dtype, n_terms, z, s, case.act, alpha)


# ---------------------------------------------------------------------------
# device runs
# ---------------------------------------------------------------------------

def run_gemm(case: wl.GemmCase, inp, path: str = "fused", out=None):
    import torch
    import conv_bias_activation_amd as ba
    A, _ = to_dev(inp["A"].reshape(case.M, case.K), case.in_dtype)
    B, _ = to_dev(inp["B"].reshape(case.K, case.N), case.in_dtype)
    bias = None if inp["bias"] is None else to_dev(inp["bias"], case.bias_dtype)[0]
    C = out if out is not None else torch.empty((case.M, case.N), dtype=torch_dtype(case.out_dtype),
                                               device="cuda")
    alpha = float(np.float32(case.alpha))
    R = None if inp.get("R") is None else to_dev(inp["R"].reshape(case.M, case.N), case.out_dtype)[0]
    if path == "fused":
        if R is None:
            ba.gemm_bias_act(A, B, bias, C, case.act, alpha)
        else:
            ba.gemm_bias_add_act(A, B, bias, R, C, case.act, alpha)
    else:
        ws = torch.empty(max(1, ba.gemm_bias_act_workspace_size(case.M, case.N) // 4),
                         dtype=torch.float32, device="cuda")
        if R is None:
            ba.gemm_bias_act_2k(A, B, bias, C, case.act, alpha, workspace=ws)
        else:
            ba.gemm_bias_add_act_2k(A, B, bias, R, C, case.act, alpha, workspace=ws)
    torch.cuda.synchronize()
    return C


def run_conv(case: wl.ConvCase, inp, path: str = "fused", out=None):
    import torch
    import conv_bias_activation_amd as ba
    x, _ = to_dev(inp["x"].reshape(case.N, case.C, case.H, case.W), case.in_dtype)
    w, _ = to_dev(inp["w"].reshape(case.Co, case.C, case.kh, case.kw), case.in_dtype)
    bias = None if inp["bias"] is None else to_dev(inp["bias"], case.bias_dtype)[0]
    Ho, Wo = case.out_hw()
    y = out if out is not None else torch.empty((case.N, case.Co, Ho, Wo),
                                               dtype=torch_dtype(case.out_dtype), device="cuda")
    R = None if inp.get("R") is None else to_dev(inp["R"].reshape(case.N, case.Co, Ho, Wo),
                                                 case.out_dtype)[0]
    args = (case.strides, case.pads, case.dilations, case.act)
    if path == "fused":
        if R is None:
            ba.conv2d_bias_act(x, w, bias, y, *args)
        else:
            ba.conv2d_bias_add_act(x, w, bias, R, y, *args)
    else:
        n = ba.conv2d_bias_act_workspace_size(case.N, case.C, case.H, case.W, case.Co, case.kh,
                                              case.kw, case.strides, case.pads, case.dilations)
        ws = torch.empty(max(1, n // 4), dtype=torch.float32, device="cuda")
        if R is None:
            ba.conv2d_bias_act_2k(x, w, bias, y, *args, workspace=ws)
        else:
            ba.conv2d_bias_add_act_2k(x, w, bias, R, y, *args, workspace=ws)
    torch.cuda.synchronize()
    return y


def check(y_vals, ref, floor, case) -> dict:
    return compare(y_vals, ref, case.in_dtype, case.out_dtype, floor)
