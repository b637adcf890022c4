"""Shared helpers of the GPU tests: move encoded inputs to the device, run the
library through its binding, and compute the oracle's reference for the same
bits."""
from __future__ import annotations

import numpy as np

import oracle as orc
from oracle.compare import compare, decode_out, gamma
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

def _needs_floor(in_dtype, out_dtype, K):
    return out_dtype != "f32" or (in_dtype == "f32" and K > 512)


def _floor(in_dtype, out_dtype, K, abs_sum):
    """Accumulation-error bound E for the acceptance rule (oracle/compare.py):
    the worst-case gamma_{K+1} * sum|a b| for 16-bit outputs; for fp32 inputs
    beyond K = 512 the probabilistic bound lambda * sqrt(K+1) * u * sum|a b|
    (Higham & Mary, 2019) with lambda = 6."""
    if out_dtype != "f32":
        return gamma(K + 1) * abs_sum
    return 6.0 * np.sqrt(K + 1) * 2.0 ** -24 * abs_sum


def gemm_reference(case: wl.GemmCase, inp, idx=None):
    """Oracle values (and the fp32 accumulation-error floor) for all outputs,
    or for the flat indices `idx`."""
    o = O()
    A = o.decode(inp["A"], case.in_dtype)
    B = o.decode(inp["B"], case.in_dtype)
    bias = o.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
    alpha = orc.f32(case.alpha)
    floor = None
    need = _needs_floor(case.in_dtype, case.out_dtype, case.K)
    absb = None if bias is None else np.abs(bias)
    R = None if inp.get("R") is None else o.decode(inp["R"].ravel(), case.out_dtype)
    terms = case.K + (R is not None)
    if idx is None:
        if R is None:
            ref = o.gemm(A, B, bias, case.act, alpha).ravel()
        else:
            ref = o.gemm_residual(A, B, bias, R.reshape(case.M, case.N), case.act, alpha).ravel()
        if need:
            s = o.gemm(np.abs(A), np.abs(B), absb, "none").ravel()
            if R is not None:
                s = s + np.abs(R)
            floor = _floor(case.in_dtype, case.out_dtype, terms, s)
    else:
        ii, jj = idx // case.N, idx % case.N
        if R is None:
            ref = o.gemm_elems(A, B, bias, ii, jj, case.act, alpha)
        else:
            ref = o.gemm_residual_elems(A, B, bias, R[idx], ii, jj, case.act, alpha)
        if need:
            s = o.gemm_elems(np.abs(A), np.abs(B), absb, ii, jj, "none")
            if R is not None:
                s = s + np.abs(R[idx])
            floor = _floor(case.in_dtype, case.out_dtype, terms, s)
    return ref, floor


def conv_reference(case: wl.ConvCase, inp, idx=None):
    o = O()
    x = o.decode(inp["x"], case.in_dtype)
    w = o.decode(inp["w"], case.in_dtype)
    bias = o.decode(inp["bias"], case.bias_dtype) if inp["bias"] is not None else None
    args = (case.strides, case.pads, case.dilations)
    K = case.C * case.kh * case.kw
    floor = None
    absb = None if bias is None else np.abs(bias)
    need = _needs_floor(case.in_dtype, case.out_dtype, K)
    R = None if inp.get("R") is None else o.decode(inp["R"].ravel(), case.out_dtype)
    terms = K + (R is not None)
    if idx is None:
        if R is None:
            ref = o.conv2d(x, w, bias, *args, case.act, orc.f32(case.alpha)).ravel()
        else:
            z = o.conv2d(x, w, bias, *args, "none").ravel()
            ref = o.residual_act(z, R, case.act, orc.f32(case.alpha))
        if need:
            s = o.conv2d(np.abs(x), np.abs(w), absb, *args, "none").ravel()
            floor = _floor(case.in_dtype, case.out_dtype, terms, s if R is None else s + np.abs(R))
    else:
        if R is None:
            ref = o.conv2d_elems(x, w, bias, *args, idx, case.act, orc.f32(case.alpha))
        else:
            ref = o.conv2d_residual_elems(x, w, bias, R[idx], *args, idx, case.act,
                                          orc.f32(case.alpha))
        if need:
            s = o.conv2d_elems(np.abs(x), np.abs(w), absb, *args, idx, "none")
            floor = _floor(case.in_dtype, case.out_dtype, terms,
                           s if R is None else s + np.abs(R[idx]))
    return ref, floor


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
