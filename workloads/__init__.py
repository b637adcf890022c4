"""Seeded synthetic inputs for the fused contraction + bias + activation.

This module only *draws* inputs: it holds none of the method's arithmetic.
Both the GPU path and the CPU oracle receive exactly the encoded bit patterns
produced here (fp16 / bf16 / fp32 words), so the two sides see identical
operands.

Values are drawn in fp32 from numpy's PCG64 (``default_rng(seed)``) in a
fixed order (A, B, bias for a GEMM; x, w, bias for a conv) and then rounded
to the operand dtype with round-to-nearest-even.

The shapes and value distributions follow the workloads the pages describe:
the MatmulLeakyRelu sample spec of "CANN pyasc MatmulLeakyRelu 融合算子实战"
(section 样例规格), the 4096^3 fused matmul+ReLU call of the ops-nn
fused_matmul_relu article (section "fused_matmul_relu底层到底做了什么"), and
conv + tanh cases covering the kernel sizes, strides, dilations and dtypes
listed in the "实战效果" section of the multimodal-ops Fused ConvTanh article.
The article's own 24 case shapes are not published, so the conv shapes here
are synthetic stand-ins of the same kinds (3x3 s1, 7x7 s2 stem, 1x1 s2,
3x3 dilation 2).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
DTYPE_SIZES = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i32": 4}
ACT_CODES = {"none": 0, "relu": 1, "leaky_relu": 2, "tanh": 3, "gelu": 4, "sigmoid": 5}


# ---------------------------------------------------------------------------
# encoders: fp32 draws -> operand words (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array -> packed words of `dtype` (uint16 for 16-bit, uint32 for f32
    and int32, uint8 for int8; integer types take integer values)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("synthetic inputs must be finite")
    if dtype == "f32":
        return a.view(np.uint32).copy()
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16).copy()
    if dtype == "bf16":
        return _f32_to_bf16_bits(a)
    if dtype in ("i8", "i32"):
        lo, hi, t = (-128, 127, np.int8) if dtype == "i8" else (-2 ** 31, 2 ** 31 - 1, np.int32)
        if not np.all((a == np.round(a)) & (a >= lo) & (a <= hi)):
            raise ValueError(f"{dtype} inputs must be integers in [{lo}, {hi}]")
        return a.astype(np.float64).astype(t).view(np.uint8 if dtype == "i8" else np.uint32).copy()
    raise ValueError(f"unknown dtype {dtype!r}; supported: f32, f16, bf16, i8, i32")


# ---------------------------------------------------------------------------
# distributions
# ---------------------------------------------------------------------------

def draw(rng: np.random.Generator, shape, dist: Tuple) -> np.ndarray:
    """dist = ("uniform", lo, hi) | ("normal", std) | ("ints", lo, hi)."""
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape).astype(np.float32)
    if kind == "normal":
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(dist[1]))
    if kind == "ints":
        return rng.integers(dist[1], dist[2] + 1, size=shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GemmCase:
    name: str
    M: int
    N: int
    K: int
    in_dtype: str
    bias_dtype: Optional[str]       # None = no bias
    out_dtype: str
    act: str
    alpha: float = 0.0
    dist_a: Tuple = ("uniform", -1.0, 1.0)
    dist_b: Tuple = ("uniform", -1.0, 1.0)
    dist_bias: Tuple = ("uniform", -1.0, 1.0)
    dist_r: Optional[Tuple] = None  # residual R [M, N] in out_dtype; None = no residual

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def alg_bytes(self) -> int:
        s = DTYPE_SIZES
        b = (self.M * self.K + self.K * self.N) * s[self.in_dtype] + self.M * self.N * s[self.out_dtype]
        if self.bias_dtype:
            b += self.N * s[self.bias_dtype]
        if self.dist_r:
            b += self.M * self.N * s[self.out_dtype]
        return b


@dataclass(frozen=True)
class ConvCase:
    name: str
    N: int
    C: int
    H: int
    W: int
    Co: int
    kh: int
    kw: int
    strides: Tuple[int, int]
    pads: Tuple[int, int, int, int]      # top, bottom, left, right
    dilations: Tuple[int, int]
    in_dtype: str
    bias_dtype: Optional[str]
    out_dtype: str
    act: str
    alpha: float = 0.0
    dist_x: Tuple = ("uniform", -1.0, 1.0)
    dist_w: Tuple = ("uniform", -1.0, 1.0)
    dist_bias: Tuple = ("uniform", -1.0, 1.0)
    dist_r: Optional[Tuple] = None  # residual R [N, Co, Ho, Wo] in out_dtype; None = no residual

    def out_hw(self) -> Tuple[int, int]:
        def od(i, k, s, p0, p1, d):
            span = i + p0 + p1 - d * (k - 1) - 1
            return span // s + 1 if span >= 0 else 0
        return (od(self.H, self.kh, self.strides[0], self.pads[0], self.pads[1], self.dilations[0]),
                od(self.W, self.kw, self.strides[1], self.pads[2], self.pads[3], self.dilations[1]))

    @property
    def flops(self) -> int:
        Ho, Wo = self.out_hw()
        return 2 * self.N * self.Co * Ho * Wo * self.C * self.kh * self.kw

    @property
    def alg_bytes(self) -> int:
        """Inputs read once (only the x elements some tap touches) + output once."""
        s = DTYPE_SIZES
        Ho, Wo = self.out_hw()
        rows = _touched(self.H, Ho, self.kh, self.strides[0], self.pads[0], self.dilations[0])
        cols = _touched(self.W, Wo, self.kw, self.strides[1], self.pads[2], self.dilations[1])
        b = self.N * self.C * rows * cols * s[self.in_dtype]
        b += self.Co * self.C * self.kh * self.kw * s[self.in_dtype]
        b += self.N * self.Co * Ho * Wo * s[self.out_dtype]
        if self.bias_dtype:
            b += self.Co * s[self.bias_dtype]
        if self.dist_r:
            b += self.N * self.Co * Ho * Wo * s[self.out_dtype]
        return b


def _touched(n_in, n_out, k, s, p, d) -> int:
    hit = np.zeros(n_in, dtype=bool)
    for o in range(n_out):
        for r in range(k):
            i = o * s - p + r * d
            if 0 <= i < n_in:
                hit[i] = True
    return int(hit.sum())


U1 = ("uniform", -1.0, 1.0)
U01 = ("uniform", -0.1, 0.1)

# The five named workloads.  Readings where a description leaves a value open
# (the conv bias dtype, the activation of the dilated conv, the meaning of the
# second normal parameter) are listed in the design notes.
CASES: Dict[str, object] = {
    # MatmulLeakyRelu sample spec: A[1024,256] f16, B[256,640] f16,
    # bias[1,640] f32, alpha f32, C[1024,640] f32.
    "gemm_leaky_1024x640x256_f16": GemmCase(
        "gemm_leaky_1024x640x256_f16", 1024, 640, 256, "f16", "f32", "f32",
        "leaky_relu", 0.001, U1, U1, U1),
    # fused matmul+ReLU at 4096^3, bf16 in/out, f32 bias.
    "gemm_relu_4096_bf16": GemmCase(
        "gemm_relu_4096_bf16", 4096, 4096, 4096, "bf16", "f32", "bf16", "relu", 0.0,
        ("normal", 1.0 / 64.0), ("normal", 1.0 / 64.0), U01),
    # conv 3x3 s1 p1 + tanh, fp16.
    "conv3x3_tanh_8x64x56_f16": ConvCase(
        "conv3x3_tanh_8x64x56_f16", 8, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1),
        "f16", "f16", "f16", "tanh", 0.0, U01, U01, U01),
    # 7x7 s2 p3 stem + tanh, fp32 (shallow K = 147).
    "conv7x7s2_tanh_16x3x224_f32": ConvCase(
        "conv7x7s2_tanh_16x3x224_f32", 16, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1),
        "f32", "f32", "f32", "tanh", 0.0, U1, U1, U1),
    # 1x1 s2 + tanh, fp32.
    "conv1x1s2_tanh_16x256x56_f32": ConvCase(
        "conv1x1s2_tanh_16x256x56_f32", 16, 256, 56, 56, 512, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1),
        "f32", "f32", "f32", "tanh", 0.0, U1, U1, U1),
    # large LeakyReLU GEMM, bf16.
    "gemm_leaky_32768x4096x1024_bf16": GemmCase(
        "gemm_leaky_32768x4096x1024_bf16", 32768, 4096, 1024, "bf16", "f32", "bf16",
        "leaky_relu", 0.01, U1, U1, U1),
    # conv 3x3 dilation 2 pad 2 + tanh, bf16.
    "conv3x3d2_tanh_32x128x28_bf16": ConvCase(
        "conv3x3d2_tanh_32x128x28_bf16", 32, 128, 28, 28, 128, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2),
        "bf16", "bf16", "bf16", "tanh", 0.0, U01, U01, U01),
    # The other element-wise activations of the matmul + activation class
    # (ops-nn article, 融合算子分类): the 4096^3 GEMM with GELU, and the
    # ConvSigmoid twin of the fp16 3x3 conv (Fused ConvTanh article, 核心问题).
    "gemm_gelu_4096_bf16": GemmCase(
        "gemm_gelu_4096_bf16", 4096, 4096, 4096, "bf16", "f32", "bf16", "gelu", 0.0,
        ("normal", 1.0 / 64.0), ("normal", 1.0 / 64.0), U01),
    "conv3x3_sigmoid_8x64x56_f16": ConvCase(
        "conv3x3_sigmoid_8x64x56_f16", 8, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1),
        "f16", "f16", "f16", "sigmoid", 0.0, U01, U01, U01),
    # The residual ("matmul + add + bias", ops-nn article, math class): the
    # 4096^3 GEMM with a bf16 residual, and the fp16 3x3 conv with an identity
    # skip (R of y's shape), the shape of a residual block.
    "gemm_relu_residual_4096_bf16": GemmCase(
        "gemm_relu_residual_4096_bf16", 4096, 4096, 4096, "bf16", "f32", "bf16", "relu", 0.0,
        ("normal", 1.0 / 64.0), ("normal", 1.0 / 64.0), U01, U01),
    # int8 operands with an int32 bias (MatmulLeakyRelu page, 补充说明), exact
    # int32 output with ReLU, at the 4096^3 shape.
    "gemm_int8_relu_4096_i32": GemmCase(
        "gemm_int8_relu_4096_i32", 4096, 4096, 4096, "i8", "i32", "i32", "relu", 0.0,
        ("ints", -128, 127), ("ints", -128, 127), ("ints", -100000, 100000)),
    "conv3x3_residual_tanh_8x64x56_f16": ConvCase(
        "conv3x3_residual_tanh_8x64x56_f16", 8, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1, 1, 1),
        (1, 1), "f16", "f16", "f16", "tanh", 0.0, U01, U01, U01, U01),
}

# 16-bit convs with filters larger than 3x3 (the pages' conv suites include
# 7x7 filters in fp16 and bf16): the fp16 3x3 conv's shape with a 5x5 and a
# 7x7 filter.  Not named workloads: parity-tested at full size and timed
# beside them.
FILTER_CASES: Dict[str, object] = {
    "conv5x5_tanh_8x64x56_f16": ConvCase(
        "conv5x5_tanh_8x64x56_f16", 8, 64, 56, 56, 64, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1),
        "f16", "f16", "f16", "tanh", 0.0, U01, U01, U01),
    "conv7x7_tanh_8x64x56_bf16": ConvCase(
        "conv7x7_tanh_8x64x56_bf16", 8, 64, 56, 56, 64, 7, 7, (1, 1), (3, 3, 3, 3), (1, 1),
        "bf16", "bf16", "bf16", "tanh", 0.0, U01, U01, U01),
}

# Which case each named workload group covers (group 1 is the small spec case,
# group 2 the 4096^3 headline, groups 4 and 5 hold two cases each).
GROUPS = {
    1: ["gemm_leaky_1024x640x256_f16"],
    2: ["gemm_relu_4096_bf16"],
    3: ["conv3x3_tanh_8x64x56_f16"],
    4: ["conv7x7s2_tanh_16x3x224_f32", "conv1x1s2_tanh_16x256x56_f32"],
    5: ["gemm_leaky_32768x4096x1024_bf16", "conv3x3d2_tanh_32x128x28_bf16"],
    6: ["gemm_gelu_4096_bf16", "conv3x3_sigmoid_8x64x56_f16"],      # epilogue extensions
    7: ["gemm_relu_residual_4096_bf16", "conv3x3_residual_tanh_8x64x56_f16"],
    8: ["gemm_int8_relu_4096_i32"],
}


def gen_gemm(case: GemmCase, seed: int):
    """Returns dict(A, B, bias[, R]) of encoded words; bias is None without
    bias; R (drawn last) only for residual cases."""
    rng = np.random.default_rng(seed)
    a = draw(rng, (case.M, case.K), case.dist_a)
    b = draw(rng, (case.K, case.N), case.dist_b)
    out = {"A": encode(a, case.in_dtype), "B": encode(b, case.in_dtype), "bias": None}
    if case.bias_dtype:
        bias = draw(rng, (case.N,), case.dist_bias)
        out["bias"] = encode(bias, case.bias_dtype)
    if case.dist_r:
        out["R"] = encode(draw(rng, (case.M, case.N), case.dist_r), case.out_dtype)
    return out


def gen_conv(case: ConvCase, seed: int):
    """Returns dict(x, w, bias[, R]) of encoded words, as gen_gemm."""
    rng = np.random.default_rng(seed)
    x = draw(rng, (case.N, case.C, case.H, case.W), case.dist_x)
    w = draw(rng, (case.Co, case.C, case.kh, case.kw), case.dist_w)
    out = {"x": encode(x, case.in_dtype), "w": encode(w, case.in_dtype), "bias": None}
    if case.bias_dtype:
        bias = draw(rng, (case.Co,), case.dist_bias)
        out["bias"] = encode(bias, case.bias_dtype)
    if case.dist_r:
        Ho, Wo = case.out_hw()
        out["R"] = encode(draw(rng, (case.N, case.Co, Ho, Wo), case.dist_r), case.out_dtype)
    return out


def sample_indices(total: int, n: int, seed: int) -> np.ndarray:
    """n distinct flat indices in [0, total), sorted (for sampled parity checks)."""
    rng = np.random.default_rng(seed + 7919)
    n = min(n, total)
    return np.sort(rng.choice(total, size=n, replace=False)).astype(np.int64)
