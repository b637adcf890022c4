"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, never against the oracle itself.

Kinds of pin used here:
  * hand-derived worked examples (tests/golden/*.json, each citing its page);
  * closed forms (identity B, tanh at ln k, bias broadcast over rows);
  * exact brute force on tiny integer inputs (Python integers / Fractions);
  * library routines on special cases (numpy float16 / float32 views,
    numpy.matmul and torch conv2d in float64);
  * invariants stated on the pages (LeakyReLU, ReLU, tanh symmetry, the bias
    fold of the Fused ConvTanh article).

The library under test can be redirected with BIASACT_ORACLE_LIB (used by the
mutation test, which plants mistakes in a copy of oracle.c).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from oracle import Oracle
from oracle.compare import ETA_ACT, compare, gamma, propagated_bound, slope_bound, tolerance, ulp
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_LIB = os.environ.get("BIASACT_ORACLE_LIB")
O = Oracle(orc.load(_LIB) if _LIB else None)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# exact decoders (IEEE-754 binary16 / binary32, bfloat16)
# --------------------------------------------------------------------------

def test_f16_decode_known_patterns():
    known = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x03FF: 1023 * 2.0 ** -24, 0x3555: 0.333251953125,
             0x0000: 0.0, 0x7C00: math.inf, 0xFC00: -math.inf}
    for bits, val in known.items():
        assert O.lib.orc_f16_to_f64(bits) == val
    assert math.copysign(1.0, O.lib.orc_f16_to_f64(0x8000)) == -1.0
    assert math.isnan(O.lib.orc_f16_to_f64(0x7E00))


def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    got = O.decode(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_decode_all_patterns():
    known = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    for b, v in known.items():
        assert O.lib.orc_bf16_to_f64(b) == v
    bits = np.arange(65536, dtype=np.uint16)
    got = O.decode(bits, "bf16")
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f32_decode_random_patterns():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:6] = [0x3F800000, 0x00000001, 0x007FFFFF, 0x80000000, 0x7F800000, 0x7F7FFFFF]
    got = O.decode(bits, "f32")
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[1] == 2.0 ** -149


# --------------------------------------------------------------------------
# activation
# --------------------------------------------------------------------------

_Z = np.array([0.0, -0.0, 1e-300, -1e-300, 0.5, -0.5, 3.0, -3.0, 1e30, -1e30, 7.25, -1e-8])


def test_leaky_relu_invariant():
    # non-negative values pass unchanged; negative values are multiplied by alpha
    for alpha in (0.001, 0.01, 0.25, 1.0, 0.0):
        y = O.act(_Z, "leaky_relu", alpha)
        pos = _Z >= 0
        assert np.array_equal(y[pos], _Z[pos])
        assert np.array_equal(y[~pos], alpha * _Z[~pos])
    # alpha = 1 is the identity; alpha = 0 agrees with ReLU
    assert np.array_equal(O.act(_Z, "leaky_relu", 1.0), _Z)
    assert np.array_equal(O.act(_Z, "leaky_relu", 0.0), O.act(_Z, "relu"))


def test_relu_and_none():
    y = O.act(_Z, "relu")
    assert np.array_equal(y, np.maximum(_Z, 0.0))
    assert not np.signbit(y).any()          # ReLU gives +0 for every non-positive input
    assert np.array_equal(O.act(_Z, "none"), _Z)


def test_tanh_closed_forms_golden():
    g = _golden("tanh_closed_forms.json")
    z = np.array([math.log(p["ln_of"]) for p in g["points"]])
    y = O.act(z, "tanh")
    for got, p in zip(y, g["points"]):
        assert abs(got - p["expect"]) <= 4e-16, (p, got)


def test_tanh_matches_page_formula_and_symmetry():
    z = np.concatenate([np.linspace(-20, 20, 4001), [1e-12, -1e-12, 1e-5, 0.0]])
    y = O.act(z, "tanh")
    f = (np.exp(z) - np.exp(-z)) / (np.exp(z) + np.exp(-z))
    assert np.all(np.abs(y - f) <= 1e-15 + 1e-15 * np.abs(f))
    assert np.array_equal(O.act(-z, "tanh"), -y)
    big = O.act(np.array([30.0, 400.0, 1e6, -1e6]), "tanh")
    assert np.array_equal(big, [1.0, 1.0, 1.0, -1.0])       # finite where the quotient overflows
    assert np.all(np.abs(O.act(np.linspace(-50, 50, 999), "tanh")) <= 1.0)


def test_sigmoid_closed_forms_golden():
    g = _golden("sigmoid_closed_forms.json")
    z = np.array([math.log(p["ln_of"]) for p in g["points"]])
    y = O.act(z, "sigmoid")
    for got, p in zip(y, g["points"]):
        assert abs(got - p["expect"]) <= 4e-16, (p, got)


def test_sigmoid_symmetry_tanh_relation_and_range():
    z = np.concatenate([np.linspace(-40, 40, 8001), [1e-12, -1e-12, 0.0]])
    y = O.act(z, "sigmoid")
    # Sigmoid(z) + Sigmoid(-z) = 1
    assert np.all(np.abs(y + O.act(-z, "sigmoid") - 1.0) <= 4.5e-16)     # two ulps of 1
    # Sigmoid(z) = (1 + tanh(z/2)) / 2, against the (separately pinned) tanh
    assert np.all(np.abs(y - 0.5 * (1.0 + O.act(z / 2.0, "tanh"))) <= 4e-16)
    # finite and in [0, 1] far out, where e^-z alone would overflow
    far = O.act(np.array([800.0, -800.0, 1e6, -1e6]), "sigmoid")
    assert np.array_equal(far, [1.0, 0.0, 1.0, 0.0])
    assert np.all((y >= 0.0) & (y <= 1.0))


def _phi_by_quadrature(z):
    """Standard normal CDF by composite Simpson integration of the density
    from 0 to z (2^14 panels; error far below 1e-14 for |z| <= 6): an
    evaluation that shares nothing with an erf routine."""
    n = 1 << 14
    t = np.linspace(0.0, z, n + 1)
    f = np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
    h = z / n
    return 0.5 + h / 3.0 * (f[0] + f[-1] + 4.0 * f[1:-1:2].sum() + 2.0 * f[2:-1:2].sum())


def test_gelu_against_quadrature_of_the_normal_density():
    # GELU(z) = z * Phi(z), the exact (erf) form
    zs = np.array([-6.0, -3.0, -2.0, -1.0, -0.5, -0.1, 0.1, 0.5, 1.0, 1.5, 2.0, 3.0, 6.0])
    y = O.act(zs, "gelu")
    for z, got in zip(zs, y):
        want = z * _phi_by_quadrature(z)
        assert abs(got - want) <= 1e-14 * max(1.0, abs(want)), (z, got, want)


def test_gelu_identities_and_limits():
    z = np.linspace(-8, 8, 1601)
    y = O.act(z, "gelu")
    # Phi(z) + Phi(-z) = 1  =>  GELU(z) - GELU(-z) = z
    assert np.all(np.abs(y - O.act(-z, "gelu") - z) <= 1e-15 * (1 + np.abs(z)))
    # GELU(z) = z/2 + z^2 / sqrt(2 pi) + O(z^4) near 0
    h = np.array([1e-3, -1e-3, 1e-4])
    c2 = (O.act(h, "gelu") - h / 2) / h ** 2
    assert np.all(np.abs(c2 - 1.0 / math.sqrt(2.0 * math.pi)) <= 2e-6)
    assert O.act(np.array([0.0]), "gelu")[0] == 0.0
    # far tails: the identity for large positive z, zero for large negative z
    far = O.act(np.array([40.0, -40.0]), "gelu")
    assert far[0] == 40.0 and abs(far[1]) < 1e-300
    # the minimum of z * Phi(z) lies between -1 and 0 and is about -0.17
    assert -0.18 < y.min() < -0.16
    # relative accuracy in the negative tail, against the quadrature:
    # Phi(z) = 1/2 - int_z^0 density, and Mills' ratio bounds
    # phi(z)/|z| * (1 - 1/z^2) < Phi(z) < phi(z)/|z| for z < 0
    for z in (-8.0, -12.0, -20.0):
        got = O.act(np.array([z]), "gelu")[0] / z
        dens = math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
        assert dens / abs(z) * (1 - 1 / z ** 2) < got < dens / abs(z), (z, got)


def test_int8_and_int32_decoders():
    # all 256 int8 patterns and random int32 patterns against numpy's views
    w8 = np.arange(256, dtype=np.uint8)
    assert np.array_equal(O.decode(w8, "i8"), w8.view(np.int8).astype(np.float64))
    w32 = np.random.default_rng(5).integers(0, 2 ** 32, 100000, dtype=np.uint64).astype(np.uint32)
    w32 = np.concatenate([w32, np.array([0, 1, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFF], np.uint32)])
    assert np.array_equal(O.decode(w32, "i32"), w32.view(np.int32).astype(np.float64))
    assert O.decode(np.array([0x80], np.uint8), "i8")[0] == -128.0
    assert O.decode(np.array([0x80000000], np.uint32), "i32")[0] == -2.0 ** 31


def test_int8_gemm_exact_with_int32_bias():
    # int8 A, B and an int32 bias ([MLR] 补充说明): the sums are integers far
    # below 2^53, so the double result is the exact integer (Python ints)
    rng = np.random.default_rng(8)
    M, N, K = 9, 11, 300
    A = rng.integers(-128, 128, (M, K))
    B = rng.integers(-128, 128, (K, N))
    bias = rng.integers(-2 ** 30, 2 ** 30, N)
    got = O.gemm(O.decode(workloads.encode(A.astype(np.float32), "i8").reshape(M, K), "i8"),
                 O.decode(workloads.encode(B.astype(np.float32), "i8").reshape(K, N), "i8"),
                 O.decode(bias.astype(np.int32).view(np.uint32), "i32"), "none")
    want = [[sum(int(A[i, k]) * int(B[k, j]) for k in range(K)) + int(bias[j]) for j in range(N)]
            for i in range(M)]
    assert got.tolist() == [[float(v) for v in r] for r in want]
    # the extreme product -128 * -128 summed 131071 times still fits int32
    assert 131071 * 16384 < 2 ** 31


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def test_gemm_golden_example():
    g = _golden("gemm_leaky_2x3x2.json")
    for act, want in g["expect"].items():
        got = O.gemm(g["A"], g["B"], g["bias"], act, g["alpha"])
        assert np.array_equal(got, np.array(want, dtype=np.float64)), act


def test_gemm_identity_B():
    rng = np.random.default_rng(0)
    M, K = 5, 7
    A = rng.uniform(-3, 3, (M, K))
    bias = rng.uniform(-1, 1, K)
    C = O.gemm(A, np.eye(K), bias, "none")
    assert np.array_equal(C, A + bias)            # A.I + bias, every row gets the same bias row
    C0 = O.gemm(A, np.eye(K), None, "none")
    assert np.array_equal(C0, A)


def test_gemm_bias_is_a_row_broadcast():
    M, N, K = 3, 5, 4
    bias = np.arange(N) - 2.0
    C = O.gemm(np.zeros((M, K)), np.ones((K, N)), bias, "none")
    assert np.array_equal(C, np.tile(bias, (M, 1)))


def _exact_gemm(A, B, bias, act, alpha):
    M, K = len(A), len(A[0])
    N = len(B[0])
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            z = sum(Fraction(A[i][k]) * Fraction(B[k][j]) for k in range(K)) + Fraction(bias[j])
            if act == "relu":
                z = z if z > 0 else Fraction(0)
            elif act == "leaky_relu":
                z = z if z >= 0 else Fraction(alpha) * z
            row.append(z)
        out.append(row)
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (7, 5, 3), (3, 7, 2), (5, 2, 7)])
def test_gemm_tiny_integer_bruteforce(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.integers(-2, 3, (M, K)).tolist()
    B = rng.integers(-2, 3, (K, N)).tolist()
    bias = rng.integers(-2, 3, N).tolist()
    for act in ("none", "relu", "leaky_relu"):
        want = _exact_gemm(A, B, bias, act, Fraction(1, 4))
        got = O.gemm(A, B, bias, act, 0.25)
        assert [[Fraction(v) for v in r] for r in got.tolist()] == want, act


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (7, 5, 3), (4, 6, 2)])
def test_gemm_residual_tiny_integer_bruteforce(M, N, K):
    # act(A.B + bias + R), the residual joining the sum before the activation
    # ("matmul + add + bias" of the ops-nn math class), exactly
    rng = np.random.default_rng(M * 37 + N * 11 + K)
    A = rng.integers(-2, 3, (M, K)).tolist()
    B = rng.integers(-2, 3, (K, N)).tolist()
    bias = rng.integers(-2, 3, N).tolist()
    R = rng.integers(-3, 4, (M, N)).tolist()
    for act in ("none", "relu", "leaky_relu"):
        base = _exact_gemm(A, B, bias, "none", None)
        want = []
        for i in range(M):
            row = []
            for j in range(N):
                z = base[i][j] + Fraction(R[i][j])
                if act == "relu":
                    z = z if z > 0 else Fraction(0)
                elif act == "leaky_relu":
                    z = z if z >= 0 else Fraction(1, 4) * z
                row.append(z)
            want.append(row)
        got = O.gemm_residual(A, B, bias, np.array(R, dtype=np.float64), act, 0.25)
        assert [[Fraction(v) for v in r] for r in got.tolist()] == want, act


def test_residual_special_cases():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((6, 9))
    B = rng.standard_normal((9, 5))
    bias = rng.standard_normal(5)
    # R = 0 gives the epilogue without a residual, bit for bit
    for act in ("none", "relu", "tanh", "gelu", "sigmoid"):
        assert np.array_equal(O.gemm_residual(A, B, bias, np.zeros((6, 5)), act),
                              O.gemm(A, B, bias, act))
    # an empty sum (K = 0) leaves act(bias + R): tanh(ln 2) = 3/5 at z = ln 2
    R = np.full((3, 5), math.log(2.0)) - np.zeros(5)
    got = O.gemm_residual(np.zeros((3, 0)), np.zeros((0, 5)), np.zeros(5), R, "tanh")
    assert np.all(np.abs(got - 0.6) <= 4e-16)
    # R = -(A.B + bias) cancels the sum: ReLU of it is +0, Sigmoid 1/2
    z = O.gemm(A, B, bias, "none")
    assert np.array_equal(O.gemm_residual(A, B, bias, -z, "relu"), np.zeros((6, 5)))
    assert np.array_equal(O.gemm_residual(A, B, bias, -z, "sigmoid"), np.full((6, 5), 0.5))
    # the residual is indexed like C (row-major [M, N]), not transposed
    Rr = np.arange(30, dtype=np.float64).reshape(6, 5)
    assert np.array_equal(O.gemm_residual(A, B, bias, Rr, "none") - z, Rr)


def test_gemm_matches_numpy_matmul():
    rng = np.random.default_rng(1)
    M, N, K = 37, 53, 61                     # all different: a transposed operand cannot fit
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    bias = rng.standard_normal(N)
    ref = A @ B + bias
    got = O.gemm(A, B, bias, "none")
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)
    got_t = O.gemm(A, B, bias, "tanh")
    assert np.allclose(got_t, np.tanh(ref), rtol=1e-13, atol=1e-14)


def test_gemm_elems_equal_full():
    rng = np.random.default_rng(2)
    M, N, K = 31, 29, 47
    A, B = rng.standard_normal((M, K)), rng.standard_normal((K, N))
    bias = rng.standard_normal(N)
    full = O.gemm(A, B, bias, "leaky_relu", 0.01)
    ii = rng.integers(0, M, 200)
    jj = rng.integers(0, N, 200)
    got = O.gemm_elems(A, B, bias, ii, jj, "leaky_relu", 0.01)
    assert np.array_equal(got, full[ii, jj])


def test_gemm_bias_fold_equals_direct_add():
    rng = np.random.default_rng(4)
    M, N, K = 19, 23, 41
    A, B = rng.uniform(-1, 1, (M, K)), rng.uniform(-1, 1, (K, N))
    bias = rng.uniform(-1, 1, N)
    for act in ("none", "relu", "leaky_relu", "tanh"):
        d = O.gemm(A, B, bias, act, 0.01)
        f = O.gemm_bias_fold(A, B, bias, act, 0.01)
        assert np.all(np.abs(d - f) <= 1e-12 * (1 + np.abs(d))), act


def test_gemm_empty_and_degenerate():
    assert O.gemm(np.zeros((0, 3)), np.zeros((3, 4)), None, "none").shape == (0, 4)
    # K = 0: the sum is empty, C = act(bias)
    C = O.gemm(np.zeros((2, 0)), np.zeros((0, 3)), [1.0, -1.0, 0.5], "relu")
    assert np.array_equal(C, [[1.0, 0.0, 0.5]] * 2)


# --------------------------------------------------------------------------
# conv2d
# --------------------------------------------------------------------------

def test_conv_golden_cases():
    g = _golden("conv_small_cases.json")
    for c in g["cases"]:
        got = O.conv2d(c["x"], c["w"], c["bias"], c["strides"], c["pads"], c["dilations"], c["act"])
        assert np.array_equal(got, np.array(c["expect"], dtype=np.float64)), c["name"]
        got2 = O.conv2d_im2col(c["x"], c["w"], c["bias"], c["strides"], c["pads"],
                               c["dilations"], c["act"])
        assert np.array_equal(got2, np.array(c["expect"], dtype=np.float64)), c["name"]


def test_conv_out_dim_formula():
    # with dilation 1 and symmetric padding: (H + 2p - k)//s + 1
    for H in (1, 5, 28, 56, 224):
        for k in (1, 3, 7):
            for s in (1, 2, 3):
                for p in (0, 1, 3):
                    want = (H + 2 * p - k) // s + 1 if H + 2 * p >= k else 0
                    assert O.conv_out_dim(H, k, s, p, p, 1) == max(want, 0)
    assert O.conv_out_dim(28, 3, 1, 2, 2, 2) == 28
    assert O.conv_out_dim(224, 7, 2, 3, 3, 1) == 112
    assert O.conv_out_dim(56, 1, 2, 0, 0, 1) == 28


_CONV_SHAPES = [
    # N, C, H, W, Co, kh, kw, strides, pads(t,b,l,r), dilations
    (1, 1, 5, 6, 1, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (2, 3, 9, 7, 4, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2)),
    (1, 2, 11, 11, 3, 5, 5, (3, 2), (2, 2, 0, 3), (1, 1)),
    (3, 4, 8, 8, 5, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)),
    (2, 3, 12, 10, 2, 3, 3, (1, 1), (2, 2, 2, 2), (2, 3)),
    (1, 3, 15, 15, 4, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)),
]


@pytest.mark.parametrize("shape", _CONV_SHAPES)
def test_conv_matches_torch_conv2d_float64(shape):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    rng = np.random.default_rng(sum(shape[:7]))
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, kh, kw))
    b = rng.standard_normal(Co)
    xt = F.pad(torch.from_numpy(x), (pd[2], pd[3], pd[0], pd[1]))   # (left, right, top, bottom)
    ref = F.conv2d(xt, torch.from_numpy(w), torch.from_numpy(b), stride=st, dilation=dl).numpy()
    got = O.conv2d(x, w, b, st, pd, dl, "none")
    assert got.shape == ref.shape
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", _CONV_SHAPES[1:4])
def test_conv_residual_matches_torch_float64(shape):
    # y = act(conv2d(x, w) + bias + R) with R [N, Co, Ho, Wo], against torch in float64
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    rng = np.random.default_rng(sum(shape[:7]) + 5)
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, kh, kw))
    b = rng.standard_normal(Co)
    xt = F.pad(torch.from_numpy(x), (pd[2], pd[3], pd[0], pd[1]))
    conv = F.conv2d(xt, torch.from_numpy(w), torch.from_numpy(b), stride=st, dilation=dl)
    R = rng.standard_normal(tuple(conv.shape))
    ref = torch.tanh(conv + torch.from_numpy(R)).numpy()
    got = O.conv2d_residual(x, w, b, R, st, pd, dl, "tanh")
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    idx = np.arange(0, got.size, 3)
    assert np.array_equal(O.conv2d_residual_elems(x, w, b, R.ravel()[idx], st, pd, dl, idx, "tanh"),
                          got.ravel()[idx])


@pytest.mark.parametrize("shape", _CONV_SHAPES)
def test_conv_direct_equals_im2col_and_fold(shape):
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    rng = np.random.default_rng(7 + sum(shape[:7]))
    x = rng.uniform(-1, 1, (N, C, H, W))
    w = rng.uniform(-1, 1, (Co, C, kh, kw))
    b = rng.uniform(-1, 1, Co)
    for act in ("none", "tanh", "leaky_relu"):
        d = O.conv2d(x, w, b, st, pd, dl, act, 0.01)
        i = O.conv2d_im2col(x, w, b, st, pd, dl, act, 0.01, fold_bias=False)
        f = O.conv2d_im2col(x, w, b, st, pd, dl, act, 0.01, fold_bias=True)
        assert np.all(np.abs(d - i) <= 1e-12 * (1 + np.abs(d)))
        assert np.all(np.abs(d - f) <= 1e-12 * (1 + np.abs(d)))


def test_conv_1x1_identity_weights():
    rng = np.random.default_rng(5)
    N, C, H, W = 2, 4, 3, 5
    x = rng.uniform(-1, 1, (N, C, H, W))
    b = rng.uniform(-1, 1, C)
    w = np.eye(C).reshape(C, C, 1, 1)
    y = O.conv2d(x, w, b, (1, 1), (0, 0, 0, 0), (1, 1), "none")
    assert np.array_equal(y, x + b.reshape(1, C, 1, 1))


def test_conv_1x1_on_1x1_images_is_a_gemm():
    rng = np.random.default_rng(6)
    N, C, Co = 6, 5, 3
    x = rng.standard_normal((N, C, 1, 1))
    w = rng.standard_normal((Co, C, 1, 1))
    b = rng.standard_normal(Co)
    y = O.conv2d(x, w, b, (1, 1), (0, 0, 0, 0), (1, 1), "none")[:, :, 0, 0]
    ref = x[:, :, 0, 0] @ w[:, :, 0, 0].T + b
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_conv_elems_equal_full():
    rng = np.random.default_rng(8)
    N, C, H, W, Co = 2, 3, 10, 9, 4
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((Co, C, 3, 3))
    b = rng.standard_normal(Co)
    args = ((2, 1), (1, 2, 0, 1), (1, 2))
    full = O.conv2d(x, w, b, *args, "tanh")
    idx = rng.choice(full.size, 60, replace=False)
    got = O.conv2d_elems(x, w, b, *args, idx, "tanh")
    assert np.array_equal(got, full.ravel()[idx])


def test_conv_rejects_invalid():
    x = np.zeros((1, 1, 3, 3))
    w = np.zeros((1, 1, 5, 5))
    with pytest.raises(ValueError):
        O.conv2d(x, w, None, (1, 1), (0, 0, 0, 0), (1, 1), "none")   # output would be empty
    with pytest.raises(ValueError):
        O.conv2d(x, np.zeros((1, 1, 1, 1)), None, (0, 1), (0, 0, 0, 0), (1, 1), "none")
    with pytest.raises(ValueError):
        O.conv2d(x, np.zeros((1, 1, 1, 1)), None, (1, 1), (-1, 0, 0, 0), (1, 1), "none")


# --------------------------------------------------------------------------
# acceptance helpers and the input generator
# --------------------------------------------------------------------------

def test_ulp_values():
    assert ulp(1.0, "bf16") == 2.0 ** -7
    assert ulp(1.0, "f16") == 2.0 ** -10
    assert ulp(65504.0, "f16") == 32.0
    assert ulp(1.5, "f16") == 2.0 ** -10
    assert ulp(0.99, "f16") == 2.0 ** -11
    assert ulp(1e-6, "f16") == 2.0 ** -24          # below the smallest fp16 normal
    assert ulp(0.0, "bf16") == 2.0 ** -133


def test_compare_flags_errors():
    ref = np.array([1.0, 2.0, 0.0])
    assert compare(ref, ref, "bf16", "f32")["ok"]
    assert not compare(ref + [0, 0.01, 0], ref, "bf16", "f32")["ok"]
    assert compare(ref + [0, 0.002, 0], ref, "bf16", "f32")["ok"]
    assert not compare(ref + [0, 4e-5, 0], ref, "f32", "f32")["ok"]
    assert not compare(np.array([1.0, np.nan, 0]), ref, "bf16", "f32")["ok"]
    # 16-bit output: one ulp passes, two fail
    assert compare(np.array([1.0 + 2 ** -7]), np.array([1.0]), "bf16", "bf16")["ok"]
    assert not compare(np.array([1.0 + 2 ** -6]), np.array([1.0]), "bf16", "bf16")["ok"]
    # 16-bit output: one ulp, or half an ulp (at |ref| + d) plus d where the
    # allowance d = L*E + ETA*|ref| exceeds half an ulp
    eta = ETA_ACT
    assert tolerance(np.array([1.0]), "bf16", "bf16")[0] == 2.0 ** -7
    assert tolerance(np.array([1.0]), "bf16", "bf16", np.array([2.0 ** -9]))[0] == 2.0 ** -7
    t = tolerance(np.array([1.0]), "bf16", "bf16", np.array([0.5]))[0]
    assert t == 0.5 * 2.0 ** -7 + 0.5 + eta               # ulp at 1.5 is still 2^-7
    t = tolerance(np.array([1.0]), "bf16", "bf16", np.array([1.0]))[0]
    assert t == 0.5 * 2.0 ** -6 + 1.0 + eta               # 2 + eta lies in the next binade
    # fp32 outputs take no accumulation allowance
    assert abs(tolerance(np.array([2.0]), "f32", "f32", np.array([1.0]))[0] - 3e-5) < 1e-18
    assert abs(tolerance(np.array([2.0]), "f32", "f32")[0] - 3e-5) < 1e-18
    assert tolerance(np.array([5.0]), "i8", "i32")[0] == 0.0


def test_slope_bound_closed_forms():
    z0 = np.zeros(1)
    assert slope_bound(z0, 0.0, "tanh")[0] == 1.0                 # tanh'(0) = 1
    assert slope_bound(z0, 0.0, "sigmoid")[0] == 0.25             # s'(0) = 1/4
    assert slope_bound(z0, 0.0, "gelu")[0] == 0.5                 # Phi(0) + 0
    # tanh'(ln 3) = 1 - (4/5)^2; the interval's point nearest 0 decides
    assert abs(slope_bound(np.array([math.log(3.0) + 0.5]), 0.5, "tanh")[0] - 9.0 / 25.0) < 1e-15
    assert abs(slope_bound(np.array([-math.log(3.0)]), 0.0, "sigmoid")[0] - 0.75 * 0.25) < 1e-15
    # GELU' peaks at sqrt(2): Phi(sqrt 2) + sqrt(2) phi(sqrt 2), an interior point of [1, 2]
    r2 = math.sqrt(2.0)
    peak = 0.5 * math.erfc(-1.0) + r2 * math.exp(-1.0) / math.sqrt(2.0 * math.pi)
    assert abs(slope_bound(np.array([1.5]), 0.5, "gelu")[0] - peak) < 1e-14
    assert slope_bound(np.array([1.5]), 0.5, "gelu")[0] > max(slope_bound(np.array([1.0]), 0.0, "gelu")[0],
                                                              slope_bound(np.array([2.0]), 0.0, "gelu")[0])
    # ReLU passes nothing below zero unless the interval reaches it; LeakyReLU alpha
    assert slope_bound(np.array([-1.0, -1.0, 0.5]), np.array([0.5, 1.5, 0.1]), "relu").tolist() == [0, 1, 1]
    assert slope_bound(np.array([-1.0, -0.1]), 0.5, "leaky_relu", 0.01).tolist() == [0.01, 1.0]
    assert slope_bound(np.array([-7.0]), 0.0, "none")[0] == 1.0
    # the propagated bound is gamma_n * S times the slope
    pb = propagated_bound(np.array([-3.0]), np.array([2.0]), 100, "leaky_relu", 0.25)[0]
    assert pb == 0.25 * gamma(100) * 2.0


def test_generator_rounding_and_determinism():
    enc = workloads.encode(np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32), "bf16")
    assert enc.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020]          # ties go to even
    assert workloads.encode(np.array([1.0, 65504.0], np.float32), "f16").tolist() == [0x3C00, 0x7BFF]
    c = workloads.CASES["gemm_leaky_1024x640x256_f16"]
    a1, a2 = workloads.gen_gemm(c, 0), workloads.gen_gemm(c, 0)
    assert np.array_equal(a1["A"], a2["A"]) and np.array_equal(a1["bias"], a2["bias"])
    assert not np.array_equal(a1["A"], workloads.gen_gemm(c, 1)["A"])
    assert a1["A"].shape == (1024, 256) and a1["B"].shape == (256, 640) and a1["bias"].dtype == np.uint32


def test_named_workloads_sizes():
    c = workloads.CASES
    assert c["gemm_relu_4096_bf16"].flops == 2 * 4096 ** 3
    assert c["conv3x3_tanh_8x64x56_f16"].out_hw() == (56, 56)
    assert c["conv7x7s2_tanh_16x3x224_f32"].out_hw() == (112, 112)
    assert c["conv1x1s2_tanh_16x256x56_f32"].out_hw() == (28, 28)
    assert c["conv3x3d2_tanh_32x128x28_bf16"].out_hw() == (28, 28)
    # 1x1 stride 2 touches a quarter of the input
    cb = c["conv1x1s2_tanh_16x256x56_f32"]
    assert cb.alg_bytes == 16 * 256 * 28 * 28 * 4 + 512 * 256 * 4 + 16 * 512 * 28 * 28 * 4 + 512 * 4
