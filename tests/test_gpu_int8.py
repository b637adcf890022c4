"""GPU parity of int8 GEMMs with an int32 bias ("CANN pyasc MatmulLeakyRelu
融合算子实战", section 补充说明: with int8 A and B the bias is int32) against
the fp64 oracle, whose sums of int8 products are exact integers.

An int32 output is compared bit for bit (integer work); floating-point
outputs take the integer sum rounded to fp32, then the activation, and are
held to the fp32-input rule (fp32 output) or one output ulp (16-bit output).
fp16 outputs use bounded activations: these sums exceed the fp16 range.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import check, gemm_reference, run_gemm, values_of, words_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    return m


INTS = ("ints", -128, 127)
BIAS = ("ints", -100000, 100000)


def _case(M, N, K, to, act, dist_a=INTS, dist_b=INTS, bias=BIAS):
    return wl.GemmCase(f"i8_{M}x{N}x{K}", M, N, K, "i8", "i32" if bias else None, to, act, 0.0625,
                       dist_a, dist_b, bias or BIAS)


SHAPES = [(1, 1, 1), (3, 5, 7), (64, 64, 128), (127, 129, 65), (200, 136, 72), (300, 520, 200),
          (33, 260, 1000), (520, 8, 24), (1024, 640, 256), (256, 512, 2048)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("to,acts", [("i32", ("none", "relu")), ("f32", ("leaky_relu", "tanh")),
                                     ("bf16", ("gelu", "relu")), ("f16", ("sigmoid", "tanh"))])
def test_int8_gemm_vs_oracle(ba, shape, to, acts):
    M, N, K = shape
    for j, act in enumerate(acts):
        case = _case(M, N, K, to, act)
        inp = wl.gen_gemm(case, seed=90 + j)
        y = run_gemm(case, inp)
        ref, floor = gemm_reference(case, inp)
        if to == "i32":
            assert np.array_equal(words_of(y, "i32").view(np.int32).astype(np.float64), ref), act
        else:
            rep = check(values_of(y, to), ref, floor, case)
            assert rep["ok"], (act, rep)


@pytest.mark.parametrize("tile", range(8))
def test_int8_every_tile_config(ba, tile):
    # id 6 is the int8 ping-pong kernel only where K and N are multiples of
    # 16 (none of these shapes): here it, and the conv-only id 7, fall back
    # to generic tiles
    ba.force_tile_config(tile)
    try:
        for (M, N, K), to in (((300, 520, 200), "i32"), ((513, 264, 1032), "i32"),
                              ((40, 1000, 72), "f32"), ((130, 70, 17), "i32")):
            case = _case(M, N, K, to, "relu")
            inp = wl.gen_gemm(case, seed=7)
            y = run_gemm(case, inp)
            ref, floor = gemm_reference(case, inp)
            if to == "i32":
                assert np.array_equal(words_of(y, "i32").view(np.int32).astype(np.float64), ref)
            else:
                assert check(values_of(y, to), ref, floor, case)["ok"]
    finally:
        ba.force_tile_config(-1)


def test_int8_extremes_are_exact(ba):
    # every product at its largest magnitude (-128 * -128 = 16384), the
    # longest reduction the planner admits for two rows, and a bias near the
    # int32 limit: the sums are exact
    K = 131071
    A = np.full((2, K), -128, np.int8)
    B = np.full((K, 3), -128, np.int8)
    B[:, 1] = 127                                 # -128 * 127 = -16256 per term
    bias = np.array([-(2 ** 31) + 2 ** 31 - K * 16384, 0, 5], np.int32)
    inp = {"A": A.view(np.uint8), "B": B.view(np.uint8), "bias": bias.view(np.uint32)}
    case = _case(2, 3, K, "i32", "none")
    y = words_of(run_gemm(case, inp), "i32").view(np.int32).reshape(2, 3)
    want = np.array([[K * 16384 + int(bias[0]), -K * 16256, K * 16384 + 5]] * 2, dtype=np.int64)
    assert np.array_equal(y.astype(np.int64), want)
    assert y.max() < 2 ** 31


def test_int8_no_bias_and_relu_invariant(ba):
    case = _case(190, 264, 333, "i32", "none", bias=None)
    inp = wl.gen_gemm(case, seed=3)
    z = words_of(run_gemm(case, inp), "i32").view(np.int32)
    ref, _ = gemm_reference(case, inp)
    assert np.array_equal(z.astype(np.float64), ref)
    rcase = _case(190, 264, 333, "i32", "relu", bias=None)
    r = words_of(run_gemm(rcase, inp), "i32").view(np.int32)
    assert np.array_equal(r, np.maximum(z, 0))


PP_SHAPES = [(300, 528, 208), (257, 272, 1040), (1, 16, 16), (520, 784, 64), (256, 256, 4096)]


@pytest.mark.parametrize("shape", PP_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("to,acts", [("i32", ("none", "relu")), ("f32", ("leaky_relu", "tanh")),
                                     ("bf16", ("gelu", "relu")), ("f16", ("sigmoid", "tanh"))])
def test_int8_ping_pong_vs_oracle(ba, shape, to, acts):
    # the 256x256 ping-pong kernel with int8 operands (transposing byte reads
    # of B, v_mfma_i32_32x32x32_i8): ragged M and N, K tails inside a 64-deep
    # k-tile, every output type, with and without a bias
    M, N, K = shape
    ba.force_tile_config(6)
    try:
        for j, act in enumerate(acts):
            case = _case(M, N, K, to, act, bias=BIAS if j == 0 else None)
            inp = wl.gen_gemm(case, seed=120 + j)
            y = run_gemm(case, inp)
            assert "ping-pong int8" in ba.last_tile_config(), ba.last_tile_config()
            ref, floor = gemm_reference(case, inp)
            if to == "i32":
                assert np.array_equal(words_of(y, "i32").view(np.int32).astype(np.float64), ref), act
            else:
                rep = check(values_of(y, to), ref, floor, case)
                assert rep["ok"], (act, rep)
    finally:
        ba.force_tile_config(-1)


def test_int8_ping_pong_misaligned_bias(ba):
    # an int32 bias one element into its buffer is read element by element,
    # an aligned one as runs of four columns: the same exact sums
    from gpu_helpers import to_dev
    M, N, K = 300, 528, 208
    case = _case(M, N, K, "i32", "relu")
    inp = wl.gen_gemm(case, seed=131)
    ref, _ = gemm_reference(case, inp)
    A, _ = to_dev(inp["A"].reshape(M, K), "i8")
    B, _ = to_dev(inp["B"].reshape(K, N), "i8")
    bias0, _ = to_dev(inp["bias"], "i32")
    outs = []
    ba.force_tile_config(6)
    try:
        for off in (0, 1):
            bias = bias0
            if off:
                buf = torch.empty(N + off, dtype=torch.int32, device="cuda")
                bias = buf[off:]
                bias.copy_(bias0)
            C = torch.empty((M, N), dtype=torch.int32, device="cuda")
            ba.gemm_bias_act(A, B, bias, C, "relu", 0.0)
            torch.cuda.synchronize()
            assert "ping-pong int8" in ba.last_tile_config(), ba.last_tile_config()
            outs.append(words_of(C, "i32"))
    finally:
        ba.force_tile_config(-1)
    for w in outs:
        assert np.array_equal(w.view(np.int32).astype(np.float64), ref)
