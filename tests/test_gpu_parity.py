"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on
the same seeded input bits, element by element.

Acceptance (oracle/compare.py): fp32 output with fp16/bf16 inputs within
1e-3*(1+|ref|); fp32 inputs within 1e-5*(1+|ref|); fp16/bf16 output within one
output ulp, or half an ulp plus the fp32 accumulation-error bound carried
through the activation's slope where that bound is the larger.  Where the
result is exact in fp32 (small-integer operands, identity B) the test demands
bit equality; fused vs two-kernel and run-to-run must be bitwise equal.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import (check, conv_reference, empty_out, gemm_reference, guard_intact, merge, run_conv,
                         run_gemm, to_dev, values_of, words_of)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    return m


# fp32 operands with a reduction longer than 512 are drawn from U(-0.1, 0.1):
# their fp32 accumulation error then stays well inside 1e-5 * (1 + |ref|)
# (the rule takes no allowance for it), where U(-1, 1) operands would put
# the error of a correct fp32 sum at the tolerance's own scale.
SMALL_F32 = ("uniform", -0.1, 0.1)


def _gcase(M, N, K, ti, to, tb, act, alpha=0.01, dist=None):
    if dist is None:
        dist = SMALL_F32 if ti == "f32" and K > 512 else ("uniform", -1.0, 1.0)
    return wl.GemmCase(f"g{M}x{N}x{K}", M, N, K, ti, tb, to, act, alpha, dist, dist, dist)


def _ccase(N, C, H, W, Co, kh, kw, st, pd, dl, ti, to, tb, act, dist=None):
    if dist is None:
        dist = SMALL_F32 if ti == "f32" and C * kh * kw > 512 else ("uniform", -0.5, 0.5)
    return wl.ConvCase(f"c{N}x{C}x{H}x{W}", N, C, H, W, Co, kh, kw, st, pd, dl, ti, tb, to, act, 0.0,
                       dist, dist, dist)


def _report(tag, rep):
    print(f"[{tag}] n={rep['n']} bad={rep['n_bad']} max_err/tol={rep['max_err_over_tol']:.3g}", flush=True)


# ---------------------------------------------------------------------------
# GEMM: small and ragged shapes, every element against the oracle
# ---------------------------------------------------------------------------

GEMM_SHAPES = [(1, 1, 1), (3, 5, 7), (64, 64, 64), (127, 129, 65), (200, 136, 72),
               (256, 256, 64), (300, 520, 200), (33, 260, 1000), (520, 8, 24), (16, 1024, 40)]
GEMM_TYPES = [("bf16", "bf16", "f32"), ("f16", "f32", "f32"), ("f16", "f16", "f16"),
              ("bf16", "f32", "bf16"), ("f32", "f32", "f32"), ("f32", "bf16", "f32")]
ACTS = ["none", "relu", "leaky_relu", "tanh", "gelu", "sigmoid"]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("types", GEMM_TYPES, ids=lambda t: "-".join(t))
def test_gemm_small_vs_oracle(ba, shape, types):
    M, N, K = shape
    ti, to, tb = types
    s0 = sum(shape) + len(ti)
    for j, act in enumerate((ACTS[s0 % 6], ACTS[(s0 + 1) % 6], ACTS[(s0 + 3) % 6])):
        case = _gcase(M, N, K, ti, to, tb, act, alpha=0.1)
        inp = wl.gen_gemm(case, seed=11 + j)
        y = values_of(run_gemm(case, inp), to)
        ref, floor = gemm_reference(case, inp)
        rep = check(y, ref, floor, case)
        _report(f"gemm {shape} {types} {act}", rep)
        assert rep["ok"], rep


@pytest.mark.parametrize("tile", range(8))
def test_gemm_every_tile_config(ba, tile):
    ba.force_tile_config(tile)
    try:
        for ti, to, (M, N, K) in (("bf16", "bf16", (300, 520, 200)), ("f16", "f32", (300, 520, 200)),
                                  ("f32", "f32", (300, 520, 200)), ("bf16", "f16", (513, 264, 1032)),
                                  ("f16", "bf16", (40, 1000, 72))):
            case = _gcase(M, N, K, ti, to, "f32", "leaky_relu", 0.05)
            inp = wl.gen_gemm(case, seed=3)
            y = values_of(run_gemm(case, inp), to)
            ref, floor = gemm_reference(case, inp)
            rep = check(y, ref, floor, case)
            _report(f"tile {tile} {ti}->{to}", rep)
            assert rep["ok"], rep
    finally:
        ba.force_tile_config(-1)


@pytest.mark.parametrize("ti,tb", [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("f16", "f32")])
def test_pp_bias_vector_and_element_loads_agree(ba, ti, tb):
    # The ping-pong kernel reads each lane's bias as runs of 4 columns (one
    # 16- or 8-byte load each) when the bias is aligned for it, and element by
    # element otherwise: bias one element into its buffer gives the same bits
    M, N, K = 300, 520, 200
    case = _gcase(M, N, K, ti, ti, tb, "gelu")
    inp = wl.gen_gemm(case, seed=23)
    ref, floor = gemm_reference(case, inp)
    A, _ = to_dev(inp["A"].reshape(M, K), ti)
    B, _ = to_dev(inp["B"].reshape(K, N), ti)
    bias0, _ = to_dev(inp["bias"], tb)
    outs = []
    ba.force_tile_config(6)
    try:
        for off in (0, 1):
            if off:
                buf = torch.empty(N + off, dtype=bias0.dtype, device="cuda")
                bias = buf[off:]
                bias.copy_(bias0)
            else:
                bias = bias0
            C = torch.empty((M, N), dtype=A.dtype, device="cuda")
            ba.gemm_bias_act(A, B, bias, C, "gelu", 0.0)
            torch.cuda.synchronize()
            assert "ping-pong" in ba.last_tile_config()
            outs.append(C)
    finally:
        ba.force_tile_config(-1)
    for C in outs:
        rep = check(values_of(C, ti), ref, floor, case)
        _report(f"pp bias {ti} {tb}", rep)
        assert rep["ok"], rep
    assert np.array_equal(words_of(outs[0], ti), words_of(outs[1], ti))


@pytest.mark.parametrize("ti", ["bf16", "f16", "f32"])
def test_gemm_short_reduction_all_k_tiles(ba, ti):
    # the 64x64 tile loads a reduction of at most four k-tiles at once; cover
    # 1..4 k-tiles, ragged tails and the first length past the limit
    ba.force_tile_config(5)
    try:
        bk = 32 if ti == "f32" else 64
        for j, K in enumerate((0, 1, bk - 3, bk, bk + 1, 3 * bk - 5, 4 * bk, 4 * bk + 1)):
            M, N = 70 + 37 * j, 130 - 9 * j
            case = _gcase(M, N, K, ti, "f32", "f32", ACTS[j % 6], 0.1)
            inp = wl.gen_gemm(case, seed=40 + j)
            y = values_of(run_gemm(case, inp), "f32")
            ref, floor = gemm_reference(case, inp)
            rep = check(y, ref, floor, case)
            _report(f"short-k {ti} K={K}", rep)
            assert rep["ok"], rep
    finally:
        ba.force_tile_config(-1)


def test_gemm_no_bias_and_k_zero(ba):
    case = wl.GemmCase("nobias", 70, 90, 130, "bf16", None, "f32", "relu")
    inp = wl.gen_gemm(case, seed=5)
    y = values_of(run_gemm(case, inp), "f32")
    ref, _ = gemm_reference(case, inp)
    assert check(y, ref, None, case)["ok"]
    # K = 0: the sum is empty, C = act(bias)
    case0 = _gcase(9, 40, 0, "f16", "f32", "f32", "leaky_relu", 0.25)
    inp0 = wl.gen_gemm(case0, seed=6)
    y0 = values_of(run_gemm(case0, inp0), "f32")
    ref0, _ = gemm_reference(case0, inp0)
    assert np.array_equal(y0, ref0.astype(np.float32).astype(np.float64))   # act(bias) exactly


def test_gemm_empty_is_a_no_op(ba):
    A = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    ba.gemm_bias_act(A, B, None, C, "relu")
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# exact cases: bit equality where fp32 arithmetic is exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ti", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("shape", [(5, 7, 3), (64, 96, 128), (130, 70, 257)])
def test_gemm_small_integers_bitwise(ba, ti, shape):
    M, N, K = shape
    for act, alpha in (("none", 0), ("relu", 0), ("leaky_relu", 0.25)):
        case = wl.GemmCase("ints", M, N, K, ti, "f32", "f32", act, alpha,
                           ("ints", -2, 2), ("ints", -2, 2), ("ints", -2, 2))
        inp = wl.gen_gemm(case, seed=21)
        y = values_of(run_gemm(case, inp), "f32")
        ref, _ = gemm_reference(case, inp)
        assert np.array_equal(y, ref), (act, np.abs(y - ref).max())


def _within_one_f32_ulp(y, want):
    # The matrix cores' accumulate step is not guaranteed to round to nearest:
    # bias + a through an identity B can land on either fp32 neighbour.
    w32 = want.astype(np.float32)
    return bool(np.all(np.abs(y - want) <= np.spacing(np.abs(w32)).astype(np.float64)))


def test_gemm_identity_b_one_ulp(ba):
    M, K = 96, 128
    rng = np.random.default_rng(0)
    a = rng.uniform(-4, 4, (M, K)).astype(np.float32)
    bias = rng.uniform(-1, 1, K).astype(np.float32)
    inp = {"A": wl.encode(a, "bf16"), "B": wl.encode(np.eye(K, dtype=np.float32), "bf16"),
           "bias": wl.encode(bias, "f32")}
    case = wl.GemmCase("eye", M, K, K, "bf16", "f32", "f32", "none")
    y = values_of(run_gemm(case, inp), "f32")
    a_bf = (inp["A"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = (bias.astype(np.float64).reshape(1, K) + a_bf).ravel()     # exact bias + a
    assert _within_one_f32_ulp(y, want)


def test_leaky_and_relu_invariants_bitwise(ba):
    base = _gcase(130, 264, 96, "bf16", "f32", "f32", "none")
    inp = wl.gen_gemm(base, seed=9)
    y_none = values_of(run_gemm(base, inp), "f32").astype(np.float32)
    for alpha in (0.001, 0.01, 0.25):
        lk = _gcase(130, 264, 96, "bf16", "f32", "f32", "leaky_relu", alpha)
        y = values_of(run_gemm(lk, inp), "f32").astype(np.float32)
        want = np.where(y_none >= 0, y_none, np.float32(alpha) * y_none)
        assert np.array_equal(y, want)
    rl = _gcase(130, 264, 96, "bf16", "f32", "f32", "relu")
    y = values_of(run_gemm(rl, inp), "f32").astype(np.float32)
    assert np.array_equal(y, np.maximum(y_none, np.float32(0)))


def test_tanh_sweep_through_k1_gemm(ba):
    z = np.array([0.0, 1e-8, 1e-6, 1e-3, 0.1, 0.5, 1.0, 2.0, 5.0, 9.0, 10.0, 15.0, 20.0,
                  88.0, 89.0, 1e4, 3.4e38], dtype=np.float32)
    z = np.concatenate([z, -z, np.linspace(-12, 12, 4047, dtype=np.float32)])
    M = z.size
    inp = {"A": wl.encode(z.reshape(M, 1), "f32"), "B": wl.encode(np.ones((1, 1), np.float32), "f32"),
           "bias": None}
    case = wl.GemmCase("tanh", M, 1, 1, "f32", None, "f32", "tanh")
    y = values_of(run_gemm(case, inp), "f32")
    ref = np.tanh(z.astype(np.float64))
    assert y.shape == ref.shape
    assert np.all(np.isfinite(y))
    ulp32 = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(y - ref) <= np.maximum(4 * ulp32, 1e-30))
    assert np.all(y[np.abs(z) >= 10] == np.sign(z[np.abs(z) >= 10]))
    yf = y.astype(np.float32)
    pos, neg = yf[:17], yf[17:34]
    assert np.array_equal(neg, -pos)


@pytest.mark.parametrize("to", ["f16", "bf16"])
def test_tanh_sweep_16bit_outputs(ba, to):
    # 16-bit outputs take the shorter tanh (series below 2^-6, the e^{2|x|}
    # identity above): z through an fp32 K = 1 GEMM, against the oracle at one
    # output ulp, across the switch point, the small-|z| range and saturation
    t = np.float32(2.0 ** -6)
    z = np.concatenate([np.array([0.0, 1e-30, 1e-8, 6e-8, 1e-5, 1e-3, 0.01, 0.5, 1.0, 4.0, 9.0, 10.0,
                                  20.0, 89.0, 1e4, 3.4e38], np.float32),
                        np.nextafter(t, np.float32(0)) * np.ones(1, np.float32), t * np.ones(1, np.float32),
                        np.nextafter(t, np.float32(1)) * np.ones(1, np.float32),
                        np.geomspace(1e-7, 12.0, 6000).astype(np.float32)])
    z = np.concatenate([z, -z])
    M = z.size
    inp = {"A": wl.encode(z.reshape(M, 1), "f32"), "B": wl.encode(np.ones((1, 1), np.float32), "f32"),
           "bias": None}
    case = wl.GemmCase("tanh16", M, 1, 1, "f32", None, to, "tanh")
    y = values_of(run_gemm(case, inp), to)
    ref, acc = gemm_reference(case, inp)
    rep = check(y, ref, acc, case)
    _report(f"tanh sweep {to}", rep)
    assert rep["ok"], rep
    half = M // 2
    assert np.array_equal(y[half:], -y[:half])               # odd


@pytest.mark.parametrize("act", ["gelu", "sigmoid"])
def test_gelu_sigmoid_sweep_through_k1_gemm(ba, act):
    # z through an fp32 K = 1 GEMM (A = z, B = 1, no bias): y = act(z) against
    # the oracle's fp64 value, over the range and the far tails
    z = np.array([0.0, 1e-8, 1e-6, 1e-3, 0.1, 0.5, 1.0, 2.0, 3.0, 5.0, 8.0, 10.0, 15.0, 20.0,
                  40.0, 88.0, 89.0, 1e4, 3.4e38], dtype=np.float32)
    z = np.concatenate([z, -z, np.linspace(-12, 12, 4041, dtype=np.float32)])
    M = z.size
    inp = {"A": wl.encode(z.reshape(M, 1), "f32"), "B": wl.encode(np.ones((1, 1), np.float32), "f32"),
           "bias": None}
    case = wl.GemmCase(act, M, 1, 1, "f32", None, "f32", act)
    y = values_of(run_gemm(case, inp), "f32")
    ref = gemm_reference(case, inp)[0]
    assert np.all(np.isfinite(y))
    ulp32 = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    zd = np.abs(z.astype(np.float64))
    if act == "sigmoid":
        # a few fp32 ulps (hardware exp2 and reciprocal), plus the rounding of
        # the fp32 exponent argument z*log2(e), which e^-z turns into a
        # relative error of |z| * 2^-24 (up to ~90 ulps at z = -88); results
        # below the fp32 normal range may flush to zero
        assert np.all(np.abs(y - ref) <= np.maximum((4 + 1.5 * zd) * ulp32, 1e-37))
        assert np.all((y >= 0) & (y <= 1))
        assert np.all(y[z >= 20] == 1.0)
    else:
        # a few fp32 ulps, plus roundings that erfc's tail (~e^-x^2) amplifies
        # by x^2: of the fp32 argument x = z/sqrt(2) (2 x^2 ulps) and of the
        # exponent -x^2 + P(t) and its base-2 scaling (about 2 x^2 ulps more);
        # a float32 emulation of the device evaluation peaks at 0.61 of this
        # bound (255 ulps at z = -12).  erfc, unlike 1 + erf, adds no
        # cancellation there.
        x2 = zd * zd / 2.0
        small = np.abs(ref) < 1e-30
        err_ulps = np.abs(y - ref)[~small] / ulp32[~small]
        assert np.all(err_ulps <= 16 + 6.0 * x2[~small]), np.max(err_ulps)
        assert np.all(np.abs(y[small]) < 1e-30)
        assert np.all(y[z >= 10] == z[z >= 10])


# ---------------------------------------------------------------------------
# conv2d
# ---------------------------------------------------------------------------

CONV_SHAPES = [
    # N, C, H, W, Co, kh, kw, strides, pads(t,b,l,r), dilations
    (1, 1, 5, 6, 1, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (2, 3, 9, 7, 4, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2)),
    (1, 5, 11, 13, 3, 5, 5, (3, 2), (2, 2, 0, 3), (1, 1)),
    (3, 16, 8, 8, 70, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)),
    (2, 12, 12, 10, 33, 3, 3, (1, 1), (2, 2, 2, 2), (2, 3)),
    (1, 3, 31, 29, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)),
    (2, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (1, 40, 9, 9, 136, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2)),
    (1, 16, 6, 20, 24, 1, 9, (1, 1), (0, 0, 4, 4), (1, 1)),     # 9 taps, not 3x3: the generic kernel
    (1, 16, 20, 6, 24, 9, 1, (1, 1), (4, 4, 0, 0), (1, 1)),
    (2, 37, 7, 9, 40, 1, 1, (1, 1), (1, 0, 2, 1), (1, 1)),      # 1x1 in padding, ragged last chunk
    (1, 70, 5, 11, 33, 1, 1, (2, 3), (0, 0, 0, 0), (1, 1)),     # 1x1, unequal strides, odd W
]
CONV_TYPES = [("f16", "f16", "f16"), ("bf16", "bf16", "bf16"), ("f32", "f32", "f32"),
              ("f16", "f32", "f32"), ("bf16", "bf16", "f32")]


@pytest.mark.parametrize("shape", CONV_SHAPES, ids=lambda s: "x".join(map(str, s[:7])))
@pytest.mark.parametrize("types", CONV_TYPES, ids=lambda t: "-".join(t))
def test_conv_small_vs_oracle(ba, shape, types):
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    ti, to, tb = types
    for j, act in enumerate(("tanh", "none", "relu", "sigmoid", "gelu")):
        case = _ccase(N, C, H, W, Co, kh, kw, st, pd, dl, ti, to, tb, act)
        inp = wl.gen_conv(case, seed=31 + j)
        y = values_of(run_conv(case, inp), to)
        ref, floor = conv_reference(case, inp)
        rep = check(y, ref, floor, case)
        _report(f"conv {shape} {types} {act}", rep)
        assert rep["ok"], rep


@pytest.mark.parametrize("tile", range(8))
def test_conv_every_tile_config(ba, tile):
    ba.force_tile_config(tile)
    try:
        for ti, to in (("f16", "f16"), ("f32", "f32")):
            for k, geo in ((3, ((1, 2), (1, 0, 1, 2), (2, 1))), (1, ((2, 1), (1, 0, 0, 1), (1, 1)))):
                case = _ccase(2, 36 if k == 1 else 20, 15, 17, 75, k, k, *geo, ti, to, ti, "tanh")
                inp = wl.gen_conv(case, seed=4)
                y = values_of(run_conv(case, inp), to)
                ref, floor = conv_reference(case, inp)
                rep = check(y, ref, floor, case)
                _report(f"conv tile {tile} {ti} {k}x{k}", rep)
                assert rep["ok"], rep
    finally:
        ba.force_tile_config(-1)


# Shapes that take the channel-last halo kernel (16-bit, C % 8 == 0, even W,
# 1x1 or 3x3): several channel chunks, ragged Co, narrow and wide outputs,
# strides, dilations, asymmetric padding.
HALO_SHAPES = [
    (2, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),
    (1, 128, 12, 10, 96, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2)),
    (3, 16, 8, 8, 70, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)),
    (1, 8, 9, 150, 33, 3, 3, (1, 1), (1, 0, 2, 1), (1, 1)),
    (2, 256, 7, 6, 130, 3, 3, (2, 1), (1, 1, 0, 1), (1, 2)),
    (1, 24, 30, 2, 64, 3, 3, (3, 1), (1, 1, 1, 1), (1, 1)),
    (2, 32, 5, 40, 17, 1, 1, (1, 2), (1, 0, 0, 1), (1, 1)),
    (2, 40, 10, 12, 48, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),      # 64-channel chunk, 40 used
    (1, 104, 9, 8, 64, 3, 3, (1, 1), (0, 1, 1, 0), (1, 1)),       # two chunks, the last partial
    (2, 16, 11, 14, 80, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1)),      # 128-row blocks, one k-step
    (1, 72, 6, 16, 200, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1)),      # three chunks, two co blocks
    (1, 64, 9, 130, 32, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1)),      # halo past one load batch
    (2, 16, 13, 18, 40, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1)),      # 5x5: one 16-channel chunk
    (1, 32, 9, 12, 64, 5, 5, (1, 1), (4, 4, 4, 4), (2, 2)),       # 5x5 dilated, two chunks
    (1, 24, 11, 20, 72, 7, 7, (1, 1), (3, 3, 3, 3), (1, 1)),      # 7x7: partial second chunk, two co blocks
    (1, 8, 17, 30, 33, 7, 7, (2, 2), (3, 2, 1, 3), (1, 1)),       # 7x7 stride 2, asymmetric pads, C = 8
]


@pytest.mark.parametrize("shape", HALO_SHAPES, ids=lambda s: "x".join(map(str, s[:7])))
@pytest.mark.parametrize("types", [("f16", "f16", "f16"), ("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                   ("f16", "bf16", "f32")], ids=lambda t: "-".join(t))
def test_conv_halo_path_vs_oracle(ba, shape, types):
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    ti, to, tb = types
    # automatic choice, then every conv-halo variant forced
    for tile, variant in ((-1, -1), (7, 0), (7, 1), (7, 2), (7, 3), (7, 4)):
        ba.force_tile_config(tile)
        ba.force_halo_variant(variant)
        try:
            for j, act in enumerate(("tanh", "relu", "gelu" if Co % 2 else "sigmoid")):
                case = _ccase(N, C, H, W, Co, kh, kw, st, pd, dl, ti, to, tb, act)
                inp = wl.gen_conv(case, seed=41 + j)
                y = values_of(run_conv(case, inp), to)
                ref, floor = conv_reference(case, inp)
                rep = check(y, ref, floor, case)
                _report(f"halo {shape} {types} {act} tile {tile} variant {variant}", rep)
                assert rep["ok"], rep
        finally:
            ba.force_tile_config(-1)
            ba.force_halo_variant(-1)


HALO32_SHAPES = [
    (2, 3, 20, 22, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)),       # stem-like: C = 3, one chunk in both buffers
    (1, 3, 30, 40, 64, 11, 11, (2, 2), (5, 5, 5, 5), (1, 1)),     # C = 3 in three chunks (128 k-pairs at most)
    (1, 5, 13, 9, 70, 5, 5, (1, 1), (2, 1, 0, 2), (1, 1)),        # odd C, asymmetric pads, 128-row block
    (2, 40, 9, 11, 33, 1, 3, (1, 2), (0, 0, 1, 1), (1, 3)),       # 1x3 filter, dilation 3, odd chunk K
    (1, 300, 6, 7, 20, 3, 3, (1, 1), (1, 1, 1, 1), (2, 1)),       # many chunks, the last partial
    (3, 16, 30, 140, 8, 3, 2, (2, 3), (1, 2, 1, 0), (1, 1)),      # 3x2 filter, wide rows
    (1, 7, 5, 300, 130, 1, 2, (1, 1), (0, 0, 0, 1), (1, 1)),      # rows past 128 columns, two co blocks
]


@pytest.mark.parametrize("shape", HALO32_SHAPES, ids=lambda s: "x".join(map(str, s[:7])))
@pytest.mark.parametrize("to", ["f32", "bf16", "f16"])
def test_conv_halo32_path_vs_oracle(ba, shape, to):
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    for tile in (-1, 7):
        ba.force_tile_config(tile)
        try:
            for j, act in enumerate(("tanh", "relu", "sigmoid" if Co % 2 else "gelu")):
                case = _ccase(N, C, H, W, Co, kh, kw, st, pd, dl, "f32", to, "f32", act)
                inp = wl.gen_conv(case, seed=71 + j)
                y = values_of(run_conv(case, inp), to)
                ref, floor = conv_reference(case, inp)
                rep = check(y, ref, floor, case)
                _report(f"halo32 {shape} {to} {act} tile {tile}", rep)
                assert rep["ok"], rep
        finally:
            ba.force_tile_config(-1)


RESIDENT_SHAPES = [
    (1, 3, 300, 130, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)),       # 600 patches, ragged second column block
    (2, 4, 600, 70, 40, 5, 5, (2, 1), (2, 2, 2, 2), (1, 2)),        # stride 2 rows, dilation 2 columns
]


@pytest.mark.parametrize("shape", RESIDENT_SHAPES, ids=lambda s: "x".join(map(str, s[:7])))
@pytest.mark.parametrize("to", ["f32", "bf16"])
def test_conv_halo32_resident_filter_vs_oracle(ba, shape, to):
    # one channel chunk, one output-channel block and more patches than the
    # 512 workgroup slots: each workgroup stages the filter once and streams
    # two or one patches' halos through its two halo buffers
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    for j, act in enumerate(("tanh", "none")):
        case = _ccase(N, C, H, W, Co, kh, kw, st, pd, dl, "f32", to, "f32", act)
        inp = wl.gen_conv(case, seed=81 + j)
        y = values_of(run_conv(case, inp), to)
        assert "resident filter" in ba.last_tile_config(), ba.last_tile_config()
        ref, floor = conv_reference(case, inp)
        rep = check(y, ref, floor, case)
        _report(f"halo32 resident {shape} {to} {act}", rep)
        assert rep["ok"], rep


def test_conv_no_bias(ba):
    case = _ccase(2, 8, 10, 10, 16, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), "bf16", "f32", None, "none")
    inp = wl.gen_conv(case, seed=2)
    y = values_of(run_conv(case, inp), "f32")
    ref, _ = conv_reference(case, inp)
    assert check(y, ref, None, case)["ok"]


def test_conv_1x1_identity_weights_one_ulp(ba):
    N, C, H, W = 2, 32, 6, 10
    rng = np.random.default_rng(1)
    x = rng.uniform(-2, 2, (N, C, H, W)).astype(np.float32)
    bias = rng.uniform(-1, 1, C).astype(np.float32)
    inp = {"x": wl.encode(x, "f16"), "w": wl.encode(np.eye(C, dtype=np.float32).reshape(C, C, 1, 1), "f16"),
           "bias": wl.encode(bias, "f32")}
    case = wl.ConvCase("eye", N, C, H, W, C, 1, 1, (1, 1), (0, 0, 0, 0), (1, 1), "f16", "f32", "f32", "none")
    y = values_of(run_conv(case, inp), "f32")
    xf = inp["x"].view(np.float16).astype(np.float64)
    want = (xf + bias.astype(np.float64).reshape(1, C, 1, 1)).ravel()
    assert _within_one_f32_ulp(y, want)


# ---------------------------------------------------------------------------
# two-kernel path, determinism, guard bands
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("types", GEMM_TYPES, ids=lambda t: "-".join(t))
def test_gemm_two_kernel_bitwise_equal_fused(ba, types):
    ti, to, tb = types
    for act in ACTS:
        case = _gcase(257, 264, 136, ti, to, tb, act, 0.02)
        inp = wl.gen_gemm(case, seed=8)
        a = words_of(run_gemm(case, inp, "fused"), to)
        b = words_of(run_gemm(case, inp, "2k"), to)
        assert np.array_equal(a, b), act


@pytest.mark.parametrize("types", CONV_TYPES, ids=lambda t: "-".join(t))
def test_conv_two_kernel_bitwise_equal_fused(ba, types):
    ti, to, tb = types
    for act in ("tanh", "relu", "none", "gelu", "sigmoid"):
        case = _ccase(2, 24, 13, 11, 40, 3, 3, (2, 1), (1, 1, 0, 2), (1, 2), ti, to, tb, act)
        inp = wl.gen_conv(case, seed=12)
        a = words_of(run_conv(case, inp, "fused"), to)
        b = words_of(run_conv(case, inp, "2k"), to)
        assert np.array_equal(a, b), act


def test_run_to_run_bitwise_determinism(ba):
    case = _gcase(520, 384, 640, "bf16", "bf16", "f32", "tanh")
    inp = wl.gen_gemm(case, seed=1)
    first = words_of(run_gemm(case, inp), "bf16")
    for _ in range(3):
        assert np.array_equal(words_of(run_gemm(case, inp), "bf16"), first)
    cc = _ccase(2, 16, 20, 20, 48, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), "f16", "f16", "f16", "tanh")
    cinp = wl.gen_conv(cc, seed=1)
    cfirst = words_of(run_conv(cc, cinp), "f16")
    for _ in range(3):
        assert np.array_equal(words_of(run_conv(cc, cinp), "f16"), cfirst)


@pytest.mark.parametrize("to", ["f32", "bf16"])
def test_guard_bands_untouched(ba, to):
    canary = 0x7FC01234 if to == "f32" else 0x7FC1
    guard = 256
    for M, N, K in ((131, 77, 50), (300, 260, 72), (64, 128, 64)):
        case = _gcase(M, N, K, "bf16", to, "f32", "relu")
        inp = wl.gen_gemm(case, seed=2)
        C, buf = empty_out((M, N), to, guard, canary)
        run_gemm(case, inp, out=C)
        assert guard_intact(buf, guard, to, canary), (M, N, K)
        ref, floor = gemm_reference(case, inp)
        assert check(values_of(C, to), ref, floor, case)["ok"]
    cc = _ccase(3, 5, 9, 11, 70, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), "bf16", to, "bf16", "tanh")
    cinp = wl.gen_conv(cc, seed=3)
    Ho, Wo = cc.out_hw()
    y, buf = empty_out((3, 70, Ho, Wo), to, guard, canary)
    run_conv(cc, cinp, out=y)
    assert guard_intact(buf, guard, to, canary)


def test_python_binding_rejects_bad_tensors(ba):
    A = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 4), dtype=torch.float16, device="cuda")
    C = torch.zeros((4, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        ba.gemm_bias_act(A, B, None, C, "relu")             # A and B types differ
    with pytest.raises(ValueError):
        ba.gemm_bias_act(A, A.t(), None, C, "relu")          # non-contiguous
    x = torch.zeros((1, 2, 5, 5), dtype=torch.float16, device="cuda")
    w = torch.zeros((3, 2, 3, 3), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, 3, 3, 3), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        ba.conv2d_bias_act(x, w, None, y, act="leaky_relu")


# ---------------------------------------------------------------------------
# the named workloads at full size: every output, seeds 0, 1 and 2
# ---------------------------------------------------------------------------

NAMED = list(wl.CASES)
CHUNK = 1 << 24          # outputs per oracle call on the GEMMs (bounds host memory)


def _log_report(name, seed, rep):
    """Print the report; with BIASACT_PARITY_LOG set, also append it there as
    one JSON line (the per-workload error record)."""
    import json
    import os
    line = {"workload": name, "seed": seed, **{k: v for k, v in rep.items() if k != "worst"}}
    print(f"[full {name} seed {seed}] {json.dumps(line)}", flush=True)
    path = os.environ.get("BIASACT_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


@pytest.mark.parametrize("seed", (0, 1, 2))
@pytest.mark.parametrize("name", NAMED + list(wl.FILTER_CASES))
def test_named_workload_full_size(ba, name, seed):
    case = wl.CASES[name] if name in wl.CASES else wl.FILTER_CASES[name]
    is_gemm = isinstance(case, wl.GemmCase)
    inp = wl.gen_gemm(case, seed) if is_gemm else wl.gen_conv(case, seed)
    y_t = run_gemm(case, inp) if is_gemm else run_conv(case, inp)
    vals = values_of(y_t, case.out_dtype)
    assert np.all(np.isfinite(vals))
    if is_gemm:
        rows = max(1, CHUNK // case.N)
        reps = []
        for r0 in range(0, case.M, rows):
            r1 = min(case.M, r0 + rows)
            ref, acc = gemm_reference(case, inp, rows=slice(r0, r1))
            reps.append(check(vals[r0 * case.N:r1 * case.N], ref, acc, case))
        rep = merge(reps)
    else:
        ref, acc = conv_reference(case, inp)
        rep = check(vals, ref, acc, case)
    _log_report(name, seed, rep)
    assert rep["ok"], rep
    # the two-kernel path gives the same bits at full size (int8 GEMMs have
    # the fused path only)
    if seed == 0 and case.in_dtype != "i8":
        y2 = run_gemm(case, inp, "2k") if is_gemm else run_conv(case, inp, "2k")
        assert np.array_equal(words_of(y2, case.out_dtype), words_of(y_t, case.out_dtype))
        del y2
    del y_t
    torch.cuda.empty_cache()


def test_matmul_leakyrelu_sample_acceptance_scale(ba):
    """The MatmulLeakyRelu sample's acceptance scale ("CANN pyasc
    MatmulLeakyRelu 融合算子实战", section 编译执行: relative and absolute
    tolerance 1e-3 over the whole output), stated here as an explicit bound
    against the oracle: |C - ref| <= 1e-3 * (1 + |ref|) for every element."""
    case = wl.CASES["gemm_leaky_1024x640x256_f16"]
    inp = wl.gen_gemm(case, 0)
    c = values_of(run_gemm(case, inp), "f32")
    ref, _ = gemm_reference(case, inp)
    assert np.all(np.abs(c - ref) <= 1e-3 * (1.0 + np.abs(ref)))
