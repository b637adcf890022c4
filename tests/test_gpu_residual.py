"""GPU parity of the residual epilogue, act(A.B + bias + R) and
act(conv2d(x, w) + bias + R), against the fp64 oracle on the same input bits.

The residual R has the output's type and shape.  Every kernel family is
covered (ping-pong, short-reduction and tiled GEMMs; the fp16/bf16 and fp32
conv-halo kernels and the generic conv), fused and two-kernel paths (bitwise
equal), in place (R is the output buffer), and with R misaligned against the
output so the kernels fall back to element-wise accesses.  The acceptance rule
is the one of the other parity tests; for 16-bit outputs the accumulation
allowance counts R as one more term of the fp32 sum.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import O, acc_bound, check, to_dev, torch_dtype, values_of, words_of
import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    m.force_halo_variant(-1)
    return m


def _residual_words(shape, dt, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return wl.encode((rng.uniform(-1.0, 1.0, shape) * scale).astype(np.float32), dt)


def _dev_out(words, dt, offset=0):
    """Device tensor of the encoded words; offset > 0 places it `offset`
    elements into a larger buffer (misaligned against a fresh allocation)."""
    t, _ = to_dev(words.ravel(), dt)
    if not offset:
        return t.view(words.shape)
    buf = torch.empty(words.size + offset, dtype=torch_dtype(dt), device="cuda")
    v = buf[offset:offset + words.size]
    v.copy_(t)
    return v.view(words.shape)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _gemm_case(M, N, K, ti, to, act):
    U = ("uniform", -1.0, 1.0)
    return wl.GemmCase(f"r{M}x{N}x{K}", M, N, K, ti, "f32", to, act, 0.05, U, U, U)


def _gemm_ref(case, inp, r_words):
    o = O()
    A = o.decode(inp["A"], case.in_dtype).reshape(case.M, case.K)
    B = o.decode(inp["B"], case.in_dtype).reshape(case.K, case.N)
    bias = o.decode(inp["bias"], case.bias_dtype)
    R = o.decode(r_words.ravel(), case.out_dtype).reshape(case.M, case.N)
    alpha = orc.f32(case.alpha)
    ref = o.gemm_residual(A, B, bias, R, case.act, alpha).ravel()
    z = (o.gemm(A, B, bias, "none") + R).ravel()
    s = (o.gemm(np.abs(A), np.abs(B), np.abs(bias), "none") + np.abs(R)).ravel()
    return ref, acc_bound(case.out_dtype, case.K + 2, z, s, case.act, alpha)


def _run_gemm(ba, case, inp, r_words, path="fused", inplace=False, r_offset=0, c_offset=0):
    A, _ = to_dev(inp["A"].reshape(case.M, case.K), case.in_dtype)
    B, _ = to_dev(inp["B"].reshape(case.K, case.N), case.in_dtype)
    bias, _ = to_dev(inp["bias"], case.bias_dtype)
    R = _dev_out(r_words.reshape(case.M, case.N), case.out_dtype, r_offset)
    if inplace:
        C = R
    else:
        buf = torch.empty(case.M * case.N + c_offset, dtype=torch_dtype(case.out_dtype), device="cuda")
        C = buf[c_offset:].view(case.M, case.N)
    alpha = float(np.float32(case.alpha))
    if path == "fused":
        ba.gemm_bias_add_act(A, B, bias, R, C, case.act, alpha)
    else:
        ws = torch.empty(max(1, ba.gemm_bias_act_workspace_size(case.M, case.N) // 4),
                         dtype=torch.float32, device="cuda")
        ba.gemm_bias_add_act_2k(A, B, bias, R, C, case.act, alpha, workspace=ws)
    torch.cuda.synchronize()
    return C


GEMM_CASES = [
    # (M, N, K, in, out, act, forced tile)
    (300, 520, 200, "bf16", "bf16", "relu", -1),
    (257, 264, 136, "f16", "f32", "gelu", -1),
    (1024, 640, 256, "f16", "f32", "leaky_relu", 5),       # short reduction, all k-tiles at once
    (512, 768, 192, "bf16", "bf16", "tanh", 6),            # ping-pong kernel
    (264, 520, 136, "f16", "f32", "gelu", 6),              # ping-pong kernel, 32-bit output in two passes
    (520, 384, 640, "f16", "f16", "sigmoid", 2),
    (200, 136, 72, "f32", "f32", "tanh", -1),
    (33, 260, 1000, "f32", "bf16", "none", -1),
]


@pytest.mark.parametrize("case_args", GEMM_CASES, ids=lambda c: "x".join(map(str, c[:3])) + "-" + c[3] + "-" + c[5])
def test_gemm_residual_vs_oracle(ba, case_args):
    M, N, K, ti, to, act, tile = case_args
    case = _gemm_case(M, N, K, ti, to, act)
    inp = wl.gen_gemm(case, seed=61)
    r = _residual_words((M, N), to, seed=62)
    ref, floor = _gemm_ref(case, inp, r)
    ba.force_tile_config(tile)
    try:
        y = _run_gemm(ba, case, inp, r)
        rep = check(values_of(y, to), ref, floor, case)
        assert rep["ok"], rep
        # the two-kernel path adds R in its second kernel: the same bits
        y2 = _run_gemm(ba, case, inp, r, "2k")
        assert np.array_equal(words_of(y, to), words_of(y2, to))
        # in place: R is the output buffer
        y3 = _run_gemm(ba, case, inp, r, inplace=True)
        assert np.array_equal(words_of(y, to), words_of(y3, to))
    finally:
        ba.force_tile_config(-1)


@pytest.mark.parametrize("ti,to", [("bf16", "bf16"), ("f16", "f32")])
def test_gemm_residual_misaligned(ba, ti, to):
    # R one element into its buffer: no longer aligned for 4-wide accesses,
    # so the kernels use element-wise residual loads (and the ping-pong
    # kernel is not taken); results are unchanged
    case = _gemm_case(512, 512, 128, ti, to, "relu")
    inp = wl.gen_gemm(case, seed=63)
    r = _residual_words((512, 512), to, seed=64)
    ref, floor = _gemm_ref(case, inp, r)
    a = _run_gemm(ba, case, inp, r)
    b = _run_gemm(ba, case, inp, r, r_offset=1)
    assert check(values_of(b, to), ref, floor, case)["ok"]
    assert np.array_equal(words_of(a, to), words_of(b, to))


@pytest.mark.parametrize("to", ["bf16", "f16"])
def test_pp_row_staged_and_direct_epilogues_agree(ba, to):
    # The ping-pong kernel writes a 16-bit output through LDS, in whole rows,
    # when C and R lie on 16-byte boundaries, and straight from the
    # accumulator layout when one of them lies 8 bytes off (still aligned for
    # its 4-wide accesses).  Both give the oracle's result and the same bits,
    # with and without a residual, over ragged M and N (N % 8 == 0).
    case = _gemm_case(300, 520, 200, "bf16", to, "tanh")
    inp = wl.gen_gemm(case, seed=66)
    r = _residual_words((300, 520), to, seed=67)
    ref, floor = _gemm_ref(case, inp, r)
    ref0, floor0 = _gemm_ref(case, inp, _residual_words((300, 520), to, seed=0, scale=0.0))
    ba.force_tile_config(6)
    try:
        staged = _run_gemm(ba, case, inp, r)
        assert check(values_of(staged, to), ref, floor, case)["ok"]
        for kw in ({"c_offset": 4}, {"r_offset": 4}):
            direct = _run_gemm(ba, case, inp, r, **kw)
            assert np.array_equal(words_of(staged, to), words_of(direct, to)), kw
        plain = []
        for off in (0, 4):                       # no residual: the plain entry point
            A, _ = to_dev(inp["A"].reshape(300, 200), "bf16")
            B, _ = to_dev(inp["B"].reshape(200, 520), "bf16")
            bias, _ = to_dev(inp["bias"], "f32")
            buf = torch.empty(300 * 520 + off, dtype=torch_dtype(to), device="cuda")
            C = buf[off:].view(300, 520)
            ba.gemm_bias_act(A, B, bias, C, case.act, float(np.float32(case.alpha)))
            torch.cuda.synchronize()
            plain.append(C)
        assert check(values_of(plain[0], to), ref0, floor0, case)["ok"]
        assert np.array_equal(words_of(plain[0], to), words_of(plain[1], to))
    finally:
        ba.force_tile_config(-1)


def test_gemm_residual_zero_equals_plain(ba):
    # R = 0 gives the plain entry point's bits (-0 residuals would not, for
    # outputs that are exactly -0)
    case = _gemm_case(260, 300, 96, "bf16", "f32", "leaky_relu")
    inp = wl.gen_gemm(case, seed=65)
    r = np.zeros((260, 300), dtype=np.uint32)
    y = _run_gemm(ba, case, inp, r)
    A, _ = to_dev(inp["A"].reshape(260, 96), "bf16")
    B, _ = to_dev(inp["B"].reshape(96, 300), "bf16")
    bias, _ = to_dev(inp["bias"], "f32")
    C = torch.empty((260, 300), dtype=torch.float32, device="cuda")
    ba.gemm_bias_act(A, B, bias, C, "leaky_relu", float(np.float32(0.05)))
    torch.cuda.synchronize()
    yv, cv = words_of(y, "f32"), words_of(C, "f32")
    nz = cv != 0x80000000                    # -0 + (+0) = +0
    assert np.array_equal(yv[nz], cv[nz])


# ---------------------------------------------------------------------------
# conv2d
# ---------------------------------------------------------------------------

def _conv_case(shape, ti, to, act):
    N, C, H, W, Co, kh, kw, st, pd, dl = shape
    U = ("uniform", -0.5, 0.5)
    return wl.ConvCase("rc", N, C, H, W, Co, kh, kw, st, pd, dl, ti, ti, to, act, 0.0, U, U, U)


def _conv_ref(case, inp, r_words):
    o = O()
    x = o.decode(inp["x"], case.in_dtype).reshape(case.N, case.C, case.H, case.W)
    w = o.decode(inp["w"], case.in_dtype).reshape(case.Co, case.C, case.kh, case.kw)
    bias = o.decode(inp["bias"], case.bias_dtype)
    Ho, Wo = case.out_hw()
    R = o.decode(r_words.ravel(), case.out_dtype).reshape(case.N, case.Co, Ho, Wo)
    args = (case.strides, case.pads, case.dilations)
    ref = o.conv2d_residual(x, w, bias, R, *args, case.act).ravel()
    K = case.C * case.kh * case.kw
    z = (o.conv2d(x, w, bias, *args, "none") + R).ravel()
    s = (o.conv2d(np.abs(x), np.abs(w), np.abs(bias), *args, "none") + np.abs(R)).ravel()
    return ref, acc_bound(case.out_dtype, K + 2, z, s, case.act, 0.0)


def _run_conv(ba, case, inp, r_words, path="fused", inplace=False, r_offset=0):
    x, _ = to_dev(inp["x"].reshape(case.N, case.C, case.H, case.W), case.in_dtype)
    w, _ = to_dev(inp["w"].reshape(case.Co, case.C, case.kh, case.kw), case.in_dtype)
    bias, _ = to_dev(inp["bias"], case.bias_dtype)
    Ho, Wo = case.out_hw()
    R = _dev_out(r_words.reshape(case.N, case.Co, Ho, Wo), case.out_dtype, r_offset)
    y = R if inplace else torch.empty((case.N, case.Co, Ho, Wo), dtype=torch_dtype(case.out_dtype),
                                      device="cuda")
    args = (case.strides, case.pads, case.dilations, case.act)
    if path == "fused":
        ba.conv2d_bias_add_act(x, w, bias, R, y, *args)
    else:
        n = ba.conv2d_bias_act_workspace_size(case.N, case.C, case.H, case.W, case.Co, case.kh,
                                              case.kw, case.strides, case.pads, case.dilations)
        ws = torch.empty(max(1, n // 4), dtype=torch.float32, device="cuda")
        ba.conv2d_bias_add_act_2k(x, w, bias, R, y, *args, workspace=ws)
    torch.cuda.synchronize()
    return y


CONV_CASES = [
    # shape, in, out, act, forced tile, expected kernel prefix
    ((2, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)), "f16", "f16", "tanh", -1, "conv-halo 9"),
    ((1, 128, 12, 10, 96, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2)), "bf16", "bf16", "relu", -1, "conv-halo 9"),
    ((3, 16, 8, 8, 70, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)), "bf16", "f32", "sigmoid", -1, "conv-halo 1"),
    ((1, 8, 9, 150, 33, 3, 3, (1, 1), (1, 0, 2, 1), (1, 1)), "f16", "f16", "gelu", -1, "conv-halo 9"),
    ((2, 3, 20, 22, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)), "f32", "f32", "tanh", -1, "conv-halo fp32"),
    ((1, 5, 13, 9, 70, 5, 5, (1, 1), (2, 1, 0, 2), (1, 1)), "f32", "bf16", "relu", -1, "conv-halo fp32"),
    ((2, 24, 13, 11, 40, 3, 3, (2, 1), (1, 1, 0, 2), (1, 2)), "f16", "f16", "tanh", 3, "conv 64x128"),
    ((2, 32, 14, 14, 48, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)), "f32", "f32", "none", -1, "conv "),
    # Ho*Wo % 4 == 0 on the generic kernel: outputs staged through LDS (and,
    # with R one element off, element-wise: the same bits)
    ((2, 32, 16, 16, 48, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)), "f32", "f32", "tanh", -1, "conv "),
    ((2, 20, 12, 12, 72, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)), "f16", "f16", "gelu", -1, "conv "),
    ((1, 36, 10, 10, 130, 1, 1, (1, 1), (1, 1, 1, 1), (1, 1)), "bf16", "bf16", "relu", 1, "conv 128x256"),
]


@pytest.mark.parametrize("case_args", CONV_CASES, ids=lambda c: "x".join(map(str, c[0][:7])) + "-" + c[1] + "-" + c[3])
def test_conv_residual_vs_oracle(ba, case_args):
    shape, ti, to, act, tile, kernel = case_args
    case = _conv_case(shape, ti, to, act)
    inp = wl.gen_conv(case, seed=71)
    Ho, Wo = case.out_hw()
    r = _residual_words((case.N, case.Co, Ho, Wo), to, seed=72, scale=0.5)
    ref, floor = _conv_ref(case, inp, r)
    ba.force_tile_config(tile)
    try:
        y = _run_conv(ba, case, inp, r)
        assert ba.last_tile_config().startswith(kernel), ba.last_tile_config()
        rep = check(values_of(y, to), ref, floor, case)
        assert rep["ok"], rep
        y2 = _run_conv(ba, case, inp, r, "2k")
        assert np.array_equal(words_of(y, to), words_of(y2, to))
        y3 = _run_conv(ba, case, inp, r, inplace=True)
        assert np.array_equal(words_of(y, to), words_of(y3, to))
        y4 = _run_conv(ba, case, inp, r, r_offset=1)            # element-wise residual loads
        assert np.array_equal(words_of(y, to), words_of(y4, to))
    finally:
        ba.force_tile_config(-1)


def test_binding_rejects_mismatched_residual(ba):
    A = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 4), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((4, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        ba.gemm_bias_add_act(A, B, None, torch.zeros((4, 4), dtype=torch.bfloat16, device="cuda"), C)
    with pytest.raises(ValueError):
        ba.gemm_bias_add_act(A, B, None, torch.zeros((4, 5), dtype=torch.float32, device="cuda"), C)
    with pytest.raises(ValueError):
        ba.gemm_bias_add_act(A, B, None, None, C)
