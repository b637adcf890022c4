"""The entry points under HIP graph capture, and the per-thread launch record.

Every entry point only queues kernels on the caller's stream (no allocation,
no synchronisation, no memset), so a caller may capture it into a graph.  The
test captures each path once, then replays the graph several times with the
program's own eager work and synchronisations between the replays (new input
values written in place), and checks every replay bitwise against an eager
call of the same entry point on the same inputs.
"""
import pytest

import workloads as wl
from gpu_helpers import check, conv_reference, gemm_reference, to_dev, torch_dtype, values_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    m.force_halo_variant(-1)
    return m


def _gemm_setup(ba, M, N, K, ti, to, act, path):
    case = wl.GemmCase(f"g{M}x{N}x{K}", M, N, K, ti, "f32", to, act, 0.05,
                       ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0))
    inp = wl.gen_gemm(case, seed=21)
    A, _ = to_dev(inp["A"].reshape(M, K), ti)
    B, _ = to_dev(inp["B"].reshape(K, N), ti)
    bias, _ = to_dev(inp["bias"], "f32")
    C = torch.empty((M, N), dtype=torch_dtype(to), device="cuda")
    ws = torch.empty(max(1, ba.gemm_bias_act_workspace_size(M, N) // 4), dtype=torch.float32,
                     device="cuda")
    if path == "fused":
        call = lambda: ba.gemm_bias_act(A, B, bias, C, act, 0.05)
    else:
        call = lambda: ba.gemm_bias_act_2k(A, B, bias, C, act, 0.05, workspace=ws)
    return case, inp, A, C, call


def _conv_setup(ba, shape, ti, to, path):
    N, C_, H, W, Co, kh, kw, st, pd, dl = shape
    case = wl.ConvCase("c", N, C_, H, W, Co, kh, kw, st, pd, dl, ti, ti, to, "tanh", 0.0,
                       ("uniform", -0.5, 0.5), ("uniform", -0.5, 0.5), ("uniform", -0.5, 0.5))
    inp = wl.gen_conv(case, seed=22)
    x, _ = to_dev(inp["x"].reshape(N, C_, H, W), ti)
    w, _ = to_dev(inp["w"].reshape(Co, C_, kh, kw), ti)
    bias, _ = to_dev(inp["bias"], ti)
    Ho, Wo = case.out_hw()
    y = torch.empty((N, Co, Ho, Wo), dtype=torch_dtype(to), device="cuda")
    n = ba.conv2d_bias_act_workspace_size(N, C_, H, W, Co, kh, kw, st, pd, dl)
    ws = torch.empty(max(1, n // 4), dtype=torch.float32, device="cuda")
    if path == "fused":
        call = lambda: ba.conv2d_bias_act(x, w, bias, y, st, pd, dl, "tanh")
    else:
        call = lambda: ba.conv2d_bias_act_2k(x, w, bias, y, st, pd, dl, "tanh", workspace=ws)
    return x, y, call


def _replays_match_eager(call, inp_t, out_t, replays=3):
    """Capture `call`, then per replay: write new input values eagerly, replay,
    and compare with an eager call on the same values."""
    call()                                       # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(5)
    base = inp_t.clone()
    for r in range(replays):
        scale = 1.0 - 0.25 * r
        inp_t.copy_(base * scale + 0.01 * r * torch.rand(base.shape, generator=gen, device="cuda",
                                                         dtype=torch.float32).to(base.dtype))
        out_t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_t.clone()
        out_t.zero_()
        call()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if got.element_size() == 2 else got.view(torch.int32),
                           out_t.view(torch.int16) if out_t.element_size() == 2
                           else out_t.view(torch.int32)), f"replay {r}"
    return True


@pytest.mark.parametrize("path", ["fused", "2k"])
@pytest.mark.parametrize("shape", [(1024, 640, 256, "f16", "f32", "leaky_relu"),
                                   (512, 768, 512, "bf16", "bf16", "relu"),
                                   (200, 136, 72, "f32", "f32", "tanh")],
                         ids=["allk", "pingpong", "fp32"])
def test_gemm_graph_replays_match_eager(ba, shape, path):
    M, N, K, ti, to, act = shape
    case, inp, A, C, call = _gemm_setup(ba, M, N, K, ti, to, act, path)
    # the ping-pong kernel is picked on its own only for grids of 256+ tiles
    ba.force_tile_config(6 if ti == "bf16" else -1)
    try:
        assert _replays_match_eager(call, A, C)
    finally:
        ba.force_tile_config(-1)
    # and the replays computed the method, not just the same bits: the last
    # input written was base * 0.5 + noise; check the first replay's inputs
    A.copy_(to_dev(inp["A"].reshape(M, K), ti)[0])
    call()
    torch.cuda.synchronize()
    ref, floor = gemm_reference(case, inp)
    assert check(values_of(C, to), ref, floor, case)["ok"]


@pytest.mark.parametrize("path", ["fused", "2k"])
@pytest.mark.parametrize("shape", [
    ((4, 64, 28, 28, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)), "f16", "f16"),
    ((2, 3, 64, 64, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)), "f32", "f32"),
    ((2, 32, 14, 14, 48, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)), "f32", "f32")],
    ids=["halo16", "halo32", "generic"])
def test_conv_graph_replays_match_eager(ba, shape, path):
    geom, ti, to = shape
    x, y, call = _conv_setup(ba, geom, ti, to, path)
    assert _replays_match_eager(call, x, y)


def test_last_tile_config_names_the_kernel(ba):
    import conv_bias_activation_amd as m
    cases = [((1024, 640, 256, "f16", "f32", "leaky_relu"), "gemm 64x64/2x2 all-k"),
             ((1024, 640, 1024, "f16", "f32", "leaky_relu"), "gemm 64x64/2x2"),
             ((512, 768, 512, "bf16", "bf16", "relu"), "gemm 256x256/2x4 ping-pong")]
    for (M, N, K, ti, to, act), want in cases:
        _, _, _, C, call = _gemm_setup(ba, M, N, K, ti, to, act, "fused")
        ba.force_tile_config(6 if want.endswith("ping-pong") else -1)
        try:
            call()
        finally:
            ba.force_tile_config(-1)
        torch.cuda.synchronize()
        got = m.last_tile_config()
        assert got == want, (got, want)
    x, y, call = _conv_setup(ba, (4, 64, 28, 28, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)), "f16",
                             "f16", "fused")
    call()
    torch.cuda.synchronize()
    assert m.last_tile_config().startswith("conv-halo 9 taps, 64 co"), m.last_tile_config()
    x, y, call = _conv_setup(ba, (2, 3, 64, 64, 64, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)), "f32",
                             "f32", "2k")
    call()
    torch.cuda.synchronize()
    assert m.last_tile_config().startswith("two-kernel: conv-halo fp32"), m.last_tile_config()


def test_tuned_path_choice_and_auto_calls(ba):
    # "measure first": tune both paths on the caller's buffers, record the
    # faster, and let the auto entry point follow it; the bits are those of
    # the fused call either way
    import conv_bias_activation_amd as m
    for (M, N, K, ti, to, act) in ((1024, 640, 256, "f16", "f32", "leaky_relu"),
                                   (512, 768, 512, "bf16", "bf16", "relu")):
        case, inp, _, C, call = _gemm_setup(ba, M, N, K, ti, to, act, "fused")
        call()
        torch.cuda.synchronize()
        want = C.clone()
        ws = torch.empty(m.gemm_bias_act_workspace_size(M, N) // 4, dtype=torch.float32,
                         device="cuda")
        dt = m.dtypes_code(ti, ti, "f32", to)
        assert m.gemm_path(M, N, K, dt, act) == "fused"          # nothing recorded yet
        A, B, bias, C2 = _gemm_tensors(case, inp)
        got = m.tune_gemm(A, B, bias, C2, act=act, alpha=0.05, workspace=ws, reps=5)
        assert got in ("fused", "2k")
        assert m.gemm_path(M, N, K, dt, act) == got
        C2.zero_()
        m.gemm_bias_act_auto(A, B, bias, C2, act, 0.05, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(C2), _bits(want))
    # conv: a problem without bias and with zero weights, y = tanh(0) = 0
    x = torch.randn((4, 64, 28, 28), device="cuda").half()
    w = torch.zeros((64, 64, 3, 3), dtype=torch.float16, device="cuda")
    y = torch.empty((4, 64, 28, 28), dtype=torch.float16, device="cuda")
    n = m.conv2d_bias_act_workspace_size(4, 64, 28, 28, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1))
    ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    got = m.tune_conv(x, w, None, y, (1, 1), (1, 1, 1, 1), (1, 1), "tanh", workspace=ws, reps=5)
    assert got in ("fused", "2k")
    dt = m.dtypes_code("f16", "f16", None, "f16")
    assert m.conv_path(4, 64, 28, 28, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), dt, "tanh") == got
    y.fill_(1.0)
    m.conv2d_bias_act_auto(x, w, None, y, (1, 1), (1, 1, 1, 1), (1, 1), "tanh", workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _gemm_tensors(case, inp):
    A, _ = to_dev(inp["A"].reshape(case.M, case.K), case.in_dtype)
    B, _ = to_dev(inp["B"].reshape(case.K, case.N), case.in_dtype)
    bias, _ = to_dev(inp["bias"], "f32")
    C = torch.empty((case.M, case.N), dtype=torch_dtype(case.out_dtype), device="cuda")
    return A, B, bias, C


def test_recorded_two_kernel_choice_matches_oracle(ba):
    # A recorded two-kernel choice: the auto entry points take the two-kernel
    # branch (and report it), and the result matches the oracle and the fused
    # call's bits; without a workspace they fall back to the fused call.
    import conv_bias_activation_amd as m
    M, N, K, ti, to, act = 520, 384, 640, "bf16", "bf16", "gelu"
    case, inp, _, C, call = _gemm_setup(ba, M, N, K, ti, to, act, "fused")
    call()
    torch.cuda.synchronize()
    want = C.clone()
    A, B, bias, C2 = _gemm_tensors(case, inp)
    ws = torch.empty(m.gemm_bias_act_workspace_size(M, N) // 4, dtype=torch.float32, device="cuda")
    dt = m.dtypes_code(ti, ti, "f32", to)
    m.set_gemm_path(M, N, K, dt, act, "2k")
    try:
        assert m.gemm_path(M, N, K, dt, act) == "2k"
        m.gemm_bias_act_auto(A, B, bias, C2, act, 0.05, workspace=ws)
        torch.cuda.synchronize()
        assert m.last_tile_config().startswith("two-kernel: "), m.last_tile_config()
        ref, acc = gemm_reference(case, inp)
        rep = check(values_of(C2, to), ref, acc, case)
        assert rep["ok"], rep
        assert torch.equal(_bits(C2), _bits(want))
        m.gemm_bias_act_auto(A, B, bias, C2, act, 0.05)
        torch.cuda.synchronize()
        assert not m.last_tile_config().startswith("two-kernel"), m.last_tile_config()
    finally:
        m.set_gemm_path(M, N, K, dt, act, None)
    # conv: fp16 3x3 with a bias, recorded two-kernel, against the oracle
    geom = (2, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1))
    Nb, C_, H, W, Co, kh, kw, st, pd, dl = geom
    ccase = wl.ConvCase("c", Nb, C_, H, W, Co, kh, kw, st, pd, dl, "f16", "f16", "f16", "tanh", 0.0,
                        ("uniform", -0.5, 0.5), ("uniform", -0.5, 0.5), ("uniform", -0.5, 0.5))
    cinp = wl.gen_conv(ccase, seed=22)
    x, y, ccall = _conv_setup(ba, geom, "f16", "f16", "fused")
    ccall()
    torch.cuda.synchronize()
    cwant = y.clone()
    w, _ = to_dev(cinp["w"].reshape(Co, C_, kh, kw), "f16")
    cb, _ = to_dev(cinp["bias"], "f16")
    y2 = torch.empty_like(y)
    n = m.conv2d_bias_act_workspace_size(*geom)
    cws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    cdt = m.dtypes_code("f16", "f16", "f16", "f16")
    m.set_conv_path(*geom, cdt, "tanh", "2k")
    try:
        m.conv2d_bias_act_auto(x, w, cb, y2, st, pd, dl, "tanh", workspace=cws)
        torch.cuda.synchronize()
        assert m.last_tile_config().startswith("two-kernel: conv-halo"), m.last_tile_config()
        ref, acc = conv_reference(ccase, cinp)
        rep = check(values_of(y2, "f16"), ref, acc, ccase)
        assert rep["ok"], rep
        assert torch.equal(_bits(y2), _bits(cwant))
    finally:
        m.set_conv_path(*geom, cdt, "tanh", None)


def test_static_rule_takes_two_kernels_for_a_misaligned_output(ba):
    # Nothing recorded, C two bytes off its allocation: the fused call loses
    # the ping-pong main loop (its epilogue needs 4-element aligned rows),
    # kernel 1 of the two-kernel path keeps it on the aligned workspace, so
    # the static rule takes the two-kernel branch.  Both paths match the
    # oracle on every output.
    import conv_bias_activation_amd as m
    M, N, K = 4096, 4096, 256
    case = wl.GemmCase("misaligned", M, N, K, "bf16", "f32", "bf16", "relu", 0.0,
                       ("normal", 1.0 / 16.0), ("normal", 1.0 / 16.0), ("uniform", -0.1, 0.1))
    inp = wl.gen_gemm(case, seed=31)
    A, _ = to_dev(inp["A"].reshape(M, K), "bf16")
    B, _ = to_dev(inp["B"].reshape(K, N), "bf16")
    bias, _ = to_dev(inp["bias"], "f32")
    buf = torch.empty(M * N + 1, dtype=torch.bfloat16, device="cuda")
    C = buf[1:].view(M, N)
    ws = torch.empty(M * N, dtype=torch.float32, device="cuda")
    dt = m.dtypes_code("bf16", "bf16", "f32", "bf16")
    assert m.gemm_path(M, N, K, dt, "relu") == "fused"           # nothing recorded
    assert m.gemm_static_path(A, B, bias, C, "relu", workspace=ws) == "2k"
    assert m.gemm_static_path(A, B, bias, C, "relu") == "fused"  # no workspace given
    ref, acc = gemm_reference(case, inp)
    m.gemm_bias_act_auto(A, B, bias, C, "relu", workspace=ws)
    torch.cuda.synchronize()
    assert m.last_tile_config() == "two-kernel: gemm 256x256/2x4 ping-pong", m.last_tile_config()
    rep = check(values_of(C, "bf16"), ref, acc, case)
    assert rep["ok"], rep
    two = C.clone()
    m.gemm_bias_act(A, B, bias, C, "relu")
    torch.cuda.synchronize()
    assert "ping-pong" not in m.last_tile_config(), m.last_tile_config()
    rep = check(values_of(C, "bf16"), ref, acc, case)
    assert rep["ok"], rep
    # both main loops sum the same 16-wide k-steps in ascending order from the bias
    assert torch.equal(_bits(C), _bits(two))
