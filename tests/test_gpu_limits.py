"""GPU parity at the size limit.

The library takes tensors below 2^31 bytes and addresses them with 32-bit
byte offsets (masked-off accesses use the offset 2^31).  These problems put
the output within half a megabyte of that limit, through the 256x256
ping-pong GEMM, the 16-bit conv-halo kernel and the generic fp32 conv, and
check sampled outputs against the oracle: random ones plus the final 2048
elements of the buffer and the first and last column of the last 64 rows.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import check, conv_reference, gemm_reference, to_dev, torch_dtype, values_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LIMIT = 1 << 31


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    m.force_halo_variant(-1)
    return m


def _idx(rows, cols, seed):
    rng = np.random.default_rng(seed)
    total = rows * cols
    last = rows - 1 - np.arange(64)
    pick = [rng.integers(0, total, 4000), np.arange(total - 2048, total), last * cols,
            last * cols + cols - 1, np.arange(64)]
    return np.unique(np.concatenate(pick)).astype(np.int64)


def _gather(t, idx):
    flat = t.reshape(-1)
    return flat[torch.from_numpy(idx).to(flat.device)]


@pytest.mark.parametrize("to,M", [("f32", 16384), ("bf16", 32768)])
def test_gemm_output_just_under_2gib(ba, to, M):
    N, K = 32760, 24
    case = wl.GemmCase(f"lim_{to}", M, N, K, "bf16", "f32", to, "relu")
    out_bytes = M * N * (4 if to == "f32" else 2)
    assert LIMIT - (1 << 20) < out_bytes < LIMIT
    inp = wl.gen_gemm(case, seed=41)
    A, _ = to_dev(inp["A"].reshape(M, K), "bf16")
    B, _ = to_dev(inp["B"].reshape(K, N), "bf16")
    bias, _ = to_dev(inp["bias"], "f32")
    C = torch.empty((M, N), dtype=torch_dtype(to), device="cuda")
    try:
        ba.gemm_bias_act(A, B, bias, C, "relu", 0.0)
        torch.cuda.synchronize()
        assert "ping-pong" in ba.last_tile_config()
        idx = _idx(M, N, 42)
        y = values_of(_gather(C, idx), to)
    finally:
        del C
        torch.cuda.empty_cache()
    ref, floor = gemm_reference(case, inp, idx=idx)
    rep = check(y, ref, floor, case)
    assert rep["ok"], rep


@pytest.mark.parametrize("ti,to,kh,N,C", [("f16", "f16", 3, 16, 16), ("f32", "f32", 1, 8, 32)])
def test_conv_output_just_under_2gib(ba, ti, to, kh, N, C):
    H = W = 512
    Co = 255
    pad = kh // 2
    case = wl.ConvCase(f"lim_{ti}", N, C, H, W, Co, kh, kh, (1, 1), (pad,) * 4, (1, 1), ti, ti, to, "tanh")
    Ho, Wo = case.out_hw()
    out_bytes = N * Co * Ho * Wo * (4 if to == "f32" else 2)
    assert LIMIT - (16 << 20) < out_bytes < LIMIT
    inp = wl.gen_conv(case, seed=43)
    x, _ = to_dev(inp["x"].reshape(N, C, H, W), ti)
    w, _ = to_dev(inp["w"].reshape(Co, C, kh, kh), ti)
    bias, _ = to_dev(inp["bias"], ti)
    y = torch.empty((N, Co, Ho, Wo), dtype=torch_dtype(to), device="cuda")
    try:
        ba.conv2d_bias_act(x, w, bias, y, (1, 1), (pad,) * 4, (1, 1), "tanh")
        torch.cuda.synchronize()
        kernel = ba.last_tile_config()
        assert kernel.startswith("conv-halo 9" if ti == "f16" else "conv "), kernel
        idx = _idx(N * Co, Ho * Wo, 44)
        yv = values_of(_gather(y, idx), to)
    finally:
        del y
        torch.cuda.empty_cache()
    ref, floor = conv_reference(case, inp, idx=idx)
    rep = check(yv, ref, floor, case)
    assert rep["ok"], rep


def _tiled(words, reps):
    # a seeded block repeated along the leading dimension: the operand's
    # last rows are known without drawing 2 GiB of random numbers
    return np.concatenate([words] * reps, axis=0)


def test_gemm_operand_a_just_under_2gib(ba):
    # A is 65536 x 16376 bf16 (2^31 - 1 MiB bytes): the rows that read its
    # tail (the last 64 output rows) and its head, against the oracle
    M, N, K = 65536, 64, 16376
    assert LIMIT - (2 << 20) < M * K * 2 < LIMIT
    blk = wl.GemmCase("lim_a_blk", 256, N, K, "bf16", "f32", "f32", "relu")
    inp = wl.gen_gemm(blk, seed=45)
    a_words = inp["A"].reshape(256, K)
    A, _ = to_dev(_tiled(a_words, M // 256), "bf16")
    B, _ = to_dev(inp["B"].reshape(K, N), "bf16")
    bias, _ = to_dev(inp["bias"], "f32")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    try:
        ba.gemm_bias_act(A, B, bias, C, "relu", 0.0)
        torch.cuda.synchronize()
        head = values_of(C[:64], "f32")
        tail = values_of(C[M - 64:], "f32")
    finally:
        del A, C
        torch.cuda.empty_cache()
    # rows 0..63 and M-64..M-1 of A are block rows 0..63 and 192..255
    for rows, y in ((slice(0, 64), head), (slice(192, 256), tail)):
        sub = wl.GemmCase("lim_a_rows", 64, N, K, "bf16", "f32", "f32", "relu")
        ref, floor = gemm_reference(sub, dict(inp, A=a_words[rows]))
        rep = check(y, ref, floor, sub)
        assert rep["ok"], rep


def test_conv_input_just_under_2gib(ba):
    # x is 63 x 64 x 512 x 512 fp16 (2^31 - 32 MiB bytes) on the conv-halo
    # kernel: the first and the last image (the tail of x) against the oracle
    N, C, H, W, Co = 63, 64, 512, 512, 8
    assert LIMIT - (64 << 20) < N * C * H * W * 2 < LIMIT
    one = wl.ConvCase("lim_x_img", 1, C, H, W, Co, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), "f16", "f16", "f16", "tanh")
    inp = wl.gen_conv(one, seed=46)
    x, _ = to_dev(_tiled(inp["x"].reshape(1, C, H, W), N), "f16")
    w, _ = to_dev(inp["w"].reshape(Co, C, 3, 3), "f16")
    bias, _ = to_dev(inp["bias"], "f16")
    y = torch.empty((N, Co, H, W), dtype=torch.float16, device="cuda")
    try:
        ba.conv2d_bias_act(x, w, bias, y, (1, 1), (1, 1, 1, 1), (1, 1), "tanh")
        torch.cuda.synchronize()
        assert ba.last_tile_config().startswith("conv-halo 9"), ba.last_tile_config()
        first = values_of(y[0], "f16")
        last = values_of(y[N - 1], "f16")
    finally:
        del x, y
        torch.cuda.empty_cache()
    ref, floor = conv_reference(one, inp)
    for yv in (first, last):
        rep = check(yv, ref, floor, one)
        assert rep["ok"], rep
