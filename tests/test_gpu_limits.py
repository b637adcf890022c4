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
