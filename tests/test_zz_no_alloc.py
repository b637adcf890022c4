"""The two-kernel GEMM entry point that allocates nothing
(gemm_bias_act_2k_noalloc: its fp32 workspace is a fixed device array in the
library), called through the C ABI and checked against gemm_bias_act_2k with a
caller workspace, bit for bit, and against the oracle, on two calls in a row,
the second with a smaller problem (the array keeps the first call's
contents)."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from gpu_helpers import check, gemm_reference, to_dev, torch_dtype, values_of, words_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _call_both(L, case, inp):
    A, _ = to_dev(inp["A"].reshape(case.M, case.K), case.in_dtype)
    B, _ = to_dev(inp["B"].reshape(case.K, case.N), case.in_dtype)
    bias, _ = to_dev(inp["bias"], case.bias_dtype)
    C_ref = torch.empty((case.M, case.N), dtype=torch_dtype(case.out_dtype), device="cuda")
    C_new = torch.full((case.M, case.N), float("nan"), dtype=torch_dtype(case.out_dtype),
                       device="cuda")
    ws = torch.empty(case.M * case.N, dtype=torch.float32, device="cuda")
    dt = (wl.DTYPE_CODES[case.in_dtype] | (wl.DTYPE_CODES[case.in_dtype] << 8)
          | (wl.DTYPE_CODES[case.bias_dtype] << 16) | (wl.DTYPE_CODES[case.out_dtype] << 24))
    act = wl.ACT_CODES[case.act]
    alpha = ctypes.c_float(np.float32(case.alpha))
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.gemm_bias_act_2k(p(A), p(B), p(bias), p(C_ref), case.M, case.N, case.K, dt, act, alpha,
                            p(ws), ws.numel() * 4, s)
    assert rc == 0, rc
    rc = L.gemm_bias_act_2k_noalloc(p(A), p(B), p(bias), p(C_new), case.M, case.N, case.K, dt, act,
                                    alpha, s)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return C_ref, C_new


def test_noalloc_two_calls_match_the_workspace_entry_point():
    import conv_bias_activation_amd as ba
    L = ba.lib
    U = ("uniform", -1.0, 1.0)
    # the second problem is smaller than the first: its outputs must not pick
    # up anything the first call left in the array
    for j, (M, N, K, ti, to, act) in enumerate(((2048, 2048, 512, "bf16", "bf16", "gelu"),
                                                (300, 520, 200, "f16", "f32", "leaky_relu"))):
        case = wl.GemmCase(f"noalloc{j}", M, N, K, ti, "f32", to, act, 0.05, U, U, U)
        inp = wl.gen_gemm(case, seed=140 + j)
        C_ref, C_new = _call_both(L, case, inp)
        assert ba.last_tile_config().startswith("two-kernel: "), ba.last_tile_config()
        assert np.array_equal(words_of(C_new, to), words_of(C_ref, to)), (M, N, K)
        ref, acc = gemm_reference(case, inp)
        rep = check(values_of(C_new, to), ref, acc, case)
        assert rep["ok"], rep
    # past the array's size: refused, nothing launched
    A = torch.zeros((4096, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 4097), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((4096, 4097), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        ba.gemm_bias_act_2k_noalloc(A, B, None, C, "relu")
