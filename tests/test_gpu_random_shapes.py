"""GPU parity on seeded random problems.

GEMMs and convs with random shapes (ragged and aligned), operand, bias and
output types, activations, strides, padding, dilation, bias and residual,
through the automatic kernel choice: every output against the fp64 oracle
under the acceptance rule of oracle/compare.py (int32 outputs bit for bit),
and the two-kernel path (floating-point operands) bit for bit against the
fused one.  The problems are
drawn once from a fixed seed, so the set is the same on every run.
"""
import numpy as np
import pytest

import workloads as wl
from gpu_helpers import check, conv_reference, gemm_reference, run_conv, run_gemm, values_of, words_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FLOAT_TYPES = [("bf16", "bf16", "f32"), ("bf16", "f32", "bf16"), ("f16", "f16", "f16"),
               ("f16", "f32", "f32"), ("f32", "f32", "f32"), ("f32", "f16", "f32"), ("bf16", "f16", "bf16")]
ACTS = ["none", "relu", "leaky_relu", "tanh", "gelu", "sigmoid"]
CONV_ACTS = ["none", "relu", "tanh", "gelu", "sigmoid"]       # the conv takes no LeakyReLU
INTS = ("ints", -128, 127)
IBIAS = ("ints", -100000, 100000)


def _dist(ti, terms):
    # fp32 operands over reductions longer than 128: U(-0.1, 0.1), so a
    # correct fp32 sum stays well inside the fp32 rule (which takes no
    # allowance for the accumulation error)
    return ("uniform", -0.1, 0.1) if ti == "f32" and terms > 128 else ("uniform", -1.0, 1.0)


def _gemm_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        int8 = rng.random() < 0.15
        M, N, K = (int(v) for v in rng.integers(1, (400, 400, 700)))
        if rng.random() < 0.4:          # aligned sizes reach the 256x256 ping-pong kernel's checks
            N, K = 8 * ((N + 7) // 8), 16 * ((K + 15) // 16)
        res = not int8 and rng.random() < 0.3
        if int8:
            to = str(rng.choice(["i32", "f32", "bf16"]))
            act = str(rng.choice(["none", "relu"] if to == "i32" else ["relu", "leaky_relu", "tanh"]))
            bias = "i32" if rng.random() < 0.8 else None
            cases.append(wl.GemmCase(f"rg{i}", M, N, K, "i8", bias, to, act, 0.0625, INTS, INTS, IBIAS))
            continue
        ti, to, tb = FLOAT_TYPES[int(rng.integers(len(FLOAT_TYPES)))]
        act = ACTS[int(rng.integers(len(ACTS)))]
        d = _dist(ti, K)
        cases.append(wl.GemmCase(f"rg{i}", M, N, K, ti, tb if rng.random() < 0.8 else None, to, act,
                                 0.01, d, d, d, ("uniform", -0.5, 0.5) if res else None))
    return cases


def _conv_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        ti, to, tb = FLOAT_TYPES[int(rng.integers(len(FLOAT_TYPES)))]
        k = int(rng.choice([1, 1, 2, 3, 3, 3, 5, 7]))
        kh, kw = (k, k) if rng.random() < 0.8 else (k, int(rng.choice([1, 3])))
        C = int(rng.choice([3, 8, 16, 24, 40, 64, 13]))
        N = int(rng.integers(1, 3))
        sh, sw = (int(v) for v in rng.integers(1, 4, size=2))
        dh, dw = (int(v) for v in rng.integers(1, 3, size=2))
        pads = tuple(int(v) for v in rng.integers(0, 4, size=4))
        # the input must cover the dilated filter once the padding is added
        H = int(rng.integers(max(1, dh * (kh - 1) + 1 - pads[0] - pads[1]), 24))
        W = int(rng.integers(max(1, dw * (kw - 1) + 1 - pads[2] - pads[3]), 24))
        if rng.random() < 0.5:
            W += W % 2                  # even widths reach the 16-bit conv-halo kernel
        Co = int(rng.integers(1, 140))
        act = CONV_ACTS[int(rng.integers(len(CONV_ACTS)))]
        res = rng.random() < 0.3
        d = _dist(ti, C * kh * kw)
        cases.append(wl.ConvCase(f"rc{i}", N, C, H, W, Co, kh, kw, (sh, sw), pads, (dh, dw), ti,
                                 tb if rng.random() < 0.8 else None, to, act, 0.01, d, d, d,
                                 ("uniform", -0.5, 0.5) if res else None))
    return cases


GEMM_CASES = _gemm_cases(64, seed=2024)
CONV_CASES = _conv_cases(64, seed=2025)


@pytest.fixture(scope="module")
def ba():
    import conv_bias_activation_amd as m
    m.force_tile_config(-1)
    m.force_halo_variant(-1)
    return m


def _compare(y, ref, floor, case):
    if case.out_dtype == "i32":
        assert np.array_equal(words_of(y, "i32").view(np.int32).astype(np.float64), ref), case
    else:
        rep = check(values_of(y, case.out_dtype), ref, floor, case)
        assert rep["ok"], (case, rep)


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"{c.name}-{c.M}x{c.N}x{c.K}-{c.in_dtype}-{c.out_dtype}")
def test_random_gemm_vs_oracle(ba, case):
    inp = wl.gen_gemm(case, seed=7)
    ref, floor = gemm_reference(case, inp)
    y = run_gemm(case, inp)
    print(f"[{case.name}] {ba.last_tile_config()}", flush=True)
    _compare(y, ref, floor, case)
    if case.in_dtype != "i8":           # the two-kernel path takes floating-point operands only
        y2 = run_gemm(case, inp, "2k")
        assert np.array_equal(words_of(y, case.out_dtype), words_of(y2, case.out_dtype))


@pytest.mark.parametrize("case", CONV_CASES,
                         ids=lambda c: f"{c.name}-{c.N}x{c.C}x{c.H}x{c.W}-{c.Co}-{c.kh}x{c.kw}-{c.in_dtype}")
def test_random_conv_vs_oracle(ba, case):
    Ho, Wo = case.out_hw()
    assert Ho > 0 and Wo > 0, case
    inp = wl.gen_conv(case, seed=8)
    ref, floor = conv_reference(case, inp)
    y = run_conv(case, inp)
    print(f"[{case.name}] {ba.last_tile_config()}", flush=True)
    _compare(y, ref, floor, case)
    y2 = run_conv(case, inp, "2k")
    assert np.array_equal(words_of(y, case.out_dtype), words_of(y2, case.out_dtype))


FORCED = [(c, i % 8, (i // 8) % 6 - 1) for i, c in enumerate(_gemm_cases(48, seed=2026) + _conv_cases(48, seed=2027))]


@pytest.mark.parametrize("case,tile,variant", FORCED,
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_random_forced_config_vs_oracle(ba, case, tile, variant):
    # every tile configuration and conv-halo variant in turn (a forced choice
    # that does not apply to a problem falls back to one that does)
    ba.force_tile_config(tile)
    ba.force_halo_variant(variant)
    try:
        if isinstance(case, wl.GemmCase):
            inp = wl.gen_gemm(case, seed=9)
            ref, floor = gemm_reference(case, inp)
            y = run_gemm(case, inp)
        else:
            inp = wl.gen_conv(case, seed=10)
            ref, floor = conv_reference(case, inp)
            y = run_conv(case, inp)
        print(f"[{case.name} tile {tile} variant {variant}] {ba.last_tile_config()}", flush=True)
    finally:
        ba.force_tile_config(-1)
        ba.force_halo_variant(-1)
    _compare(y, ref, floor, case)
