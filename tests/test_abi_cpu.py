"""C-ABI checks that need no GPU: the library loads, exports every function
that include/biasact.h declares, and rejects invalid arguments before any HIP
call (so every error path is reachable here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "biasact.h")

ba = pytest.importorskip("conv_bias_activation_amd")
L = ba.lib

F32, F16, BF16 = 0, 1, 2


def _dt(a, b, bias, out):
    return a | (b << 8) | (bias << 16) | (out << 24)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("gemm_bias_act", "conv2d_bias_act", "gemm_bias_act_2k", "conv2d_bias_act_2k",
                 "gemm_bias_act_workspace_size", "conv2d_bias_act_workspace_size",
                 "biasact_status_string", "biasact_force_tile_config", "gemm_bias_add_act",
                 "conv2d_bias_add_act", "gemm_bias_add_act_2k", "conv2d_bias_add_act_2k"):
        assert must in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(L, name), f"libbiasact.so does not export {name}"


def test_status_strings():
    assert L.biasact_status_string(0) == b"ok"
    for s in (1, 2, 3, 99):
        assert len(L.biasact_status_string(s)) > 0


def test_last_tile_config_before_any_launch():
    buf = ctypes.create_string_buffer(64)
    assert L.biasact_last_tile_config(buf, 64) == 0 and buf.value == b"none"
    assert L.biasact_last_tile_config(None, 64) == 1
    assert L.biasact_last_tile_config(buf, 0) == 1
    small = ctypes.create_string_buffer(3)
    assert L.biasact_last_tile_config(small, 3) == 0 and small.value == b"no"


def test_last_hip_error_starts_clear():
    # nothing has failed a launch on this thread: hipSuccess and a fixed text
    assert L.biasact_last_hip_error() == 0
    assert L.biasact_last_hip_error_string() == b"no HIP error"


def test_one_hip_runtime_beside_torch():
    # importing the package before torch must still leave one libamdhip64 in
    # the process (the library binds to torch's instance)
    import subprocess
    import sys
    code = ("import conv_bias_activation_amd, torch\n"
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(paths)); print(sorted(paths))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.splitlines()[0] == "1", r.stdout


def test_tile_table_introspection():
    n = ba.num_tile_configs()
    assert n >= 5
    names = [ba.tile_config_name(i) for i in range(n)]
    assert names[0] == "256x256/2x2"
    assert len(set(names)) == n
    with pytest.raises(ValueError):
        ba.tile_config_name(n)
    assert 0 <= ba.gemm_tile_config(4096, 4096, 4096, _dt(BF16, BF16, F32, BF16)) < n
    assert ba.gemm_tile_config(4096, 4096, 4096, _dt(BF16, BF16, F32, BF16)) == 6   # ping-pong kernel
    assert ba.gemm_tile_config(4096, 4096, 4096, _dt(F32, F32, F32, F32)) == 0
    ba.force_tile_config(3)
    try:
        assert ba.gemm_tile_config(4096, 4096, 4096, 0) == 3
    finally:
        ba.force_tile_config(-1)
    with pytest.raises(ValueError):
        ba.force_tile_config(n)


def test_conv_tile_balances_the_busiest_cu():
    f32 = _dt(F32, F32, F32, F32)
    # 16 x 512 x 28 x 28 output (the 1x1 stride-2 conv of 16 x 256 x 56 x 56):
    # 128x128 tiles make 392 workgroups, two on some CUs (32768 outputs);
    # 64x64 tiles make 1568, seven on some CUs (28672): an eighth less
    assert ba.tile_config_name(ba.conv_tile_config(16, 512, 28, 28, 256, f32)) == "64x64/2x2"
    # 16 x 512 x 32 x 32: 128x256 gives 256 workgroups, one per CU; every
    # smaller tile gives the busiest CU the same 32768 outputs
    assert ba.tile_config_name(ba.conv_tile_config(16, 512, 32, 32, 256, f32)) == "128x256/2x2"
    # Co <= 64: 8 x 64 x 56 x 56 positions, 64x64 tiles (392 workgroups) as before
    assert ba.tile_config_name(ba.conv_tile_config(8, 64, 56, 56, 576, f32)) == "64x64/2x2"


def test_halo_variant_override_range():
    for v in (-1, 0, 1, 2, 3, 4):
        ba.force_halo_variant(v)
    ba.force_halo_variant(-1)
    for v in (-2, 5):
        with pytest.raises(ValueError):
            ba.force_halo_variant(v)


def test_workspace_sizes():
    assert L.gemm_bias_act_workspace_size(4096, 4096) == 4096 * 4096 * 4
    assert L.gemm_bias_act_workspace_size(-1, 3) == 0
    i32 = lambda *v: (ctypes.c_int32 * len(v))(*v)
    n = L.conv2d_bias_act_workspace_size(8, 64, 56, 56, 64, 3, 3, i32(1, 1), i32(1, 1, 1, 1), i32(1, 1))
    assert n == 8 * 64 * 56 * 56 * 4
    assert L.conv2d_bias_act_workspace_size(1, 1, 2, 2, 1, 5, 5, i32(1, 1), i32(0, 0, 0, 0), i32(1, 1)) == 0


# Fake (never dereferenced) device pointers: every call below fails validation
# before anything is launched.
P = ctypes.c_void_p(0x1000)
NUL = ctypes.c_void_p(0)


def gemm(A=P, B=P, bias=P, C=P, M=4, N=4, K=4, dt=_dt(F16, F16, F32, F32), act=2, alpha=0.1):
    return L.gemm_bias_act(A, B, bias, C, M, N, K, dt, act, alpha, NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(A=NUL), 1), (dict(B=NUL), 1), (dict(C=NUL), 1),
    (dict(M=-1), 1), (dict(N=-2), 1), (dict(K=-3), 1),
    (dict(act=6), 1), (dict(act=-1), 1),
    (dict(dt=_dt(F16, BF16, F32, F32)), 2),           # A and B differ
    (dict(dt=_dt(3, 3, F32, F32)), 2),                # unknown type
    (dict(dt=_dt(F16, F16, BF16, F32)), 2),           # bias neither f32 nor the input type
    (dict(dt=_dt(F16, F16, F32, 7)), 2),              # unknown output type
    (dict(M=1 << 20, K=1 << 11, dt=_dt(F32, F32, F32, F32)), 2),   # A is 2^33 bytes
])
def test_gemm_rejects(kw, code):
    assert gemm(**kw) == code


def test_gemm_empty_problem_is_ok_without_launch():
    assert gemm(M=0) == 0 and gemm(N=0) == 0


def test_residual_entry_points_validate():
    dt = _dt(BF16, BF16, F32, BF16)
    # a null residual with a non-empty output is invalid; empty outputs launch nothing
    assert L.gemm_bias_add_act(P, P, P, NUL, P, 4, 4, 4, dt, 1, 0.0, NUL) == 1
    assert L.gemm_bias_add_act(P, P, P, NUL, P, 0, 4, 4, dt, 1, 0.0, NUL) == 0
    assert L.gemm_bias_add_act_2k(P, P, P, NUL, P, 4, 4, 4, dt, 1, 0.0, P, 64, NUL) == 1
    # the other checks are those of the plain entry point
    assert L.gemm_bias_add_act(P, P, P, P, P, 4, 4, 4, dt, 6, 0.0, NUL) == 1
    assert L.gemm_bias_add_act(P, P, P, P, P, 4, 4, 4, _dt(F16, BF16, F32, F32), 1, 0.0, NUL) == 2
    c = (ctypes.c_int32 * 2)(1, 1), (ctypes.c_int32 * 4)(1, 1, 1, 1), (ctypes.c_int32 * 2)(1, 1)
    cdt = _dt(F16, F16, F16, F16)
    assert L.conv2d_bias_add_act(P, P, P, NUL, P, 1, 3, 8, 8, 4, 3, 3, *c, cdt, 3, NUL) == 1
    assert L.conv2d_bias_add_act(P, P, P, P, P, 1, 3, 8, 8, 4, 3, 3, *c, cdt, 2, NUL) == 2
    assert L.conv2d_bias_add_act_2k(P, P, P, NUL, P, 1, 3, 8, 8, 4, 3, 3, *c, cdt, 3, P, 4096,
                                    NUL) == 1


I8, I32 = 3, 4


def test_int8_type_rules():
    dt = _dt(I8, I8, I32, I32)
    # valid int8 problems fail only later, at launch, on this machine; the
    # planner's rejections come first and need no GPU
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, _dt(I8, I8, F32, F32), 1, 0.0, NUL) == 2  # bias must be int32
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, _dt(I8, F16, I32, I32), 1, 0.0, NUL) == 2
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, _dt(F16, F16, I32, F32), 1, 0.0, NUL) == 2  # int32 bias needs int8
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, _dt(F16, F16, F32, I32), 1, 0.0, NUL) == 2  # int32 out needs int8
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, dt, 3, 0.0, NUL) == 2     # tanh into int32
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 4, dt, 2, 0.1, NUL) == 2     # leaky into int32
    assert L.gemm_bias_act(P, P, P, P, 4, 4, 131072, dt, 1, 0.0, NUL) == 2   # K past the int32-safe bound
    assert L.gemm_bias_act(P, P, P, P, 0, 4, 4, dt, 1, 0.0, NUL) == 0     # empty: nothing launched
    # the fused GEMM only
    assert L.gemm_bias_act_2k(P, P, P, P, 4, 4, 4, dt, 1, 0.0, P, 64, NUL) == 2
    assert L.gemm_bias_add_act(P, P, P, P, P, 4, 4, 4, dt, 1, 0.0, NUL) == 2
    c = (ctypes.c_int32 * 2)(1, 1), (ctypes.c_int32 * 4)(1, 1, 1, 1), (ctypes.c_int32 * 2)(1, 1)
    assert L.conv2d_bias_act(P, P, P, P, 1, 3, 8, 8, 4, 3, 3, *c, _dt(I8, I8, I32, I32), 1, NUL) == 2
    # int8 takes the 256x256 ping-pong kernel where K and N are multiples of 16
    # and its grid covers every CU; otherwise a tiled kernel, never the tiled 256x256
    assert ba.gemm_tile_config(4096, 4096, 4096, dt) == 6
    assert ba.gemm_tile_config(4096, 4096, 4104, dt) == 1
    assert ba.gemm_tile_config(1024, 1024, 1024, dt) not in (0, 6)


def test_path_selection_defaults_to_fused():
    # nothing tuned: the static rule is the fused path for every problem
    for M, N, K in ((1, 1, 1), (4096, 4096, 4096), (1024, 640, 256)):
        assert L.biasact_gemm_path(M, N, K, _dt(BF16, BF16, F32, BF16), 1) == 0
    c = (ctypes.c_int32 * 2)(1, 1), (ctypes.c_int32 * 4)(1, 1, 1, 1), (ctypes.c_int32 * 2)(1, 1)
    assert L.biasact_conv_path(8, 64, 56, 56, 64, 3, 3, *c, _dt(F16, F16, F16, F16), 3) == 0
    assert L.biasact_conv_path(8, 64, 56, 56, 64, 3, 3, None, c[1], c[2], 0, 3) == -1
    # tuning validates before any launch
    path = ctypes.c_int(-1)
    assert L.biasact_tune_gemm(P, P, P, P, 4, 4, 4, _dt(BF16, BF16, F32, BF16), 1, 0.0, NUL, 0, 5,
                               NUL, None) == 1
    assert L.biasact_tune_gemm(P, P, P, P, 4, 4, 4, _dt(BF16, BF16, F32, BF16), 9, 0.0, NUL, 0, 5,
                               NUL, ctypes.byref(path)) == 1
    assert L.gemm_bias_act_auto(NUL, P, P, P, 4, 4, 4, _dt(BF16, BF16, F32, BF16), 1, 0.0, NUL, 0,
                                NUL) == 1


def test_gemm_2k_workspace_checks():
    dt = _dt(BF16, BF16, F32, BF16)
    assert L.gemm_bias_act_2k(P, P, P, P, 4, 4, 4, dt, 1, 0.0, NUL, 64, NUL) == 1
    assert L.gemm_bias_act_2k(P, P, P, P, 4, 4, 4, dt, 1, 0.0, P, 63, NUL) == 1
    assert L.gemm_bias_act_2k(P, P, P, P, 4, 4, 4, dt, 9, 0.0, P, 64, NUL) == 1


def _i32(*v):
    return (ctypes.c_int32 * len(v))(*v)


def conv(x=P, w=P, bias=P, y=P, N=1, C=3, H=8, W=8, Co=4, kh=3, kw=3, st=(1, 1), pd=(1, 1, 1, 1),
         dl=(1, 1), dt=_dt(F16, F16, F16, F16), act=3):
    return L.conv2d_bias_act(x, w, bias, y, N, C, H, W, Co, kh, kw, _i32(*st), _i32(*pd), _i32(*dl),
                             dt, act, NUL)


@pytest.mark.parametrize("kw,code", [
    (dict(x=NUL), 1), (dict(w=NUL), 1), (dict(y=NUL), 1),
    (dict(N=-1), 1), (dict(C=0), 1), (dict(H=0), 1), (dict(Co=0), 1), (dict(kh=0), 1),
    (dict(st=(0, 1)), 1), (dict(st=(1, -2)), 1), (dict(dl=(0, 1)), 1),
    (dict(pd=(-1, 0, 0, 0)), 1), (dict(pd=(0, 0, 0, -1)), 1),
    (dict(H=2, W=2, pd=(0, 0, 0, 0)), 1),             # 3x3 filter on a 2x2 image: empty output
    (dict(act=7), 1),
    (dict(act=2), 2),                                 # no alpha on the conv entry point
    (dict(dt=_dt(F16, F32, F16, F16)), 2),
    (dict(N=64, C=1024, H=256, W=256, dt=_dt(F32, F32, F32, F32)), 2),   # x >= 2^31 bytes
])
def test_conv_rejects(kw, code):
    assert conv(**kw) == code


def test_conv_empty_batch_is_ok_without_launch():
    assert conv(N=0) == 0


def test_null_attribute_arrays_rejected():
    c_null = ctypes.POINTER(ctypes.c_int32)()
    rc = L.conv2d_bias_act(P, P, P, P, 1, 3, 8, 8, 4, 3, 3, c_null, _i32(1, 1, 1, 1), _i32(1, 1),
                           _dt(F16, F16, F16, F16), 3, NUL)
    assert rc == 1


def test_python_binding_raises_value_error_on_bad_names():
    with pytest.raises(ValueError):
        ba.dtypes_code("f64", "f64", None, "f32")
    with pytest.raises(ValueError):
        ba._binding._act("swish")
    assert ba.conv_out_hw(224, 224, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)) == (112, 112)
    assert ba.conv_out_hw(2, 2, 3, 3, (1, 1), (0, 0, 0, 0), (1, 1)) is None


def test_conv_out_dims_query():
    # the library's one output-size rule (no launch): floor((H + pt + pb -
    # dh*(kh-1) - 1) / sh) + 1, likewise for W
    ho, wo = ctypes.c_int64(-1), ctypes.c_int64(-1)
    q = lambda H, W, kh, kw, st, pd, dl: L.conv2d_bias_act_out_dims(
        H, W, kh, kw, _i32(*st), _i32(*pd), _i32(*dl), ctypes.byref(ho), ctypes.byref(wo))
    assert q(224, 224, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1)) == 0 and (ho.value, wo.value) == (112, 112)
    assert q(28, 28, 3, 3, (1, 1), (2, 2, 2, 2), (2, 2)) == 0 and (ho.value, wo.value) == (28, 28)
    assert q(9, 7, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2)) == 0 and (ho.value, wo.value) == (4, 8)
    assert q(56, 56, 1, 1, (2, 2), (0, 0, 0, 0), (1, 1)) == 0 and (ho.value, wo.value) == (28, 28)
    assert q(2, 2, 3, 3, (1, 1), (0, 0, 0, 0), (1, 1)) == 1          # empty output
    assert q(8, 8, 3, 3, (0, 1), (1, 1, 1, 1), (1, 1)) == 1          # stride < 1
    assert q(8, 8, 3, 3, (1, 1), (1, 1, -1, 1), (1, 1)) == 1         # pad < 0
    assert q(0, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)) == 1
    assert q(1 << 31, 8, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1)) == 2
    assert L.conv2d_bias_act_out_dims(8, 8, 3, 3, _i32(1, 1), _i32(1, 1, 1, 1), _i32(1, 1),
                                      None, ctypes.byref(wo)) == 1
    # the binding takes its shapes from the library
    assert ba.conv_out_hw(9, 7, 3, 2, (2, 1), (1, 0, 2, 1), (1, 2)) == (4, 8)


def test_static_path_rule():
    # fused unless the output's alignment keeps the fused GEMM off the
    # ping-pong main loop that kernel 1 keeps when writing an aligned workspace
    dt = _dt(BF16, BF16, F32, BF16)
    A = ctypes.c_void_p(0x10000)
    C_al, C_mis = ctypes.c_void_p(0x20000), ctypes.c_void_p(0x20002)
    ws, ws_mis = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x40004)
    big = 4096 * 4096 * 4
    sp = lambda C, M, N, K, w, n, d=dt: L.biasact_gemm_static_path(A, A, A, C, M, N, K, d, 1, w, n)
    assert sp(C_al, 4096, 4096, 4096, ws, big) == 0            # aligned: fused ping-pong
    assert sp(C_mis, 4096, 4096, 4096, ws, big) == 1           # misaligned C: two kernels
    assert sp(C_mis, 4096, 4096, 4096, NUL, 0) == 0            # no workspace
    assert sp(C_mis, 4096, 4096, 4096, ws, big - 4) == 0       # workspace too small
    assert sp(C_mis, 4096, 4096, 4096, ws_mis, big) == 0       # workspace not 16-byte aligned
    assert sp(C_mis, 1024, 640, 256, ws, big) == 0             # small grid: no ping-pong either way
    assert sp(C_mis, 4096, 4096, 4096, ws, big, _dt(F32, F32, F32, F32)) == 0
    assert sp(C_mis, 4096, 4096, 4100, ws, big) == 0           # K % 8: no ping-pong either way
    assert sp(NUL, 4096, 4096, 4096, ws, big) == 0             # invalid: fused (the call will reject it)


def test_recorded_path_roundtrip():
    dt = _dt(F16, F16, F32, F16)
    assert L.biasact_gemm_path(77, 88, 99, dt, 3) == 0
    assert L.biasact_set_gemm_path(77, 88, 99, dt, 3, 1) == 0
    assert L.biasact_gemm_path(77, 88, 99, dt, 3) == 1
    assert L.biasact_gemm_path(77, 88, 99, dt, 4) == 0              # another activation
    assert L.biasact_set_gemm_path(77, 88, 99, dt, 3, -1) == 0       # forget
    assert L.biasact_gemm_path(77, 88, 99, dt, 3) == 0
    assert L.biasact_set_gemm_path(77, 88, 99, dt, 3, 2) == 1
    c = (_i32(1, 1), _i32(1, 1, 1, 1), _i32(1, 1))
    cdt = _dt(F16, F16, F16, F16)
    assert L.biasact_set_conv_path(3, 8, 9, 9, 5, 3, 3, *c, cdt, 3, 1) == 0
    assert L.biasact_conv_path(3, 8, 9, 9, 5, 3, 3, *c, cdt, 3) == 1
    assert L.biasact_set_conv_path(3, 8, 9, 9, 5, 3, 3, *c, cdt, 3, -1) == 0
    assert L.biasact_conv_path(3, 8, 9, 9, 5, 3, 3, *c, cdt, 3) == 0
    assert L.biasact_set_conv_path(3, 8, 9, 9, 5, 3, 3, None, c[1], c[2], cdt, 3, 1) == 1
    assert ba.set_gemm_path(5, 6, 7, dt, "tanh", "2k") is None
    assert ba.gemm_path(5, 6, 7, dt, "tanh") == "2k"
    ba.set_gemm_path(5, 6, 7, dt, "tanh", None)
    assert ba.gemm_path(5, 6, 7, dt, "tanh") == "fused"


def test_noalloc_entry_point_checks_before_any_hip_call():
    dt = _dt(BF16, BF16, F32, BF16)
    f = L.gemm_bias_act_2k_noalloc
    assert f(P, P, P, P, 8192, 4096, 64, dt, 1, 0.0, NUL) == 2       # 128 MiB workspace > 64 MiB
    assert f(P, P, P, P, 4096, 4097, 64, dt, 1, 0.0, NUL) == 2       # just past the limit
    assert f(NUL, P, P, P, 64, 64, 64, dt, 1, 0.0, NUL) == 1
    assert f(P, P, P, P, 64, 64, 64, dt, 9, 0.0, NUL) == 1
    assert f(P, P, P, P, 64, 64, 64, _dt(3, 3, 4, 4), 1, 0.0, NUL) == 2   # int8: fused only
    assert f(P, P, P, P, 0, 64, 64, dt, 1, 0.0, NUL) == 0              # empty: nothing to launch
