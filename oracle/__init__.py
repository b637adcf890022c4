"""fp64 CPU oracle for act(A.B + bias) and act(conv2d(x, w) + bias).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library and its
Python binding never import it; it never imports them.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only marshals numpy arrays into it.  ``build()`` compiles the C file with gcc
(``-O2 -ffp-contract=off -fopenmp``, no fast-math).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4}
ACT_CODES = {"none": 0, "relu": 1, "leaky_relu": 2, "tanh": 3, "gelu": 4, "sigmoid": 5}

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
             "-std=c11", "-Wall"]


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle into a shared library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, *extra_flags, "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def _bind(lib):
    i64 = ctypes.c_int64
    lib.orc_decode.argtypes = [ctypes.c_int, ctypes.c_void_p, i64, _D]
    lib.orc_act_array.argtypes = [ctypes.c_int, ctypes.c_double, _D, _D, i64]
    lib.orc_act_array.restype = None
    lib.orc_residual_act.argtypes = [_D, _D, _D, i64, ctypes.c_int, ctypes.c_double]
    lib.orc_gemm_bias_act.argtypes = [_D, _D, _D, _D, i64, i64, i64, ctypes.c_int, ctypes.c_double]
    lib.orc_gemm_bias_act_elems.argtypes = [_D, _D, _D, i64, i64, i64, _I64, _I64, i64,
                                            ctypes.c_int, ctypes.c_double, _D]
    lib.orc_gemm_bias_fold.argtypes = [_D, _D, _D, _D, i64, i64, i64, ctypes.c_int, ctypes.c_double]
    lib.orc_conv_out_dim.argtypes = [i64] * 6
    lib.orc_conv_out_dim.restype = i64
    conv_common = [_D, _D, _D]
    shape = [i64] * 7 + [_I64, _I64, _I64]
    lib.orc_conv2d_bias_act.argtypes = conv_common + [_D] + shape + [ctypes.c_int, ctypes.c_double]
    lib.orc_conv2d_bias_act_elems.argtypes = conv_common + shape + [_I64, i64, ctypes.c_int,
                                                                    ctypes.c_double, _D]
    lib.orc_conv2d_im2col.argtypes = conv_common + [_D] + shape + [ctypes.c_int, ctypes.c_double,
                                                                   ctypes.c_int]
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    lib.orc_num_threads.argtypes = []
    for name in ("orc_decode", "orc_gemm_bias_act", "orc_gemm_bias_act_elems", "orc_gemm_bias_fold",
                 "orc_conv2d_bias_act", "orc_conv2d_bias_act_elems", "orc_conv2d_im2col",
                 "orc_num_threads"):
        getattr(lib, name).restype = ctypes.c_int
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f64.restype = ctypes.c_double
    lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f64.restype = ctypes.c_double
    lib.orc_f32_to_f64.argtypes = [ctypes.c_uint32]
    lib.orc_f32_to_f64.restype = ctypes.c_double
    return lib


def load(path: Optional[str] = None):
    """Load (building first if absent) the oracle library.  With `path`, load
    that library instead of the default one (used by mutation tests)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(_D)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


class Oracle:
    """Thin marshalling layer over one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # -- decoding ----------------------------------------------------------
    def decode(self, words: np.ndarray, dtype: str) -> np.ndarray:
        words = np.ascontiguousarray(words)
        want = {"f32": np.uint32, "i32": np.uint32, "i8": np.uint8}.get(dtype, np.uint16)
        if words.dtype != want:
            raise ValueError(f"{dtype} words must be {np.dtype(want).name}")
        out = np.empty(words.shape, dtype=np.float64)
        _check(self.lib.orc_decode(DTYPE_CODES[dtype], words.ctypes.data_as(ctypes.c_void_p),
                                   words.size, _dp(out)), "decode")
        return out

    # -- activation --------------------------------------------------------
    def act(self, z: np.ndarray, act: str, alpha: float = 0.0) -> np.ndarray:
        z = _f64(z)
        y = np.empty_like(z)
        self.lib.orc_act_array(ACT_CODES[act], float(alpha), _dp(z), _dp(y), z.size)
        return y

    def residual_act(self, z, r, act: str, alpha: float = 0.0) -> np.ndarray:
        """act(z + r) elementwise; z is a pre-activation (contraction + bias)."""
        z = _f64(z)
        r = _f64(r).reshape(z.shape)
        y = np.empty_like(z)
        _check(self.lib.orc_residual_act(_dp(z), _dp(r), _dp(y), z.size, ACT_CODES[act],
                                         float(alpha)), "residual_act")
        return y

    # -- GEMM --------------------------------------------------------------
    def gemm(self, A, B, bias, act: str, alpha: float = 0.0) -> np.ndarray:
        A, B = _f64(A), _f64(B)
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError("inner dimensions differ")
        bias = None if bias is None else _f64(bias).reshape(N)
        C = np.empty((M, N), dtype=np.float64)
        _check(self.lib.orc_gemm_bias_act(_dp(A), _dp(B), _dp(bias), _dp(C), M, N, K,
                                          ACT_CODES[act], float(alpha)), "gemm")
        return C

    def gemm_elems(self, A, B, bias, ii, jj, act: str, alpha: float = 0.0) -> np.ndarray:
        A, B = _f64(A), _f64(B)
        M, K = A.shape
        N = B.shape[1]
        bias = None if bias is None else _f64(bias).reshape(N)
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        jj = np.ascontiguousarray(jj, dtype=np.int64)
        out = np.empty(ii.size, dtype=np.float64)
        _check(self.lib.orc_gemm_bias_act_elems(_dp(A), _dp(B), _dp(bias), M, N, K,
                                                ii.ctypes.data_as(_I64), jj.ctypes.data_as(_I64),
                                                ii.size, ACT_CODES[act], float(alpha), _dp(out)),
               "gemm_elems")
        return out

    def gemm_residual(self, A, B, bias, R, act: str, alpha: float = 0.0) -> np.ndarray:
        """C = act(A.B + bias + R), R of C's shape."""
        return self.residual_act(self.gemm(A, B, bias, "none"), R, act, alpha)

    def gemm_residual_elems(self, A, B, bias, R_flat_at, ii, jj, act: str, alpha: float = 0.0):
        """The elements (ii, jj) of act(A.B + bias + R); R_flat_at holds R at those elements."""
        return self.residual_act(self.gemm_elems(A, B, bias, ii, jj, "none"), R_flat_at, act, alpha)

    def gemm_bias_fold(self, A, B, bias, act: str, alpha: float = 0.0) -> np.ndarray:
        A, B = _f64(A), _f64(B)
        M, K = A.shape
        N = B.shape[1]
        bias = None if bias is None else _f64(bias).reshape(N)
        C = np.empty((M, N), dtype=np.float64)
        _check(self.lib.orc_gemm_bias_fold(_dp(A), _dp(B), _dp(bias), _dp(C), M, N, K,
                                           ACT_CODES[act], float(alpha)), "gemm_bias_fold")
        return C

    # -- conv2d ------------------------------------------------------------
    def conv_out_dim(self, n_in, k, stride, pad_lo, pad_hi, dil) -> int:
        return int(self.lib.orc_conv_out_dim(n_in, k, stride, pad_lo, pad_hi, dil))

    @staticmethod
    def _conv_args(x, w, strides, pads, dilations):
        x, w = _f64(x), _f64(w)
        N, C, H, W = x.shape
        Co, C2, kh, kw = w.shape
        if C != C2:
            raise ValueError("channel counts differ")
        st = np.ascontiguousarray(strides, dtype=np.int64)
        pd = np.ascontiguousarray(pads, dtype=np.int64)
        dl = np.ascontiguousarray(dilations, dtype=np.int64)
        if st.size != 2 or pd.size != 4 or dl.size != 2:
            raise ValueError("strides[2], pads[4] (top, bottom, left, right), dilations[2]")
        return x, w, (N, C, H, W, Co, kh, kw), st, pd, dl

    def conv_out_shape(self, x_shape, w_shape, strides, pads, dilations):
        N, C, H, W = x_shape
        Co, _, kh, kw = w_shape
        Ho = self.conv_out_dim(H, kh, strides[0], pads[0], pads[1], dilations[0])
        Wo = self.conv_out_dim(W, kw, strides[1], pads[2], pads[3], dilations[1])
        return (N, Co, Ho, Wo)

    def conv2d(self, x, w, bias, strides, pads, dilations, act: str, alpha: float = 0.0):
        x, w, dims, st, pd, dl = self._conv_args(x, w, strides, pads, dilations)
        y = np.empty(self.conv_out_shape(x.shape, w.shape, st, pd, dl), dtype=np.float64)
        bias = None if bias is None else _f64(bias).reshape(dims[4])
        _check(self.lib.orc_conv2d_bias_act(_dp(x), _dp(w), _dp(bias), _dp(y), *dims,
                                            st.ctypes.data_as(_I64), pd.ctypes.data_as(_I64),
                                            dl.ctypes.data_as(_I64), ACT_CODES[act], float(alpha)),
               "conv2d")
        return y

    def conv2d_elems(self, x, w, bias, strides, pads, dilations, idx, act: str, alpha: float = 0.0):
        x, w, dims, st, pd, dl = self._conv_args(x, w, strides, pads, dilations)
        bias = None if bias is None else _f64(bias).reshape(dims[4])
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        out = np.empty(idx.size, dtype=np.float64)
        _check(self.lib.orc_conv2d_bias_act_elems(_dp(x), _dp(w), _dp(bias), *dims,
                                                  st.ctypes.data_as(_I64), pd.ctypes.data_as(_I64),
                                                  dl.ctypes.data_as(_I64), idx.ctypes.data_as(_I64),
                                                  idx.size, ACT_CODES[act], float(alpha), _dp(out)),
               "conv2d_elems")
        return out

    def conv2d_residual(self, x, w, bias, R, strides, pads, dilations, act: str,
                        alpha: float = 0.0):
        """y = act(conv2d(x, w) + bias + R), R of y's shape."""
        z = self.conv2d(x, w, bias, strides, pads, dilations, "none")
        return self.residual_act(z, R, act, alpha)

    def conv2d_residual_elems(self, x, w, bias, R_flat_at, strides, pads, dilations, idx,
                              act: str, alpha: float = 0.0):
        z = self.conv2d_elems(x, w, bias, strides, pads, dilations, idx, "none")
        return self.residual_act(z, R_flat_at, act, alpha)

    def conv2d_im2col(self, x, w, bias, strides, pads, dilations, act: str, alpha: float = 0.0,
                      fold_bias: bool = False):
        x, w, dims, st, pd, dl = self._conv_args(x, w, strides, pads, dilations)
        y = np.empty(self.conv_out_shape(x.shape, w.shape, st, pd, dl), dtype=np.float64)
        bias = None if bias is None else _f64(bias).reshape(dims[4])
        _check(self.lib.orc_conv2d_im2col(_dp(x), _dp(w), _dp(bias), _dp(y), *dims,
                                          st.ctypes.data_as(_I64), pd.ctypes.data_as(_I64),
                                          dl.ctypes.data_as(_I64), ACT_CODES[act], float(alpha),
                                          int(fold_bias)), "conv2d_im2col")
        return y

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.orc_set_num_threads(int(n))


def f32(x: float) -> float:
    """The fp32 value of a Python float (alpha is an fp32 scalar on the pages)."""
    return float(np.float32(x))
