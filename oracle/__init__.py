"""fp64 CPU oracle for the dense projection Y = X . W^T (+ bias) (-> GELU).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product path (``dense_linear_projection_amd``) never imports it, and the two
share no code: the oracle is plain C built with gcc (``proj_oracle.c``), the
product is HIP built with hipcc.

The arithmetic lives in ``proj_oracle.c``; this module only loads it and
marshals numpy arrays.  ``compare`` holds the acceptance rule.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "proj_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

EPI_NONE, EPI_BIAS, EPI_GELU, EPI_BIAS_GELU = 0, 1, 2, 3
OUT_F32, OUT_BF16 = 0, 1


def build() -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double, ascending sums)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-pthread", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        L.oracle_proj_f64.argtypes = [u16p, u16p, u16p, ctypes.c_int, i64, i64, i64, dp, ctypes.c_int]
        L.oracle_proj_f64.restype = ctypes.c_int
        L.oracle_proj_f64_at.argtypes = [u16p, u16p, u16p, ctypes.c_int, i64, i64, i64,
                                         i64p, i64p, i64, dp, ctypes.c_int]
        L.oracle_proj_f64_at.restype = ctypes.c_int
        f32p = ctypes.POINTER(ctypes.c_float)
        L.oracle_proj_f64_w32.argtypes = [u16p, f32p, u16p, ctypes.c_int, i64, i64, i64, dp, ctypes.c_int]
        L.oracle_proj_f64_w32.restype = ctypes.c_int
        L.oracle_hilo_split.argtypes = [f32p, i64, u16p, u16p]
        L.oracle_hilo_split.restype = None
        L.oracle_round_out.argtypes = [dp, i64, ctypes.c_int, ctypes.c_void_p]
        L.oracle_round_out.restype = ctypes.c_int
        L.oracle_f64_to_bf16_array.argtypes = [dp, i64, u16p]
        L.oracle_bf16_to_f64_array.argtypes = [u16p, i64, dp]
        L.oracle_gelu_tanh_array.argtypes = [dp, i64, dp]
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_gelu_tanh.argtypes = [ctypes.c_double]
        L.oracle_gelu_tanh.restype = ctypes.c_double
        _lib = L
    return _lib


def _u16(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def proj_f64(X, W, bias=None, epi=EPI_NONE, nthreads=None) -> np.ndarray:
    """Exact-as-double result of epi(X . W^T + bias) for bf16 bit arrays.

    X: uint16 [M, K] bf16 bits; W: uint16 [N, K]; bias: uint16 [N] or None.
    Returns float64 [M, N], before rounding to the output type.
    """
    X, W, bias = _u16(X), _u16(W), _u16(bias)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ: X has K=%d, W has K=%d" % (K, K2))
    out = np.empty((M, N), dtype=np.float64)
    rc = lib().oracle_proj_f64(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16),
                               _ptr(bias, ctypes.c_uint16), int(epi), M, N, K,
                               _ptr(out, ctypes.c_double), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def proj_f64_at(X, W, rows, cols, bias=None, epi=EPI_NONE, nthreads=None) -> np.ndarray:
    """The same cell values as proj_f64, only at the (rows[i], cols[i]) pairs."""
    X, W, bias = _u16(X), _u16(W), _u16(bias)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(rows.shape, dtype=np.float64)
    rc = lib().oracle_proj_f64_at(_ptr(X, ctypes.c_uint16), _ptr(W, ctypes.c_uint16),
                                  _ptr(bias, ctypes.c_uint16), int(epi), M, N, K,
                                  _ptr(rows, ctypes.c_int64), _ptr(cols, ctypes.c_int64),
                                  rows.size, _ptr(out, ctypes.c_double),
                                  int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def proj_f64_w32(X, W32, bias=None, epi=EPI_NONE, nthreads=None) -> np.ndarray:
    """As proj_f64 with fp32 weights: X uint16 [M, K] bf16 bits, W32 float32
    [N, K] values (the router's reference product)."""
    X, bias = _u16(X), _u16(bias)
    W32 = np.ascontiguousarray(W32, dtype=np.float32)
    M, K = X.shape
    N, K2 = W32.shape
    if K != K2:
        raise ValueError("inner dimensions differ: X has K=%d, W has K=%d" % (K, K2))
    out = np.empty((M, N), dtype=np.float64)
    rc = lib().oracle_proj_f64_w32(_ptr(X, ctypes.c_uint16), _ptr(W32, ctypes.c_float),
                                   _ptr(bias, ctypes.c_uint16), int(epi), M, N, K,
                                   _ptr(out, ctypes.c_double), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def hilo_split(W32):
    """(hi, lo): uint16 bf16 bit arrays of W32's shape with hi = bf16(w) and
    lo = bf16(w - hi), both rounded to nearest even."""
    W32 = np.ascontiguousarray(W32, dtype=np.float32)
    hi = np.empty(W32.shape, dtype=np.uint16)
    lo = np.empty(W32.shape, dtype=np.uint16)
    lib().oracle_hilo_split(_ptr(W32, ctypes.c_float), W32.size, _ptr(hi, ctypes.c_uint16),
                            _ptr(lo, ctypes.c_uint16))
    return hi, lo


def round_out(s: np.ndarray, out_dtype: int) -> np.ndarray:
    """Round oracle doubles to the output type: float32 array, or uint16 bf16 bits."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    if out_dtype == OUT_F32:
        dst = np.empty(s.shape, dtype=np.float32)
    elif out_dtype == OUT_BF16:
        dst = np.empty(s.shape, dtype=np.uint16)
    else:
        raise ValueError("unknown output type")
    rc = lib().oracle_round_out(_ptr(s, ctypes.c_double), s.size, int(out_dtype),
                                dst.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("unknown output type")
    return dst


def f64_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f64_to_bf16_array(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_uint16))
    return out


def bf16_to_f64(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oracle_bf16_to_f64_array(_ptr(b, ctypes.c_uint16), b.size, _ptr(out, ctypes.c_double))
    return out


def gelu_tanh(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_gelu_tanh_array(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_double))
    return out


def reference(X, W, bias=None, epi=EPI_NONE, out_dtype=OUT_F32, nthreads=None):
    """(r, s): r = oracle result rounded to the output type, as float64 values,
    and s = the unrounded double result."""
    s = proj_f64(X, W, bias, epi, nthreads)
    r = round_out(s, out_dtype)
    if out_dtype == OUT_BF16:
        r = bf16_to_f64(r)
    return r.astype(np.float64), s
