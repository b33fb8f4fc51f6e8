"""CPU oracle for RMSNorm, fused residual-add + RMSNorm, LayerNorm and row softmax.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the GPU library (``row_reduction_rmsnorm_amd``) and neither imports the
other.  The arithmetic lives in ``oracle.c`` (fp64, plain definitions); this
module only moves numpy arrays in and out of it.  ``online_ref`` holds a
pure-Python fp64 twin of the online normaliser for tiny brute-force rows.

Every function here is pinned by ``tests/test_oracle_pins.py`` against the
pages' worked examples, invariants, brute force and library routines.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
F32 = 0
BF16 = 1
_DTYPES = {"f32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16}

_dp = ctypes.POINTER(ctypes.c_double)


def _lib():
    global _LIB
    if _LIB is None:
        path = os.environ.get("ORACLE_LIB_OVERRIDE")  # mutation tests only
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        lib = ctypes.CDLL(path)
        i64 = ctypes.c_int64
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_double
        lib.oracle_round_f32.argtypes = [ctypes.c_double]
        lib.oracle_round_f32.restype = ctypes.c_double
        lib.oracle_round_array.argtypes = [ctypes.c_int, i64, _dp, _dp]
        lib.oracle_rmsnorm.argtypes = [i64, i64, _dp, _dp, ctypes.c_double, _dp]
        lib.oracle_layernorm.argtypes = [i64, i64, _dp, _dp, _dp, ctypes.c_double, _dp]
        lib.oracle_fused_add_rmsnorm.argtypes = [i64, i64, _dp, _dp, _dp, ctypes.c_double,
                                                 ctypes.c_int, _dp, _dp]
        lib.oracle_softmax.argtypes = [i64, i64, _dp, _dp]
        lib.oracle_log_softmax.argtypes = [i64, i64, _dp, _dp]
        lib.oracle_softmax_stats.argtypes = [i64, i64, _dp, _dp, _dp]
        for f in ("oracle_rmsnorm", "oracle_fused_add_rmsnorm", "oracle_softmax",
                  "oracle_softmax_stats", "oracle_layernorm", "oracle_log_softmax"):
            getattr(lib, f).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_dp)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def num_threads() -> int:
    """Host threads the oracle's row loops use."""
    return int(_lib().oracle_num_threads())


def round_bf16(a):
    """Round fp64 values to bfloat16 (ties to even); returns fp64 holding bf16 values."""
    a = _f64(a)
    out = np.empty_like(a)
    _lib().oracle_round_array(BF16, a.size, _ptr(a), _ptr(out))
    return out


def round_f32(a):
    a = _f64(a)
    out = np.empty_like(a)
    _lib().oracle_round_array(F32, a.size, _ptr(a), _ptr(out))
    return out


def round_io(a, dtype):
    return round_bf16(a) if _DTYPES[dtype] == BF16 else round_f32(a)


def rmsnorm(x, gamma, eps):
    """y[M,H] in fp64 for x[M,H] (or [H]), gamma[H]."""
    x = _f64(x)
    gamma = _f64(gamma)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    M, H = x2.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must have shape [H]")
    y = np.empty_like(x2)
    _check(_lib().oracle_rmsnorm(M, H, _ptr(x2), _ptr(gamma), float(eps), _ptr(y)), "rmsnorm")
    return y.reshape(shape)


def layernorm(x, gamma, beta, eps):
    """y[M,H] in fp64 for x[M,H] (or [H]), gamma[H], beta[H] or None."""
    x = _f64(x)
    gamma = _f64(gamma)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    M, H = x2.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must have shape [H]")
    bp = None
    if beta is not None:
        beta = _f64(beta)
        if beta.shape != (H,):
            raise ValueError("beta must have shape [H]")
        bp = _ptr(beta)
    y = np.empty_like(x2)
    _check(_lib().oracle_layernorm(M, H, _ptr(x2), _ptr(gamma), bp, float(eps), _ptr(y)),
           "layernorm")
    return y.reshape(shape)


def fused_add_rmsnorm(x, residual, gamma, eps, io_dtype):
    """Returns (residual_out, y): residual_out holds I/O-dtype values, y is fp64."""
    x = _f64(x)
    r = _f64(residual)
    gamma = _f64(gamma)
    if x.shape != r.shape:
        raise ValueError("x and residual must have the same shape")
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    r2 = r.reshape(-1, shape[-1])
    M, H = x2.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must have shape [H]")
    h = np.empty_like(x2)
    y = np.empty_like(x2)
    rc = _lib().oracle_fused_add_rmsnorm(M, H, _ptr(x2), _ptr(r2), _ptr(gamma), float(eps),
                                         _DTYPES[io_dtype], _ptr(h), _ptr(y))
    _check(rc, "fused_add_rmsnorm")
    return h.reshape(shape), y.reshape(shape)


def softmax(x):
    """Row softmax in fp64 over the last axis."""
    x = _f64(x)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    M, N = x2.shape
    y = np.empty_like(x2)
    _check(_lib().oracle_softmax(M, N, _ptr(x2), _ptr(y)), "softmax")
    return y.reshape(shape)


def log_softmax(x):
    """Row log-softmax in fp64 over the last axis."""
    x = _f64(x)
    shape = x.shape
    x2 = x.reshape(-1, shape[-1])
    M, N = x2.shape
    y = np.empty_like(x2)
    _check(_lib().oracle_log_softmax(M, N, _ptr(x2), _ptr(y)), "log_softmax")
    return y.reshape(shape)


def softmax_stats(x):
    """Per-row (m, d) of the safe softmax: m = max, d = sum exp(x - m)."""
    x = _f64(x)
    x2 = x.reshape(-1, x.shape[-1])
    M, N = x2.shape
    m = np.empty(M)
    d = np.empty(M)
    _check(_lib().oracle_softmax_stats(M, N, _ptr(x2), _ptr(m), _ptr(d)), "softmax_stats")
    return m, d
