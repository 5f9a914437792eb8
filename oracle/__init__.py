"""CPU oracle for FP32 row reductions -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library (``row_reductions_amd``)
never imports it and shares no code with it.

The arithmetic lives in plain C (``oracle.c``, double accumulation, plus the
FP32 ordered-fold replay); this module only builds that file with gcc and
marshals numpy arrays into it.  Definitions and citations are in
``oracle.h``.  Pins: ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_softmax_f64.argtypes = [P, P, I64, I64]
        lib.oracle_rmsnorm_f64.argtypes = [P, P, P, I64, I64, ctypes.c_double]
        lib.oracle_layernorm_f64.argtypes = [P, P, P, P, I64, I64, ctypes.c_double]
        lib.oracle_layernorm_stats_f64.argtypes = [P, P, P, I64, I64]
        lib.oracle_cross_entropy_f64.argtypes = [P, P, P, I64, I64]
        lib.oracle_add_layernorm_f64.argtypes = [P, P, P, P, P, P, I64, I64, ctypes.c_double]
        lib.oracle_add_layernorm_f64.restype = ctypes.c_int
        lib.oracle_row_sum_f64.argtypes = [P, P, I64, I64]
        lib.oracle_row_minmax_f32.argtypes = [P, P, P, I64, I64]
        lib.oracle_row_sum_f64.restype = None
        lib.oracle_row_minmax_f32.restype = None
        lib.oracle_rmsnorm_fold_f32.argtypes = [P, P, P, I64, I64, ctypes.c_float]
        lib.oracle_layernorm_fold_f32.argtypes = [P, P, P, P, I64, I64, ctypes.c_float]
        lib.oracle_fold_left_f32.argtypes = [P, I64, ctypes.c_int]
        lib.oracle_fold_left_f32.restype = ctypes.c_float
        lib.oracle_ordered_sum_f32.argtypes = [P, I64, ctypes.c_int, ctypes.c_int]
        lib.oracle_ordered_sum_f32.restype = ctypes.c_float
        lib.oracle_rmsnorm_ordered_f32.argtypes = [P, P, P, I64, I64, ctypes.c_float, ctypes.c_int]
        lib.oracle_rmsnorm_ordered_f32.restype = None
        lib.oracle_layernorm_ordered_f32.argtypes = [P, P, P, P, I64, I64, ctypes.c_float, ctypes.c_int]
        lib.oracle_layernorm_ordered_f32.restype = ctypes.c_int
        for f in ("oracle_softmax_f64", "oracle_rmsnorm_f64", "oracle_layernorm_f64",
                  "oracle_layernorm_stats_f64", "oracle_cross_entropy_f64",
                  "oracle_rmsnorm_fold_f32", "oracle_layernorm_fold_f32"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _opt_vec(a, cols):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    assert a.shape[0] == cols
    return a


def eps_as_f32(eps: float) -> float:
    """The eps value a float32 kernel argument actually carries."""
    return float(np.float32(eps))


def softmax(x) -> np.ndarray:
    x = _f32(x)
    y = np.empty(x.shape, dtype=np.float64)
    _load().oracle_softmax_f64(_ptr(x), _ptr(y), x.shape[0], x.shape[1])
    return y


def rmsnorm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    y = np.empty(x.shape, dtype=np.float64)
    _load().oracle_rmsnorm_f64(_ptr(x), _ptr(g), _ptr(y), x.shape[0], x.shape[1],
                               eps_as_f32(eps))
    return y


def layernorm(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    b = _opt_vec(beta, x.shape[1])
    y = np.empty(x.shape, dtype=np.float64)
    _load().oracle_layernorm_f64(_ptr(x), _ptr(g), _ptr(b), _ptr(y), x.shape[0],
                                 x.shape[1], eps_as_f32(eps))
    return y


def add_layernorm(x, residual, gamma=None, beta=None, eps: float = 1e-5, with_sum: bool = False):
    """Fused residual LayerNorm: layernorm(fl32(x + residual)) in double; with
    ``with_sum`` also the FP32 combined tensor."""
    x = _f32(x)
    r = _f32(residual)
    assert r.shape == x.shape
    g = _opt_vec(gamma, x.shape[1])
    b = _opt_vec(beta, x.shape[1])
    y = np.empty(x.shape, dtype=np.float64)
    s = np.empty(x.shape, dtype=np.float32) if with_sum else None
    rc = _load().oracle_add_layernorm_f64(_ptr(x), _ptr(r), _ptr(g), _ptr(b), _ptr(y), _ptr(s),
                                          x.shape[0], x.shape[1], eps_as_f32(eps))
    if rc != 0:
        raise MemoryError("oracle_add_layernorm_f64: row scratch")
    return (y, s) if with_sum else y


def layernorm_stats(x):
    x = _f32(x)
    mu = np.empty(x.shape[0], dtype=np.float64)
    var = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_layernorm_stats_f64(_ptr(x), _ptr(mu), _ptr(var), x.shape[0], x.shape[1])
    return mu, var


def cross_entropy(logits, labels) -> np.ndarray:
    x = _f32(logits)
    lab = np.ascontiguousarray(labels, dtype=np.int64).reshape(-1)
    assert lab.shape[0] == x.shape[0]
    out = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_cross_entropy_f64(_ptr(x), _ptr(lab), _ptr(out), x.shape[0], x.shape[1])
    return out


def row_sum(x) -> np.ndarray:
    """Per-row sum in double."""
    x = _f32(x)
    out = np.empty(x.shape[0], dtype=np.float64)
    _load().oracle_row_sum_f64(_ptr(x), _ptr(out), x.shape[0], x.shape[1])
    return out


def row_minmax(x):
    """Per-row (minimum, maximum), exact FP32 values."""
    x = _f32(x)
    lo = np.empty(x.shape[0], dtype=np.float32)
    hi = np.empty(x.shape[0], dtype=np.float32)
    _load().oracle_row_minmax_f32(_ptr(x), _ptr(lo), _ptr(hi), x.shape[0], x.shape[1])
    return lo, hi


def rmsnorm_fold_f32(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    y = np.empty(x.shape, dtype=np.float32)
    _load().oracle_rmsnorm_fold_f32(_ptr(x), _ptr(g), _ptr(y), x.shape[0], x.shape[1],
                                    ctypes.c_float(eps))
    return y


def layernorm_fold_f32(x, gamma=None, beta=None, eps: float = 1e-5) -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    b = _opt_vec(beta, x.shape[1])
    y = np.empty(x.shape, dtype=np.float32)
    _load().oracle_layernorm_fold_f32(_ptr(x), _ptr(g), _ptr(b), _ptr(y), x.shape[0],
                                      x.shape[1], ctypes.c_float(eps))
    return y


def fold_left_f32(x, kind: int = 0) -> float:
    """FP32 left fold of a 1-D array: kind 0 sums x_j, kind 1 sums x_j*x_j."""
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    return float(_load().oracle_fold_left_f32(_ptr(a), a.shape[0], kind))


#: the ordered reduction policies and their codes in the replay functions
ORDERED_POLICIES = {"ordered_fold": 1, "ordered_tree": 2, "fold_right": 3}


def ordered_sum_f32(x, policy: str, kind: int = 0) -> float:
    """FP32 sum of a 1-D array in the order of an ordered policy: kind 0
    sums x_j, kind 1 sums x_j*x_j."""
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    return float(_load().oracle_ordered_sum_f32(_ptr(a), a.shape[0], kind, ORDERED_POLICIES[policy]))


def rmsnorm_ordered_f32(x, gamma=None, eps: float = 1e-6, policy: str = "ordered_fold") -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    y = np.empty(x.shape, dtype=np.float32)
    _load().oracle_rmsnorm_ordered_f32(_ptr(x), _ptr(g), _ptr(y), x.shape[0], x.shape[1], ctypes.c_float(eps),
                                       ORDERED_POLICIES[policy])
    return y


def layernorm_ordered_f32(x, gamma=None, beta=None, eps: float = 1e-5, policy: str = "ordered_fold") -> np.ndarray:
    x = _f32(x)
    g = _opt_vec(gamma, x.shape[1])
    b = _opt_vec(beta, x.shape[1])
    y = np.empty(x.shape, dtype=np.float32)
    rc = _load().oracle_layernorm_ordered_f32(_ptr(x), _ptr(g), _ptr(b), _ptr(y), x.shape[0], x.shape[1],
                                              ctypes.c_float(eps), ORDERED_POLICIES[policy])
    if rc != 0:
        raise MemoryError("oracle_layernorm_ordered_f32: row scratch")
    return y


def run(op: str, inputs: dict, eps=None) -> np.ndarray:
    """Oracle output of ``op`` for a ``synth`` input dict (double results)."""
    if op == "softmax":
        return softmax(inputs["x"])
    if op == "rmsnorm":
        return rmsnorm(inputs["x"], inputs.get("gamma"), eps)
    if op == "layernorm":
        return layernorm(inputs["x"], inputs.get("gamma"), inputs.get("beta"), eps)
    if op == "cross_entropy":
        return cross_entropy(inputs["logits"], inputs["labels"])
    if op == "add_layernorm":
        return add_layernorm(inputs["x"], inputs["residual"], inputs.get("gamma"), inputs.get("beta"), eps)
    raise ValueError(op)
