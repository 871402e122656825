"""ctypes front end of the CPU fp64 oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg; never by the library.  Every function takes and
returns numpy float64 arrays holding the exact values of the inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIBRARY names another build of oracle.c (the host-sanitizer build of
# the test suite); by default the in-tree one.
_LIB = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra",
             "-shared", "-fPIC"]


def build(force: bool = True, cc: str = "gcc", extra_flags=(), out: str | None = None) -> str:
    """Compile oracle.c (plain C, no GPU code); by default with gcc into the
    in-tree liboracle.so."""
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run([cc, *GCC_FLAGS, *extra_flags, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        i64, dbl, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_bn_forward_train.argtypes = [i64, i64, i64, p, p, p, dbl, dbl, p, p, p, p]
        lib.oracle_bn_backward.argtypes = [i64, i64, i64, p, p, p, dbl, p, p]
        lib.oracle_bn_act_forward_train.argtypes = [i64, i64, i64, p, p, p, dbl, dbl, ctypes.c_int,
                                                     dbl, p, p, p, p]
        lib.oracle_bn_act_backward.argtypes = [i64, i64, i64, p, p, p, p, dbl, ctypes.c_int, dbl, p, p]
        lib.oracle_bn_infer.argtypes = [i64, i64, i64, p, p, p, p, p, dbl, ctypes.c_int, dbl, p]
        lib.oracle_layernorm_stats.argtypes = [i64, i64, p, dbl, p, p]
        lib.oracle_layernorm_forward.argtypes = [i64, i64, p, p, p, dbl, p, p, p]
        lib.oracle_rmsnorm_forward.argtypes = [i64, i64, p, p, dbl, p, p]
        lib.oracle_layernorm_backward.argtypes = [i64, i64, p, p, p, p, p, p, p, p]
        lib.oracle_bda_layernorm_backward.argtypes = [i64, i64, p, p, p, p, p, p, p, dbl, p, p, p,
                                                       p, p]
        lib.oracle_rmsnorm_rms.argtypes = [i64, i64, p, dbl, p]
        lib.oracle_rmsnorm_backward.argtypes = [i64, i64, p, p, p, p, dbl, p, p]
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        for f in ("oracle_bn_forward_train", "oracle_bn_backward", "oracle_bn_act_forward_train",
                  "oracle_bn_act_backward", "oracle_bn_infer", "oracle_layernorm_stats",
                  "oracle_layernorm_forward", "oracle_layernorm_backward",
                  "oracle_bda_layernorm_backward", "oracle_rmsnorm_rms",
                  "oracle_rmsnorm_forward", "oracle_rmsnorm_backward", "oracle_set_threads"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _d(a):
    """Contiguous float64 copy-or-view of a."""
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: bad arguments (rc={rc})")


def _threads(n):
    """Threads for the next call's independent loops (channels, rows, column
    blocks); the results do not depend on it."""
    _check(_load().oracle_set_threads(int(n)), "oracle_set_threads")


def bn_forward_train(x, gamma, beta, *, eps=1e-5, momentum=0.1,
                     running_mean=None, running_var=None, threads=1):
    """x: [N,C,H,W] (or [N,C,HW]).  Returns (y, stats[4,C], rm', rv').
    rm'/rv' are None when the running statistics are not given."""
    _threads(threads)
    x = _d(x)
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    g, b = _d(gamma), _d(beta)
    rm = None if running_mean is None else _d(running_mean).copy()
    rv = None if running_var is None else _d(running_var).copy()
    y = np.empty_like(x)
    stats = np.empty((4, C), np.float64)
    rc = _load().oracle_bn_forward_train(N, C, HW, _ptr(x), _ptr(g), _ptr(b),
                                         momentum, eps, _ptr(rm), _ptr(rv),
                                         _ptr(y), _ptr(stats))
    _check(rc, "oracle_bn_forward_train")
    return y, stats, rm, rv


def bn_backward(x, dy, gamma, *, eps=1e-5, threads=1):
    """Returns (dx, grads[4,C] = (dgamma, dbeta, k1, k2))."""
    _threads(threads)
    x, dy = _d(x), _d(dy)
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    g = _d(gamma)
    dx = np.empty_like(x)
    grads = np.empty((4, C), np.float64)
    rc = _load().oracle_bn_backward(N, C, HW, _ptr(x), _ptr(dy), _ptr(g), eps,
                                    _ptr(dx), _ptr(grads))
    _check(rc, "oracle_bn_backward")
    return dx, grads


ACTS = {"none": 0, "relu": 1, "leaky_relu": 2}


def bn_act_forward_train(x, gamma, beta, act, slope=0.01, *, eps=1e-5, momentum=0.1,
                         running_mean=None, running_var=None):
    """BatchNorm2d + activation forward.  Returns (y, stats[4,C], rm', rv')."""
    x = _d(x)
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    g, b = _d(gamma), _d(beta)
    rm = None if running_mean is None else _d(running_mean).copy()
    rv = None if running_var is None else _d(running_var).copy()
    y = np.empty_like(x)
    stats = np.empty((4, C), np.float64)
    rc = _load().oracle_bn_act_forward_train(N, C, HW, _ptr(x), _ptr(g), _ptr(b), momentum, eps,
                                             ACTS[act], slope, _ptr(rm), _ptr(rv), _ptr(y),
                                             _ptr(stats))
    _check(rc, "oracle_bn_act_forward_train")
    return y, stats, rm, rv


def bn_act_backward(x, dy, gamma, beta, act, slope=0.01, *, eps=1e-5):
    """Returns (dx, grads[4,C]) of y = act(BatchNorm(x))."""
    x, dy = _d(x), _d(dy)
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    g, b = _d(gamma), _d(beta)
    dx = np.empty_like(x)
    grads = np.empty((4, C), np.float64)
    rc = _load().oracle_bn_act_backward(N, C, HW, _ptr(x), _ptr(dy), _ptr(g), _ptr(b), eps,
                                        ACTS[act], slope, _ptr(dx), _ptr(grads))
    _check(rc, "oracle_bn_act_backward")
    return dx, grads


def bn_infer(x, gamma, beta, running_mean, running_var, act="none", slope=0.01, *, eps=1e-5):
    """BatchNorm2d inference (+ activation) from the running statistics."""
    x = _d(x)
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    g = None if gamma is None else _d(gamma)
    b = None if beta is None else _d(beta)
    rm, rv = _d(running_mean), _d(running_var)
    y = np.empty_like(x)
    rc = _load().oracle_bn_infer(N, C, HW, _ptr(x), _ptr(g), _ptr(b), _ptr(rm), _ptr(rv), eps,
                                 ACTS[act], slope, _ptr(y))
    _check(rc, "oracle_bn_infer")
    return y


def layernorm_stats(x, *, eps=1e-5, threads=1):
    """x: [rows, cols].  Returns (mean[rows], rstd[rows])."""
    _threads(threads)
    x = _d(x)
    rows, cols = x.shape
    mean = np.empty(rows, np.float64)
    rstd = np.empty(rows, np.float64)
    _check(_load().oracle_layernorm_stats(rows, cols, _ptr(x), eps, _ptr(mean), _ptr(rstd)),
           "oracle_layernorm_stats")
    return mean, rstd


def layernorm_forward(x, w=None, b=None, *, eps=1e-5):
    """Returns (y, mean[rows], rstd[rows])."""
    x = _d(x)
    rows, cols = x.shape
    w = None if w is None else _d(w)
    b = None if b is None else _d(b)
    y = np.empty_like(x)
    mean = np.empty(rows, np.float64)
    rstd = np.empty(rows, np.float64)
    _check(_load().oracle_layernorm_forward(rows, cols, _ptr(x), _ptr(w), _ptr(b), eps, _ptr(y),
                                            _ptr(mean), _ptr(rstd)), "oracle_layernorm_forward")
    return y, mean, rstd


def layernorm_backward(x, dy, mean, rstd, w=None, *, threads=1):
    """Returns (dx, dweight, dbias)."""
    _threads(threads)
    x, dy, mean, rstd = _d(x), _d(dy), _d(mean), _d(rstd)
    w = None if w is None else _d(w)
    rows, cols = x.shape
    dx = np.empty_like(x)
    dw = np.empty(cols, np.float64)
    db = np.empty(cols, np.float64)
    _check(_load().oracle_layernorm_backward(rows, cols, _ptr(x), _ptr(dy), _ptr(mean),
                                             _ptr(rstd), _ptr(w), _ptr(dx), _ptr(dw), _ptr(db)),
           "oracle_layernorm_backward")
    return dx, dw, db


def bda_layernorm_backward(x, dy, mean, rstd, w=None, dresidual=None, mask=None, scale=1.0):
    """Backward of bias + dropout + add + LayerNorm.  mask: 0/1 array (any
    integer or bool dtype) or None.  Returns (dh, da, dweight, dbias, dbias_in)."""
    x, dy, mean, rstd = _d(x), _d(dy), _d(mean), _d(rstd)
    w = None if w is None else _d(w)
    dres = None if dresidual is None else _d(dresidual)
    m = None if mask is None else np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)
    rows, cols = x.shape
    dh = np.empty_like(x)
    da = np.empty_like(x)
    dw = np.empty(cols, np.float64)
    db = np.empty(cols, np.float64)
    dbi = np.empty(cols, np.float64)
    _check(_load().oracle_bda_layernorm_backward(rows, cols, _ptr(x), _ptr(dy), _ptr(mean),
                                                 _ptr(rstd), _ptr(w), _ptr(dres), _ptr(m), scale,
                                                 _ptr(dh), _ptr(da), _ptr(dw), _ptr(db), _ptr(dbi)),
           "oracle_bda_layernorm_backward")
    return dh, da, dw, db, dbi


def rmsnorm_rms(x, *, eps=1e-5, threads=1):
    _threads(threads)
    x = _d(x)
    rows, cols = x.shape
    rms = np.empty(rows, np.float64)
    _check(_load().oracle_rmsnorm_rms(rows, cols, _ptr(x), eps, _ptr(rms)), "oracle_rmsnorm_rms")
    return rms


def rmsnorm_forward(x, w=None, *, eps=1e-5):
    """Returns (y, rms[rows])."""
    x = _d(x)
    rows, cols = x.shape
    w = None if w is None else _d(w)
    y = np.empty_like(x)
    rms = np.empty(rows, np.float64)
    _check(_load().oracle_rmsnorm_forward(rows, cols, _ptr(x), _ptr(w), eps, _ptr(y), _ptr(rms)),
           "oracle_rmsnorm_forward")
    return y, rms


def rmsnorm_backward(x, dy, w, rms=None, *, eps=1e-5, threads=1):
    """Returns (dx, dweight).  rms=None recomputes rms from x with eps;
    w=None means weight 1."""
    _threads(threads)
    x, dy = _d(x), _d(dy)
    w = None if w is None else _d(w)
    rms = None if rms is None else _d(rms)
    rows, cols = x.shape
    dx = np.empty_like(x)
    dw = np.empty(cols, np.float64)
    _check(_load().oracle_rmsnorm_backward(rows, cols, _ptr(x), _ptr(dy), _ptr(w), _ptr(rms),
                                           eps, _ptr(dx), _ptr(dw)),
           "oracle_rmsnorm_backward")
    return dx, dw
