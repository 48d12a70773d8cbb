"""ctypes front end of the C oracle (TEST INFRASTRUCTURE ONLY).

Inputs are float32 numpy arrays (converted to C-contiguous float32); results
are float64 numpy arrays.  Every function forwards to the literal C
definitions in fconv_oracle.c; nothing is computed here.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long


def load():
    """Loads oracle/liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    _I = ctypes.c_int
    lib.oracle_conv2d_sizes_ex.argtypes = [_L, _L, _L, _L, _I, _i64p, _i64p, _i64p, _i64p]
    lib.oracle_conv2d_sizes_ex.restype = ctypes.c_int
    lib.oracle_conv2d_pool_sigmoid_sum_ex.argtypes = [
        _f32p, _L, _L, _L, _L, _f32p, _L, _L, _f32p, _L, _I, _I, _I, _i64p, _L, _f64p, _f64p, _f64p, _I]
    lib.oracle_conv2d_pool_sigmoid_sum_ex.restype = ctypes.c_int
    lib.oracle_conv2d_pooled_at_ex.argtypes = [
        _f32p, _L, _L, _L, _L, _f32p, _L, _L, _f32p, _L, _I, _I, _I, _i64p, _L, _f64p]
    lib.oracle_conv2d_pooled_at_ex.restype = ctypes.c_int
    lib.oracle_dwsep_tout.argtypes = [_L, _L, _L]
    lib.oracle_dwsep_tout.restype = _L
    lib.oracle_dwsep_tout_ex.argtypes = [_L, _L, _L, _L, _L]
    lib.oracle_dwsep_tout_ex.restype = _L
    lib.oracle_dwsep_conv1d_ex.argtypes = [
        _f32p, _L, _L, _L, _f32p, _L, _f32p, _L, _f32p, _L, _L, _L, _i64p, _L, _f64p, ctypes.c_int]
    lib.oracle_dwsep_conv1d_ex.restype = ctypes.c_int
    lib.oracle_dwsep_conv1d_at_ex.argtypes = [
        _f32p, _L, _L, _L, _f32p, _L, _f32p, _L, _f32p, _L, _L, _L, _i64p, _L, _f64p]
    lib.oracle_dwsep_conv1d_at_ex.restype = ctypes.c_int
    lib.oracle_dwsep_conv1d.argtypes = [
        _f32p, _L, _L, _L, _f32p, _L, _f32p, _L, _f32p, _L, _i64p, _L, _f64p, ctypes.c_int]
    lib.oracle_dwsep_conv1d.restype = ctypes.c_int
    lib.oracle_dwsep_conv1d_at.argtypes = [
        _f32p, _L, _L, _L, _f32p, _L, _f32p, _L, _f32p, _L, _i64p, _L, _f64p]
    lib.oracle_dwsep_conv1d_at.restype = ctypes.c_int
    _lib = lib
    return lib


def _threads(nthreads):
    if nthreads:
        return int(nthreads)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _fp(a):
    return None if a is None else a.ctypes.data_as(_f32p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


POOL_AVG, POOL_MAX = 0, 1


def conv2d_sizes(H, W, K, pool, ceil_mode=False):
    """(Hc, Wc, PH, PW) for a valid stride-1 conv of kernel K then a pool of size pool (floor or ceil mode)."""
    lib = load()
    out = [ctypes.c_long() for _ in range(4)]
    _check(lib.oracle_conv2d_sizes_ex(H, W, K, pool, int(bool(ceil_mode)), *[ctypes.byref(o) for o in out]),
           "conv2d_sizes")
    return tuple(o.value for o in out)


def conv2d_pool_sigmoid_sum(x, w, b, pool, batch_idx=None, want_part=False, want_pooled=False, nthreads=None,
                            pool_mode=POOL_AVG, relu=False, ceil_mode=False):
    """Literal Conv2d -> [ReLU] -> AvgPool2d or MaxPool2d(pool) -> sigmoid -> sum over (C, H, W).

    x [B,Cin,H,W], w [Cout,Cin,K,K], b [Cout] or None.  Returns out [nb]
    (float64), plus part [nb,Cout] and/or the pre-sigmoid pooled map
    [nb,Cout,PH,PW] when asked for.
    """
    lib = load()
    x, w = _f32(x), _f32(w)
    b = None if b is None else _f32(b)
    B, Cin, H, W = x.shape
    Cout, Cin2, K, K2 = w.shape
    if Cin2 != Cin or K2 != K or (b is not None and b.shape != (Cout,)):
        raise ValueError("shape mismatch")
    _, _, PH, PW = conv2d_sizes(H, W, K, pool, ceil_mode)
    if batch_idx is None:
        idx = None
        nb = B
    else:
        idx = np.ascontiguousarray(batch_idx, dtype=np.int64)
        nb = idx.size
    out = np.zeros(nb, dtype=np.float64)
    part = np.zeros((nb, Cout), dtype=np.float64) if want_part else None
    pooled = np.zeros((nb, Cout, PH, PW), dtype=np.float64) if want_pooled else None
    rc = lib.oracle_conv2d_pool_sigmoid_sum_ex(
        _fp(x), B, Cin, H, W, _fp(w), Cout, K, _fp(b), pool, int(pool_mode), int(bool(relu)), int(bool(ceil_mode)),
        None if idx is None else idx.ctypes.data_as(_i64p), nb,
        out.ctypes.data_as(_f64p),
        None if part is None else part.ctypes.data_as(_f64p),
        None if pooled is None else pooled.ctypes.data_as(_f64p),
        _threads(nthreads))
    _check(rc, "conv2d_pool_sigmoid_sum")
    res = [out]
    if want_part:
        res.append(part)
    if want_pooled:
        res.append(pooled)
    return res[0] if len(res) == 1 else tuple(res)


def conv2d_pooled_at(x, w, b, pool, idx, pool_mode=POOL_AVG, relu=False, ceil_mode=False):
    """Pre-sigmoid pooled values at positions idx [n,4] = (b, co, ph, pw)."""
    lib = load()
    x, w = _f32(x), _f32(w)
    b = None if b is None else _f32(b)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 4)
    out = np.zeros(idx.shape[0], dtype=np.float64)
    rc = lib.oracle_conv2d_pooled_at_ex(_fp(x), B, Cin, H, W, _fp(w), Cout, K, _fp(b), pool, int(pool_mode),
                                        int(bool(relu)), int(bool(ceil_mode)), idx.ctypes.data_as(_i64p),
                                        idx.shape[0], out.ctypes.data_as(_f64p))
    _check(rc, "conv2d_pooled_at")
    return out


def dwsep_tout(T, K, pad, stride=1, dilation=1):
    return int(load().oracle_dwsep_tout_ex(T, K, pad, stride, dilation))


def dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, batch_idx=None, nthreads=None, stride=1, dilation=1):
    """Literal depthwise Conv1d(K, pad, stride, dilation) -> pointwise 1x1 Conv1d + bias; y [nb,O,Tout] float64."""
    lib = load()
    x, w_dw, w_pw = _f32(x), _f32(w_dw), _f32(w_pw)
    b_pw = None if b_pw is None else _f32(b_pw)
    B, C, T = x.shape
    C2, K = w_dw.shape
    O, C3 = w_pw.shape
    if C2 != C or C3 != C or (b_pw is not None and b_pw.shape != (O,)):
        raise ValueError("shape mismatch")
    Tout = dwsep_tout(T, K, pad, stride, dilation)
    if Tout < 1:
        raise ValueError("empty output")
    if batch_idx is None:
        idx, nb = None, B
    else:
        idx = np.ascontiguousarray(batch_idx, dtype=np.int64)
        nb = idx.size
    y = np.zeros((nb, O, Tout), dtype=np.float64)
    rc = lib.oracle_dwsep_conv1d_ex(_fp(x), B, C, T, _fp(w_dw), K, _fp(w_pw), O, _fp(b_pw), pad, stride, dilation,
                                    None if idx is None else idx.ctypes.data_as(_i64p), nb,
                                    y.ctypes.data_as(_f64p), _threads(nthreads))
    _check(rc, "dwsep_conv1d")
    return y


def dwsep_conv1d_at(x, w_dw, w_pw, b_pw, pad, idx, stride=1, dilation=1):
    """y at positions idx [n,3] = (b, o, t), each from the definition."""
    lib = load()
    x, w_dw, w_pw = _f32(x), _f32(w_dw), _f32(w_pw)
    b_pw = None if b_pw is None else _f32(b_pw)
    B, C, T = x.shape
    _, K = w_dw.shape
    O, _ = w_pw.shape
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 3)
    y = np.zeros(idx.shape[0], dtype=np.float64)
    rc = lib.oracle_dwsep_conv1d_at_ex(_fp(x), B, C, T, _fp(w_dw), K, _fp(w_pw), O, _fp(b_pw), pad, stride,
                                       dilation, idx.ctypes.data_as(_i64p), idx.shape[0], y.ctypes.data_as(_f64p))
    _check(rc, "dwsep_conv1d_at")
    return y
