"""fp64 CPU oracle for the fused convolution hot path.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers.  The product library never
imports, links or runs anything here, and nothing here imports the product package.

The arithmetic lives in ``oracle.c`` (plain nested loops, fp64 accumulation, OpenMP
only across independent outputs).  This module only marshals numpy arrays into it.
Each wrapper names the page passage its C function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_DIR = Path(__file__).resolve().parent
_SRC = _DIR / "oracle.c"
_LIB = _DIR / "liboracle.so"
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = False) -> Path:
    """Compile oracle.c into liboracle.so with gcc (-O2 -fopenmp)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-o", str(tmp), str(_SRC), "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(str(_LIB))
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_out_len.restype = _i64
        lib.oracle_out_len.argtypes = [_i64] * 5
        lib.oracle_conv3d.argtypes = [_f32p, _f32p, _f32p, _f64p] + [_i64] * 9
        lib.oracle_mish_tanh.argtypes = [_f64p, _f64p, _i64]
        lib.oracle_conv3d_mish_tanh.argtypes = [_f32p, _f32p, _f32p, _f64p] + [_i64] * 9
        lib.oracle_conv3d_mish_tanh_at.argtypes = (
            [_f32p, _f32p, _f32p, _i64p, _i64, _f64p] + [_i64] * 9)
        lib.oracle_conv3d_div_maxpool_gap_bias_sum.argtypes = (
            [_f32p, _f32p, _f32p, ctypes.c_double, _i64, _f32p, _f64p] + [_i64] * 7)
        lib.oracle_conv3d_div_maxpool.argtypes = (
            [_f32p, _f32p, _f32p, ctypes.c_double, _i64, _f64p] + [_i64] * 7)
        lib.oracle_dwsep_conv2d.argtypes = (
            [_f32p, _f32p, _f32p, _f32p, _f32p, _f64p, _f64p] + [_i64] * 9)
        lib.oracle_dwsep_conv2d_at.argtypes = (
            [_f32p, _f32p, _f32p, _f32p, _f32p, _i64p, _i64, _f64p] + [_i64] * 9)
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_f32p)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (code %d)" % (what, rc))


def threads() -> int:
    """OpenMP threads the oracle runs on (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_threads())


def out_len(n, k, stride=1, pad=0, dilation=1) -> int:
    """floor((n + 2p - d(k-1) - 1)/s) + 1 (page l1_p86 output-size formula)."""
    return int(_load().oracle_out_len(n, k, stride, pad, dilation))


def conv3d(x, w, b=None, stride=1, pad=0):
    """Cross-correlation Conv3d (+bias) in fp64; page l2_p47 naive kernel."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(b)
    N, C, D, H, W = x.shape
    O, C2, k, k2, k3 = w.shape
    assert C2 == C and k == k2 == k3
    shp = (N, O) + tuple(out_len(s, k, stride, pad) for s in (D, H, W))
    y = np.empty(shp, np.float64)
    _check(lib.oracle_conv3d(xp, wp, bp, y.ctypes.data_as(_f64p), N, C, D, H, W, O, k,
                             stride, pad), "conv3d")
    return y


def mish_tanh(v):
    """tanh(v * tanh(softplus(v))) with the threshold-20 softplus (page l2_p47)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    _check(_load().oracle_mish_tanh(v.ctypes.data_as(_f64p), out.ctypes.data_as(_f64p),
                                    v.size), "mish_tanh")
    return out


def conv3d_mish_tanh(x, w, b=None, stride=1, pad=0):
    """y = tanh(mish(conv3d(x) + b)) over the whole output (page l2_p47)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(b)
    N, C, D, H, W = x.shape
    O, _, k, _, _ = w.shape
    shp = (N, O) + tuple(out_len(s, k, stride, pad) for s in (D, H, W))
    y = np.empty(shp, np.float64)
    _check(lib.oracle_conv3d_mish_tanh(xp, wp, bp, y.ctypes.data_as(_f64p), N, C, D, H, W,
                                       O, k, stride, pad), "conv3d_mish_tanh")
    return y


def conv3d_mish_tanh_at(x, w, b, idx, stride=1, pad=0):
    """conv3d_mish_tanh only at flat output indices ``idx`` (sampled parity)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(w)
    b, bp = _f32(b)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    N, C, D, H, W = x.shape
    O, _, k, _, _ = w.shape
    out = np.empty(idx.shape, np.float64)
    _check(lib.oracle_conv3d_mish_tanh_at(xp, wp, bp, idx.ctypes.data_as(_i64p), idx.size,
                                          out.ctypes.data_as(_f64p), N, C, D, H, W, O, k,
                                          stride, pad), "conv3d_mish_tanh_at")
    return out


def conv3d_div_maxpool_gap_bias_sum(x, w, conv_b, divisor, pool, bias):
    """out[n] = sum_c(mean(maxpool((conv(x)+cb)/divisor)) + bias[c]) (page l2_p8)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(w)
    conv_b, cbp = _f32(conv_b)
    bias, biasp = _f32(np.asarray(bias).reshape(-1))
    N, C, D, H, W = x.shape
    O, _, k, _, _ = w.shape
    out = np.empty((N,), np.float64)
    _check(lib.oracle_conv3d_div_maxpool_gap_bias_sum(
        xp, wp, cbp, float(divisor), pool, biasp, out.ctypes.data_as(_f64p),
        N, C, D, H, W, O, k), "conv3d_div_maxpool_gap_bias_sum")
    return out


def conv3d_div_maxpool(x, w, conv_b, divisor, pool):
    """y = maxpool_pool((conv(x)+cb)/divisor), the pooled tensor [N,O,PD,PH,PW] (page l2_p8,
    the fused conv + divide + max-pool output)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(w)
    conv_b, cbp = _f32(conv_b)
    N, C, D, H, W = x.shape
    O, _, k, _, _ = w.shape
    dims = [out_len(out_len(s, k, 1, 0, 1), pool, pool, 0, 1) for s in (D, H, W)]
    y = np.empty((N, O, *dims), np.float64)
    _check(lib.oracle_conv3d_div_maxpool(xp, wp, cbp, float(divisor), pool,
                                         y.ctypes.data_as(_f64p), N, C, D, H, W, O, k),
           "conv3d_div_maxpool")
    return y


def dwsep_conv2d(x, dw_w, dw_b, pw_w, pw_b, stride=1, pad=1, dilation=1):
    """Depthwise KxK then pointwise 1x1, full output (page l1_p86)."""
    lib = _load()
    x, xp = _f32(x)
    dw_w, dwp = _f32(dw_w)
    dw_b, dbp = _f32(dw_b)
    pw_w, pwp = _f32(pw_w)
    pw_b, pbp = _f32(pw_b)
    N, C, H, W = x.shape
    K = dw_w.shape[-1]
    O = pw_w.shape[0]
    Ho, Wo = out_len(H, K, stride, pad, dilation), out_len(W, K, stride, pad, dilation)
    y = np.empty((N, O, Ho, Wo), np.float64)
    scratch = np.empty((N, C, Ho, Wo), np.float64)
    _check(lib.oracle_dwsep_conv2d(xp, dwp, dbp, pwp, pbp, y.ctypes.data_as(_f64p),
                                   scratch.ctypes.data_as(_f64p), N, C, H, W, O, K, stride,
                                   pad, dilation), "dwsep_conv2d")
    return y


def dwsep_conv2d_at(x, dw_w, dw_b, pw_w, pw_b, idx, stride=1, pad=1, dilation=1):
    """dwsep_conv2d only at flat output indices ``idx`` (sampled parity)."""
    lib = _load()
    x, xp = _f32(x)
    dw_w, dwp = _f32(dw_w)
    dw_b, dbp = _f32(dw_b)
    pw_w, pwp = _f32(pw_w)
    pw_b, pbp = _f32(pw_b)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    N, C, H, W = x.shape
    K = dw_w.shape[-1]
    O = pw_w.shape[0]
    out = np.empty(idx.shape, np.float64)
    _check(lib.oracle_dwsep_conv2d_at(xp, dwp, dbp, pwp, pbp, idx.ctypes.data_as(_i64p),
                                      idx.size, out.ctypes.data_as(_f64p), N, C, H, W, O, K,
                                      stride, pad, dilation), "dwsep_conv2d_at")
    return out
