"""Plain CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it
and shares no code with it.

The arithmetic lives in ``oracle.c`` (double-precision seven-loop
convolution and two-pass GroupNorm, see the header of that file for the
passages it follows).  This module compiles it with gcc, loads it with
ctypes and marshals numpy arrays.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(delta kernel, all-ones tap counts, per-channel 2-D correlation from scipy,
explicit im2col x matmul, scatter-form brute force, torch float64 conv and
group_norm on the CPU, GroupNorm closed-form invariants, the pages' printed
geometry in ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# GCONV_SANITIZED=1 selects the AddressSanitizer/UndefinedBehaviorSanitizer
# build (see build(sanitize=True)); the process must then preload clang's
# ASan runtime, as tests/sanitize_host.py does.
_SANITIZED = os.environ.get("GCONV_SANITIZED") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZED else "liboracle.so")
_lib = None
CLANG = "/opt/rocm/llvm/bin/clang"
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                  "-shared-libsan", "-g"]


def build(force: bool = False, sanitize: bool = None) -> str:
    """Compile oracle.c -> liboracle.so with gcc (-O2, no fast-math), or with
    sanitize -> liboracle_san.so with clang, AddressSanitizer and
    UndefinedBehaviorSanitizer (-O1, the same OpenMP loops)."""
    if sanitize is None:
        sanitize = _SANITIZED
    lib = os.path.join(_HERE, "liboracle_san.so" if sanitize else "liboracle.so")
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        if sanitize:
            cmd = [CLANG, "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"] + SANITIZE_FLAGS + \
                  [_SRC, "-o", tmp, "-lm"]
        else:
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i, p, d = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.oracle_out_dim.argtypes = [i, i, i, i, i]
        lib.oracle_out_dim.restype = i
        lib.oracle_conv2d.argtypes = [i] * 11 + [p, p, p, p, p, i]
        lib.oracle_conv2d.restype = i
        lib.oracle_conv2d_points.argtypes = [i] * 11 + [p, p, p, ctypes.c_int64, p, p, p, i]
        lib.oracle_conv2d_points.restype = i
        lib.oracle_fused_gn.argtypes = [i] * 11 + [p] * 6 + [i, d, p, p, i]
        lib.oracle_fused_gn.restype = i
        lib.oracle_conv2d_2d.argtypes = [i] * 14 + [p, p, p, p, p, i]
        lib.oracle_conv2d_2d.restype = i
        lib.oracle_conv2d_points_2d.argtypes = [i] * 14 + [p, p, p, ctypes.c_int64, p, p, p, i]
        lib.oracle_conv2d_points_2d.restype = i
        lib.oracle_fused_gn_2d.argtypes = [i] * 14 + [p] * 6 + [i, d, p, p, i]
        lib.oracle_fused_gn_2d.restype = i
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def out_dim(n: int, k: int, stride: int, pad: int, dil: int) -> int:
    return _load().oracle_out_dim(n, k, stride, pad, dil)


def _pair(v):
    """An int for both axes or an (h, w) pair."""
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise ValueError("expected an int or an (h, w) pair, got %r" % (v,))
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _axes(stride, pad, dil):
    (sh, sw), (ph, pw), (dh, dw) = _pair(stride), _pair(pad), _pair(dil)
    return sh, sw, ph, pw, dh, dw


def _geom(x, w, groups):
    N, C, H, W = x.shape
    K, cin, R, S = w.shape
    if cin * groups != C:
        raise ValueError("weight shape %s does not match C=%d, groups=%d" % (w.shape, C, groups))
    return N, C, H, W, K, R, S


def conv2d(x, w, bias=None, stride=1, pad=0, dil=1, groups=1, threads=None, want_bound=True):
    """Returns (y, A): y the float64 conv output, A = sum |x*w| per output.
    stride, pad and dil are ints or (h, w) pairs."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    N, C, H, W, K, R, S = _geom(x, w, groups)
    sh, sw, ph, pw, dh, dw = _axes(stride, pad, dil)
    Ho, Wo = out_dim(H, R, sh, ph, dh), out_dim(W, S, sw, pw, dw)
    y = np.empty((N, K, Ho, Wo), dtype=np.float64)
    A = np.empty_like(y) if want_bound else None
    rc = _load().oracle_conv2d_2d(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups,
                                  _ptr(x), _ptr(w), _ptr(bias), _ptr(y), _ptr(A),
                                  threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_conv2d rejected the geometry (rc=%d)" % rc)
    return y, A


def conv2d_points(x, w, idx, bias=None, stride=1, pad=0, dil=1, groups=1, threads=None):
    """Conv output and bound at flat NCHW output indices `idx` (int64)."""
    x, w, bias = _f32(x), _f32(w), _f32(bias)
    N, C, H, W, K, R, S = _geom(x, w, groups)
    sh, sw, ph, pw, dh, dw = _axes(stride, pad, dil)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    y = np.empty(idx.shape, dtype=np.float64)
    A = np.empty_like(y)
    rc = _load().oracle_conv2d_points_2d(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups,
                                         _ptr(x), _ptr(w), _ptr(bias), idx.size, _ptr(idx),
                                         _ptr(y), _ptr(A), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_conv2d_points rejected the input (rc=%d)" % rc)
    return y, A


def fused_gn(x, w, bias, scale, gamma, beta, gn_groups, eps=1e-5, stride=1, pad=0, dil=1,
             groups=1, threads=None, want_v=False):
    """conv -> +bias -> *scale -> sigmoid -> GroupNorm.  Returns out (and v)."""
    x, w = _f32(x), _f32(w)
    bias, scale, gamma, beta = _f32(bias), _f32(scale), _f32(gamma), _f32(beta)
    N, C, H, W, K, R, S = _geom(x, w, groups)
    sh, sw, ph, pw, dh, dw = _axes(stride, pad, dil)
    Ho, Wo = out_dim(H, R, sh, ph, dh), out_dim(W, S, sw, pw, dw)
    out = np.empty((N, K, Ho, Wo), dtype=np.float64)
    v = np.empty_like(out) if want_v else None
    rc = _load().oracle_fused_gn_2d(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups,
                                    _ptr(x), _ptr(w), _ptr(bias), _ptr(scale), _ptr(gamma),
                                    _ptr(beta), gn_groups, float(eps), _ptr(v), _ptr(out),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_fused_gn rejected the input (rc=%d)" % rc)
    return (out, v) if want_v else out
