"""CPU reference for transposed convolution (ConvTranspose1d/2d, dense and grouped).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__ and
the CPU-baseline leg of bench.py may import this package.  The GPU library
never imports, links or calls it, and the two share no code.

The arithmetic lives in plain C (ctconv_oracle.c, double precision,
single-threaded); this module builds it with gcc and wraps it with ctypes.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ctconv_oracle.c")
_LIB = os.path.join(_HERE, "libctconv_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-D_GNU_SOURCE",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64p = ctypes.POINTER(ctypes.c_int64)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.ctconv_oracle_output_shape.argtypes = [ctypes.c_int] + [i64p] * 7
        lib.ctconv_oracle_conv_transpose.argtypes = (
            [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + [i64p] * 6 + [dp] * 4)
        lib.ctconv_oracle_points.argtypes = (
            [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + [i64p] * 6
            + [dp] * 3 + [i64p, ctypes.c_int64, dp])
        lib.ctconv_oracle_conv_transpose_grouped.argtypes = (
            [ctypes.c_int] + [ctypes.c_int64] * 4 + [i64p] * 6 + [dp] * 4)
        lib.ctconv_oracle_points_grouped.argtypes = (
            [ctypes.c_int] + [ctypes.c_int64] * 4 + [i64p] * 6
            + [dp] * 3 + [i64p, ctypes.c_int64, dp])
        lib.ctconv_oracle_istft_ola.argtypes = [ctypes.c_int64] * 4 + [dp, dp]
        lib.ctconv_oracle_rfft.argtypes = [ctypes.c_int64, dp, dp, dp]
        lib.ctconv_oracle_elu.argtypes = [ctypes.c_int64, dp, dp]
        lib.ctconv_oracle_elu.restype = None
        _lib = lib
    return _lib


def _i64(v: Sequence[int]):
    a = (ctypes.c_int64 * len(v))(*[int(t) for t in v])
    return a


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctypes.c_double))
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _per_dim(v, ndim):
    if isinstance(v, (int, np.integer)):
        return [int(v)] * ndim
    v = [int(t) for t in v]
    assert len(v) == ndim
    return v


def output_shape(in_spatial, kernel, stride, padding=0, output_padding=0, dilation=1):
    ndim = len(in_spatial)
    args = [_per_dim(a, ndim) for a in (in_spatial, kernel, stride, padding,
                                        output_padding, dilation)]
    out = (ctypes.c_int64 * ndim)()
    rc = _load().ctconv_oracle_output_shape(ndim, *[_i64(a) for a in args], out)
    if rc != 0:
        raise ValueError("invalid transposed-convolution parameters")
    return tuple(int(v) for v in out)


def conv_transpose(x, w, bias=None, stride=1, padding=0, output_padding=0, dilation=1):
    """y = ConvTranspose(x, w, bias) in float64 by the scatter definition.

    x [N, C_in, *sp], w [C_in, C_out, *k], bias [C_out] or None.
    """
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    ndim = x.ndim - 2
    N, C_in = x.shape[:2]
    C_out = w.shape[1]
    assert w.shape[0] == C_in and w.ndim == ndim + 2
    k = list(w.shape[2:])
    s, p, op, d = (_per_dim(a, ndim) for a in (stride, padding, output_padding, dilation))
    osp = output_shape(x.shape[2:], k, s, p, op, d)
    y = np.empty((N, C_out) + osp, dtype=np.float64)
    rc = _load().ctconv_oracle_conv_transpose(
        ndim, N, C_in, C_out, _i64(x.shape[2:]), _i64(k), _i64(s), _i64(p), _i64(op),
        _i64(d), _dp(x), _dp(w), _dp(b), _dp(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def conv_transpose_points(x, w, bias, idx, stride=1, padding=0, output_padding=0,
                          dilation=1):
    """Selected outputs; idx is an int array [P, 4] of (n, co, oy, ox) (1-D: oy = 0)."""
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    ndim = x.ndim - 2
    N, C_in = x.shape[:2]
    C_out = w.shape[1]
    k = list(w.shape[2:])
    s, p, op, d = (_per_dim(a, ndim) for a in (stride, padding, output_padding, dilation))
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    out = np.empty(idx.shape[0], dtype=np.float64)
    rc = _load().ctconv_oracle_points(
        ndim, N, C_in, C_out, _i64(x.shape[2:]), _i64(k), _i64(s), _i64(p), _i64(op),
        _i64(d), _dp(x), _dp(w), _dp(b),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.shape[0], _dp(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def conv_transpose_grouped(x, w, bias=None, groups=1, stride=1, padding=0, output_padding=0,
                           dilation=1):
    """Grouped ConvTranspose in float64 by the scatter definition.

    x [N, C_in, *sp], w [C_in, C_out / groups, *k], bias [C_out] or None;
    groups = C_in is the depthwise case.
    """
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    ndim = x.ndim - 2
    N, C_in = x.shape[:2]
    assert w.shape[0] == C_in and w.ndim == ndim + 2
    C_out = w.shape[1] * groups
    k = list(w.shape[2:])
    s, p, op, d = (_per_dim(a, ndim) for a in (stride, padding, output_padding, dilation))
    osp = output_shape(x.shape[2:], k, s, p, op, d)
    y = np.empty((N, C_out) + osp, dtype=np.float64)
    rc = _load().ctconv_oracle_conv_transpose_grouped(
        ndim, N, C_in, C_out, groups, _i64(x.shape[2:]), _i64(k), _i64(s), _i64(p), _i64(op),
        _i64(d), _dp(x), _dp(w), _dp(b), _dp(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def conv_transpose_grouped_points(x, w, bias, idx, groups=1, stride=1, padding=0,
                                  output_padding=0, dilation=1):
    """Selected outputs of the grouped case; idx [P, 4] of (n, co, oy, ox) (1-D: oy = 0)."""
    x = _f64(x)
    w = _f64(w)
    b = None if bias is None else _f64(bias)
    ndim = x.ndim - 2
    N, C_in = x.shape[:2]
    C_out = w.shape[1] * groups
    k = list(w.shape[2:])
    s, p, op, d = (_per_dim(a, ndim) for a in (stride, padding, output_padding, dilation))
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    out = np.empty(idx.shape[0], dtype=np.float64)
    rc = _load().ctconv_oracle_points_grouped(
        ndim, N, C_in, C_out, groups, _i64(x.shape[2:]), _i64(k), _i64(s), _i64(p), _i64(op),
        _i64(d), _dp(x), _dp(w), _dp(b),
        idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), idx.shape[0], _dp(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def istft_ola(spec, n_fft: int, hop: int):
    """Overlap-add inverse STFT of spec [N, n_fft + 2, T] (real | imaginary channels)."""
    spec = _f64(spec)
    N, C, T = spec.shape
    assert C == n_fft + 2
    y = np.empty((N, (T - 1) * hop + n_fft), dtype=np.float64)
    rc = _load().ctconv_oracle_istft_ola(N, n_fft, hop, T, _dp(spec), _dp(y))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def rfft(frame):
    frame = _f64(frame)
    n = frame.shape[0]
    re = np.empty(n // 2 + 1)
    im = np.empty(n // 2 + 1)
    if _load().ctconv_oracle_rfft(n, _dp(frame), _dp(re), _dp(im)) != 0:
        raise ValueError("length must be a power of two")
    return re, im


def elu(x):
    x = _f64(x)
    y = np.empty_like(x)
    _load().ctconv_oracle_elu(x.size, _dp(x), _dp(y))
    return y


def rel_l2(a, ref) -> float:
    """||a - ref||_2 / ||ref||_2 in float64 (max |a| when ref is all zero)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((a - ref) ** 2)))
    if den == 0.0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return num / den
