"""numpy wrappers around the plain fp64 CPU oracle in oracle.c.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only users. The product path never imports
this module, and this module imports nothing from the product package.

All fp16 tensors are passed and returned as numpy uint16 bit patterns; trellis
codes are uint32 words (format described at the top of oracle.c).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None

# A test may point the loader at another build of the same source (the
# mutation tests run the pins against deliberately broken copies, in their
# own process); nothing else sets this.
_OVERRIDE_ENV = "EXL3_ORACLE_LIB_OVERRIDE"


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get(_OVERRIDE_ENV)
        if not path:
            path = build()
        L = ctypes.CDLL(path)
        L.oracle_f16_to_f64.argtypes = [_u16p, _f64p, _i64]
        L.oracle_f64_to_f16.argtypes = [_f64p, _u16p, _i64]
        L.oracle_trellis_states.argtypes = [_u32p, _i64, _i64, _i64, _u16p]
        L.oracle_reconstruct.argtypes = [_u32p, _u16p, _u16p, _i64, _i64, _i64, _i64, _i64, _u16p]
        L.oracle_hadamard_matrix.argtypes = [_i8p]
        L.oracle_had128.argtypes = [_u16p, _i64, _i64, ctypes.c_void_p, ctypes.c_void_p, _u16p]
        L.oracle_exl3_linear.argtypes = [_u16p, _i64, _i64p, _i64, _u32p, _u16p, _u16p, _u16p,
                                         _u16p, _i64, _i64, _i64, _u16p]
        L.oracle_padded_width.argtypes = [_i64, _i64]
        L.oracle_padded_width.restype = _i64
        L.oracle_logits.argtypes = [_u16p, _i64, _i64p, _i64, _u16p, _i64, _i64, _i64, _u16p, _i64p]
        L.oracle_head_logits.argtypes = [_u16p, _i64, _i64p, _i64, _u32p, _u16p, _u16p, _u16p, _u16p,
                                         _i64, _i64, _i64, _i64, _u16p, _i64p]
        _lib = L
    return _lib


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


def f16_to_f64(h) -> np.ndarray:
    h = _u16(h)
    out = np.empty(h.shape, np.float64)
    lib().oracle_f16_to_f64(h.ravel(), out.ravel(), h.size)
    return out


def f64_to_f16(d) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float64)
    out = np.empty(d.shape, np.uint16)
    lib().oracle_f64_to_f16(d.ravel(), out.ravel(), d.size)
    return out


def _codes(codes, K: int, N: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint32)
    if not 1 <= bits <= 8 or codes.size != K * N * bits // 32:
        raise ValueError("codes must hold K*N*bits/32 words, bits in 1..8")
    return codes


def trellis_states(codes, K: int, N: int, bits: int = 4) -> np.ndarray:
    out = np.empty((K, N), np.uint16)
    lib().oracle_trellis_states(_codes(codes, K, N, bits), K, N, bits, out)
    return out


def reconstruct(codes, cb, scale, K: int, N: int, n0: int = 0, n_count: int | None = None, bits: int = 4):
    if n_count is None:
        n_count = N - n0
    out = np.empty((K, n_count), np.uint16)
    lib().oracle_reconstruct(_codes(codes, K, N, bits), _u16(cb), _u16(scale), K, N, bits, n0, n_count, out)
    return out


def hadamard_matrix() -> np.ndarray:
    h = np.empty((128, 128), np.int8)
    lib().oracle_hadamard_matrix(h)
    return h


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def had128(x, sign_pre=None, sign_post=None) -> np.ndarray:
    x = _u16(x)
    rows, cols = x.shape
    sp = None if sign_pre is None else _u16(sign_pre)
    sq = None if sign_post is None else _u16(sign_post)
    out = np.empty_like(x)
    lib().oracle_had128(x, rows, cols, _ptr(sp), _ptr(sq), out)
    return out


def exl3_linear(x, layer: dict, cb, rows=None) -> np.ndarray:
    """Layer output for the listed rows of x (all rows by default)."""
    x = _u16(x)
    M, K = x.shape
    N = layer["N"]
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    y = np.empty((len(rows), N), np.uint16)
    bits = int(layer.get("bits", 4))
    lib().oracle_exl3_linear(x, M, rows, len(rows), _codes(layer["codes"], K, N, bits),
                             _u16(cb), _u16(layer["scale"]), _u16(layer["sign_k"]),
                             _u16(layer["sign_n"]), K, N, bits, y)
    return y


def padded_width(n_valid: int, w_rows: int) -> int:
    return int(lib().oracle_padded_width(n_valid, w_rows))


def logits(x, w, n_valid: int, rows=None):
    """(logits over the padded width, argmax) for the listed rows of x."""
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    w_rows = w.shape[0]
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    n_pad = padded_width(n_valid, w_rows)
    out = np.empty((len(rows), n_pad), np.uint16)
    am = np.empty(len(rows), np.int64)
    lib().oracle_logits(x, M, rows, len(rows), w, w_rows, K, n_valid, out, am)
    return out, am


def head_logits(x, layer: dict, cb, n_valid: int, rows=None):
    """(logits over the padded width, argmax) of a trellis-quantized head for
    the listed rows of x: the layer output's first padded_width(n_valid, N)
    columns, pads -inf, first maximum."""
    x = _u16(x)
    M, K = x.shape
    N = layer["N"]
    if not 1 <= n_valid <= N:
        raise ValueError("n_valid = %d outside [1, %d]" % (n_valid, N))
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    bits = int(layer.get("bits", 4))
    n_pad = padded_width(n_valid, N)
    out = np.empty((len(rows), n_pad), np.uint16)
    am = np.empty(len(rows), np.int64)
    lib().oracle_head_logits(x, M, rows, len(rows), _codes(layer["codes"], K, N, bits), _u16(cb),
                             _u16(layer["scale"]), _u16(layer["sign_k"]), _u16(layer["sign_n"]), K, N, bits,
                             n_valid, out, am)
    return out, am
