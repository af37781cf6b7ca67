"""ctypes binding of libexl3.so: the same entry points as include/exl3.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libexl3.so. torch supplies device memory and the current stream.
There is no fallback: if the library is missing or the device is not gfx950,
calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexl3.so")

EXL3_OK, EXL3_EINVAL, EXL3_ESHAPE, EXL3_ESCRATCH, EXL3_EWIDTH, EXL3_EHIP, EXL3_EARCH = range(7)
LAYOUT_KN, LAYOUT_NK = 0, 1
MAX_CHUNK_COLS = 32768
DEFAULT_PREFILL_MIN_M = 128

EXPORTS = (
    "exl3_linear",
    "exl3_linear_scratch_bytes",
    "exl3_head_logits_argmax",
    "exl3_head_scratch_bytes",
    "exl3_reconstruct",
    "had_r_128",
    "logits_pad_mask_argmax",
    "logits_padded_width",
    "logits_scratch_bytes",
    "exl3_decode_states",
    "exl3_strerror",
)


class Exl3Layer(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("codebook", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("sign_k", ctypes.c_void_p),
        ("sign_n", ctypes.c_void_p),
        ("K", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("bits", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libexl3.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.exl3_linear.argtypes = [ctypes.POINTER(Exl3Layer), vp, i64, vp, vp, sz, i32, vp]
        L.exl3_linear.restype = ctypes.c_int
        L.exl3_linear_scratch_bytes.argtypes = [i32, i32, i64, i32]
        L.exl3_linear_scratch_bytes.restype = sz
        L.exl3_head_logits_argmax.argtypes = [ctypes.POINTER(Exl3Layer), vp, i64, i64, vp, i64, vp, vp, sz, i32, vp]
        L.exl3_head_logits_argmax.restype = ctypes.c_int
        L.exl3_head_scratch_bytes.argtypes = [i32, i32, i64, i64, i32]
        L.exl3_head_scratch_bytes.restype = sz
        L.exl3_reconstruct.argtypes = [ctypes.POINTER(Exl3Layer), i32, i32, vp, i64, i32, vp]
        L.exl3_reconstruct.restype = ctypes.c_int
        L.had_r_128.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.had_r_128.restype = ctypes.c_int
        L.logits_pad_mask_argmax.argtypes = [vp, i64, i32, vp, i64, i64, vp, i64, vp, vp, sz, vp]
        L.logits_pad_mask_argmax.restype = ctypes.c_int
        L.logits_padded_width.argtypes = [i64, i64]
        L.logits_padded_width.restype = i64
        L.logits_scratch_bytes.argtypes = [i64, i32, i64, i64]
        L.logits_scratch_bytes.restype = sz
        L.exl3_decode_states.argtypes = [ctypes.POINTER(Exl3Layer), vp, vp]
        L.exl3_decode_states.restype = ctypes.c_int
        L.exl3_strerror.argtypes = [ctypes.c_int]
        L.exl3_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def check(status: int) -> None:
    if status == EXL3_OK:
        return
    msg = lib().exl3_strerror(status).decode()
    if status in (EXL3_EINVAL, EXL3_ESHAPE, EXL3_ESCRATCH, EXL3_EWIDTH):
        raise ValueError("exl3 status %d: %s" % (status, msg))
    raise RuntimeError("exl3 status %d: %s" % (status, msg))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def to_device_u16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device)


def to_device_u32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).to(device)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


class Layer:
    """A quantized layer resident in device memory."""

    def __init__(self, codes, codebook, scale, sign_k=None, sign_n=None, K=None, N=None, bits=4, device="cuda"):
        def dev(a, conv):
            if a is None or isinstance(a, torch.Tensor):
                return a
            return conv(a, device)

        self.codes = dev(codes, to_device_u32)
        self.codebook = dev(codebook, to_device_u16)
        self.scale = dev(scale, to_device_u16)
        self.sign_k = dev(sign_k, to_device_u16)
        self.sign_n = dev(sign_n, to_device_u16)
        self.K, self.N, self.bits = int(K), int(N), int(bits)
        self._c = Exl3Layer(_ptr(self.codes), _ptr(self.codebook), _ptr(self.scale), _ptr(self.sign_k),
                            _ptr(self.sign_n), self.K, self.N, self.bits)

    @classmethod
    def from_numpy(cls, spec: dict, codebook, device="cuda"):
        return cls(spec["codes"], codebook, spec["scale"], spec.get("sign_k"), spec.get("sign_n"),
                   K=spec["K"], N=spec["N"], bits=spec.get("bits", 4), device=device)

    @property
    def c(self):
        return ctypes.byref(self._c)


def linear_scratch_bytes(K: int, N: int, M: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M) -> int:
    return int(lib().exl3_linear_scratch_bytes(K, N, M, prefill_min_m))


def linear(x: torch.Tensor, layer: Layer, prefill_min_m: int = DEFAULT_PREFILL_MIN_M, scratch=None, out=None,
           stream=None) -> torch.Tensor:
    """y = layer(x): x is M x K fp16 (or int16 bit patterns) on the device."""
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, layer.N), dtype=x.dtype, device=x.device)
    need = linear_scratch_bytes(layer.K, layer.N, M, prefill_min_m)
    if scratch is None:
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check(lib().exl3_linear(layer.c, _ptr(x), M, _ptr(out), _ptr(scratch), scratch.numel(), prefill_min_m,
                            _stream(stream)))
    return out


def head_scratch_bytes(K: int, N: int, M: int, n_valid: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M) -> int:
    return int(lib().exl3_head_scratch_bytes(K, N, M, n_valid, prefill_min_m))


def head_logits_argmax(x: torch.Tensor, layer: Layer, n_valid: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M,
                       scratch=None, logits=None, argmax=None, stream=None):
    """(logits over the padded width, argmax) of a trellis-quantized head."""
    M = x.shape[0]
    n_pad = logits_padded_width(n_valid, layer.N)
    if logits is None:
        logits = torch.empty((M, max(n_pad, 8)), dtype=x.dtype, device=x.device)
    if argmax is None:
        argmax = torch.empty(M, dtype=torch.int64, device=x.device)
    if scratch is None:
        need = head_scratch_bytes(layer.K, layer.N, M, n_valid, prefill_min_m)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    check(lib().exl3_head_logits_argmax(layer.c, _ptr(x), M, n_valid, _ptr(logits), logits.stride(0), _ptr(argmax),
                                        _ptr(scratch), scratch.numel(), prefill_min_m, _stream(stream)))
    return logits, argmax


def reconstruct(layer: Layer, n0: int = 0, n_count: int | None = None, layout: int = LAYOUT_KN, out=None,
                ldw: int | None = None, stream=None) -> torch.Tensor:
    if n_count is None:
        n_count = layer.N - n0
    if out is None:
        shape = (layer.K, n_count) if layout == LAYOUT_KN else (n_count, layer.K)
        out = torch.empty(shape, dtype=torch.int16, device=layer.codes.device)
        ldw = shape[1]
    check(lib().exl3_reconstruct(layer.c, n0, n_count, _ptr(out), ldw, layout, _stream(stream)))
    return out


def decode_states(layer: Layer, stream=None) -> torch.Tensor:
    out = torch.empty((layer.K, layer.N), dtype=torch.int16, device=layer.codes.device)
    check(lib().exl3_decode_states(layer.c, _ptr(out), _stream(stream)))
    return out


def had_r_128(x: torch.Tensor, sign_pre=None, sign_post=None, out=None, stream=None) -> torch.Tensor:
    rows, cols = x.shape
    if out is None:
        out = torch.empty_like(x)
    check(lib().had_r_128(_ptr(x), _ptr(out), rows, cols, _ptr(sign_pre), _ptr(sign_post), _stream(stream)))
    return out


def logits_padded_width(n_valid: int, w_rows: int) -> int:
    return int(lib().logits_padded_width(n_valid, w_rows))


def logits_scratch_bytes(M: int, K: int, n_valid: int, w_rows: int) -> int:
    return int(lib().logits_scratch_bytes(M, K, n_valid, w_rows))


def logits_pad_mask_argmax(x: torch.Tensor, w: torch.Tensor, n_valid: int, scratch=None, logits=None,
                           ld_logits: int | None = None, argmax=None, stream=None):
    M, K = x.shape
    w_rows = w.shape[0]
    n_pad = logits_padded_width(n_valid, w_rows)
    if logits is None:
        logits = torch.empty((M, max(n_pad, 1)), dtype=x.dtype, device=x.device)
    if ld_logits is None:
        ld_logits = logits.stride(0)
    if argmax is None:
        argmax = torch.empty(M, dtype=torch.int64, device=x.device)
    if scratch is None:
        scratch = torch.empty(max(logits_scratch_bytes(M, K, n_valid, w_rows), 1), dtype=torch.uint8, device=x.device)
    check(lib().logits_pad_mask_argmax(_ptr(x), M, K, _ptr(w), w_rows, n_valid, _ptr(logits), ld_logits,
                                       _ptr(argmax), _ptr(scratch), scratch.numel(), _stream(stream)))
    return logits, argmax
