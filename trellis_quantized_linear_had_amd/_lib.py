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
NOALLOC_SCRATCH_BYTES = 48 * 1024 * 1024
DEFAULT_PREFILL_MIN_M = 128

EXPORTS = (
    "exl3_linear",
    "exl3_linear_scratch_bytes",
    "exl3_linear_noalloc",
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
        L.exl3_linear_noalloc.argtypes = [ctypes.POINTER(Exl3Layer), vp, i64, vp, i32, vp]
        L.exl3_linear_noalloc.restype = ctypes.c_int
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


_F16 = (torch.float16, torch.int16)  # fp16 values or their bit patterns


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _tensor(t, name: str, dtypes, shape=None, min_numel=None) -> None:
    """Shape, dtype and layout checks (before any device check, so they run
    anywhere): the C ABI receives bare pointers and cannot check these."""
    _require(isinstance(t, torch.Tensor), "%s must be a torch.Tensor" % name)
    _require(t.dtype in dtypes, "%s has dtype %s; expected one of %s" % (name, t.dtype, ", ".join(map(str, dtypes))))
    _require(t.is_contiguous(), "%s must be contiguous" % name)
    if shape is not None:
        _require(tuple(t.shape) == tuple(shape), "%s has shape %s; expected %s" % (name, tuple(t.shape), tuple(shape)))
    if min_numel is not None:
        _require(t.numel() >= min_numel, "%s holds %d elements; at least %d are needed" % (name, t.numel(), min_numel))


def _on(device, *named) -> None:
    """Every tensor on `device`, a GPU."""
    for name, t in named:
        if t is None:
            continue
        _require(t.is_cuda, "%s must be on a GPU (it is on %s)" % (name, t.device))
        _require(t.device == device, "%s is on %s; expected %s" % (name, t.device, device))


def _empty(shape, dtype, device, stream):
    """A temporary for one call. Allocated on the call's stream, so the caching
    allocator does not hand the memory to other work on the current stream
    while the call's kernels may still use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _scratch(scratch, need: int, device, stream):
    if scratch is None:
        return _empty(max(need, 1), torch.uint8, device, stream)
    _tensor(scratch, "scratch", (torch.uint8, torch.int8))
    _require(scratch.numel() >= need, "scratch holds %d bytes; this call needs %d" % (scratch.numel(), need))
    return scratch


def to_device_u16(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 bit patterns -> int16 device tensor holding the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(device)


def to_device_u32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).to(device)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


class Layer:
    """A quantized layer resident in device memory. The tensors are checked
    here for dtype, layout, size and device, once."""

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
        _require(self.K > 0 and self.N > 0 and self.K % 128 == 0 and self.N % 128 == 0,
                 "K = %d and N = %d must be positive multiples of 128" % (self.K, self.N))
        _require(1 <= self.bits <= 8, "bits = %d; 1 to 8 bits per weight are supported" % self.bits)
        _tensor(self.codes, "codes", (torch.int32, torch.uint32), min_numel=self.K * self.N * self.bits // 32)
        _tensor(self.codebook, "codebook", _F16, min_numel=65536)
        _tensor(self.scale, "scale", _F16, min_numel=self.N)
        if self.sign_k is not None:
            _tensor(self.sign_k, "sign_k", _F16, min_numel=self.K)
        if self.sign_n is not None:
            _tensor(self.sign_n, "sign_n", _F16, min_numel=self.N)
        self.device = self.codes.device
        if self.device.type == "cuda":
            _on(self.device, ("codebook", self.codebook), ("scale", self.scale), ("sign_k", self.sign_k),
                ("sign_n", self.sign_n))
        self._c = Exl3Layer(_ptr(self.codes), _ptr(self.codebook), _ptr(self.scale), _ptr(self.sign_k),
                            _ptr(self.sign_n), self.K, self.N, self.bits)

    @classmethod
    def from_numpy(cls, spec: dict, codebook, device="cuda"):
        return cls(spec["codes"], codebook, spec["scale"], spec.get("sign_k"), spec.get("sign_n"),
                   K=spec["K"], N=spec["N"], bits=spec.get("bits", 4), device=device)

    @property
    def c(self):
        return ctypes.byref(self._c)


def _rows_of(x: torch.Tensor, K: int, name: str = "x") -> int:
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "%s must be a 2-D tensor (rows x %d)" % (name, K))
    _tensor(x, name, _F16)
    _require(x.shape[1] == K, "%s has %d columns; the layer takes K = %d" % (name, x.shape[1], K))
    return int(x.shape[0])


def linear_scratch_bytes(K: int, N: int, M: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M) -> int:
    return int(lib().exl3_linear_scratch_bytes(K, N, M, prefill_min_m))


def linear(x: torch.Tensor, layer: Layer, prefill_min_m: int = DEFAULT_PREFILL_MIN_M, scratch=None, out=None,
           stream=None) -> torch.Tensor:
    """y = layer(x): x is M x K fp16 (or int16 bit patterns) on the device."""
    M = _rows_of(x, layer.K)
    if out is not None:
        _tensor(out, "out", _F16, shape=(M, layer.N))
    if scratch is not None:
        _tensor(scratch, "scratch", (torch.uint8, torch.int8))
    _on(layer.device, ("x", x), ("out", out), ("scratch", scratch))
    if out is None:
        out = _empty((M, layer.N), x.dtype, x.device, stream)
    scratch = _scratch(scratch, linear_scratch_bytes(layer.K, layer.N, M, prefill_min_m), x.device, stream)
    check(lib().exl3_linear(layer.c, _ptr(x), M, _ptr(out), _ptr(scratch), scratch.numel(), prefill_min_m,
                            _stream(stream)))
    return out


def linear_noalloc(x: torch.Tensor, layer: Layer, prefill_min_m: int = DEFAULT_PREFILL_MIN_M, out=None,
                   stream=None) -> torch.Tensor:
    """layer(x) through the allocation-free entry point (the library's own
    per-GPU scratch of NOALLOC_SCRATCH_BYTES; calls on one GPU must not
    overlap). `out` must be given where nothing may be allocated."""
    M = _rows_of(x, layer.K)
    if out is not None:
        _tensor(out, "out", _F16, shape=(M, layer.N))
    _on(layer.device, ("x", x), ("out", out))
    if out is None:
        out = _empty((M, layer.N), x.dtype, x.device, stream)
    check(lib().exl3_linear_noalloc(layer.c, _ptr(x), M, _ptr(out), prefill_min_m, _stream(stream)))
    return out


def head_scratch_bytes(K: int, N: int, M: int, n_valid: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M) -> int:
    return int(lib().exl3_head_scratch_bytes(K, N, M, n_valid, prefill_min_m))


def head_logits_argmax(x: torch.Tensor, layer: Layer, n_valid: int, prefill_min_m: int = DEFAULT_PREFILL_MIN_M,
                       scratch=None, logits=None, argmax=None, stream=None):
    """(logits over the padded width, argmax) of a trellis-quantized head."""
    M = _rows_of(x, layer.K)
    _require(1 <= n_valid <= layer.N, "n_valid = %d must be in [1, N = %d]" % (n_valid, layer.N))
    n_pad = logits_padded_width(n_valid, layer.N)
    if logits is not None:
        _require(logits.dim() == 2 and logits.shape[0] >= M and logits.shape[1] >= n_pad and logits.stride(1) == 1,
                 "logits must be (>= M) x (>= %d) with unit column stride" % n_pad)
        _require(logits.dtype in _F16, "logits has dtype %s" % logits.dtype)
    if argmax is not None:
        _tensor(argmax, "argmax", (torch.int64,), min_numel=M)
    if scratch is not None:
        _tensor(scratch, "scratch", (torch.uint8, torch.int8))
    _on(layer.device, ("x", x), ("logits", logits), ("argmax", argmax), ("scratch", scratch))
    if logits is None:
        logits = _empty((M, max(n_pad, 8)), x.dtype, x.device, stream)
    if argmax is None:
        argmax = _empty(M, torch.int64, x.device, stream)
    scratch = _scratch(scratch, head_scratch_bytes(layer.K, layer.N, M, n_valid, prefill_min_m), x.device, stream)
    check(lib().exl3_head_logits_argmax(layer.c, _ptr(x), M, n_valid, _ptr(logits), logits.stride(0), _ptr(argmax),
                                        _ptr(scratch), scratch.numel(), prefill_min_m, _stream(stream)))
    return logits, argmax


def reconstruct(layer: Layer, n0: int = 0, n_count: int | None = None, layout: int = LAYOUT_KN, out=None,
                ldw: int | None = None, stream=None) -> torch.Tensor:
    if n_count is None:
        n_count = layer.N - n0
    _require(layout in (LAYOUT_KN, LAYOUT_NK), "unknown layout %r" % (layout,))
    rows, cols = (layer.K, n_count) if layout == LAYOUT_KN else (n_count, layer.K)
    if out is None:
        _on(layer.device, ("codes", layer.codes))
        out = _empty((rows, cols), torch.int16, layer.device, stream)
        ldw = cols
    else:
        _require(out.dtype in _F16 and out.dim() == 2, "out must be a 2-D fp16 or int16 tensor")
        if ldw is None:
            ldw = out.stride(0)
        _require(out.stride(1) == 1 and out.stride(0) == ldw, "out must have unit column stride and row stride ldw")
        _require(out.shape[0] >= rows and out.shape[1] >= cols,
                 "out has shape %s; at least (%d, %d) is needed" % (tuple(out.shape), rows, cols))
        _on(layer.device, ("out", out))
    check(lib().exl3_reconstruct(layer.c, n0, n_count, _ptr(out), ldw, layout, _stream(stream)))
    return out


def decode_states(layer: Layer, stream=None) -> torch.Tensor:
    _on(layer.device, ("codes", layer.codes))
    out = _empty((layer.K, layer.N), torch.int16, layer.device, stream)
    check(lib().exl3_decode_states(layer.c, _ptr(out), _stream(stream)))
    return out


def had_r_128(x: torch.Tensor, sign_pre=None, sign_post=None, out=None, stream=None) -> torch.Tensor:
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor")
    _tensor(x, "x", _F16)
    rows, cols = x.shape
    for name, t in (("sign_pre", sign_pre), ("sign_post", sign_post)):
        if t is not None:
            _tensor(t, name, _F16, min_numel=cols)
    if out is not None:
        _tensor(out, "out", _F16, shape=(rows, cols))
    _on(x.device, ("x", x), ("sign_pre", sign_pre), ("sign_post", sign_post), ("out", out))
    if out is None:
        out = _empty((rows, cols), x.dtype, x.device, stream)
    check(lib().had_r_128(_ptr(x), _ptr(out), rows, cols, _ptr(sign_pre), _ptr(sign_post), _stream(stream)))
    return out


def logits_padded_width(n_valid: int, w_rows: int) -> int:
    return int(lib().logits_padded_width(n_valid, w_rows))


def logits_scratch_bytes(M: int, K: int, n_valid: int, w_rows: int) -> int:
    return int(lib().logits_scratch_bytes(M, K, n_valid, w_rows))


def logits_pad_mask_argmax(x: torch.Tensor, w: torch.Tensor, n_valid: int, scratch=None, logits=None,
                           ld_logits: int | None = None, argmax=None, stream=None):
    _require(isinstance(w, torch.Tensor) and w.dim() == 2, "w must be a 2-D tensor (rows x K)")
    _tensor(w, "w", _F16)
    w_rows, K = int(w.shape[0]), int(w.shape[1])
    M = _rows_of(x, K)
    n_pad = logits_padded_width(n_valid, w_rows)
    _require(n_pad > 0, "n_valid = %d must be in [1, w_rows = %d]" % (n_valid, w_rows))
    if logits is not None:
        _require(logits.dim() == 2 and logits.shape[0] >= M and logits.stride(1) == 1 and logits.dtype in _F16,
                 "logits must be an (>= M) x (>= n_pad) fp16 or int16 tensor with unit column stride")
        if ld_logits is None:
            ld_logits = logits.stride(0)
        _require(ld_logits == logits.stride(0) and logits.shape[1] >= n_pad,
                 "logits has %d columns and row stride %d; ld_logits %s and n_pad %d"
                 % (logits.shape[1], logits.stride(0), ld_logits, n_pad))
    if argmax is not None:
        _tensor(argmax, "argmax", (torch.int64,), min_numel=M)
    if scratch is not None:
        _tensor(scratch, "scratch", (torch.uint8, torch.int8))
    _on(x.device, ("x", x), ("w", w), ("logits", logits), ("argmax", argmax), ("scratch", scratch))
    if logits is None:
        logits = _empty((M, n_pad), x.dtype, x.device, stream)
        ld_logits = n_pad
    if argmax is None:
        argmax = _empty(M, torch.int64, x.device, stream)
    scratch = _scratch(scratch, logits_scratch_bytes(M, K, n_valid, w_rows), x.device, stream)
    check(lib().logits_pad_mask_argmax(_ptr(x), M, K, _ptr(w), w_rows, n_valid, _ptr(logits), ld_logits,
                                       _ptr(argmax), _ptr(scratch), scratch.numel(), _stream(stream)))
    return logits, argmax
