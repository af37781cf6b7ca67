"""ctypes binding of libexl3_measure.so (measure/measure.h): per-kernel timing
of libexl3's calls with caller-owned HIP events, and the ceiling probes.
Benchmarks and their tests use it; the product binding (_lib) does not."""
from __future__ import annotations

import ctypes
import os

from . import _lib

MEASURE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libexl3_measure.so")
DECODE, GEMM, LOGITS, RECONSTRUCT = 0, 1, 2, 3
VARIANT_AUTO, VARIANT_FUSED, VARIANT_RECON_GEMM, VARIANT_DEQUANT_GEMM, VARIANT_DEQUANT_WHOLE = 0, 1, 2, 3, 4
VARIANT_DEQUANT_GEMM8, VARIANT_DEQUANT8_WHOLE = 5, 6  # the eight-wave dequant-GEMM (split tail, whole units)
PROBE_WORKGROUPS = 256
PROBE_SINK_BYTES = 256 * 32 * 256 * 4
EXPORTS = (
    "exl3m_events_create",
    "exl3m_events_destroy",
    "exl3m_elapsed_ms",
    "exl3m_linear_marked",
    "exl3m_linear_scratch_bytes",
    "exl3m_head_marked",
    "exl3m_logits_marked",
    "exl3m_probe_lds_gather",
    "exl3m_probe_mfma",
    "exl3m_probe_stream",
    "exl3m_strerror",
)

_m = None


def mlib() -> ctypes.CDLL:
    global _m
    if _m is None:
        if not os.path.exists(MEASURE_PATH):
            raise ImportError("libexl3_measure.so is not built (%s); run __graft_entry__.build()" % MEASURE_PATH)
        L = ctypes.CDLL(MEASURE_PATH)
        vp, i32, i64, sz, ip = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        vpp = ctypes.POINTER(ctypes.c_void_p)
        L.exl3m_events_create.argtypes = [ip, vpp]
        L.exl3m_events_destroy.argtypes = [ip, vpp]
        L.exl3m_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
        L.exl3m_linear_marked.argtypes = [ctypes.POINTER(_lib.Exl3Layer), vp, i64, vp, vp, sz, i32, vp, ip, ip, vpp,
                                          vpp, ctypes.POINTER(ip), ip]
        L.exl3m_head_marked.argtypes = [ctypes.POINTER(_lib.Exl3Layer), vp, i64, i64, vp, i64, vp, vp, sz, i32, vp,
                                        ip, ip, vpp, vpp, ctypes.POINTER(ip)]
        L.exl3m_logits_marked.argtypes = [vp, i64, i32, vp, i64, i64, vp, i64, vp, vp, sz, vp, ip, ip, vpp, vpp,
                                          ctypes.POINTER(ip)]
        L.exl3m_probe_lds_gather.argtypes = [i64, vp, vp, vp]
        L.exl3m_probe_mfma.argtypes = [i64, vp, vp, vp]
        L.exl3m_probe_stream.argtypes = [i32, vp, vp, i64, vp, vp]
        L.exl3m_linear_scratch_bytes.argtypes = [i32, i32, i64, i32, ip]
        L.exl3m_strerror.argtypes = [ip]
        L.exl3m_strerror.restype = ctypes.c_char_p
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = ip
        L.exl3m_linear_scratch_bytes.restype = sz
        _m = L
    return _m


def linear_scratch_bytes(K: int, N: int, M: int, variant: int, prefill_min_m: int = 128) -> int:
    return int(mlib().exl3m_linear_scratch_bytes(K, N, M, prefill_min_m, variant))


def check(status: int) -> None:
    if status == _lib.EXL3_OK:
        return
    msg = mlib().exl3m_strerror(status).decode()
    if status in (_lib.EXL3_EINVAL, _lib.EXL3_ESHAPE, _lib.EXL3_ESCRATCH, _lib.EXL3_EWIDTH):
        raise ValueError("exl3 status %d: %s" % (status, msg))
    raise RuntimeError("exl3 status %d: %s" % (status, msg))


def linear_forced(layer, x, M, y, scratch, stream, variant):
    """One exl3_linear call (device tensors x, y, scratch) with the kernel
    sequence forced to `variant` instead of the row-count dispatch; scratch
    holds linear_scratch_bytes(K, N, M, variant). Nothing is timed."""
    used = ctypes.c_int(0)
    check(mlib().exl3m_linear_marked(layer.c, x.data_ptr(), M, y.data_ptr(), scratch.data_ptr(), scratch.numel(),
                                     128, stream, DECODE, 0, None, None, ctypes.byref(used), variant))


class KernelTimer:
    """Event pairs around every launch of one kind inside library calls.

    Each marked call records up to `per_call` pairs on its stream; read()
    waits for them and returns (summed milliseconds, launch count)."""

    def __init__(self, pairs: int = 256, per_call: int = 64):
        self.n = pairs
        self.per_call = per_call
        arr = ctypes.c_void_p * pairs
        self.start, self.stop = arr(), arr()
        check(mlib().exl3m_events_create(pairs, self.start))
        check(mlib().exl3m_events_create(pairs, self.stop))
        self.pending = {}  # kind -> number of pairs recorded since the last read
        self.next = 0

    def _slot(self):
        if self.next + self.per_call > self.n:
            raise RuntimeError("KernelTimer: read() before more than %d pairs are recorded" % self.n)
        off = self.next
        vpp = ctypes.POINTER(ctypes.c_void_p)
        s = ctypes.cast(ctypes.byref(self.start, off * ctypes.sizeof(ctypes.c_void_p)), vpp)
        e = ctypes.cast(ctypes.byref(self.stop, off * ctypes.sizeof(ctypes.c_void_p)), vpp)
        return off, s, e

    def linear(self, layer, x, M, y, scratch, prefill_min_m, stream, kind, variant=VARIANT_AUTO):
        off, s, e = self._slot()
        used = ctypes.c_int(0)
        check(mlib().exl3m_linear_marked(layer.c, x.data_ptr(), M, y.data_ptr(), scratch.data_ptr(), scratch.numel(),
                                         prefill_min_m, stream, kind, self.per_call, s, e, ctypes.byref(used),
                                         variant))
        self._record(kind, off, used.value)

    def linear_variant(self, layer, x, M, y, scratch, stream, variant):
        """One exl3_linear call with the kernel sequence forced, unmarked."""
        linear_forced(layer, x, M, y, scratch, stream, variant)

    def head(self, layer, x, M, n_valid, lg, ld, am, scratch, prefill_min_m, stream, kind):
        off, s, e = self._slot()
        used = ctypes.c_int(0)
        check(mlib().exl3m_head_marked(layer.c, x.data_ptr(), M, n_valid, lg.data_ptr(), ld, am.data_ptr(),
                                       scratch.data_ptr(), scratch.numel(), prefill_min_m, stream, kind,
                                       self.per_call, s, e, ctypes.byref(used)))
        self._record(kind, off, used.value)

    def logits(self, x, M, K, w, w_rows, n_valid, lg, ld, am, scratch, stream, kind=LOGITS):
        off, s, e = self._slot()
        used = ctypes.c_int(0)
        check(mlib().exl3m_logits_marked(x.data_ptr(), M, K, w.data_ptr(), w_rows, n_valid, lg.data_ptr(), ld,
                                         am.data_ptr(), scratch.data_ptr(), scratch.numel(), stream, kind,
                                         self.per_call, s, e, ctypes.byref(used)))
        self._record(kind, off, used.value)

    def _record(self, kind, off, used):
        self.pending.setdefault(kind, []).extend(range(off, off + used))
        self.next += used

    def read(self, kind):
        ms_total, idx = 0.0, self.pending.pop(kind, [])
        for i in idx:
            ms = ctypes.c_float(0.0)
            check(mlib().exl3m_elapsed_ms(self.start[i], self.stop[i], ctypes.byref(ms)))
            ms_total += ms.value
        if not self.pending:
            self.next = 0
        return ms_total, len(idx)

    def close(self):
        if self.n:
            check(mlib().exl3m_events_destroy(self.n, self.start))
            check(mlib().exl3m_events_destroy(self.n, self.stop))
            self.n = 0
