"""Shared test helpers: tolerance checks and device-tensor plumbing."""
from __future__ import annotations

import sys

import numpy as np
import pytest

# Per-row output tolerance: max_n |y - y_ref| <= 2e-3 * max_n |y_ref| (fp16
# output, fp32 accumulation).
Y_REL_TOL = 2e-3


def val(h) -> np.ndarray:
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def assert_rows_close(y_gpu_u16, y_ref_u16, tol=Y_REL_TOL, what="y"):
    g, r = val(y_gpu_u16), val(y_ref_u16)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "%s has non-finite values" % what
    err = np.max(np.abs(g - r), axis=1)
    scale = np.max(np.abs(r), axis=1)
    worst = int(np.argmax(err / np.maximum(scale, 1e-30)))
    assert np.all(err <= tol * scale), (
        "%s: row %d max|err| %.3e > %.1e * rowmax %.3e" % (what, worst, err[worst], tol, scale[worst]))
    return float(np.max(err / np.maximum(scale, 1e-30)))


def ulp_diff(a_u16, b_u16) -> np.ndarray:
    """Distance in fp16 units in the last place (same-sign finite values)."""
    a = np.asarray(a_u16, np.uint16).astype(np.int32)
    b = np.asarray(b_u16, np.uint16).astype(np.int32)

    def ordered(x):
        return np.where(x & 0x8000, -(x & 0x7FFF), x)

    return np.abs(ordered(a) - ordered(b))


def ulp16(ref_u16) -> np.ndarray:
    """Spacing of fp16 values at |ref| (2^-24 in the subnormal range)."""
    v = np.abs(val(ref_u16))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -14)))
    return np.exp2(e - 10)


def assert_logits_close(lg_u16, ref_u16, K: int):
    """fp16 logits from fp32 accumulation against the fp64 oracle: one fp16
    rounding step plus the worst-case fp32 accumulation error over K terms,
    with partial sums bounded by the row's largest logit."""
    g, r = val(lg_u16), val(ref_u16)
    assert np.all(np.isfinite(g))
    rowmax = np.max(np.abs(r), axis=1, keepdims=True)
    tol = ulp16(ref_u16) + K * 2.0 ** -24 * rowmax
    bad = np.abs(g - r) > tol
    assert not np.any(bad), (np.argwhere(bad)[:5], g[bad][:5], r[bad][:5])


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # Where a GPU is present the native library must be there: import failures are errors.
    from trellis_quantized_linear_had_amd import _lib

    _lib.lib()
    return torch


# exl3_linear's kernel sequences: the decode-GEMM ("fused"), reconstruct +
# GEMM ("recon") and the dequant-GEMMs ("dq8", eight waves, and "dq", four
# waves, forced only; 4 bits only). At 4 bits the dispatch takes the
# eight-wave dequant-GEMM from 33 rows on the fused side and up to 1024 rows
# on the prefill side.
DQ_FUSED_MIN_ROWS, DQ_PREFILL_MAX_ROWS = 33, 1024


def route(bits: int, M: int, pm: int) -> str:
    prefill = pm > 0 and M >= pm
    if bits == 4 and (M <= DQ_PREFILL_MAX_ROWS if prefill else M >= DQ_FUSED_MIN_ROWS):
        return "dq8"
    return "recon" if prefill else "fused"


def linear_forced(lay, x, route_name: str, out=None, scratch=None, sync: bool = True):
    """exl3_linear with its kernel sequence forced (through the measurement
    library); x is a host uint16 array or a device tensor. Returns the host
    output if sync, else the device output."""
    import torch

    from trellis_quantized_linear_had_amd import _lib, _measure

    variant = {"fused": _measure.VARIANT_FUSED, "recon": _measure.VARIANT_RECON_GEMM,
               "dq": _measure.VARIANT_DEQUANT_GEMM, "dq_whole": _measure.VARIANT_DEQUANT_WHOLE,
               "dq8": _measure.VARIANT_DEQUANT_GEMM8, "dq8_whole": _measure.VARIANT_DEQUANT8_WHOLE}[route_name]
    xd = x if isinstance(x, torch.Tensor) else _lib.to_device_u16(x)
    M = xd.shape[0]
    if out is None:
        out = torch.full((M, lay.N), 0x7E7E, dtype=torch.int16, device="cuda")
    if scratch is None:
        scratch = torch.empty(max(1, _measure.linear_scratch_bytes(lay.K, lay.N, M, variant)), dtype=torch.uint8,
                              device="cuda")
    _measure.linear_forced(lay, xd, M, out, scratch, torch.cuda.current_stream().cuda_stream, variant)
    if not sync:
        return out
    torch.cuda.synchronize()
    return _lib.to_host_u16(out)


def announce(name: str):
    print("[gpu-case] %s" % name, file=sys.__stderr__, flush=True)
