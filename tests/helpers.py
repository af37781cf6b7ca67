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


def announce(name: str):
    print("[gpu-case] %s" % name, file=sys.__stderr__, flush=True)
