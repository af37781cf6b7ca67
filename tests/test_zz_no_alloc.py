"""The allocation-free entry point (exl3_linear_noalloc: the library's own
per-GPU scratch array instead of a caller-owned buffer) gives exactly
exl3_linear's output, on two calls in a row with the second smaller (the
array keeps the first call's contents), on the fused and the prefill path;
calls whose scratch exceeds the array are refused before any launch."""
import numpy as np
import pytest

import workloads as WL
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


@pytest.fixture(scope="module")
def X(T):
    import trellis_quantized_linear_had_amd as X

    return X


def both(T, X, lay, x, pm):
    from trellis_quantized_linear_had_amd import _lib

    xd = _lib.to_device_u16(x)
    ref = X.linear(xd, lay, prefill_min_m=pm)
    out = T.full((x.shape[0], lay.N), 0x5555, dtype=T.int16, device="cuda")
    X.linear_noalloc(xd, lay, prefill_min_m=pm, out=out)
    T.cuda.synchronize()
    return _lib.to_host_u16(out), _lib.to_host_u16(ref)


@pytest.mark.parametrize("K,N,Ms,pm", [
    (5120, 17408, (16, 4), 128),     # the decode configuration: prologue-rotation fused path
    (5120, 17408, (33, 20), 0),      # decode-GEMM with row groups, forced fused side
    (17408, 5120, (127, 64), 128),   # dequant-GEMM with its split-K tail, the largest fused-side scratch
    (256, 256, (200, 130), 128),     # dequant-GEMM on the prefill side
    (256, 256, (1100, 1030), 128),   # prefill path (reconstruct + GEMM)
])
def test_noalloc_matches_linear_two_calls(T, X, K, N, Ms, pm):
    lay = X.Layer.from_numpy(WL.layer(81, K, N), WL.codebook())
    for M in Ms:  # the second call is smaller and sees the first call's leftovers
        H.announce("noalloc K%d N%d M=%d pm=%d" % (K, N, M, pm))
        assert X.linear_scratch_bytes(K, N, M, pm) <= X.NOALLOC_SCRATCH_BYTES
        got, ref = both(T, X, lay, WL.activations(81, M, K), pm)
        assert np.array_equal(got, ref), (M, int(np.count_nonzero(got != ref)))


def test_noalloc_refuses_calls_beyond_its_scratch(T, X):
    from trellis_quantized_linear_had_amd import _lib

    K, N, M = 5120, 17408, 2048   # prefill: the fp16 weight slice alone is 178 MB
    H.announce("noalloc oversize K%d N%d M=%d" % (K, N, M))
    assert X.linear_scratch_bytes(K, N, M) > X.NOALLOC_SCRATCH_BYTES
    lay = X.Layer.from_numpy(WL.layer(82, K, N), WL.codebook())
    x = _lib.to_device_u16(WL.activations(82, M, K))
    out = T.full((M, N), 0x1234, dtype=T.int16, device="cuda")
    with pytest.raises(ValueError, match="exl3_linear_noalloc holds"):
        X.linear_noalloc(x, lay, out=out)
    T.cuda.synchronize()
    assert bool((out == 0x1234).all())   # refused before any launch
