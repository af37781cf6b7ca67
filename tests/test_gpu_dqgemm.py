"""GPU parity of the dequant-in-GEMM (the trellis decode inside the MFMA
loop, exl3_linear's kernel sequence forced through the measurement library)
against the oracle: within the per-row tolerance over row counts that take
one to eight row fragments per pass and several passes, with split-K, and
bit for bit on the decoded states (the inputs of tests/exact_decode.py).
Both kernels: the four-wave one (1 to 8 row fragments of 32 per pass) and
the eight-wave one (256-row passes, Xr staged in LDS)."""
import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import exact_decode as E
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


@pytest.fixture(scope="module")
def X(T):
    import trellis_quantized_linear_had_amd as X

    return X


def run_dq(T, X, lay, x, M, variant=None):
    from trellis_quantized_linear_had_amd import _lib, _measure

    if variant is None:
        variant = _measure.VARIANT_DEQUANT_GEMM
    xd = _lib.to_device_u16(x)
    y = T.full((M, lay.N), 0x7E7E, dtype=T.int16, device="cuda")
    scr = T.empty(_measure.linear_scratch_bytes(lay.K, lay.N, M, variant), dtype=T.uint8, device="cuda")
    kt = _measure.KernelTimer(pairs=4, per_call=2)
    try:
        kt.linear_variant(lay, xd, M, y, scr, T.cuda.current_stream().cuda_stream, variant)
    finally:
        kt.close()
    T.cuda.synchronize()
    return _lib.to_host_u16(y)


def variant_of(eight, whole):
    from trellis_quantized_linear_had_amd import _measure

    return {(False, False): _measure.VARIANT_DEQUANT_GEMM, (False, True): _measure.VARIANT_DEQUANT_WHOLE,
            (True, False): _measure.VARIANT_DEQUANT_GEMM8, (True, True): _measure.VARIANT_DEQUANT8_WHOLE}[eight, whole]


@pytest.mark.parametrize("eight", [False, True])
@pytest.mark.parametrize("whole", [False, True])
@pytest.mark.parametrize("K,N", [(128, 128), (256, 256), (1024, 384), (512, 1152)])
@pytest.mark.parametrize("M", [1, 17, 40, 100, 128, 200, 256, 300, 513])
def test_dqgemm_matches_oracle(T, X, K, N, M, whole, eight):
    """Both output stages: whole units (scales, rotation and signs in the
    kernel) and K-split tail pieces summed by the fixup. K = 128: four 32-k
    steps, split into pieces of two (the loop's two-step remainder); N = 128:
    half of each workgroup's waves past the last column."""
    H.announce("dqgemm K%d N%d M=%d whole=%d eight=%d" % (K, N, M, whole, eight))
    L = WL.layer(90, K, N)
    cb = WL.codebook()
    x = WL.activations(90, M, K)
    y = run_dq(T, X, X.Layer.from_numpy(L, cb), x, M, variant_of(eight, whole))
    H.assert_rows_close(y, O.exl3_linear(x, L, cb), what="dqgemm M=%d" % M)


@pytest.mark.parametrize("eight", [False, True])
@pytest.mark.parametrize("whole", [False, True])
@pytest.mark.parametrize("M", [40, 256, 300])
def test_dqgemm_states_bit_exact(T, X, M, whole, eight):
    K, N = 512, 768
    H.announce("dqgemm exact decode K%d N%d M=%d whole=%d eight=%d" % (K, N, M, whole, eight))
    L = E.unit_layer(91, K, N, 4)
    st = O.trellis_states(L["codes"], K, N, 4)
    order = np.random.default_rng(M).permutation(K)
    for kind in ("lo", "hi"):
        lay = X.Layer.from_numpy(L, E.codebook(kind))
        for c0 in range(0, K, M):
            ks = order[c0:c0 + M]
            if len(ks) < M:
                ks = np.concatenate([ks, order[:M - len(ks)]])
            got = run_dq(T, X, lay, E.unit_rows(ks, K, L["sign_k"]), M, variant_of(eight, whole))
            want = E.expected_y(st, ks, kind, L["sign_n"])
            assert np.array_equal(got, want), (kind, c0, int(np.count_nonzero(got != want)))


@pytest.mark.parametrize("eight", [False, True])
@pytest.mark.parametrize("M", [64, 256, 384, 512, 1024, 2048])
def test_dqgemm_full_geometry_sampled(T, X, M, eight):
    """K5120 x N17408 on sampled rows (every 256-row pass). At M = 384 and 512
    the eight-wave kernel's 136 units of 256 rows take the stream-K tail
    (runs crossing unit boundaries, one partial per unit a run touches)."""
    from tests.test_gpu_configs import sample_rows

    K, N = 5120, 17408
    H.announce("dqgemm K%d N%d M=%d eight=%d" % (K, N, M, eight))
    L = WL.layer(WL.SEED_PREFILL, K, N, 0)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_PREFILL, M, K, 0)
    rows = sample_rows(M)
    y = run_dq(T, X, X.Layer.from_numpy(L, cb), x, M, variant_of(eight, False))
    H.assert_rows_close(y[rows], O.exl3_linear(x, L, cb, rows), what="dqgemm full M=%d" % M)
