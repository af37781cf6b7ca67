"""GPU parity at the full sizes of the five workload configurations, in the
launch configuration the benchmark times. Where the oracle cannot do every
row in seconds it checks a fixed subset of rows (first, last and spread
rows); rows are independent, so a subset is a sample of the same outputs."""
import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    return H.require_gpu()


@pytest.fixture(scope="module")
def X(T):
    import trellis_quantized_linear_had_amd as X

    return X


@pytest.fixture(scope="module")
def cb():
    return WL.codebook()


def sample_rows(M):
    """The first and last three rows plus one row in every 64-row block (so
    every 64-row quarter of every 256-row GEMM tile is compared), at a
    different offset in each block."""
    if M <= 12:
        return np.arange(M, dtype=np.int64)
    blocks = [min(64 * b + (37 * b + 11) % 64, M - 1) for b in range((M + 63) // 64)]
    return np.unique(np.concatenate([[0, 1, 2], blocks, [M - 3, M - 2, M - 1]])).astype(np.int64)


def test_sample_rows_cover_every_tile_quarter():
    for M in (128, 256, 1024, 2048, 4096):
        r = sample_rows(M)
        assert set(r // 64) == set(range((M + 63) // 64)) and set(r // 256) == set(range((M + 255) // 256))


def gpu_linear(X, lay, x, pm):
    from trellis_quantized_linear_had_amd import _lib

    return _lib.to_host_u16(X.linear(_lib.to_device_u16(x), lay, prefill_min_m=pm))


def test_tiny_config(T, X, cb):
    c = WL.TINY
    L = WL.layer(c["seed"], c["K"], c["N"])
    lay = X.Layer.from_numpy(L, cb)
    for M in c["M"]:
        H.announce("tiny M=%d" % M)
        x = WL.activations(c["seed"], M, c["K"])
        ref = O.exl3_linear(x, L, cb)
        H.assert_rows_close(gpu_linear(X, lay, x, 128), ref)


def test_decode_config(T, X, cb):
    c = WL.DECODE
    L = WL.layer(c["seed"], c["K"], c["N"], 0)
    lay = X.Layer.from_numpy(L, cb)
    for M in c["M"]:
        H.announce("decode K5120 N17408 M=%d" % M)
        x = WL.activations(c["seed"], M, c["K"])
        y = gpu_linear(X, lay, x, 128)
        ref = O.exl3_linear(x, L, cb)
        H.assert_rows_close(y, ref)
        assert np.array_equal(y, gpu_linear(X, lay, x, 128))  # bit-identical rerun


@pytest.mark.parametrize("geom", [0, 1])
def test_prefill_config(T, X, cb, geom):
    c = WL.PREFILL
    K, N = c["geometries"][geom]
    L = WL.layer(c["seed"], K, N, geom)
    lay = X.Layer.from_numpy(L, cb)
    for M in c["M"]:
        H.announce("prefill K%d N%d M=%d" % (K, N, M))
        x = WL.activations(c["seed"], M, K, geom)
        rows = sample_rows(M)
        ref = O.exl3_linear(x, L, cb, rows)
        y = gpu_linear(X, lay, x, 128)
        H.assert_rows_close(y[rows], ref, what="prefill M=%d" % M)
        if H.route(4, M, 128) != "recon":  # the dequant-GEMM's rows: reconstruct + GEMM forced too
            H.assert_rows_close(H.linear_forced(lay, x, "recon")[rows], ref, what="recon M=%d" % M)
        if M == 128:  # at the threshold the decode-GEMM must agree too
            H.assert_rows_close(H.linear_forced(lay, x, "fused")[rows], ref, what="fused M=128")


def test_wide_config(T, X, cb):
    c = WL.WIDE
    L = WL.layer(c["seed"], c["K"], c["N"])
    lay = X.Layer.from_numpy(L, cb)
    M = c["M"][0]
    H.announce("wide K5120 N32768 M=%d" % M)
    assert X.linear_scratch_bytes(c["K"], c["N"], M) == M * c["K"] * 2 + 32768 * c["K"] * 2
    x = WL.activations(c["seed"], M, c["K"])
    rows = sample_rows(M)
    ref = O.exl3_linear(x, L, cb, rows)
    y = gpu_linear(X, lay, x, 128)
    H.assert_rows_close(y[rows], ref)


@pytest.fixture(scope="module")
def logits_inputs():
    c = WL.LOGITS
    return WL.logits_weights(c["seed"], c["w_rows"], c["K"])


@pytest.mark.parametrize("M", WL.LOGITS["M"])
def test_logits_config(T, X, logits_inputs, M):
    from trellis_quantized_linear_had_amd import _lib

    c = WL.LOGITS
    H.announce("logits K5120 n_valid=248077 w_rows=248320 M=%d" % M)
    w = logits_inputs
    x = WL.activations(c["seed"], M, c["K"])
    wd = _lib.to_device_u16(w)
    lg, am = X.logits_pad_mask_argmax(_lib.to_device_u16(x), wd, c["n_valid"])
    lg = _lib.to_host_u16(lg)
    am = am.cpu().numpy()
    del wd
    ref_lg, ref_am = O.logits(x, w, c["n_valid"])
    assert lg.shape == (M, 248192)
    assert np.all(lg[:, 248077:] == 0xFC00)
    H.assert_logits_close(lg[:, :248077], ref_lg[:, :248077], c["K"])
    assert np.array_equal(am, ref_am)
