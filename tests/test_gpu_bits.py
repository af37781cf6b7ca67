"""GPU parity at every width from 1 to 8 bits per weight (the stand-in
trellis generalised: a window at bit bits*i of a 256*bits-bit tile; vLLM PR
#316 names 4-bit MLP and 6-bit lm_head layers): trellis states and both
reconstruct layouts bit-exact, the layer on both paths within the per-row
tolerance, against the CPU oracle through the C ABI."""
import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import helpers as H

pytestmark = pytest.mark.gpu

BITS = list(range(1, 9))


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


def dev16(a):
    from trellis_quantized_linear_had_amd import _lib

    return _lib.to_device_u16(a)


def host16(t):
    from trellis_quantized_linear_had_amd import _lib

    return _lib.to_host_u16(t)


@pytest.mark.parametrize("bits", BITS)
def test_decode_states_bit_exact(T, X, cb, bits):
    H.announce("decode_states bits=%d K256 N384" % bits)
    K, N = 256, 384
    L = WL.layer(31, K, N, 0, bits)
    got = host16(X.decode_states(X.Layer.from_numpy(L, cb)))
    assert np.array_equal(got, O.trellis_states(L["codes"], K, N, bits))


@pytest.mark.parametrize("bits", BITS)
def test_reconstruct_both_layouts_bit_exact(T, X, cb, bits):
    H.announce("reconstruct KN+NK bits=%d K384 N512 slice 128+272" % bits)
    K, N, n0, nc, pad = 384, 512, 128, 272, 8
    L = WL.layer(32, K, N, 0, bits)
    lay = X.Layer.from_numpy(L, cb)
    ref = O.reconstruct(L["codes"], cb, L["scale"], K, N, n0, nc, bits)
    assert np.array_equal(host16(X.reconstruct(lay, n0, nc, X.LAYOUT_KN)), ref)
    out = T.full((nc, K + pad), -1, dtype=T.int16, device="cuda")
    X.reconstruct(lay, n0, nc, X.LAYOUT_NK, out=out, ldw=K + pad)
    got = host16(out)
    assert np.array_equal(got[:, :K], ref.T)
    assert np.all(got[:, K:] == 0xFFFF)


@pytest.mark.parametrize("bits", (3, 8))
def test_reconstruct_nk_over_several_launches(T, X, cb, bits):
    # K4096 x N17408 is 69632 units of 4 x 1 tiles: more than one launch holds
    # at 3 bits (65536) and at 8 bits (45056)
    H.announce("reconstruct NK bits=%d K4096 N17408 (several launches)" % bits)
    K, N = 4096, 17408
    L = WL.layer(33, K, N, 0, bits)
    got = host16(X.reconstruct(X.Layer.from_numpy(L, cb), 0, N, X.LAYOUT_NK))
    assert np.array_equal(got, O.reconstruct(L["codes"], cb, L["scale"], K, N, bits=bits).T)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [1, 16, 40, 100])
def test_linear_both_paths(T, X, cb, bits, M):
    H.announce("linear bits=%d K256 N384 M=%d" % (bits, M))
    K, N = 256, 384
    L = WL.layer(34, K, N, 0, bits)
    x = WL.activations(34, M, K)
    ref = O.exl3_linear(x, L, cb)
    lay = X.Layer.from_numpy(L, cb)
    for r in ("fused", "recon") + (("dq", "dq8") if bits == 4 else ()):
        H.assert_rows_close(H.linear_forced(lay, x, r), ref, what=r)
    for pm in (0, 1):  # the dispatch at this width
        want = H.linear_forced(lay, x, H.route(bits, M, pm))
        assert np.array_equal(host16(X.linear(dev16(x), lay, prefill_min_m=pm)), want), pm


@pytest.mark.parametrize("bits,M,pm", [(6, 1, 128), (6, 16, 128), (6, 2048, 128), (2, 16, 128), (8, 64, 128)])
def test_linear_full_size_sampled_rows(T, X, cb, bits, M, pm):
    H.announce("linear bits=%d K5120 N17408 M=%d (sampled rows)" % (bits, M))
    K, N = 5120, 17408
    L = WL.layer(35, K, N, 0, bits)
    x = WL.activations(35, M, K)
    rows = np.unique(np.array([0, M // 2, M - 1], np.int64))
    y = host16(X.linear(dev16(x), X.Layer.from_numpy(L, cb), prefill_min_m=pm))
    H.assert_rows_close(y[rows], O.exl3_linear(x, L, cb, rows))


@pytest.mark.parametrize("M", [512, 300])
def test_linear_fused_many_passes_other_width(T, X, cb, M):
    """The fused decode path forced (prefill_min_m = 0) at 6 bits on the MLP
    geometry with many passes of four row groups (the reduction of every pass
    but the last goes through the LDS left beside the codebook); sampled rows
    in every 64-row block against the oracle."""
    H.announce("linear bits=6 K5120 N17408 M=%d fused (sampled rows)" % M)
    K, N = 5120, 17408
    L = WL.layer(39, K, N, 0, 6)
    x = WL.activations(39, M, K)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(5, M, 64)])).astype(np.int64)
    y = host16(X.linear(dev16(x), X.Layer.from_numpy(L, cb), prefill_min_m=0))
    H.assert_rows_close(y[rows], O.exl3_linear(x, L, cb, rows))


def test_linear_deterministic_other_width(T, X, cb):
    H.announce("linear determinism bits=5")
    K, N = 1024, 2048
    L = WL.layer(36, K, N, 0, 5)
    lay = X.Layer.from_numpy(L, cb)
    for M in (8, 70, 300):
        x = dev16(WL.activations(36, M, K))
        first = host16(X.linear(x, lay))
        for _ in range(3):
            assert np.array_equal(host16(X.linear(x, lay)), first)


@pytest.mark.parametrize("bits,M", [(4, 8), (4, 16), (6, 16)])
def test_linear_wide_layer_small_m(T, X, cb, bits, M):
    """K5120 x N32768 at M <= 16: the planner takes the decode plan without
    the prologue rotation here (a separate rotation pass, no k-split), the
    one wide layers get; sampled rows against the oracle."""
    H.announce("linear bits=%d K5120 N32768 M=%d (sampled rows)" % (bits, M))
    K, N = 5120, 32768
    L = WL.layer(37, K, N, 0, bits)
    x = WL.activations(37, M, K)
    rows = np.array([0, M - 1], np.int64)
    y = host16(X.linear(dev16(x), X.Layer.from_numpy(L, cb)))
    H.assert_rows_close(y[rows], O.exl3_linear(x, L, cb, rows))


@pytest.mark.parametrize("bits,M", [(6, 1), (6, 4), (6, 16), (3, 4)])
def test_linear_four_tile_waves(T, X, cb, bits, M):
    """K512 x N12800: the planner gives each wave four n-tiles at these
    widths (the prologue rotation included); every row against the oracle."""
    H.announce("linear bits=%d K512 N12800 M=%d" % (bits, M))
    K, N = 512, 12800
    L = WL.layer(38, K, N, 0, bits)
    x = WL.activations(38, M, K)
    y = host16(X.linear(dev16(x), X.Layer.from_numpy(L, cb)))
    H.assert_rows_close(y, O.exl3_linear(x, L, cb))
