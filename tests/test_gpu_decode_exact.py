"""Bit-exact check of the decoded trellis states inside the fused decode-GEMM
(and the prefill path) through the public C ABI.

With the inputs of tests/exact_decode.py -- x rows that rotate exactly to
unit vectors e_k, unit column scales and an integer codebook (each state's
low byte, then its high byte) -- every output is an exact function of the
states the kernel decoded, so the GPU output must equal the output computed
from the oracle's states bit for bit. Every k of the layer is covered, at
every width 1..8, for the row counts that select each kind of fused pass (the
prologue rotation at M <= 16, two and four row groups per pass above) and
for several widths N, so the planner takes different tile counts per wave."""
import numpy as np
import pytest

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


def run(X, lay, x, pm):
    """pm: a threshold for exl3_linear's dispatch, or the name of a kernel
    sequence to force."""
    from trellis_quantized_linear_had_amd import _lib

    if isinstance(pm, str):
        return H.linear_forced(lay, x, pm)
    return _lib.to_host_u16(X.linear(_lib.to_device_u16(x), lay, prefill_min_m=pm))


def check_all_k(X, L, K, N, bits, M, pms, what):
    st = O.trellis_states(L["codes"], K, N, bits)
    order = np.random.default_rng(K + N + bits + M).permutation(K)  # rows hit k in mixed order
    for kind in ("lo", "hi"):
        lay = X.Layer.from_numpy(L, E.codebook(kind))
        for c0 in range(0, K, M):
            ks = order[c0:c0 + M]
            if len(ks) < M:  # a full last call: pad with k already covered
                ks = np.concatenate([ks, order[:M - len(ks)]])
            x = E.unit_rows(ks, K, L["sign_k"])
            want = E.expected_y(st, ks, kind, L["sign_n"])
            for pm in pms:
                got = run(X, lay, x, pm)
                if not np.array_equal(got, want):
                    bad = np.argwhere(got != want)
                    m, n = bad[0]
                    raise AssertionError("%s %s pm=%s: %d outputs differ; first at row %d (k=%d), column %d"
                                         % (what, kind, pm, len(bad), m, ks[m], n))


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("N", [128, 1152, 2560])
@pytest.mark.parametrize("M", [16, 40, 100])
def test_fused_decode_states_bit_exact(T, X, bits, N, M):
    """The fused side (prefill_min_m = 0), the decode-GEMM forced where that
    side takes the dequant-GEMM (4 bits, M = 100), and at M = 40 also the
    prefill side (prefill_min_m = 1) on the same rows."""
    K = 256
    H.announce("exact decode bits=%d K%d N%d M=%d" % (bits, K, N, M))
    L = E.unit_layer(60 + bits, K, N, bits)
    pms = (0, 1) if M == 40 else (0,)
    if H.route(bits, M, 0) != "fused":
        pms += ("fused",)
    check_all_k(X, L, K, N, bits, M, pms, "K%d N%d bits=%d M=%d" % (K, N, bits, M))


def test_fused_decode_states_bit_exact_full_geometry(T, X):
    """The decode configuration's geometry (K5120 x N17408, 4 bits) in the
    launch configuration the benchmark times (M = 16, default threshold):
    64 k spread over K, each checked over all 17408 columns."""
    K, N, bits = 5120, 17408, 4
    H.announce("exact decode K5120 N17408 M=16 (64 k)")
    L = E.unit_layer(70, K, N, bits)
    st = O.trellis_states(L["codes"], K, N, bits)
    ks_all = np.concatenate([np.arange(0, K, 80), [K - 1]])[:64]
    for kind in ("lo", "hi"):
        lay = X.Layer.from_numpy(L, E.codebook(kind))
        for c0 in range(0, len(ks_all), 16):
            ks = ks_all[c0:c0 + 16]
            got = run(X, lay, E.unit_rows(ks, K, L["sign_k"]), 128)
            assert np.array_equal(got, E.expected_y(st, ks, kind, L["sign_n"])), (kind, c0)


def test_head_decode_states_bit_exact(T, X):
    """The quantized head reads codes with the full layer's row stride over
    its first n_pad columns only: the same exactness there."""
    from trellis_quantized_linear_had_amd import _lib

    K, N, bits, n_valid = 512, 2048, 6, 1000   # n_pad = 1024
    H.announce("exact decode head K512 N2048 n_valid=1000")
    L = E.unit_layer(71, K, N, bits)
    st = O.trellis_states(L["codes"], K, N, bits)
    ks = np.arange(3, K, 37)
    for kind in ("lo", "hi"):
        lay = X.Layer.from_numpy(L, E.codebook(kind))
        lg, _ = X.head_logits_argmax(_lib.to_device_u16(E.unit_rows(ks, K, L["sign_k"])), lay, n_valid,
                                     prefill_min_m=0)
        lg = _lib.to_host_u16(lg)
        want = E.expected_y(st, ks, kind, L["sign_n"])
        assert np.array_equal(lg[:, :n_valid], want[:, :n_valid]), kind
