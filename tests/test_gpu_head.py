"""GPU parity of the trellis-quantized output head (the layer's first n_pad
columns, pads -inf, first maximum) against the CPU oracle through the C ABI:
logits within the per-row tolerance on the valid columns, pads exactly -inf,
columns past n_pad untouched, the argmax exactly the first maximum of the
returned logits and, where it differs from the oracle's, a near tie there."""
import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import helpers as H

pytestmark = pytest.mark.gpu

SENTINEL = 0x7E7E


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


def check_head(lg, am, ref_lg, ref_am, n_valid, rowmax=None):
    """lg: rows x ld (ld >= n_pad) from the GPU; ref_lg: rows x n_pad;
    rowmax: the largest |value| of each row of the layer output (the
    tolerance's scale; by default the valid logits' own)."""
    n_pad = ref_lg.shape[1]
    g, r = H.val(lg[:, :n_valid]), H.val(ref_lg[:, :n_valid])
    assert np.all(np.isfinite(g))
    if rowmax is None:
        rowmax = np.max(np.abs(r), axis=1)
    err = np.max(np.abs(g - r), axis=1)
    assert np.all(err <= H.Y_REL_TOL * rowmax), (err, rowmax)
    assert np.all(lg[:, n_valid:n_pad] == 0xFC00), "pad columns are not -inf"
    assert np.all(lg[:, n_pad:] == SENTINEL), "columns past the padded width were written"
    g = H.val(lg[:, :n_pad])
    # the selection is exactly the first maximum of the returned logits
    assert np.array_equal(am, np.argmax(g, axis=1))
    assert np.all(am < n_valid)
    r = H.val(ref_lg)
    for i in range(len(am)):
        if am[i] != ref_am[i]:
            # a near tie: the chosen column is within tolerance of the row maximum
            assert r[i, ref_am[i]] - r[i, am[i]] <= 2 * H.Y_REL_TOL * rowmax[i], (i, am[i], ref_am[i])


def run_head(T, X, x, lay, n_valid, M, ld, pm):
    lg = T.full((M, ld), SENTINEL, dtype=T.int16, device="cuda")
    am = T.full((M,), -7, dtype=T.int64, device="cuda")
    X.head_logits_argmax(dev16(x), lay, n_valid, prefill_min_m=pm, logits=lg, argmax=am)
    T.cuda.synchronize()
    return host16(lg), am.cpu().numpy()


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("n_valid", [777, 1024, 1, 129])
@pytest.mark.parametrize("M", [1, 5, 16, 64, 130])
def test_head_small(T, X, cb, bits, n_valid, M):
    H.announce("head bits=%d K256 N1024 n_valid=%d M=%d" % (bits, n_valid, M))
    K, N = 256, 1024
    L = WL.layer(41, K, N, 0, bits)
    x = WL.activations(41, M, K)
    ref_lg, ref_am = O.head_logits(x, L, cb, n_valid)
    # the per-row tolerance scales with the layer output's row (all N columns)
    rowmax = np.max(np.abs(H.val(O.exl3_linear(x, L, cb))), axis=1)
    n_pad = ref_lg.shape[1]
    lg, am = run_head(T, X, x, X.Layer.from_numpy(L, cb), n_valid, M, n_pad + 8, 128)
    check_head(lg, am, ref_lg, ref_am, n_valid, rowmax)


@pytest.mark.parametrize("pm", [0, 1])
def test_head_both_paths_agree_with_linear(T, X, cb, pm):
    """n_valid = N: the head's logits are the layer output itself (the same
    kernels, so bit-identical), and nothing is masked."""
    H.announce("head vs linear K512 N1536 M=24 pm=%d" % pm)
    K, N, M = 512, 1536, 24
    L = WL.layer(42, K, N, 0, 4)
    lay = X.Layer.from_numpy(L, cb)
    x = WL.activations(42, M, K)
    y = host16(X.linear(dev16(x), lay, prefill_min_m=pm))
    lg, am = run_head(T, X, x, lay, N, M, N, pm)
    assert np.array_equal(lg, y)
    assert np.array_equal(am, np.argmax(H.val(y), axis=1))


def test_head_leading_columns_equal_linear(T, X, cb):
    """The decode path over the first n_pad columns of a wider layer agrees
    with those columns of the whole layer (its k-split may differ with the
    width, so within tolerance rather than bit for bit)."""
    H.announce("head leading columns K1024 N4096 n_valid=1500 M=8")
    K, N, M, n_valid = 1024, 4096, 8, 1500
    L = WL.layer(43, K, N, 0, 5)
    lay = X.Layer.from_numpy(L, cb)
    x = WL.activations(43, M, K)
    y = host16(X.linear(dev16(x), lay, prefill_min_m=0))
    lg, am = run_head(T, X, x, lay, n_valid, M, 1536, 0)
    H.assert_rows_close(lg[:, :n_valid], y[:, :n_valid], what="leading columns")
    assert np.all(lg[:, n_valid:] == 0xFC00)


@pytest.mark.parametrize("pm", [0, 1])
def test_head_nan_rule(T, X, cb, pm):
    """NaN logits in the head on both paths: a NaN column scale makes its
    whole rotation block NaN, a NaN row of x its whole output; the first NaN
    wins (NumPy's and torch's argmax) and a pad column is never selected.
    Same inputs as the oracle's pin."""
    H.announce("head NaN rule pm=%d" % pm)
    L = WL.layer(31, 128, 512)
    L = dict(L, scale=L["scale"].copy())
    L["scale"][300] = 0x7E00
    x = WL.activations(31, 3, 128).copy()
    x[1] = 0x7E00
    for extra in (None, 5):
        if extra is not None:
            L["scale"][extra] = 0x7E00
        _, ref_am = O.head_logits(x, L, cb, 400)
        lg, am = run_head(T, X, x, X.Layer.from_numpy(L, cb), 400, 3, 512, pm)
        assert np.array_equal(am, ref_am), (am, ref_am)
        assert np.array_equal(am, np.argmax(H.val(lg), axis=1))
        assert np.all(lg[:, 400:] == 0xFC00)


def test_head_empty_batch_is_a_no_op(T, X, cb):
    H.announce("head M=0")
    K, N = 256, 512
    lay = X.Layer.from_numpy(WL.layer(44, K, N), cb)
    lg = T.full((1, 512), SENTINEL, dtype=T.int16, device="cuda")
    am = T.full((1,), -7, dtype=T.int64, device="cuda")
    X.head_logits_argmax(T.empty((0, K), dtype=T.int16, device="cuda"), lay, 300, logits=lg, argmax=am)
    T.cuda.synchronize()
    assert np.all(host16(lg) == SENTINEL) and int(am[0]) == -7


@pytest.fixture(scope="module")
def full_head(cb):
    # the padded-logits geometry with the weight as 4-bit trellis codes
    K, N, M, n_valid = 5120, 248320, 16, 248077
    L = WL.layer(45, K, N, 0, 4)
    x = WL.activations(45, M, K)
    rows = np.array([0, M - 1], np.int64)
    ref_lg, ref_am = O.head_logits(x, L, cb, n_valid, rows)
    return L, x, rows, ref_lg, ref_am, n_valid


@pytest.mark.parametrize("M,pm", [(16, 128), (16, 1), (1, 128)])
def test_head_full_size_sampled_rows(T, X, cb, full_head, M, pm):
    H.announce("head K5120 N248320 n_valid=248077 M=%d pm=%d (sampled rows)" % (M, pm))
    L, x, rows, ref_lg, ref_am, n_valid = full_head
    n_pad = ref_lg.shape[1]
    lg, am = run_head(T, X, x[:M], X.Layer.from_numpy(L, cb), n_valid, M, n_pad, pm)
    keep = rows[rows < M]
    check_head(lg[keep], am[keep], ref_lg[:len(keep)], ref_am[:len(keep)], n_valid)
    assert np.all(am < n_valid) and np.all(lg[:, n_valid:] == 0xFC00)
