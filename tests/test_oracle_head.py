"""Pins for the oracle's quantized output head (a trellis layer projected to
the padded logits width, pads -inf, first maximum selected). The expected
values come from the layer computed as a sequence of numpy matmuls with
scipy's Hadamard matrix, the pad rule of the logits projection and numpy's
argmax (first occurrence of the maximum)."""
import numpy as np
import pytest
import scipy.linalg

import workloads as WL
from oracle import oracle as O

H = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128)


def val(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def blockdiag(n):
    return scipy.linalg.block_diag(*([H] * (n // 128)))


def library_layer(x, L, cb):
    K, N, bits = L["K"], L["N"], L.get("bits", 4)
    W = val(O.reconstruct(L["codes"], cb, L["scale"], K, N, bits=bits))
    xr = val(f16((val(x) * val(L["sign_k"])) @ blockdiag(K).T))
    yr = val(f16(xr @ W))
    return f16((yr @ blockdiag(N).T) * val(L["sign_n"]))


def expected_head(y_full, n_valid):
    N = y_full.shape[1]
    n_pad = min((n_valid + 127) // 128 * 128, N)
    lg = y_full[:, :n_pad].copy()
    lg[:, n_valid:] = 0xFC00
    return lg, np.argmax(val(lg[:, :n_valid]), axis=1)


@pytest.mark.parametrize("bits", [4, 6])
@pytest.mark.parametrize("n_valid", [777, 1024, 1, 129, 896])
def test_head_matches_library_sequence(bits, n_valid):
    K, N, M = 256, 1024, 4
    L = WL.layer(WL.SEED_TINY, K, N, bits=bits)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY + 3, M, K)
    lg_ref, am_ref = expected_head(library_layer(x, L, cb), n_valid)
    lg, am = O.head_logits(x, L, cb, n_valid)
    assert lg.shape == lg_ref.shape
    assert np.array_equal(lg, lg_ref)
    assert np.array_equal(am, am_ref)


def test_head_row_subset_and_widths():
    K, N, M = 256, 640, 6
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY + 4, M, K)
    full_lg, full_am = O.head_logits(x, L, cb, 300)
    assert full_lg.shape == (M, 384)
    rows = np.array([5, 1, 3], np.int64)
    lg, am = O.head_logits(x, L, cb, 300, rows)
    assert np.array_equal(lg, full_lg[rows]) and np.array_equal(am, full_am[rows])
    # width equals the layer width once n_valid passes its last 128 block
    assert O.head_logits(x, L, cb, 600)[0].shape == (M, 640)


def test_head_zero_input_selects_column_zero():
    K, N = 256, 512
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    x = np.zeros((2, K), np.uint16)
    lg, am = O.head_logits(x, L, cb, 300)
    assert np.all(val(lg[:, :300]) == 0.0)
    assert np.all(lg[:, 300:] == 0xFC00)
    assert np.array_equal(am, [0, 0])


def test_head_layer_maximum_in_the_pad_region_cannot_win():
    """n_valid is put just below the column where the full layer output of a
    row peaks, so that column (and any larger one in its 128 block) is a pad:
    the selection must come from the valid columns instead."""
    K, N, M = 256, 1024, 8
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY + 5, M, K)
    y = library_layer(x, L, cb)
    done = 0
    for r in range(M):
        j = int(np.argmax(val(y[r])))
        if j % 128 == 0:
            continue
        lg, am = O.head_logits(x[r:r + 1], L, cb, j)
        assert lg.shape[1] > j and lg[0, j] == 0xFC00
        assert am[0] < j and am[0] == int(np.argmax(val(y[r, :j])))
        done += 1
    assert done >= 4


def test_head_rejects_bad_widths():
    K, N = 256, 256
    L = WL.layer(WL.SEED_TINY, K, N)
    x = WL.activations(WL.SEED_TINY, 1, K)
    with pytest.raises(ValueError):
        O.head_logits(x, L, WL.codebook(), 0)
    with pytest.raises(ValueError):
        O.head_logits(x, L, WL.codebook(), N + 1)


def test_nan_head_logits_follow_numpy_argmax():
    """A NaN column scale makes the whole 128-column rotation block NaN in
    every row; a NaN row of x makes its whole output NaN. The first NaN
    wins (NumPy's and torch's argmax); pads are never selected."""
    cb = WL.codebook()
    L = WL.layer(31, 128, 512)
    L = dict(L, scale=L["scale"].copy())
    L["scale"][300] = 0x7E00           # block 2 (columns 256..383) NaN
    x = WL.activations(31, 3, 128).copy()
    x[1] = 0x7E00
    lg, am = O.head_logits(x, L, cb, 400)   # n_pad = 512
    v = val(lg)
    assert np.all(np.isnan(v[:, 256:384])) and np.all(np.isnan(v[1, :400]))
    assert np.array_equal(am, np.argmax(v, axis=1))
    assert list(am) == [256, 0, 256]
    L["scale"][5] = 0x7E00             # block 0 NaN as well: column 0 first
    lg, am = O.head_logits(x, L, cb, 400)
    assert np.all(am == 0) and np.all(lg[:, 400:] == 0xFC00)
