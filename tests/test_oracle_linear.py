"""Pins for the oracle's full layer: associativity against an explicit dense
effective weight built with library matmuls, and closed forms."""
import numpy as np
import scipy.linalg

import workloads as WL
from oracle import oracle as O
from tests import brute_trellis as BT

H = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128)


def val(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def blockdiag(n):
    return scipy.linalg.block_diag(*([H] * (n // 128)))


def test_matches_library_sequence_tiny():
    K, N, M = 256, 384, 5
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY, M, K)
    W = val(O.reconstruct(L["codes"], cb, L["scale"], K, N))
    sk, sn = val(L["sign_k"]), val(L["sign_n"])
    HK, HN = blockdiag(K), blockdiag(N)
    # the same four materialisation points, computed with numpy matmuls
    xr = val(f16((val(x) * sk) @ HK.T))
    yr = val(f16(xr @ W))
    y_ref = f16((yr @ HN.T) * sn)
    y = O.exl3_linear(x, L, cb)
    assert np.array_equal(y, y_ref)
    # associativity: one dense effective weight, no intermediate rounding
    Weff = np.diag(sk) @ HK.T @ W @ HN.T @ np.diag(sn)
    y_exact = val(x) @ Weff
    rowmax = np.max(np.abs(y_exact), axis=1, keepdims=True)
    assert np.all(np.abs(val(y) - y_exact) <= 2e-3 * rowmax)


def test_row_subset_equals_full():
    K, N, M = 256, 256, 16
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY, M, K)
    full = O.exl3_linear(x, L, cb)
    rows = np.array([15, 0, 7], np.int64)
    assert np.array_equal(O.exl3_linear(x, L, cb, rows), full[rows])


def test_zero_codes_rank_one_closed_form():
    K, N, M = 256, 256, 3
    L = dict(WL.layer(WL.SEED_TINY, K, N))
    L["codes"] = np.zeros(K * N // 8, np.uint32)
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY, M, K)
    xr = val(O.had128(x, L["sign_k"]))
    w_col = val(f16(val(cb[:1])[0] * val(L["scale"])))     # every row of W is this vector
    yr = val(f16(xr.sum(axis=1, keepdims=True) * w_col[None, :]))
    y_ref = O.had128(f16(yr), None, L["sign_n"])
    assert np.array_equal(O.exl3_linear(x, L, cb), y_ref)


def test_matches_library_sequence_other_widths():
    # W from the brute-force shift register and numpy's exact float32 product
    # (one fp16 rounding), then the same matmul sequence as above
    K, N, M = 128, 256, 3
    cb = WL.codebook()
    x = WL.activations(WL.SEED_TINY, M, K)
    HK, HN = blockdiag(K), blockdiag(N)
    for bits in (3, 6):
        L = WL.layer(WL.SEED_TINY, K, N, 0, bits)
        st = BT.states_matrix(L["codes"], K, N, bits)
        W = (cb[st].view(np.float16).astype(np.float32) *
             L["scale"].view(np.float16).astype(np.float32)[None, :]).astype(np.float16).astype(np.float64)
        sk, sn = val(L["sign_k"]), val(L["sign_n"])
        xr = val(f16((val(x) * sk) @ HK.T))
        yr = val(f16(xr @ W))
        y_ref = f16((yr @ HN.T) * sn)
        assert np.array_equal(O.exl3_linear(x, L, cb), y_ref), bits
