"""Pins for the oracle's 128-point Walsh-Hadamard rotation."""
import numpy as np
import scipy.linalg

import workloads as WL
from oracle import oracle as O

H = scipy.linalg.hadamard(128).astype(np.float64)  # natural (Sylvester) order


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def val(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def test_matrix_is_sylvester_and_orthogonal():
    h = O.hadamard_matrix().astype(np.int64)
    assert np.array_equal(h, H.astype(np.int64))
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def test_unit_vectors_give_scaled_columns():
    x = np.zeros((128, 256), np.uint16)
    for j in range(128):
        x[j, j] = 0x3C00            # 1.0 in block 0
        x[j, 128 + (j * 7) % 128] = 0xC000  # -2.0 in block 1
    out = val(O.had128(x))
    for j in range(128):
        assert np.array_equal(out[j, :128], val(f16(H[:, j] / np.sqrt(128))))
        assert np.array_equal(out[j, 128:], val(f16(-2.0 * H[:, (j * 7) % 128] / np.sqrt(128))))


def test_constant_block_concentrates_in_first_output():
    c = val(f16([0.3]))[0]
    x = np.full((1, 128), f16([0.3])[0], np.uint16)
    out = val(O.had128(x))[0]
    assert out[0] == val(f16([c * np.sqrt(128)]))[0]
    assert np.all(out[1:] == 0.0)


def test_matches_library_matmul_with_signs():
    r = np.random.default_rng(11)
    x = WL.activations(99, 7, 512)
    sp = WL.signs(99, 2, 512)
    sq = WL.signs(99, 3, 512)
    ref = np.empty((7, 512))
    xv, spv, sqv = val(x), val(sp), val(sq)
    for b in range(0, 512, 128):
        ref[:, b:b + 128] = ((xv[:, b:b + 128] * spv[b:b + 128]) @ H.T / np.sqrt(128)) * sqv[b:b + 128]
    assert np.array_equal(O.had128(x, sp, sq), f16(ref))
    assert np.array_equal(O.had128(x, sp, None), f16(
        np.concatenate([(xv[:, b:b + 128] * spv[b:b + 128]) @ H.T / np.sqrt(128) for b in range(0, 512, 128)], 1)))
    del r


def test_involution_and_parseval():
    x = WL.activations(98, 5, 384)
    once = O.had128(x)
    twice = O.had128(once)
    xv = val(x)
    # two fp16 roundings of an orthonormal map: error well under 2^-9 of the row scale
    assert np.max(np.abs(val(twice) - xv)) <= 2.0 ** -9 * np.max(np.abs(xv))
    for b in range(0, 384, 128):
        n0 = np.linalg.norm(xv[:, b:b + 128], axis=1)
        n1 = np.linalg.norm(val(once)[:, b:b + 128], axis=1)
        assert np.allclose(n0, n1, rtol=2e-3)
