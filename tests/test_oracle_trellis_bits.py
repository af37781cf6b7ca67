"""Pins for the oracle's trellis decode at every supported width (1..8 bits
per weight): hand-worked closed forms, the halfword-aligned windows, the
brute-force shift register on multi-tile inputs, and reconstruct through
identity codebooks."""
import json
import os

import numpy as np
import pytest

import workloads as WL
from oracle import oracle as O
from tests import brute_trellis as BT

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "trellis_bits_closed_forms.json")))
BITS = range(1, 9)


def _one_tile(words, bits):
    return O.trellis_states(np.asarray(words, np.uint32), 16, 16, bits)


def _step(states, i):
    return int(states[i % 16, i // 16])


@pytest.mark.parametrize("bits", BITS)
def test_single_bit_tail_biting(bits):
    words = [0] * (8 * bits)
    words[0] = 1
    st = _one_tile(words, bits)
    nz = {i: _step(st, i) for i in range(256) if _step(st, i)}
    assert nz == {int(i): int(v, 16) for i, v in GOLD["single_bit0"][str(bits)].items()}


def test_byte_ramp_8_bits():
    words = [(4 * w) | (4 * w + 1) << 8 | (4 * w + 2) << 16 | (4 * w + 3) << 24 for w in range(64)]
    st = _one_tile(words, 8)
    for i, v in GOLD["byte_ramp_b8"]["states"].items():
        assert _step(st, int(i)) == int(v, 16), i


def test_bit_ramp_1_bit():
    st = _one_tile([0xFFFF0000] * 8, 1)
    for i, v in GOLD["bit_ramp_b1"]["states"].items():
        assert _step(st, int(i)) == int(v, 16), i


@pytest.mark.parametrize("bits", BITS)
def test_halfword_aligned_windows(bits):
    # where the window starts on a 16-bit boundary it is that halfword
    r = np.random.default_rng(10 + bits)
    words = r.integers(0, 2**32, 8 * bits, dtype=np.uint32)
    halves = words.view(np.uint16)  # little-endian: halfword j = bits 16j .. 16j+15
    st = _one_tile(words, bits)
    checked = 0
    for i in range(256):
        if (bits * i) % 16 == 0:
            assert _step(st, i) == int(halves[bits * i // 16]), i
            checked += 1
    assert checked >= 16


@pytest.mark.parametrize("bits", BITS)
def test_brute_force_matches_oracle_multi_tile(bits):
    for K, N, seed in ((32, 48, 1), (48, 32, 2)):
        codes = np.random.default_rng([seed, bits]).integers(0, 2**32, K * N * bits // 32, dtype=np.uint32)
        assert np.array_equal(O.trellis_states(codes, K, N, bits), BT.states_matrix(codes, K, N, bits))


@pytest.mark.parametrize("bits", (1, 3, 6, 8))
def test_reconstruct_identity_codebooks(bits):
    K, N = 32, 128
    codes = np.random.default_rng(20 + bits).integers(0, 2**32, K * N * bits // 32, dtype=np.uint32)
    s = np.arange(65536)
    cb_lo = (s & 255).astype(np.float16).view(np.uint16)
    cb_hi = (s >> 8).astype(np.float16).view(np.uint16)
    one = np.full(N, 0x3C00, np.uint16)
    lo = O.reconstruct(codes, cb_lo, one, K, N, bits=bits).view(np.float16).astype(np.int64)
    hi = O.reconstruct(codes, cb_hi, one, K, N, bits=bits).view(np.float16).astype(np.int64)
    assert np.array_equal(hi * 256 + lo, BT.states_matrix(codes, K, N, bits).astype(np.int64))


def test_workload_code_sizes_and_streams():
    for bits in BITS:
        L = WL.layer(WL.SEED_TINY, 128, 256, 0, bits)
        assert L["bits"] == bits and L["codes"].size == 128 * 256 * bits // 32
    # the 4-bit codes are the original stream; other widths draw their own
    assert np.array_equal(WL.layer(WL.SEED_TINY, 128, 256)["codes"], WL.layer(WL.SEED_TINY, 128, 256, 0, 4)["codes"])


def test_code_size_checked():
    with pytest.raises(ValueError):
        O.trellis_states(np.zeros(8 * 3, np.uint32), 16, 16, 4)
    with pytest.raises(ValueError):
        O.trellis_states(np.zeros(8 * 9, np.uint32), 16, 16, 9)
