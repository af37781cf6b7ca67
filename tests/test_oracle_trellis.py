"""Pins for the oracle's trellis decode and reconstruct (bit-exact)."""
import json
import os

import numpy as np

import workloads as WL
from oracle import oracle as O
from tests import brute_trellis as BT

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "trellis_closed_forms.json")))


def _one_tile(words):
    return O.trellis_states(np.asarray(words, np.uint32), 16, 16)


def _step(states, i):
    # step i of a single tile sits at row i % 16, column i // 16
    return int(states[i % 16, i // 16])


def test_closed_form_nibble_ramp_mod8():
    g = GOLD["nibble_ramp_mod8"]
    st = _one_tile([int(g["word"], 16)] * 32)
    for i, v in g["states"].items():
        assert _step(st, int(i)) == int(v, 16), i


def test_closed_form_single_bit_tail_biting():
    g = GOLD["single_bit0"]["nonzero_states"]
    words = [0] * 32
    words[0] = 1
    st = _one_tile(words)
    nz = {i: _step(st, i) for i in range(256) if _step(st, i)}
    assert nz == {int(i): int(v, 16) for i, v in g.items()}


def test_closed_form_step_orientation_k_fastest():
    g = GOLD["nibble_ramp_mod16"]
    even, odd = (int(w, 16) for w in g["words_even_odd"])
    st = _one_tile([even if j % 2 == 0 else odd for j in range(32)])
    # the state depends only on the row (k mod 16), never on the column
    assert np.all(st == st[:, :1])
    for r, v in g["state_by_row"].items():
        assert int(st[int(r), 7]) == int(v, 16)


def test_tile_order_k_major():
    K, N = 32, 48  # 2 x 3 tiles
    codes = np.concatenate([np.full(32, t * 0x11111111, np.uint32) for t in range(6)])
    st = O.trellis_states(codes, K, N)
    for kt in range(2):
        for nt in range(3):
            blk = st[kt * 16:(kt + 1) * 16, nt * 16:(nt + 1) * 16]
            assert np.all(blk == (kt * 3 + nt) * 0x1111)


def test_word_aligned_windows():
    r = np.random.default_rng(3)
    words = r.integers(0, 2**32, 32, dtype=np.uint32)
    st = _one_tile(words)
    for d in range(32):
        assert _step(st, 8 * d) == int(words[d]) & 0xFFFF
        assert _step(st, 8 * d + 4) == int(words[d]) >> 16


def test_brute_force_matches_oracle_random():
    for K, N, seed in ((16, 16, 1), (32, 48, 2), (48, 32, 3)):
        codes = np.random.default_rng(seed).integers(0, 2**32, K * N // 8, dtype=np.uint32)
        assert np.array_equal(O.trellis_states(codes, K, N), BT.states_matrix(codes, K, N))


def test_reconstruct_recovers_states_with_identity_codebooks():
    K, N = 64, 128
    codes = np.random.default_rng(5).integers(0, 2**32, K * N // 8, dtype=np.uint32)
    s = np.arange(65536)
    cb_lo = (s & 255).astype(np.float16).view(np.uint16)
    cb_hi = (s >> 8).astype(np.float16).view(np.uint16)
    one = np.full(N, 0x3C00, np.uint16)
    lo = O.reconstruct(codes, cb_lo, one, K, N).view(np.float16).astype(np.int64)
    hi = O.reconstruct(codes, cb_hi, one, K, N).view(np.float16).astype(np.int64)
    assert np.array_equal(hi * 256 + lo, BT.states_matrix(codes, K, N).astype(np.int64))


def test_reconstruct_single_rounding_against_numpy():
    # The product of two fp16 values is exact in float32, so numpy's float32
    # multiply followed by its float16 cast is one correct rounding.
    L = WL.layer(WL.SEED_TINY, 256, 256)
    cb = WL.codebook()
    st = BT.states_matrix(L["codes"][: 32 * 16 * 2], 32, 256)  # first two tile rows
    ref = (cb[st].view(np.float16).astype(np.float32) *
           L["scale"].view(np.float16).astype(np.float32)[None, :]).astype(np.float16).view(np.uint16)
    got = O.reconstruct(L["codes"], cb, L["scale"], 256, 256)[:32]
    assert np.array_equal(got, ref)


def test_reconstruct_slice_and_zero_codes():
    K, N = 128, 256
    L = WL.layer(WL.SEED_TINY, K, N)
    cb = WL.codebook()
    full = O.reconstruct(L["codes"], cb, L["scale"], K, N)
    part = O.reconstruct(L["codes"], cb, L["scale"], K, N, 128, 64)
    assert np.array_equal(part, full[:, 128:192])
    zero = np.zeros(K * N // 8, np.uint32)
    w0 = O.reconstruct(zero, cb, L["scale"], K, N)
    expect = (np.float32(cb[:1].view(np.float16)[0]) *
              L["scale"].view(np.float16).astype(np.float32)).astype(np.float16).view(np.uint16)
    assert np.array_equal(w0, np.broadcast_to(expect, (K, N)))
