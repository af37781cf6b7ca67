"""Pins for the oracle's padded-width logits projection, pad mask and argmax."""
import json
import os

import numpy as np

from oracle import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "logits_widths.json")))


def val(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def test_widths_from_the_page():
    n_pad = O.padded_width(GOLD["n_valid"], GOLD["w_rows"])
    assert n_pad == GOLD["n_pad"]
    assert n_pad - GOLD["n_valid"] == GOLD["masked_columns"]
    assert n_pad <= GOLD["w_rows"]


def test_width_rule_edges():
    assert O.padded_width(256, 1000) == 256          # already aligned: mask is a no-op
    assert O.padded_width(257, 1000) == 384
    assert O.padded_width(257, 300) == 300           # clamped by the weight rows
    assert O.padded_width(1, 1) == 1


def _case(seed, M, K, w_rows, n_valid):
    r = np.random.default_rng(seed)
    x = f16(0.05 * r.standard_normal((M, K)))
    w = f16(0.02 * r.standard_normal((w_rows, K)))
    return x, w


def test_values_mask_and_argmax_small():
    x, w = _case(1, 4, 96, 300, 257)
    lg, am = O.logits(x, w, 257)
    assert lg.shape == (4, 300)
    ref = f16(val(x) @ val(w[:257]).T)
    assert np.array_equal(lg[:, :257], ref)
    assert np.all(lg[:, 257:] == 0xFC00)
    assert np.array_equal(am, np.argmax(val(lg), axis=1))


def test_planted_pad_row_cannot_win_and_nan_poison_is_ignored():
    x, w = _case(2, 3, 64, 400, 300)   # n_pad = 384
    w = w.copy()
    w[310] = f16(5 * val(x[0]))        # a pad row aligned with row 0 of x: it wins without the mask
    plain = val(x) @ val(w).T
    assert np.argmax(plain[0, :384]) == 310
    _, am_ref = O.logits(x, w, 300)
    w2 = w.copy()
    w2[300:384] = 0x7E00               # NaN in the pad rows
    w2[384:] = 0x7E00                  # NaN beyond the padded width
    lg2, am2 = O.logits(x, w2, 300)
    assert np.array_equal(am2, am_ref)
    assert np.all(lg2[:, 300:] == 0xFC00)
    assert np.all(am_ref < 300)


def test_ties_resolve_to_lowest_index():
    x, w = _case(3, 2, 64, 256, 256)
    w = w.copy()
    lg, am = O.logits(x, w, 256)
    for i in range(2):
        best = int(am[i])
        w[200] = w[best]
        w[best + 1 if best + 1 < 200 else 0] = w[best]
    lg2, am2 = O.logits(x, w, 256)
    for i in range(2):
        m = np.max(val(lg2[i]))
        assert am2[i] == np.min(np.nonzero(val(lg2[i]) == m)[0])


def nan_logits_case():
    """Inputs whose logits hold NaNs: a NaN weight row makes its column NaN in
    every row of x, a NaN row of x makes every logit of that row NaN, and a
    huge weight row overflows one logit to +inf (a NaN must still beat it)."""
    x, w = _case(4, 4, 128, 400, 300)  # n_pad = 384
    x, w = x.copy(), w.copy()
    w[137] = 0x7E00                    # column 137: NaN everywhere
    w[50] = f16(np.sign(val(x[0])) * 60000.0)  # row 0, column 50: +inf
    x[2] = 0x7E00                      # row 2: every logit NaN
    return x, w


def test_nan_logits_follow_numpy_argmax():
    """NaN rule (NumPy's and torch's argmax): a NaN ranks above every number
    and the first NaN wins; selection never reaches the pad columns."""
    x, w = nan_logits_case()
    lg, am = O.logits(x, w, 300)
    v = val(lg)
    assert np.isinf(v[0, 50]) and v[0, 50] > 0
    assert np.all(np.isnan(v[:, 137])) and np.all(np.isnan(v[2, :300]))
    assert np.array_equal(am, np.argmax(v, axis=1))
    assert list(am) == [137, 137, 0, 137]
    w0 = w.copy()
    w0[0] = 0x7E00                     # a NaN in column 0 wins at once
    lg0, am0 = O.logits(x, w0, 300)
    assert np.array_equal(am0, np.argmax(val(lg0), axis=1)) and np.all(am0 == 0)
    wall = w.copy()
    wall[:300] = 0x7E00                # every decodable logit NaN: still column 0, never a pad
    lga, ama = O.logits(x, wall, 300)
    assert np.all(ama == 0) and np.all(lga[:, 300:] == 0xFC00)
