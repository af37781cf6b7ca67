"""CPU pins of the exact-decode inputs (tests/exact_decode.py): the oracle's
input rotation of each unit row is exactly e_k, the integer codebooks give
back the state bytes through the oracle's reconstruct, and the expected
output agrees with the oracle's layer (fp64, one rounding) to within one fp16
unit in the last place -- the two differ only in the fp32 product the
kernels use before their fp16 rounding."""
import numpy as np

from oracle import oracle as O
from tests import exact_decode as E
from tests import helpers as HL


def test_unit_rows_rotate_to_unit_vectors():
    L = E.unit_layer(51, 384, 256, 4)
    ks = [0, 1, 127, 128, 200, 255, 256, 383]
    x = E.unit_rows(ks, 384, L["sign_k"])
    xr = O.had128(x, sign_pre=L["sign_k"])
    want = np.zeros((len(ks), 384), np.uint16)
    want[np.arange(len(ks)), ks] = 0x3C00
    assert np.array_equal(xr, want)


def test_integer_codebooks_recover_state_bytes():
    L = E.unit_layer(52, 256, 256, 5)
    st = O.trellis_states(L["codes"], 256, 256, 5).astype(np.int64)
    for kind, want in (("lo", st & 255), ("hi", st >> 8)):
        w = O.reconstruct(L["codes"], E.codebook(kind), L["scale"], 256, 256, bits=5)
        assert np.array_equal(HL.val(w), want.astype(np.float64))


def test_expected_output_matches_the_oracle_layer():
    for bits in (1, 4, 7):
        L = E.unit_layer(53, 256, 384, bits)
        ks = np.arange(0, 256, 9)
        x = E.unit_rows(ks, 256, L["sign_k"])
        st = O.trellis_states(L["codes"], 256, 384, bits)
        for kind in ("lo", "hi"):
            y = E.expected_y(st, ks, kind, L["sign_n"])
            ref = O.exl3_linear(x, L, E.codebook(kind))
            assert np.max(HL.ulp_diff(y, ref)) <= 1, bits
            assert np.mean(y == ref) > 0.99


def test_a_single_wrong_state_changes_the_output():
    """The check is sensitive: changing one state byte by one moves every
    output of its 128-column block."""
    L = E.unit_layer(54, 128, 256, 4)
    st = O.trellis_states(L["codes"], 128, 256, 4)
    ks = [5, 77]
    y = E.expected_y(st, ks, "lo", L["sign_n"])
    bad = st.copy()
    bad[77, 200] ^= 1
    y2 = E.expected_y(bad, ks, "lo", L["sign_n"])
    assert np.array_equal(y[0], y2[0])
    assert np.count_nonzero(y[1, 128:] != y2[1, 128:]) > 100 and np.array_equal(y[1, :128], y2[1, :128])
