"""Pins for the oracle's own fp16 conversions against numpy's float16 casts."""
import numpy as np

from oracle import oracle as O


def test_f16_to_f64_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    got = O.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _check(d):
    got = O.f64_to_f16(d)
    ref = d.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (d[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_f64_to_f16_roundtrip_all_finite():
    h = np.arange(65536, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    v = v[np.isfinite(v)]
    _check(v)


def test_f64_to_f16_midpoints_ties_to_even():
    # exact midpoints between consecutive positive fp16 values, and 1 ulp (fp64) either side
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2
    for d in (mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid):
        _check(d)


def test_f64_to_f16_random_and_boundaries():
    r = np.random.default_rng(7)
    d = np.exp2(r.uniform(-30, 17, 200000)) * r.choice([-1.0, 1.0], 200000)
    _check(d)
    edges = np.array([65504.0, 65519.999, 65520.0, 65536.0, 1e300, -65520.0,
                      2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                      2.0 ** -26, 0.0, -0.0, 3 * 2.0 ** -26, np.inf, -np.inf])
    _check(edges)
    assert O.f64_to_f16(np.array([np.nan]))[0] & 0x7C00 == 0x7C00
