"""Every synthetic input of the five workload configurations is pinned by
SHA-256 (tests/golden/input_sha256.json, written by
tests/golden/make_input_sha256.py): a change in numpy's random streams or in
workloads.py would otherwise move the inputs and every expected value
together, unnoticed."""
import json
import os

from tests.golden import make_input_sha256 as G


def test_inputs_match_their_pinned_digests():
    want = json.load(open(G.OUT))
    got = G.input_digests()
    assert set(got) == set(want)
    bad = sorted(k for k in want if got[k] != want[k])
    assert not bad, bad
    assert len(want) > 100 and os.path.getsize(G.OUT) < 64 * 1024
