"""Writes tests/golden/input_sha256.json: the SHA-256 of every synthetic
input array of the five workload configurations, as workloads.py generates
them (the byte images of the uint16 / uint32 arrays). The test
tests/test_inputs_pinned.py recomputes them, so a change in numpy's streams
or in the generators cannot move the inputs (and every expected value with
them) unnoticed. Run from the repository root:
    python tests/golden/make_input_sha256.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_sha256.json")


def sha(a) -> str:
    return hashlib.sha256(a.tobytes()).hexdigest()


def layer_digests(prefix, spec, out):
    for key in ("codes", "scale", "sign_k", "sign_n"):
        out["%s.%s" % (prefix, key)] = sha(spec[key])


def input_digests() -> dict:
    out = {"codebook": sha(W.codebook())}
    t = W.TINY
    layer_digests("tiny", W.layer(t["seed"], t["K"], t["N"]), out)
    for M in t["M"]:
        out["tiny.x.M%d" % M] = sha(W.activations(t["seed"], M, t["K"]))
    d = W.DECODE
    for s in range(12):  # the benchmark's rotating sets; the tests use set 0
        layer_digests("decode.set%d" % s, W.layer(d["seed"], d["K"], d["N"], s), out)
    for M in d["M"]:
        out["decode.x.M%d" % M] = sha(W.activations(d["seed"], M, d["K"]))
    p = W.PREFILL
    for g, (K, N) in enumerate(p["geometries"]):
        layer_digests("prefill.g%d" % g, W.layer(p["seed"], K, N, g), out)
        for M in p["M"]:
            out["prefill.g%d.x.M%d" % (g, M)] = sha(W.activations(p["seed"], M, K, g))
    K, N = p["geometries"][0]
    for s in range(2, 12, 2):  # the benchmark's rotating sets 0, 2, .., 10 (set 0 is g0)
        layer_digests("prefill.set%d" % s, W.layer(p["seed"], K, N, s), out)
    w = W.WIDE
    layer_digests("wide", W.layer(w["seed"], w["K"], w["N"]), out)
    out["wide.x.M2048"] = sha(W.activations(w["seed"], 2048, w["K"]))
    lc = W.LOGITS
    wl = W.logits_weights(lc["seed"], lc["w_rows"], lc["K"], threads=8)
    step = W.LOGITS_CHUNK_ROWS
    with ThreadPoolExecutor(8) as ex:  # one digest per generator chunk
        chunks = list(ex.map(lambda r0: sha(wl[r0:r0 + step]), range(0, lc["w_rows"], step)))
    out["logits.w.chunks"] = hashlib.sha256("".join(chunks).encode()).hexdigest()
    for M in lc["M"]:
        out["logits.x.M%d" % M] = sha(W.activations(lc["seed"], M, lc["K"]))
    return out


if __name__ == "__main__":
    d = input_digests()
    with open(OUT, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print("%d digests -> %s" % (len(d), OUT))
