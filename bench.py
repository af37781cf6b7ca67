#!/usr/bin/env python3
"""Benchmark of the EXL3-style trellis-quantized linear hot path on one MI355X.

One step is one pass of the whole hot path over synthetic inputs of the
pages' shapes, every call through the C ABI on the current stream:
  * four decode-shaped calls of exl3_linear at M = 1, 4, 8, 16 on the
    K5120 x N17408 gate/up geometry (fused decode-GEMM path; the weight set
    rotates through 12 independent sets, 535 MB of packed codes, so the
    256 MB last-level cache cannot serve them);
  * one prefill-shaped call at M = 2048 on the same geometry (input rotation,
    reconstruct to fp16, MFMA GEMM with the output rotation; 6 rotating sets);
  * one padded-logits call at M = 16 (K 5120, 248077 decodable columns padded
    to 248192 inside 248320 weight rows, -inf pad mask, argmax).
All inputs are resident in HBM before the timed region. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import workloads as W

DEC_M = (1, 4, 8, 16)
K, N = 5120, 17408
PREFILL_M = 2048
LOGITS_M = 16
CODE_BYTES = K * N // 2                 # packed 4-bit codes of one layer: 44,564,480 B
PREFILL_FLOP = 2 * PREFILL_M * K * N    # 365,072,220,160
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 skips it)")
    ap.add_argument("--no-logits", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib

    lib = _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    # ------------------------------------------------------------ inputs
    t_setup = time.time()
    cb = W.codebook()
    dec_layers = [X.Layer.from_numpy(W.layer(W.SEED_DECODE, K, N, s), cb) for s in range(12)]
    pre_layers = [X.Layer.from_numpy(W.layer(W.SEED_PREFILL, K, N, 2 * s), cb) for s in range(6)]
    xs = {M: _lib.to_device_u16(W.activations(W.SEED_DECODE, M, K)) for M in DEC_M}
    xp = _lib.to_device_u16(W.activations(W.SEED_PREFILL, PREFILL_M, K, 0))
    ys = {M: torch.empty((M, N), dtype=torch.int16, device=dev) for M in DEC_M}
    yp = torch.empty((PREFILL_M, N), dtype=torch.int16, device=dev)
    dec_scratch = torch.empty(X.linear_scratch_bytes(K, N, max(DEC_M)), dtype=torch.uint8, device=dev)
    pre_scratch = torch.empty(X.linear_scratch_bytes(K, N, PREFILL_M), dtype=torch.uint8, device=dev)
    lc = W.LOGITS
    n_valid, w_rows = lc["n_valid"], lc["w_rows"]
    n_pad = X.logits_padded_width(n_valid, w_rows)
    if not args.no_logits:
        wl = _lib.to_device_u16(W.logits_weights(lc["seed"], w_rows, K, threads=16))
        xl = _lib.to_device_u16(W.activations(lc["seed"], LOGITS_M, K))
        lg = torch.empty((LOGITS_M, n_pad), dtype=torch.int16, device=dev)
        am = torch.empty(LOGITS_M, dtype=torch.int64, device=dev)
        lg_scratch = torch.empty(X.logits_scratch_bytes(LOGITS_M, K, n_valid, w_rows), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("inputs resident in %.1f s" % (time.time() - t_setup))

    def call_linear(layer, x, M, y, scratch):
        _lib.check(lib.exl3_linear(layer.c, x.data_ptr(), M, y.data_ptr(), scratch.data_ptr(), scratch.numel(),
                                   128, sh))

    def call_logits():
        _lib.check(lib.logits_pad_mask_argmax(xl.data_ptr(), LOGITS_M, K, wl.data_ptr(), w_rows, n_valid,
                                              lg.data_ptr(), n_pad, am.data_ptr(), lg_scratch.data_ptr(),
                                              lg_scratch.numel(), sh))

    # Events only at segment boundaries (an event record is itself a timed
    # packet on the stream): [decode x4] [prefill] [logits].
    n_marks = 3 + (0 if args.no_logits else 1)

    def step(i, marks=None):
        if marks:
            marks[0].record(stream)
        for j, M in enumerate(DEC_M):
            call_linear(dec_layers[(len(DEC_M) * i + j) % 12], xs[M], M, ys[M], dec_scratch)
        if marks:
            marks[1].record(stream)
        call_linear(pre_layers[i % 6], xp, PREFILL_M, yp, pre_scratch)
        if marks:
            marks[2].record(stream)
        if not args.no_logits:
            call_logits()
            if marks:
                marks[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(n_marks)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, marks[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed %d steps in %.3f s" % (args.steps, wall))

    parts = np.array([[marks[i][j].elapsed_time(marks[i][j + 1]) for j in range(n_marks - 1)]
                      for i in range(args.steps)])
    mean = parts.mean(axis=0)
    dec_seg_ms = float(mean[0])
    pre_ms = float(mean[1])
    log_ms = None if args.no_logits else float(mean[2])

    # Per-row-count decode time: back-to-back calls between one event pair.
    dec_ms = {}
    for M in DEC_M:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 48
        e0.record(stream)
        for r in range(reps):
            call_linear(dec_layers[r % 12], xs[M], M, ys[M], dec_scratch)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms[M] = e0.elapsed_time(e1) / reps

    value = len(DEC_M) * CODE_BYTES / (dec_seg_ms * 1e-3) / 1e9
    pre_tflops = PREFILL_FLOP / (pre_ms * 1e-3) / 1e12
    logits_bytes = n_pad * K * 2
    rooflines = {
        "decode_m16": {"bound": "hbm", "achieved": CODE_BYTES / (dec_ms[16] * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "us": dec_ms[16] * 1e3,
                       "per_launch": "44564480 B packed codes (K5120 x N17408 x 0.5 B)"},
        "prefill_m2048": {"bound": "mfma", "achieved": pre_tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "us": pre_ms * 1e3, "per_launch": "2*2048*5120*17408 FLOP incl. rotations + reconstruct"},
    }
    if log_ms is not None:
        rooflines["logits_m16"] = {"bound": "hbm", "achieved": logits_bytes / (log_ms * 1e-3) / 1e9,
                                   "peak": HBM_PEAK_GBPS, "unit": "GB/s", "us": log_ms * 1e3,
                                   "per_launch": "%d B fp16 weight rows read (248192 x 5120 x 2)" % logits_bytes}
    for r in rooflines.values():
        r["frac"] = r["achieved"] / r["peak"]
    # the dominant part of the step by GPU time
    times = {"decode_m16": dec_ms[16], "prefill_m2048": pre_ms}
    if log_ms is not None:
        times["logits_m16"] = log_ms
    dom = max(times, key=times.get)
    roof = dict(rooflines[dom])
    roof["kernel"] = dom
    roof["traffic"] = None

    result = {
        "metric": "decode GB/s + us/call at M=1..16; prefill TFLOP/s at M=2048, K5120xN17408",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode K5120xN17408 M=1,4,8,16 (12 rotating weight sets) + prefill K5120xN17408 M=2048 "
                        "(6 rotating sets) + padded logits K5120 n_valid=248077 n_pad=248192 M=16",
            "global_batch": PREFILL_M, "parallelism": "none (1 GPU)",
        },
        "decode_us_per_call": {str(M): round(dec_ms[M] * 1e3, 2) for M in DEC_M},
        "decode_GBps_per_call": {str(M): round(CODE_BYTES / (dec_ms[M] * 1e-3) / 1e9, 1) for M in DEC_M},
        "prefill_us_per_call": round(pre_ms * 1e3, 2),
        "prefill_tflops": round(pre_tflops, 1),
        "logits_us_per_call": None if log_ms is None else round(log_ms * 1e3, 2),
        "roofline": roof,
        "rooflines": rooflines,
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, log)
    print(json.dumps(result), flush=True)


def cpu_baseline(target_s: float, log):
    """The plain fp64 oracle timed on the host cores on a bounded sample of
    the same workload: whole decode calls at M = 16 on the K5120 x N17408
    layer (every weight decoded once per call), repeated until the target
    time is reached."""
    from oracle import oracle as O

    cb = W.codebook()
    L = W.layer(W.SEED_DECODE, K, N, 0)
    x = W.activations(W.SEED_DECODE, 16, K)
    O.lib()
    calls, t0 = 0, time.perf_counter()
    while True:
        O.exl3_linear(x, L, cb)
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 50:
            break
    gbps = calls * CODE_BYTES / el / 1e9
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    log("oracle: %d decode calls in %.2f s" % (calls, el))
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d oracle decode call(s), M=16, K5120xN17408 (89.1M weights decoded per call), %.1f s"
                      % (calls, el)}


if __name__ == "__main__":
    main()
