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
# reconstruct of the K5120 x N17408 slice: codes read, fp16 W^T written, column
# scales read: 44,564,480 + 178,257,920 + 34,816 B
RECON_BYTES = K * N // 2 + K * N * 2 + N * 2
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
# Secondary roof of the trellis kernels: one random 16-bit codebook read from
# LDS per weight. The gather probe's rate per CU per clock for addresses
# independent across lanes (measured in every run; 9.06 on the last boxes)
# times 256 CUs at the 2.4 GHz peak clock gives the weights per second, and
# 0.5 byte of packed 4-bit codes per weight the GB/s (2.78 TB/s at 9.06).
PEAK_CLOCK_HZ = 2.4e9


def lds_gather_roof_gbps(per_cu_clk: float, bits: int = 4) -> float:
    return per_cu_clk * 256 * PEAK_CLOCK_HZ * bits / 8 / 1e9


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample (0 skips it)")
    ap.add_argument("--no-logits", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--pmc-summary", nargs=3, metavar=("KIND", "FETCH_CSV", "WRITE_CSV"), default=None,
                    help="print the traffic summary (markdown with a JSON block) of two rocprofv3 --pmc "
                         "counter_collection.csv files taken over --pmc-workload KIND")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: time the fused and prefill paths over M on both MLP "
                         "geometries (crossover) and the wide projection, and print a markdown summary")
    ap.add_argument("--sweep-bits", type=int, default=4, choices=range(1, 9), metavar="BITS",
                    help="width of the --sweep layers; other than 4 adds a K5120 x N5120 projection and stops at "
                         "M = 1024")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the bench line: run the library's probes (LDS gathers, MFMA loop, HBM "
                         "streams) and print the measured ceilings")
    ap.add_argument("--bits-sweep", action="store_true",
                    help="instead of the bench line: time decode (M = 1, 16) and prefill (M = 2048) calls and the "
                         "decode and reconstruct kernels at every width 1..8 bits per weight, K5120 x N17408, and "
                         "print a markdown summary")
    ap.add_argument("--head", action="store_true",
                    help="instead of the bench line: time the trellis-quantized output head (the padded-logits "
                         "geometry, 4 and 6 bits per weight) at M = 1, 4, 16, 64 beside the dense fp16 logits "
                         "projection, and print a markdown summary")
    ap.add_argument("--dq-sweep", action="store_true",
                    help="instead of the bench line: time the three kernel sequences of exl3_linear (fused "
                         "decode-GEMM, reconstruct + GEMM, dequant-in-GEMM) over M on both MLP geometries, with the "
                         "main kernel alone, and print a markdown summary")
    ap.add_argument("--pmc-workload", choices=("logits", "gemm", "decode", "reconstruct", "gemm_tail", "dq"),
                    default=None,
                    help="run only a counter-collection workload: two 1 GiB device copies (calibration) then "
                         "three calls of the named path; prints nothing else")
    return ap.parse_args()


def main():
    args = parse()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib, _measure

    if args.pmc_workload:
        pmc_workload(args.pmc_workload)
        return
    if args.sweep:
        print(sweep(args.sweep_bits))
        return
    if args.bits_sweep:
        print(bits_sweep())
        return
    if args.head:
        print(head_sweep())
        return
    if args.dq_sweep:
        print(dq_sweep())
        return
    if args.ceilings:
        c = ceilings()
        print("| ceiling | value |\n|---|---|")
        for k, v in c.items():
            print("| %s | %s |" % (k, "%.4g" % v if isinstance(v, float) else v))
        return

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

    # Per-kernel times: the library's event hook brackets the main kernel of
    # each call on this stream (decode GEMM, full-tile prefill GEMM, logits
    # GEMM); a separate loop after the timed steps, so the hook's event
    # records never sit inside the timed region.
    reps = 12
    kern_us = {}
    kt = _measure.KernelTimer()
    try:
        for M in DEC_M:
            for r in range(reps):
                kt.linear(dec_layers[r % 12], xs[M], M, ys[M], dec_scratch, 128, sh, _measure.DECODE)
            ms, n = kt.read(_measure.DECODE)
            kern_us["decode_gemm_kernel M=%d" % M] = ms / n * 1e3
        for kind, key in ((_measure.GEMM, "gemm_had_kernel<0> M=2048"),
                          (_measure.RECONSTRUCT, "reconstruct_nk_kernel K5120xN17408")):
            for r in range(reps // 2):
                kt.linear(pre_layers[r % 6], xp, PREFILL_M, yp, pre_scratch, 128, sh, kind)
            ms, n = kt.read(kind)
            kern_us[key] = ms / n * 1e3
        if not args.no_logits:
            for r in range(reps // 2):
                kt.logits(xl, LOGITS_M, K, wl, w_rows, n_valid, lg, n_pad, am, lg_scratch, sh)
            ms, n = kt.read(_measure.LOGITS)
            kern_us["logits_kernel M=16"] = ms / n * 1e3
    finally:
        kt.close()
    torch.cuda.synchronize()

    # Algorithmic work per launch: packed codes read by the decode GEMM; 2MNK
    # FLOP over the full-tile launch's 512 of 544 256x256 tiles; fp16 weight
    # rows read by the logits GEMM.
    tiles = (N // 256) * (PREFILL_M // 256)       # 544 output tiles of 256 x 256
    full_tiles = tiles // 256 * 256                 # 512 run at full K; the rest are split along K
    gemm_full_flop = 2 * 256 * 256 * K * full_tiles
    ceil = ceilings(log)
    gather_roof = lds_gather_roof_gbps(ceil["lds_gather_lookups_per_cu_clk"])
    kernels = {}
    for M in DEC_M:
        us = kern_us["decode_gemm_kernel M=%d" % M]
        gbps = CODE_BYTES / (us * 1e-6) / 1e9
        kernels["decode_gemm_kernel M=%d" % M] = {
            "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "us": us, "per_launch": "%d B packed codes (K5120 x N17408 x 0.5 B)" % CODE_BYTES,
            "lds_gather_roof_GBps": gather_roof, "lds_gather_frac": gbps / gather_roof}
    us = kern_us["gemm_had_kernel<0> M=2048"]
    kernels["gemm_had_kernel<0> M=2048"] = {
        "bound": "mfma", "achieved": gemm_full_flop / (us * 1e-6) / 1e12, "peak": MFMA_F16_PEAK_TFLOPS,
        "unit": "TFLOP/s", "us": us, "per_launch": "%d FLOP (2*256*256*5120 x %d full tiles)" % (gemm_full_flop, full_tiles)}
    us = kern_us["reconstruct_nk_kernel K5120xN17408"]
    kernels["reconstruct_nk_kernel K5120xN17408"] = {
        "bound": "hbm", "achieved": RECON_BYTES / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "us": us, "per_launch": "%d B: packed codes read + fp16 W^T written + column scales read" % RECON_BYTES}
    if not args.no_logits:
        us = kern_us["logits_kernel M=16"]
        kernels["logits_kernel M=16"] = {
            "bound": "hbm", "achieved": logits_bytes / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "us": us, "per_launch": "%d B fp16 weight rows read (248192 x 5120 x 2)" % logits_bytes}
    for k, r in kernels.items():
        r["frac"] = r["achieved"] / r["peak"]
        r["traffic"] = stored_traffic(k)
        if k.startswith("decode"):
            r["measured_ceiling"] = {"what": "LDS random-gather probe, GB/s of 4-bit codes",
                                     "value": ceil["lds_gather_GBps_4bit_codes"]}
        elif k.startswith("gemm"):
            r["measured_ceiling"] = {"what": "independent fp16 MFMA loop, TFLOP/s", "value": ceil["mfma_f16_TFLOPs"]}
        elif k.startswith("logits"):
            r["measured_ceiling"] = {"what": "HBM read stream, GB/s", "value": ceil["hbm_read_GBps"]}
        else:  # reconstruct: its reads at the read-stream rate plus its writes at the write-stream rate
            t_ceil = (K * N // 2 + N * 2) / ceil["hbm_read_GBps"] + K * N * 2 / ceil["hbm_write_GBps"]
            r["measured_ceiling"] = {"what": "HBM read + write streams, GB/s for this mix",
                                     "value": RECON_BYTES / t_ceil}
        r["frac_of_measured_ceiling"] = r["achieved"] / r["measured_ceiling"]["value"]
    # the dominant kernel: most GPU time per step (the decode GEMM runs once
    # per row count, the others once)
    step_us = {k: v["us"] for k, v in kernels.items() if not k.startswith("decode")}
    step_us["decode_gemm_kernel"] = sum(kernels["decode_gemm_kernel M=%d" % M]["us"] for M in DEC_M)
    dom = max(step_us, key=step_us.get)
    dom_key = "decode_gemm_kernel M=16" if dom == "decode_gemm_kernel" else dom
    roof = {k: kernels[dom_key][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof["traffic"] = stored_traffic(dom_key)
    roof["kernel"] = dom_key
    roof["us"] = kernels[dom_key]["us"]
    roof["per_launch"] = kernels[dom_key]["per_launch"]

    # The metric's own paths beside the dominant kernel: the decode call and
    # its decode-GEMM kernel (packed 4-bit codes against HBM and against the
    # LDS-gather ceiling), the prefill call (2MKN over the whole call) and its
    # full-tile GEMM launch.
    dec_call_gbps = {M: CODE_BYTES / (dec_ms[M] * 1e-3) / 1e9 for M in DEC_M}
    gk = kernels["gemm_had_kernel<0> M=2048"]
    metric_roofs = {
        "decode_call": {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "achieved": {str(M): round(v, 1) for M, v in dec_call_gbps.items()},
            "frac": {str(M): round(v / HBM_PEAK_GBPS, 4) for M, v in dec_call_gbps.items()},
            "frac_of_lds_gather_probe": {str(M): round(v / ceil["lds_gather_GBps_4bit_codes"], 4)
                                         for M, v in dec_call_gbps.items()},
            "per_call": "%d B packed codes" % CODE_BYTES},
        "decode_kernel": {
            "bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBPS,
            "achieved": {str(M): round(kernels["decode_gemm_kernel M=%d" % M]["achieved"], 1) for M in DEC_M},
            "frac": {str(M): round(kernels["decode_gemm_kernel M=%d" % M]["achieved"] / HBM_PEAK_GBPS, 4)
                     for M in DEC_M},
            "frac_of_lds_gather_probe": {str(M): round(kernels["decode_gemm_kernel M=%d" % M]["achieved"]
                                                       / ceil["lds_gather_GBps_4bit_codes"], 4) for M in DEC_M}},
        "prefill_call": {
            "bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_F16_PEAK_TFLOPS, "achieved": round(pre_tflops, 1),
            "frac": round(pre_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "frac_of_mfma_probe": round(pre_tflops / ceil["mfma_f16_TFLOPs"], 4),
            "per_call": "%d FLOP (2 x 2048 x 5120 x 17408), whole call" % PREFILL_FLOP},
        "prefill_gemm_full_tiles": {
            "bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_F16_PEAK_TFLOPS, "achieved": round(gk["achieved"], 1),
            "frac": round(gk["frac"], 4), "frac_of_mfma_probe": round(gk["frac_of_measured_ceiling"], 4),
            "us": round(gk["us"], 2), "per_launch": gk["per_launch"]},
    }

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
        "metric_rooflines": metric_roofs,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "ceilings": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in ceil.items()},
        "cpu_baseline": None,
    }

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, log)
    print(json.dumps(result), flush=True)


COPY_BYTES = 1 << 30
DQ_PMC_M = 256
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "trellis_quantized_linear_had_amd", "csrc")
# kernel name in the counter files, the key used in the bench line, and the
# sources whose change makes a stored traffic figure stale
PMC_KERNELS = {
    "logits": ("exl3::logits_kernel", "logits_kernel M=16", ("logits.hip", "common.h")),
    "gemm": ("exl3::gemm_had_kernel<0>", "gemm_had_kernel<0> M=2048", ("gemm_f16.hip", "epilogue.h", "common.h")),
    "decode": ("exl3::decode_gemm_kernel<6, true, 1, 4>", "decode_gemm_kernel M=16",
               ("decode_gemm.hip", "decode_plan.h", "trellis.h", "common.h")),
    "reconstruct": ("exl3::reconstruct_nk_kernel<4>", "reconstruct_nk_kernel K5120xN17408",
                    ("reconstruct.hip", "trellis.h", "common.h")),
    # the down-projection geometry, where all 160 tiles run as stream-K pieces
    "gemm_tail": ("exl3::gemm_had_kernel<1>", "gemm_had_kernel<1> K17408xN5120 M=2048",
                  ("gemm_f16.hip", "epilogue.h", "common.h")),
    # the eight-wave dequant-GEMM at M = 256 (the dispatch's choice there): 68 units of 256 rows x 256
    # columns, each split in three k pieces
    "dq": ("exl3::dqgemm2_kernel<16, true>", "dqgemm2_kernel<16,true> K5120xN17408 M=256",
           ("dqgemm.hip", "dq_plan.h", "epilogue.h", "trellis.h", "common.h")),
}


def sources_sha256(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def pmc_summary(kind: str, fetch_csv: str, write_csv: str) -> str:
    """Per-dispatch HBM traffic of one kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    workload's 1 GiB device copy (COPY_BYTES read and written)."""
    import csv

    kname, key, srcs = PMC_KERNELS[kind]

    def per_kernel(path):
        out = {}
        for r in sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"])):
            out.setdefault(r["Kernel_Name"].split("(")[0].replace("void ", ""), []).append(float(r["Counter_Value"]))
        return out

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    copy = "__amd_rocclr_copyBuffer"
    # the calibration copies are the workload's first two copy dispatches
    # (host-to-device uploads of the inputs add small ones later)
    fetch[copy], write[copy] = fetch[copy][:2], write[copy][:2]
    f_scale = COPY_BYTES / (sum(fetch[copy]) / len(fetch[copy]) * 1024)
    w_scale = COPY_BYTES / (sum(write[copy]) / len(write[copy]) * 1024)
    f_kib = sum(fetch[kname]) / len(fetch[kname])
    w_kib = sum(write[kname]) / len(write[kname])
    fetch_b, write_b = f_kib * 1024 * f_scale, w_kib * 1024 * w_scale
    rec = {"kernel": key, "source_sha256": sources_sha256(srcs), "fetch_kib_raw": round(f_kib, 1),
           "write_kib_raw": round(w_kib, 1), "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b), "traffic_bytes": round(fetch_b + write_b),
           "dispatches": [len(fetch[kname]), len(write[kname])]}
    lines = ["| counter | copy of 1 GiB (KiB) | scale | `%s` per dispatch (KiB) | scaled bytes |" % kname,
             "|---|---|---|---|---|",
             "| FETCH_SIZE | %.1f | %.5f | %.1f | %d |" % (sum(fetch[copy]) / len(fetch[copy]), f_scale, f_kib, fetch_b),
             "| WRITE_SIZE | %.1f | %.5f | %.1f | %d |" % (sum(write[copy]) / len(write[copy]), w_scale, w_kib, write_b)]
    return "\n".join(lines) + "\n\n```json\n" + json.dumps(rec) + "\n```\n"


def stored_traffic(key: str):
    """HBM bytes per launch of a kernel from its committed counter summary
    (profiles/*traffic*.md), or None if there is none or the kernel's sources
    changed since the counters were taken."""
    import glob
    import re

    kind = next((k for k, v in PMC_KERNELS.items() if v[1] == key), None)
    if kind is None:
        return None
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.md"))):
        for block in re.findall(r"```json\n(.*?)\n```", open(path).read(), re.S):
            rec = json.loads(block)
            if rec.get("kernel") == key and rec.get("source_sha256") == sources_sha256(PMC_KERNELS[kind][2]):
                return rec["traffic_bytes"]
    return None


def pmc_workload(kind: str):
    """Counter-collection workload: a plain 1 GiB device-to-device copy twice
    (reads and writes COPY_BYTES each: the calibration of FETCH_SIZE /
    WRITE_SIZE), then three calls of one path at the bench's shapes."""
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    lib = _lib.lib()
    sh = torch.cuda.current_stream().cuda_stream
    cb = W.codebook()
    if kind == "logits":
        lc = W.LOGITS
        n_valid, w_rows = lc["n_valid"], lc["w_rows"]
        n_pad = X.logits_padded_width(n_valid, w_rows)
        wl = _lib.to_device_u16(W.logits_weights(lc["seed"], w_rows, K, threads=16))
        xl = _lib.to_device_u16(W.activations(lc["seed"], LOGITS_M, K))
        lg = torch.empty((LOGITS_M, n_pad), dtype=torch.int16, device=dev)
        am = torch.empty(LOGITS_M, dtype=torch.int64, device=dev)
        scr = torch.empty(X.logits_scratch_bytes(LOGITS_M, K, n_valid, w_rows), dtype=torch.uint8, device=dev)
        for _ in range(3):
            _lib.check(lib.logits_pad_mask_argmax(xl.data_ptr(), LOGITS_M, K, wl.data_ptr(), w_rows, n_valid,
                                                  lg.data_ptr(), n_pad, am.data_ptr(), scr.data_ptr(), scr.numel(), sh))
    else:
        pre = kind in ("gemm", "reconstruct", "gemm_tail", "dq")  # these run inside the prefill call
        M = DQ_PMC_M if kind == "dq" else PREFILL_M if pre else max(DEC_M)
        Kw, Nw = (N, K) if kind == "gemm_tail" else (K, N)
        layer = X.Layer.from_numpy(W.layer(W.SEED_PREFILL if pre else W.SEED_DECODE, Kw, Nw, 0), cb)
        x = _lib.to_device_u16(W.activations(W.SEED_PREFILL if pre else W.SEED_DECODE, M, Kw, 0))
        y = torch.empty((M, Nw), dtype=torch.int16, device=dev)
        scr = torch.empty(X.linear_scratch_bytes(Kw, Nw, M), dtype=torch.uint8, device=dev)
        for _ in range(3):
            _lib.check(lib.exl3_linear(layer.c, x.data_ptr(), M, y.data_ptr(), scr.data_ptr(), scr.numel(), 128, sh))
    torch.cuda.synchronize()
    print("[bench] pmc workload %s done" % kind, file=sys.stderr, flush=True)


def interleaved_us(calls, reps, rounds=3):
    """Microseconds per call of each entry of `calls` (name -> one(i) that
    enqueues call i): every callable warmed up, then `rounds` rounds that
    time `reps` back-to-back calls of each in turn between one event pair;
    the least of a callable's rounds is its figure, so a clock still ramping
    up (or a neighbour's leftovers in the caches) does not bias whichever
    callable happens to run first."""
    import torch

    for one in calls.values():
        for i in range(2):
            one(i)
    torch.cuda.synchronize()
    best = {}
    for _ in range(rounds):
        for name, one in calls.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                one(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            best[name] = min(best.get(name, us), us)
    return best


def sweep(bits: int = 4) -> str:
    """exl3_linear's kernel sequences over M, each forced through the
    measurement library (decode-GEMM, reconstruct + GEMM and, at 4 bits, the
    dequant-GEMM), beside the default dispatch (threshold 128), 6 rotating
    weight sets per geometry (267 MB of 4-bit codes at the MLP geometries,
    above the 256 MB MALL), back-to-back calls between one event pair per
    cell. At 4 bits: both MLP geometries, then the wide projection K5120 x
    N32768 at M = 2048 (one 32768-column slice) with its scratch bytes. At
    another width: the MLP geometries and a square K5120 x N5120 projection
    (attention-sized), M up to 1024, to locate that width's crossover."""
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib, _measure

    lib = _lib.lib()
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    cb = W.codebook()

    def caller(layers, x, M, y, scr, variant=None):
        def one(i):
            lay = layers[i % len(layers)]
            if variant is None:
                _lib.check(lib.exl3_linear(lay.c, x.data_ptr(), M, y.data_ptr(), scr.data_ptr(), scr.numel(), 128,
                                           sh))
            else:
                _measure.linear_forced(lay, x, M, y, scr, sh, variant)
        return one

    names = {_measure.VARIANT_FUSED: "decode-GEMM", _measure.VARIANT_RECON_GEMM: "reconstruct+GEMM",
             _measure.VARIANT_DEQUANT_GEMM: "dequant-GEMM", _measure.VARIANT_DEQUANT_GEMM8: "dequant-GEMM, 8 waves"}
    variants = [_measure.VARIANT_FUSED, _measure.VARIANT_RECON_GEMM] + (
        [_measure.VARIANT_DEQUANT_GEMM, _measure.VARIANT_DEQUANT_GEMM8] if bits == 4 else [])
    out = ["| geometry | bits | M | " + " | ".join("%s µs" % names[v] for v in variants) +
           " | default dispatch µs | fastest | default TFLOP/s |",
           "|---|---|---|" + "---|" * len(variants) + "---|---|---|"]
    cross = {}
    geoms = ((5120, 17408), (17408, 5120)) if bits == 4 else ((5120, 17408), (17408, 5120), (5120, 5120))
    Ms = (16, 32, 33, 48, 64, 96, 128, 192, 256, 384, 512, 1024, 2048, 4096) if bits == 4 else (
        16, 32, 64, 96, 128, 192, 256, 512, 1024)
    for gi, (Kg, Ng) in enumerate(geoms):
        layers = [X.Layer.from_numpy(W.layer(W.SEED_PREFILL, Kg, Ng, 2 * s + gi, bits), cb) for s in range(6)]
        for M in Ms:
            x = _lib.to_device_u16(W.activations(W.SEED_PREFILL, M, Kg, gi))
            y = torch.empty((M, Ng), dtype=torch.int16, device=dev)
            need = max([X.linear_scratch_bytes(Kg, Ng, M, 128)] +
                       [_measure.linear_scratch_bytes(Kg, Ng, M, v) for v in variants])
            scr = torch.empty(need, dtype=torch.uint8, device=dev)
            calls = {v: caller(layers, x, M, y, scr, v) for v in variants
                     if not (v == _measure.VARIANT_FUSED and M > 1024)}
            calls["default"] = caller(layers, x, M, y, scr)
            t = interleaved_us(calls, 6)
            dflt = t.pop("default")
            fastest = min(t, key=t.get)
            if (_measure.VARIANT_FUSED in t and t[_measure.VARIANT_RECON_GEMM] < t[_measure.VARIANT_FUSED]
                    and (Kg, Ng) not in cross):
                cross[(Kg, Ng)] = M
            out.append("| K%d×N%d | %d | %d | %s | %.1f | %s | %.1f |" % (
                Kg, Ng, bits, M, " | ".join("%.1f" % t[v] if v in t else "—" for v in variants), dflt,
                names[fastest], 2 * M * Kg * Ng / dflt / 1e6))
            print("[bench] sweep K%d N%d M%d done" % (Kg, Ng, M), file=sys.stderr, flush=True)
            del x, y, scr
        del layers
        torch.cuda.empty_cache()
    lines = ["\n".join(out), ""]
    if bits == 4:
        # context: the vendor library's fp16 GEMM alone (torch.matmul, fp32
        # accumulation) at the same shapes, with W^T as the N x K operand the
        # prefill GEMM reads; no rotations, no reconstruct
        lines.append("| library GEMM alone (torch.matmul fp16) | M | µs | TFLOP/s |")
        lines.append("|---|---|---|---|")
        for Kg, Ng in geoms:
            wt = (0.05 * torch.randn(Ng, Kg, device=dev)).half()
            for M in (2048, 4096):
                xa = (0.05 * torch.randn(M, Kg, device=dev)).half()
                for _ in range(3):
                    xa @ wt.t()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(10):
                    xa @ wt.t()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / 10 * 1e3
                lines.append("| K%d×N%d | %d | %.1f | %.1f |" % (Kg, Ng, M, us, 2 * M * Kg * Ng / us / 1e6))
                del xa
            del wt
        lines.append("")
    for (Kg, Ng), M in cross.items():
        lines.append("Crossover K%d×N%d, %d bits: reconstruct + GEMM is faster than the decode-GEMM from M = %d on "
                     "(among the M measured)." % (Kg, Ng, bits, M))
    if bits != 4:
        return "\n".join(lines)
    Kw, Nw, Mw = 5120, 32768, 2048
    layers = [X.Layer.from_numpy(W.layer(W.SEED_WIDE, Kw, Nw, s), cb) for s in range(3)]
    x = _lib.to_device_u16(W.activations(W.SEED_WIDE, Mw, Kw))
    y = torch.empty((Mw, Nw), dtype=torch.int16, device=dev)
    need = X.linear_scratch_bytes(Kw, Nw, Mw)
    scr = torch.empty(need, dtype=torch.uint8, device=dev)
    us = interleaved_us({"default": caller(layers, x, Mw, y, scr)}, 6)["default"]
    lines.append("")
    lines.append("Wide projection K%d×N%d, M = %d (one 32768-column slice): %.1f µs per call, %.1f TFLOP/s; "
                 "scratch %d B (x̃ %d B + fp16 W slice %d B + GEMM-tail partials %d B)" % (
                     Kw, Nw, Mw, us, 2 * Mw * Kw * Nw / us / 1e6, need, Mw * Kw * 2, Kw * Nw * 2,
                     need - Mw * Kw * 2 - Kw * Nw * 2))
    return "\n".join(lines)


def ceilings(log=None) -> dict:
    """Measured ceilings on this GPU, from the library's probes: random 16-bit
    LDS reads (the trellis codebook gathers), independent fp16 MFMAs (the
    prefill GEMM's instruction, on operands that change every iteration) for
    about 40 ms so the clock settles, and HBM streams: 1 GiB read flat, 2.5 GiB
    read in the padded-logits row pattern (the read ceiling is the faster of
    the two), 1 GiB written, and a 1 GiB device copy through torch.
    Each is the best of three runs; the compute probes also report the shader
    clock their loops ran at (s_memtime cycles over s_memrealtime time)."""
    import torch

    from trellis_quantized_linear_had_amd import _measure

    lib = _measure.mlib()
    sh = torch.cuda.current_stream().cuda_stream
    dev = torch.device("cuda:0")
    sink = torch.empty(_measure.PROBE_SINK_BYTES, dtype=torch.uint8, device=dev)
    clocks = torch.zeros(4 * _measure.PROBE_WORKGROUPS, dtype=torch.int64, device=dev)

    def timed(fn, reps=3):
        best, best_clk = None, None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            _measure.check(fn())
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = clocks.cpu().numpy().view(np.uint64).reshape(-1, 4).astype(np.float64)
            cyc = c[:, 1] - c[:, 0]
            ghz = float(np.mean(cyc / ((c[:, 3] - c[:, 2]) / 100e6)) / 1e9) if np.all(c[:, 3] > c[:, 2]) else None
            if best is None or ms < best:
                best, best_clk = ms, (float(np.mean(cyc)), ghz)
        return best, best_clk

    out = {}
    it = 4000
    ms, (cyc, ghz) = timed(lambda: lib.exl3m_probe_lds_gather(it, sink.data_ptr(), clocks.data_ptr(), sh))
    per_wg = 1024 * 16 * it
    out["lds_gather_lookups_per_cu_clk"] = per_wg / cyc
    out["lds_gather_clock_GHz"] = ghz
    out["lds_gather_lookups_per_s"] = _measure.PROBE_WORKGROUPS * per_wg / (ms * 1e-3)
    out["lds_gather_GBps_4bit_codes"] = out["lds_gather_lookups_per_s"] * 0.5 / 1e9
    it = 100000
    ms, (cyc, ghz) = timed(lambda: lib.exl3m_probe_mfma(it, sink.data_ptr(), clocks.data_ptr(), sh))
    out["mfma_f16_TFLOPs"] = _measure.PROBE_WORKGROUPS * 8 * 8 * it * 32768 / (ms * 1e-3) / 1e12
    out["mfma_clock_GHz"] = ghz
    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf2 = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _measure.check(lib.exl3m_probe_stream(1, 0, buf.data_ptr(), nbytes, sink.data_ptr(), sh))
    ms, _ = timed(lambda: lib.exl3m_probe_stream(0, buf.data_ptr(), 0, nbytes, sink.data_ptr(), sh))
    out["hbm_read_flat_GBps"] = nbytes / (ms * 1e-3) / 1e9
    # row pattern over 2048 waves of 128 rows of 10240 bytes (2.5 GiB): two
    # 4-wave workgroups per CU, all resident at once
    rbytes = 2048 * 128 * 10240
    rows = torch.empty(rbytes, dtype=torch.uint8, device=dev)
    _measure.check(lib.exl3m_probe_stream(1, 0, rows.data_ptr(), rbytes, sink.data_ptr(), sh))
    used = rbytes // (10240 * 128) * (10240 * 128)
    ms, _ = timed(lambda: lib.exl3m_probe_stream(2, rows.data_ptr(), 0, rbytes, sink.data_ptr(), sh))
    out["hbm_read_rows_GBps"] = used / (ms * 1e-3) / 1e9
    out["hbm_read_GBps"] = max(out["hbm_read_flat_GBps"], out["hbm_read_rows_GBps"])
    del rows
    ms, _ = timed(lambda: lib.exl3m_probe_stream(1, 0, buf.data_ptr(), nbytes, sink.data_ptr(), sh))
    out["hbm_write_GBps"] = nbytes / (ms * 1e-3) / 1e9
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        buf2.copy_(buf)
        e1.record()
        torch.cuda.synchronize()
        best = min(best or 1e30, e0.elapsed_time(e1))
    out["hbm_copy_GBps"] = 2 * nbytes / (best * 1e-3) / 1e9
    del buf, buf2, sink, clocks
    torch.cuda.empty_cache()
    if log:
        log("ceilings measured")
    return out


def dq_sweep() -> str:
    """exl3_linear's kernel sequences forced at the same shapes: the fused
    decode-GEMM, reconstruct + GEMM, and both dequant-in-GEMM kernels (four
    waves of 1..8 row fragments, eight waves of 256-row passes), over M on
    both MLP geometries (6 rotating 4-bit weight sets, 267 MB of codes);
    whole calls back to back between one event pair, and each dequant-GEMM
    kernel alone (event pairs around its launches)."""
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib, _measure

    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    cb = W.codebook()
    out = ["| geometry | M | fused µs | reconstruct+GEMM µs | dequant-GEMM µs | same, whole units µs | its kernels µs | "
           "8-wave dequant-GEMM µs | its kernels µs | best dequant call TFLOP/s | best kernels GB/s of codes |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    kt = _measure.KernelTimer(pairs=512, per_call=4)
    for g, (k, n) in enumerate(((5120, 17408), (17408, 5120))):
        layers = [X.Layer.from_numpy(W.layer(W.SEED_PREFILL, k, n, 2 * s), cb) for s in range(6)]
        for M in (16, 32, 33, 48, 64, 96, 128, 192, 256, 384, 512, 1024, 2048):
            x = _lib.to_device_u16(W.activations(W.SEED_PREFILL, M, k, g))
            y = torch.empty((M, n), dtype=torch.int16, device=dev)
            scr = torch.empty(max(_measure.linear_scratch_bytes(k, n, M, v) for v in (1, 2, 3, 4, 5)),
                              dtype=torch.uint8, device=dev)
            def forced(var):
                return lambda i: kt.linear_variant(layers[i % 6], x, M, y, scr, sh, var)
            vs = [v for v in (_measure.VARIANT_FUSED, _measure.VARIANT_RECON_GEMM, _measure.VARIANT_DEQUANT_GEMM,
                              _measure.VARIANT_DEQUANT_WHOLE, _measure.VARIANT_DEQUANT_GEMM8)
                  if not (v == _measure.VARIANT_FUSED and M > 256)]
            row = interleaved_us({v: forced(v) for v in vs}, 12 if M <= 256 else 6)
            row.setdefault(_measure.VARIANT_FUSED, None)
            kus = {}
            for v in (_measure.VARIANT_DEQUANT_GEMM, _measure.VARIANT_DEQUANT_GEMM8):
                for i in range(6):
                    kt.linear(layers[i % 6], x, M, y, scr, 128, sh, _measure.DECODE, v)
                ms, cnt = kt.read(_measure.DECODE)
                kus[v] = ms / cnt * 1e3
            best = min((_measure.VARIANT_DEQUANT_GEMM, _measure.VARIANT_DEQUANT_GEMM8), key=lambda v: row[v])
            out.append("| K%dxN%d | %d | %s | %.1f | %.1f | %.1f | %.1f | %.1f | %.1f | %.0f | %.0f |" % (
                k, n, M, "—" if row[_measure.VARIANT_FUSED] is None else "%.1f" % row[_measure.VARIANT_FUSED],
                row[_measure.VARIANT_RECON_GEMM], row[_measure.VARIANT_DEQUANT_GEMM],
                row[_measure.VARIANT_DEQUANT_WHOLE], kus[_measure.VARIANT_DEQUANT_GEMM],
                row[_measure.VARIANT_DEQUANT_GEMM8], kus[_measure.VARIANT_DEQUANT_GEMM8],
                2 * M * k * n / row[best] / 1e6, k * n / 2 / kus[best] / 1e3))
            print("[bench] dq-sweep K%d N%d M=%d done" % (k, n, M), file=sys.stderr, flush=True)
            del x, y, scr
        del layers
        torch.cuda.empty_cache()
    kt.close()
    return "\n".join(out)


def bits_sweep() -> str:
    """Every width 1..8 at K5120 x N17408: decode calls at M = 1 and 16 and a
    prefill call at M = 2048, each over enough rotating weight sets that their
    codes (K N bits / 8 bytes each) exceed 512 MB, beyond the 256 MB MALL;
    back-to-back calls between one event pair, then the decode and
    reconstruct kernels alone through the library's event hook. Rates use
    the algorithmic bytes of the width: packed codes for decode; codes +
    fp16 W^T + scales for reconstruct."""
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib, _measure

    lib = _lib.lib()
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    cb = W.codebook()
    gather_clk = ceilings()["lds_gather_lookups_per_cu_clk"]

    def time_calls(layers, x, M, y, scr, reps):
        def one(i):
            _lib.check(lib.exl3_linear(layers[i % len(layers)].c, x.data_ptr(), M, y.data_ptr(), scr.data_ptr(),
                                       scr.numel(), 128, sh))
        for i in range(2):
            one(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            one(i)
        e1.record()
        torch.cuda.synchronize()
        call_us = e0.elapsed_time(e1) / reps * 1e3
        kt = _measure.KernelTimer()
        kern = {}
        try:
            for kind in (_measure.DECODE, _measure.RECONSTRUCT):
                for i in range(reps):
                    kt.linear(layers[i % len(layers)], x, M, y, scr, 128, sh, kind)
                kern[kind] = kt.read(kind)
        finally:
            kt.close()
        kern_us = {k: (ms / n * 1e3 if n else None) for k, (ms, n) in kern.items()}
        return call_us, kern_us

    out = ["| bits | code bytes | decode M=1 µs | GB/s | decode kernel µs | GB/s | of 8 TB/s | of LDS-gather roof | "
           "decode M=16 µs | prefill M=2048 µs | TFLOP/s | reconstruct kernel µs | TB/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for bits in range(1, 9):
        code_bytes = K * N * bits // 8
        nsets = min(48, -(-512 * 2**20 // code_bytes))
        layers = [X.Layer.from_numpy(W.layer(W.SEED_DECODE, K, N, s, bits), cb) for s in range(nsets)]
        row = {}
        for M in (1, 16, PREFILL_M):
            x = _lib.to_device_u16(W.activations(W.SEED_DECODE, M, K))
            y = torch.empty((M, N), dtype=torch.int16, device=dev)
            scr = torch.empty(X.linear_scratch_bytes(K, N, M), dtype=torch.uint8, device=dev)
            row[M] = time_calls(layers, x, M, y, scr, 24 if M < 128 else 6)
            del x, y, scr
        roof = lds_gather_roof_gbps(gather_clk, bits)  # one gather per weight: bits / 8 bytes of codes
        dk = row[1][1][_measure.DECODE]
        rk = row[PREFILL_M][1][_measure.RECONSTRUCT]
        rbytes = K * N * bits // 8 + K * N * 2 + N * 2
        out.append("| %d | %d | %.1f | %.0f | %.1f | %.0f | %.1f %% | %.1f %% | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            bits, code_bytes, row[1][0], code_bytes / row[1][0] / 1e3, dk, code_bytes / dk / 1e3,
            100 * code_bytes / dk / 1e3 / HBM_PEAK_GBPS, 100 * code_bytes / dk / 1e3 / roof, row[16][0],
            row[PREFILL_M][0], PREFILL_FLOP / row[PREFILL_M][0] / 1e6, rk, rbytes / rk / 1e6))
        print("[bench] bits-sweep %d done (%d weight sets)" % (bits, nsets), file=sys.stderr, flush=True)
        del layers
        torch.cuda.empty_cache()
    return "\n".join(out)


def head_sweep() -> str:
    """The output head of the padded-logits geometry (K5120, n_valid 248077
    inside 248320 rows, padded width 248192) held as trellis codes at 4 and 6
    bits per weight: the head call (decode path: decode GEMM over the first
    n_pad columns, output stage, pad mask and argmax) and its decode kernel
    alone, at M = 1, 4, 16, 64, beside the dense fp16 logits projection of
    the same geometry at M = 16. Each code set (636 / 953 MB) exceeds the
    256 MB MALL by itself. Rates use the packed codes of the first n_pad
    columns."""
    import torch

    import trellis_quantized_linear_had_amd as X
    from trellis_quantized_linear_had_amd import _lib, _measure

    lib = _lib.lib()
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    cb = W.codebook()
    gather_clk = ceilings()["lds_gather_lookups_per_cu_clk"]
    lc = W.LOGITS
    n_valid, rows = lc["n_valid"], lc["w_rows"]
    n_pad = X.logits_padded_width(n_valid, rows)
    assert lc["K"] == K

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    out = ["| bits | M | code bytes (n_pad cols) | head call µs | GB/s | decode kernel µs | GB/s | of 8 TB/s | "
           "of LDS-gather roof | output stage + mask + argmax µs |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for bits in (4, 6):
        lay = X.Layer.from_numpy(W.layer(lc["seed"], K, rows, 0, bits), cb)
        code_bytes = K * n_pad * bits // 8
        roof = lds_gather_roof_gbps(gather_clk, bits)
        for M in (1, 4, 16, 64):
            x = _lib.to_device_u16(W.activations(lc["seed"], M, K))
            lg = torch.empty((M, n_pad), dtype=torch.int16, device=dev)
            am = torch.empty(M, dtype=torch.int64, device=dev)
            scr = torch.empty(X.head_scratch_bytes(K, rows, M, n_valid), dtype=torch.uint8, device=dev)

            def call():
                _lib.check(lib.exl3_head_logits_argmax(lay.c, x.data_ptr(), M, n_valid, lg.data_ptr(), n_pad,
                                                       am.data_ptr(), scr.data_ptr(), scr.numel(), 128, sh))
            call_us = timed(call, 20)
            kt = _measure.KernelTimer()
            try:
                for _ in range(20):
                    kt.head(lay, x, M, n_valid, lg, n_pad, am, scr, 128, sh, _measure.DECODE)
                ms, n = kt.read(_measure.DECODE)
            finally:
                kt.close()
            dk = ms / n * 1e3
            out.append("| %d | %d | %d | %.1f | %.0f | %.1f | %.0f | %.1f %% | %.1f %% | %.1f |" % (
                bits, M, code_bytes, call_us, code_bytes / call_us / 1e3, dk, code_bytes / dk / 1e3,
                100 * code_bytes / dk / 1e3 / HBM_PEAK_GBPS, 100 * code_bytes / dk / 1e3 / roof, call_us - dk))
            print("[bench] head bits=%d M=%d done" % (bits, M), file=sys.stderr, flush=True)
            del x, lg, am, scr
        del lay
        torch.cuda.empty_cache()
    # the dense fp16 projection of the same geometry, for comparison
    M = LOGITS_M
    wl = _lib.to_device_u16(W.logits_weights(lc["seed"], rows, K, threads=16))
    x = _lib.to_device_u16(W.activations(lc["seed"], M, K))
    lg = torch.empty((M, n_pad), dtype=torch.int16, device=dev)
    am = torch.empty(M, dtype=torch.int64, device=dev)
    scr = torch.empty(X.logits_scratch_bytes(M, K, n_valid, rows), dtype=torch.uint8, device=dev)

    def dense():
        _lib.check(lib.logits_pad_mask_argmax(x.data_ptr(), M, K, wl.data_ptr(), rows, n_valid, lg.data_ptr(), n_pad,
                                              am.data_ptr(), scr.data_ptr(), scr.numel(), sh))
    dense_us = timed(dense, 20)
    wbytes = n_pad * K * 2
    out.append("")
    out.append("Dense fp16 logits projection, same geometry, M = %d: %.1f µs per call (%d weight bytes, %.0f GB/s)."
               % (M, dense_us, wbytes, wbytes / dense_us / 1e3))
    return "\n".join(out)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s: float, log):
    """The plain fp64 oracle, as it stands, timed on the host cores. The
    headline value: whole decode calls at M = 16 on the K5120 x N17408 layer
    (every weight decoded once per call), repeated for about target_s
    seconds. Beside it, one timing per configuration of the workload (decode
    at each M; both prefill geometries and the wide projection on a labelled
    subset of 16 of the 2048 rows -- the oracle decodes the whole weight once
    per call and then computes each listed row; the padded logits at M = 1
    in full and at M = 16 on 2 of its rows), with the rate on the work
    actually done."""
    from oracle import oracle as O

    cb = W.codebook()
    O.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    per_config = []

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    L = W.layer(W.SEED_DECODE, K, N, 0)
    x16 = W.activations(W.SEED_DECODE, 16, K)
    calls, t0 = 0, time.perf_counter()
    while True:
        O.exl3_linear(x16, L, cb)
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 50:
            break
    gbps = calls * CODE_BYTES / el / 1e9
    log("oracle: %d decode calls in %.2f s" % (calls, el))
    per_config.append({"config": "decode K5120xN17408 M=16", "rows": "all 16", "seconds": round(el / calls, 3),
                       "rate": round(gbps, 4), "unit": "GB/s of packed codes"})
    for M in (1, 4, 8):
        x = W.activations(W.SEED_DECODE, M, K)
        sec = timed(lambda: O.exl3_linear(x, L, cb))
        per_config.append({"config": "decode K5120xN17408 M=%d" % M, "rows": "all %d" % M, "seconds": round(sec, 3),
                           "rate": round(CODE_BYTES / sec / 1e9, 4), "unit": "GB/s of packed codes"})
    rows = np.arange(0, 2048, 128, dtype=np.int64)  # 16 of the 2048 rows, one per 128-row block
    cases = [("prefill K5120xN17408 M=2048", W.PREFILL["seed"], 5120, 17408, (0,)),
             ("prefill K17408xN5120 M=2048", W.PREFILL["seed"], 17408, 5120, (1,)),
             ("wide K5120xN32768 M=2048", W.WIDE["seed"], 5120, 32768, ())]
    for name, seed, k, n, extra in cases:
        Lc = W.layer(seed, k, n, *extra)
        x = W.activations(seed, 2048, k, *extra)
        sec = timed(lambda: O.exl3_linear(x, Lc, cb, rows))
        per_config.append({"config": name, "rows": "16 of 2048 (every 128th)", "seconds": round(sec, 3),
                           "rate": round(2 * len(rows) * k * n / sec / 1e9, 4),
                           "unit": "GFLOP/s on the rows computed (the weight decode included)"})
    lc = W.LOGITS
    wl = W.logits_weights(lc["seed"], lc["w_rows"], lc["K"], threads=threads)
    for M, rws in ((1, None), (16, np.array([0, 15], np.int64))):
        x = W.activations(lc["seed"], M, lc["K"])
        sec = timed(lambda: O.logits(x, wl, lc["n_valid"], rws))
        nr = M if rws is None else len(rws)
        per_config.append({"config": "padded logits K5120 n_valid=248077 M=%d" % M,
                           "rows": "all 1" if rws is None else "2 of 16 (first, last)", "seconds": round(sec, 3),
                           "rate": round(nr * 248192 * lc["K"] * 2 / sec / 1e9, 4),
                           "unit": "GB/s of fp16 weight rows per computed row"})
    del wl
    log("oracle: per-configuration timings done")
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": "%d oracle decode call(s), M=16, K5120xN17408 (89.1M weights decoded per call), %.1f s"
                      % (calls, el),
            "per_config": per_config}


if __name__ == "__main__":
    main()
