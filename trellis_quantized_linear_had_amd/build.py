"""Builds libexl3.so (the product library) and libexl3_measure.so (timing
marks and ceiling probes for benchmarks, linked against libexl3.so) in-tree
with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libexl3.so")
MEASURE_LIB = os.path.join(PKG, "libexl3_measure.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources(sub: str = "csrc") -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, sub, "*.hip")))


def _run(cmd: list[str]) -> subprocess.CompletedProcess:
    return subprocess.run(cmd, capture_output=True, text=True)


def _compile(srcs: list[str], objdir: str, extra_flags: list[str] | None, verbose: bool) -> list[str]:
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in srcs]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    cmds = [[HIPCC, *FLAGS, *(extra_flags or []), *inc, "-c", src, "-o", obj] for src, obj in zip(srcs, objs)]
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(_run, cmds))
    failed = [r for r in results if r.returncode != 0]
    for r in (failed if failed else (results if verbose else [])):
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed: %s" % ", ".join(os.path.basename(c[-3]) for c, r in zip(cmds, results)
                                                       if r.returncode != 0))
    return objs


def _link(objs: list[str], out: str, extra: list[str]) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    res = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *extra, "-o", tmp])
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking %s failed" % out)
    os.replace(tmp, out)


def build(extra_flags: list[str] | None = None, out: str = LIB, verbose: bool = False,
          measure_out: str | None = MEASURE_LIB) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link
    the product library and, unless measure_out is None, the measurement
    library next to it (always recompiles)."""
    objdir = tempfile.mkdtemp(prefix="exl3_build_")
    try:
        srcs = sources("csrc")
        msrcs = sources("measure") if measure_out else []
        objs = _compile(srcs + msrcs, objdir, extra_flags, verbose)
        _link(objs[:len(srcs)], out, [])
        if measure_out:
            # resolved at load time from the directory the measurement library sits in
            _link(objs[len(srcs):], measure_out,
                  ["-L", os.path.dirname(out), "-l:" + os.path.basename(out), "-Wl,-rpath,$ORIGIN"])
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build())
