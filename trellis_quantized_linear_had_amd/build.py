"""Builds libexl3.so in-tree with hipcc for gfx950."""
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
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd: list[str]) -> subprocess.CompletedProcess:
    return subprocess.run(cmd, capture_output=True, text=True)


def build(extra_flags: list[str] | None = None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc per source, in parallel) and link
    them into one shared library (always recompiles)."""
    objdir = tempfile.mkdtemp(prefix="exl3_build_")
    try:
        srcs = sources()
        objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in srcs]
        cmds = [[HIPCC, *FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
                for src, obj in zip(srcs, objs)]
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, cmds))
        failed = [r for r in results if r.returncode != 0]
        for r in (failed if failed else (results if verbose else [])):
            sys.stderr.write(r.stdout + r.stderr)
        if failed:
            raise RuntimeError("hipcc failed building %s" % out)
        tmp = out + ".tmp%d" % os.getpid()
        res = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("linking %s failed" % out)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build())
