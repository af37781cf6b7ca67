"""Builds libexl3.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libexl3.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(extra_flags: list[str] | None = None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source into one shared library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building %s" % out)
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
