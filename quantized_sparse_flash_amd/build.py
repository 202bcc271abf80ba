"""Build libqsa.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python -m quantized_sparse_flash_amd.build

compiles every ``csrc/*.hip`` with hipcc for gfx950 into one shared library
next to this file.  Packed fp32 VALU instructions are disabled for the
device code (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_PATH = os.path.join(PKG_DIR, "libqsa.so")
ARCH = os.environ.get("QSA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqsa)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile libqsa.so for gfx950; always recompiles.  Returns its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # no NaN inputs are supported (scores, codes and scales are finite),
           # so max/min need no NaN canonicalisation; infinities are still used
           "-fno-honor-nans",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
