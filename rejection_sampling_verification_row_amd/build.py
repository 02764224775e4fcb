"""Build libspecverify.so in-tree with hipcc for gfx950.

    python -m rejection_sampling_verification_row_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = [os.path.join(CSRC, "sv_kernels.hip"), os.path.join(CSRC, "specverify.cpp")]
HEADERS = [os.path.join(CSRC, "sv_internal.h"), os.path.join(INCLUDE, "specverify.h")]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                       # no implicit fma: kernels agree bit for bit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",   # no packed fp32 math
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def command(out: str = LIB) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, *FLAGS, "-I" + INCLUDE, "-I" + CSRC, *SOURCES,
            "-o", out]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the library (always when force, else only when missing or stale)."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"  # host pass only
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
