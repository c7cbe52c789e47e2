"""Compile the HIP library libspecverify.so in-tree, for gfx950 only."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "spec_verify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                       # rounding exactly as written
    "-Xarch_device", "-fno-honor-nans",        # logits carry no NaN (documented); drops max canonicalisation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = True, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    # keep only real diagnostics (the host pass does not know the gfx feature flag)
    noise = "packed-fp32-ops"
    warn = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l
                     and "is not a recognized feature for this target" not in l)
    if verbose and warn.strip():
        print(warn)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
