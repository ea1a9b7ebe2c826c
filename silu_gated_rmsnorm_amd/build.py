"""Build ``libgated_rmsnorm.so`` in-tree with hipcc for gfx950.

Usage: ``python -m silu_gated_rmsnorm_amd.build`` (or ``build_library()``).
"""
from __future__ import annotations

import os
import pathlib
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_NAME = "libgated_rmsnorm.so"
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all device code; hipcc's host
# pass prints a harmless warning that it does not know the feature.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(str(p) for p in CSRC.glob("*.hip"))


def build_library(verbose: bool = False) -> pathlib.Path:
    hipcc = os.environ.get("HIPCC", "hipcc")
    out = PKG / LIB_NAME
    tmp = out.with_name(LIB_NAME + ".tmp")
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *sources(),
           "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-q" not in sys.argv))
