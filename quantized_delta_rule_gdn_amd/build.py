"""Build step for libdamp.so (the gfx950 HIP kernels plus the C-ABI host layer).

    python -m quantized_delta_rule_gdn_amd.build [--resource-usage]

Compiles in-tree with hipcc for gfx950 only; the library lands next to this file, where the
Python binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdamp.so")
SOURCES = [os.path.join(CSRC, "damp_api.hip"), os.path.join(CSRC, "step_kernels.hip"),
           os.path.join(CSRC, "calib_kernels.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    # arithmetic exactly as written: explicit fmaf where a fused multiply-add is meant
    "-ffp-contract=off",
    # no NaN inputs are supported: lets fmaxf skip the NaN-quieting canonicalisation
    "-fno-honor-nans",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and (verbose or resource_usage):
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
