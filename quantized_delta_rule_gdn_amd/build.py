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
SOURCES = [os.path.join(CSRC, f) for f in
           ("damp_api.hip", "step_kernels.hip", "window_kernels.hip", "calib_kernels.hip",
            "stq_kernels.hip", "order_kernels.hip")]

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
    # a variable read before every path has set it is an error (it becomes an address)
    "-Werror=uninitialized",
    "-Werror=sometimes-uninitialized",
    "-Werror=conditional-uninitialized",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# The host layer validates caller data (NaN included), so it keeps IEEE NaN semantics; it holds
# no device arithmetic.
HOST_ONLY = {"damp_api.hip"}


def _compile(src: str, obj: str, extra: list[str]) -> tuple[int, str]:
    flags = [f for f in FLAGS if f != "-shared"]
    if os.path.basename(src) in HOST_ONLY:
        flags = [f for f in flags if f != "-fno-honor-nans"]
    res = subprocess.run([HIPCC, *flags, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
    return res.returncode, res.stdout + res.stderr


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then link."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    noise = "is not a recognized feature for this target"
    with tempfile.TemporaryDirectory(prefix="damp_build_") as tmpd:
        objs = [os.path.join(tmpd, os.path.basename(s) + ".o") for s in SOURCES]
        if verbose:
            print(f"{HIPCC} {' '.join(FLAGS)} -c <each of {len(SOURCES)} sources>", flush=True)
        jobs = min(len(SOURCES), os.cpu_count() or 1, 16)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
        msgs = []
        for (rc, out), src in zip(results, SOURCES):
            lines = [ln for ln in out.splitlines() if noise not in ln]
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(lines))
            msgs.extend(lines)
        if msgs and (verbose or resource_usage):
            print("\n".join(msgs))
        tmp = LIB + ".tmp"
        res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    build_c_callers()
    return LIB


# C programs the tests run against the library (tests/c): one that includes the header as
# pedantic C99 and calls the host-side entry points, one that takes a GPU step through the C ABI
# with the HIP runtime only. Built next to their sources; skipped where gcc or the sources are
# missing.
C_DIR = os.path.join(ROOT, "tests", "c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_callers() -> list[str]:
    import shutil
    if shutil.which("gcc") is None:
        return []
    rpath = "-Wl,-rpath,$ORIGIN/../../quantized_delta_rule_gdn_amd"
    inc = ["-I", os.path.join(ROOT, "include")]
    jobs = [
        ("abi_from_c", ["-std=c99", "-pedantic"], []),
        ("step_from_c", ["-std=gnu11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")],
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]),
    ]
    built = []
    for name, cflags, libs in jobs:
        exe = os.path.join(C_DIR, name)
        if not os.path.exists(os.path.join(C_DIR, name + ".c")):   # a copy without the tests
            continue
        cmd = ["gcc", *cflags, "-Wall", "-Wextra", "-Werror", *inc, os.path.join(C_DIR, name + ".c"),
               "-L", PKG, "-ldamp", *libs, rpath, "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"gcc failed on {name}.c:\n" + res.stdout + res.stderr)
        built.append(exe)
    return built


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv, verbose=True)
