"""Build libep.so (the HIP kernels and the C ABI of include/ep.h) for gfx950.

Usage: python -m combine_get_layout_amd.build   (or build() from Python)

Every HIP source is compiled with hipcc for gfx950 only. Packed fp32 vector
instructions are switched off (-packed-fp32-ops); fp32 denormals are kept
(hipcc's default); floating-point contraction is off so the only fused
multiply-adds are the explicit ones.

EP_HIPCC_DEFINES (environment, optional) adds preprocessor definitions, e.g.
EP_HIPCC_DEFINES="-DEP_DSP_PERSIST=2", to build one of the measured kernel
alternatives that the sources keep behind compile-time switches (the
default build uses none).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libep.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "layout.hip", "dispatch.hip", "hier.hip", "combine.hip", "combine2.hip",
           "source.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # -Wno-pass-failed: two `#pragma unroll` loops over top-k lanes are not
    # fully unrolled in one instantiation each (the lane count known only at
    # run time; 16 lanes in the expand kernel). The compiler reports that as a
    # warning; the code is the same either way and uses no scratch.
    "-Wall", "-Wno-unused-result", "-Wno-pass-failed", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _defines() -> list:
    extra = os.environ.get("EP_HIPCC_DEFINES", "").split()
    bad = [d for d in extra if not d.startswith("-D")]
    if bad:
        raise ValueError(f"EP_HIPCC_DEFINES takes -DNAME[=VALUE] items only: {bad}")
    return extra


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *_defines(), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libep.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
