"""Build the native parts of the package, in-tree.

* ``libmxfp.so``      - the HIP library (gfx950 kernels + the C ABI declared in include/mxfp.h),
                        compiled with hipcc.
* ``synth/libmxsynth.so`` - the seeded input generator (plain C, gcc, OpenMP).

Every call compiles from source (no staleness check): the build is a few seconds per file.
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libmxfp.so")
SYNTH_PATH = os.path.join(PKG, "synth", "libmxsynth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Device code flags.  -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU
# instructions; the host pass does not know the feature and warns, which is harmless.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_synth(verbose: bool = False) -> str:
    src = os.path.join(PKG, "synth", "synth.c")
    _run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
          src, "-o", SYNTH_PATH + ".tmp", "-lm"], verbose)
    os.replace(SYNTH_PATH + ".tmp", SYNTH_PATH)
    return SYNTH_PATH


def build_hip(verbose: bool = False, jobs: int = 8) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [HIPCC, *HIP_FLAGS, *inc, "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd)))
        if len(procs) >= jobs:
            s0, p0 = procs.pop(0)
            if p0.wait():
                raise RuntimeError(f"hipcc failed on {s0}")
    for s0, p0 in procs:
        if p0.wait():
            raise RuntimeError(f"hipcc failed on {s0}")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB_PATH + ".tmp"],
         verbose)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def build(verbose: bool = False) -> None:
    build_synth(verbose)
    build_hip(verbose)


if __name__ == "__main__":
    build(verbose=True)
