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


SYNTH_SAN_PATH = os.path.join(PKG, "synth", "libmxsynth_san.so")


def build_synth(verbose: bool = False, sanitize: bool = False) -> str:
    """The input generator; sanitize=True builds libmxsynth_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer (selected by MXSYNTH_LIB, with libasan preloaded)."""
    src = os.path.join(PKG, "synth", "synth.c")
    out = SYNTH_SAN_PATH if sanitize else SYNTH_PATH
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"] if sanitize else []
    _run(["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fopenmp", "-ffp-contract=off", "-Wall",
          "-shared", "-fPIC", *san, src, "-o", out + ".tmp", "-lm"], verbose)
    os.replace(out + ".tmp", out)
    return out


VARIANT_DIR = os.path.join(PKG, "variants")


def build_hip(verbose: bool = False, jobs: int = 8, defines=(), variant: str = "") -> str:
    """Compile every HIP source and link libmxfp.so.  With `variant`, the sources are compiled
    with the extra `defines` (compile-time knobs such as MX_RING_PP=0) into
    fp4_block_scaled_amd/variants/libmxfp_<variant>.so instead, which a process loads when the
    environment variable MXFP_LIB names it."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)
    if variant and not variant.replace("_", "").isalnum():
        raise ValueError("variant names are letters, digits and underscores")
    objdir = os.path.join(ROOT, "_build", variant) if variant else os.path.join(ROOT, "_build")
    out = os.path.join(VARIANT_DIR, f"libmxfp_{variant}.so") if variant else LIB_PATH
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    dflags = [f"-D{d}" for d in defines]
    procs, objs = [], []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [HIPCC, *HIP_FLAGS, *dflags, *inc, "-c", s, "-o", o]
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
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> None:
    build_synth(verbose)
    build_hip(verbose)


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build the native libraries")
    ap.add_argument("--variant", default="", help="build variants/libmxfp_<VARIANT>.so with -D knobs")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="KNOB=VALUE")
    a = ap.parse_args()
    if a.variant:
        print(build_hip(verbose=True, defines=a.defines, variant=a.variant))
    else:
        build(verbose=True)
