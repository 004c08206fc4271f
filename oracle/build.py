"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/libmxref.so.

Building the checker is not using it: this only produces the shared object that the tests load.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]
SAN_LIB_PATH = os.path.join(HERE, "libmxref_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libmxref.so; with sanitize=True, libmxref_san.so instrumented with AddressSanitizer
    and UndefinedBehaviorSanitizer (loaded by setting MXREF_LIB, with libasan preloaded)."""
    src = os.path.join(HERE, "mxref.c")
    out = SAN_LIB_PATH if sanitize else os.path.join(HERE, "libmxref.so")
    cmd = ["gcc", "-std=c11", "-O1" if sanitize else "-O2", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-shared", "-fPIC",
           *(SANITIZE_FLAGS if sanitize else []), src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
