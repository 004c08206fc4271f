"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/libmxref.so.

Building the checker is not using it: this only produces the shared object that the tests load.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "mxref.c")
    out = os.path.join(HERE, "libmxref.so")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
