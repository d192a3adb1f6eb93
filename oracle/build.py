"""Build the CPU oracle library (test infrastructure only).

gcc, -O2, OpenMP, -ffp-contract=off so that no multiply-add is fused, no
fast-math.  The library is written next to this file as libheal_oracle.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "heal_oracle.c")
LIB = os.path.join(HERE, "libheal_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
