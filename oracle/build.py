"""Build the float64 CPU oracle (test infrastructure) into oracle/libnorm_oracle.so.

Plain gcc, no fast-math, so every operation keeps IEEE double semantics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "norm_oracle.c")
OUT = os.path.join(HERE, "libnorm_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-std=c11", "-D_GNU_SOURCE", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
