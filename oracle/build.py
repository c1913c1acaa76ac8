"""Build the float64 CPU oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure only; see the header of oracle.c.  Compiled for the
generic x86-64 baseline (no -march=native) so the library built in one
container runs on any x86-64 host.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-fPIC", "-shared",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
