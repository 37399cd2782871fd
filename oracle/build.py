"""Build the fp64 CPU oracle library (test infrastructure only).

Compiles ``gdn_oracle.c`` with the host C compiler and OpenMP into
``libgdn_oracle.so`` next to this file.  No fast-math: the oracle keeps IEEE
fp64 semantics and a fixed operation order, so its results do not depend on
the build.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
