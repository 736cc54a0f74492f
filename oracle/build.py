"""Build the fp64 CPU oracle (test infrastructure) with plain gcc.

Run as ``python oracle/build.py``; ``__graft_entry__.build()`` calls ``build()``.
No fast-math and no FMA contraction, so every double operation in oracle.c is
one IEEE operation in the order written.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
