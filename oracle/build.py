"""Compile the fp64 CPU oracle (tp_oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: the checker, not part of the product library.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # No -ffast-math: every sum keeps its written order and IEEE semantics.
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-fvisibility=hidden", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
