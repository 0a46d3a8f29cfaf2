"""Compile the oracle's C core (test infrastructure only).

Builds ``oracle/liboracle.so`` from ``oracle/gdn_oracle.c`` with the system gcc,
fp64 throughout, OpenMP across independent (request, value head) units.
No fast-math: the oracle must follow IEEE fp64 semantics.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
