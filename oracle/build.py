"""Builds the oracle's shared library (plain C, gcc, OpenMP) in place.

Test infrastructure: see the header of oracle.c for who may use it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    """Compile oracle.c to liboracle.so next to it and return the path.

    -ffp-contract=off keeps every multiply and add a separately rounded double
    operation, as written; no fast-math.
    """
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
